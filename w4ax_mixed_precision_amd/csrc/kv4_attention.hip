// KV4 decode attention (QoQ/QServe article, section "KV4注意力Kernel优化", and
// section "运行时设计"; COMET article: the KV cache held at 4 bits). Keys and
// values are cached per (head, token) as d unsigned 4-bit codes with an fp16
// step and an 8-bit zero point beside them, chosen at run time from each
// vector's own range; a decode step attends one query per head over the
// cached tokens.
//
// Cache layout in HBM, per kv head h and token slot t (capacity tcap):
//   codes  [h][t][d/2] bytes, channel 2i in the low nibble of byte i and 2i+1
//          in the high nibble (one 32-bit word = 8 consecutive channels);
//   step   [h][t] fp16 bits, zero [h][t] bytes.
//
// Quantizer: d / 8 lanes per vector, each holding 8 channels (one 16-byte
// load, one 32-bit code store); the range comes from min / max reductions
// over those lanes.
//
// Attention: the page's point is that decode attention is memory bound, so
// dequantization must cost few operations per code. Here a workgroup (4
// waves) takes one kv head, the G <= 2 query heads of it that it serves, and a
// chunk of 256 to 1024 cached tokens; d / CPL lanes share a token, each
// reading CPL codes (16 bytes for d >= 32), so a wave load covers contiguous
// cache rows. The zero point comes out of both products as a whole: the key
// product is s (q.u - z sum(q)) and the value sum is
// sum p s u - sum p s z, so a code costs a byte-to-float conversion (shared by
// the G queries) and one multiply-add per query. The chunk keeps its own
// maximum and sum, and a second kernel combines the chunks (the split-softmax
// identity: out = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c).
// Grouped-query heads at d = 128 take a matrix-instruction form instead
// (kv4_attn_mfma_kernel below), which converts each code once for all the
// query heads of its kv head.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "kv4_internal.h"

namespace comet {
namespace {

constexpr int kKvThreads = 256;   // 4 waves
constexpr int kKvChunkMax = 1024; // cached tokens per attention workgroup, at most
// Smallest query-head group on the matrix-instruction kernel: with one query
// head per kv head the 16-row tile is 15/16 empty and the vector kernel is
// faster (LLaMA-7B multi-head decode shape: 94-98 against 78-82 us).
constexpr int kKvMfmaMinGroup = 2;


__device__ __forceinline__ void unpack8(uint4 p, float* x) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
        x[2 * i + 1] = h2f(static_cast<uint16_t>(w[i] >> 16));
    }
}

// The value of lane (lane xor O): quad permutes for 1 and 2, a swizzle
// within 32 lanes up to 16, a permute across the halves for 32.
template <int O>
__device__ __forceinline__ float xor_get(float v) {
    const int x = __float_as_int(v);
    if constexpr (O == 1)
        return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));   // quad_perm [1, 0, 3, 2]
    else if constexpr (O == 2)
        return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));   // quad_perm [2, 3, 0, 1]
    else if constexpr (O < 32)
        return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x1F | (O << 10)));     // bitmask mode: lane ^ O
    else
        return __shfl_xor(v, O);
}

template <int O>
__device__ __forceinline__ float xor_add(float v) { return v + xor_get<O>(v); }

// Minimum and maximum over aligned groups of n lanes (n a power of two, uniform).
template <int O>
__device__ __forceinline__ void xor_minmax(float& lo, float& hi) {
    lo = fminf(lo, xor_get<O>(lo));
    hi = fmaxf(hi, xor_get<O>(hi));
}
__device__ __forceinline__ void group_minmax(float& lo, float& hi, int n) {
    if (n > 1) xor_minmax<1>(lo, hi);
    if (n > 2) xor_minmax<2>(lo, hi);
    if (n > 4) xor_minmax<4>(lo, hi);
    if (n > 8) xor_minmax<8>(lo, hi);
    if (n > 16) xor_minmax<16>(lo, hi);
    if (n > 32) xor_minmax<32>(lo, hi);
}

// Cache quantizer: d / 8 lanes per vector (8 channels each, one 16-byte
// load), 64 / (d / 8) vectors per wave; the range by a min / max reduction
// over the vector's lanes.
__global__ __launch_bounds__(kKvThreads) void kv4_quant_kernel(const uint16_t* __restrict__ X, int nvec, int H,
                                                               int d, int ldx, int pos, int tcap,
                                                               uint8_t* __restrict__ codes,
                                                               uint16_t* __restrict__ step,
                                                               uint8_t* __restrict__ zero) {
    const int lane = threadIdx.x & 63;
    const int D = d >> 3;                                // lanes (32-bit code words) per vector
    const int vpw = 64 / D;                              // vectors per wave
    const int first = (blockIdx.x * (kKvThreads / 64) + (threadIdx.x >> 6)) * vpw;
    if (first >= nvec) return;                           // whole wave
    const int v = first + lane / D;
    const int j = lane & (D - 1);
    const bool act = v < nvec;                           // whole groups of D lanes
    const int tok = act ? v / H : 0, h = act ? v - tok * H : 0;
    float x[8];
    if (act) {
        unpack8(*reinterpret_cast<const uint4*>(X + static_cast<size_t>(tok) * ldx + static_cast<size_t>(h) * d +
                                                8 * j),
                x);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = 0.0f;
    }
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        lo = fminf(lo, x[c]);
        hi = fmaxf(hi, x[c]);
    }
    group_minmax(lo, hi, D);
    if (!act) return;
    const size_t slot = static_cast<size_t>(h) * tcap + pos + tok;
    uint32_t word = 0;
    uint16_t s16 = 0;
    int z = 0;
    if (lo != hi) {
        const float dd = hi - lo;
        const float inv = 15.0f / dd;
        s16 = __half_as_ushort(__float2half_rn(opaque(dd / 15.0f)));
        if (s16 == 0) s16 = 1;                           // smallest fp16 subnormal
        z = static_cast<int>(rintf(-lo * inv));
        z = z < 0 ? 0 : (z > 15 ? 15 : z);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            int u = static_cast<int>(rintf(x[c] * inv)) + z;
            u = u < 0 ? 0 : (u > 15 ? 15 : u);
            word |= static_cast<uint32_t>(u) << (4 * c);
        }
    }
    *reinterpret_cast<uint32_t*>(codes + slot * static_cast<size_t>(d >> 1) + 4 * j) = word;
    if (j == 0) {
        step[slot] = s16;
        zero[slot] = static_cast<uint8_t>(z);
    }
}

// G per-query values reduced over the workgroup (maximum or sum), wave by
// wave and then through LDS; every thread gets the results.
template <int G, bool kMax>
__device__ __forceinline__ void block_reduce(float* v, float (*wred)[4]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float x = __shfl_xor(v[g], o);
            v[g] = kMax ? fmaxf(v[g], x) : v[g] + x;
        }
        if ((threadIdx.x & 63) == 0) wred[g][threadIdx.x >> 6] = v[g];
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g)
        v[g] = kMax ? fmaxf(fmaxf(wred[g][0], wred[g][1]), fmaxf(wred[g][2], wred[g][3]))
                    : (wred[g][0] + wred[g][1]) + (wred[g][2] + wred[g][3]);
    __syncthreads();
}

// CPL / 2 bytes of codes (CPL channels) at p, as 32-bit words.
template <int NW>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* w) {
    if constexpr (NW == 1) {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else if constexpr (NW == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x;
        w[1] = v.y;
    } else {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    }
}

// The CPL codes of NW words as floats: the even channels of a word are its low
// nibbles and the odd channels its high nibbles, so two masks put each in a
// byte of its own and one byte-to-float conversion takes each code.
// (The byte conversions are written out: left to the compiler, the masks let
// it narrow each byte to a 4-bit field extract followed by a conversion.)
template <int B>
__device__ __forceinline__ float ubyte_to_float(uint32_t x) {
    float r;
    if constexpr (B == 0)
        asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (B == 1)
        asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (B == 2)
        asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
    else
        asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

template <int NW>
__device__ __forceinline__ void codes_to_float(const uint32_t* w, float* x) {
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const uint32_t ev = w[k] & 0x0F0F0F0Fu;
        const uint32_t od = (w[k] >> 4) & 0x0F0F0F0Fu;
        x[8 * k + 0] = ubyte_to_float<0>(ev);
        x[8 * k + 1] = ubyte_to_float<0>(od);
        x[8 * k + 2] = ubyte_to_float<1>(ev);
        x[8 * k + 3] = ubyte_to_float<1>(od);
        x[8 * k + 4] = ubyte_to_float<2>(ev);
        x[8 * k + 5] = ubyte_to_float<2>(od);
        x[8 * k + 6] = ubyte_to_float<3>(ev);
        x[8 * k + 7] = ubyte_to_float<3>(od);
    }
}

// Sum over aligned groups of n lanes (n a power of two, uniform).
__device__ __forceinline__ float group_sum(float v, int n) {
    if (n > 1) v = xor_add<1>(v);
    if (n > 2) v = xor_add<2>(v);
    if (n > 4) v = xor_add<4>(v);
    if (n > 8) v = xor_add<8>(v);
    if (n > 16) v = xor_add<16>(v);
    if (n > 32) v = xor_add<32>(v);
    return v;
}

// Sum over the lanes that share lane mod n (n a power of two, uniform).
__device__ __forceinline__ float stride_sum(float v, int n) {
    if (n < 2) v = xor_add<1>(v);
    if (n < 4) v = xor_add<2>(v);
    if (n < 8) v = xor_add<4>(v);
    if (n < 16) v = xor_add<8>(v);
    if (n < 32) v = xor_add<16>(v);
    if (n < 64) v = xor_add<32>(v);
    return v;
}

// 32-channel key slices on fp16 dot products (v_dot2c_f32_f16, FP32 sum):
// a code word's 8 codes become four fp16 pairs of u - z, exact integers in
// [-15, 15] (a byte permute places each code under the fp16 exponent of 1024,
// 0x64NN = 1024 + NN, and a packed fp16 add of -(1024 + z) leaves u - z), in
// the channel order (0, 2), (4, 6), (1, 3), (5, 7) that the query pairs are
// held in. Both operands are normal fp16 numbers (or zero), whose products
// the instruction sums to within about one FP32 rounding; the zero point is
// inside the operand, so no z sum q term cancels afterwards.
typedef _Float16 kv_half2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float fdot2_bits(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(kv_half2, a), __builtin_bit_cast(kv_half2, b), c, false);
}
__device__ __forceinline__ uint32_t pk_add_half2(uint32_t a, uint32_t b) {
    const kv_half2 r = __builtin_bit_cast(kv_half2, a) + __builtin_bit_cast(kv_half2, b);
    return __builtin_bit_cast(uint32_t, r);
}
constexpr uint32_t kCodeBias = 0x64646464u;   // fp16 bits 0x64NN = 1024 + NN for NN < 1024

// Wave priority from progress through the workgroup's two token loops (done
// of total steps): 3 in the first quarter down to 0 in the last. When every
// workgroup of a launch is resident at once (eight per CU), equal priorities
// let the oldest waves win the issue arbitration, so the last-dispatched
// workgroups of each CU fall behind and finish alone; letting the waves that
// are behind go first evens them out (LLaMA-7B decode shape: 64.6 to 59.3
// us). The per-length call, which runs in two rounds, does not use it (45.6
// against 47.1 us with it).
__device__ __forceinline__ void progress_priority(int done, int total) {
    const int lv = (4 * done) / total;
    if (lv == 0)
        __builtin_amdgcn_s_setprio(3);
    else if (lv == 1)
        __builtin_amdgcn_s_setprio(2);
    else if (lv == 2)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// One (kv head, G of its query heads, chunk of 256 tokens). A lane holds CPL
// channels of one token (d / CPL lanes share a token); each code is converted
// once and feeds the G queries, so a grouped-query cache is read once for G
// heads. Partial outputs (unnormalized),
// chunk maxima and sums go to the workspace.
// Tokens of kv head hk: T, or with per-head lengths Tk[hk] clamped to [0, T].
__device__ __forceinline__ int head_tokens(const int* Tk, int hk, int T) {
    return Tk ? imin(imax(Tk[hk], 0), T) : T;
}

template <int CPL, int G, int kDim>              // kDim: d, or 0 for any d
__global__ __launch_bounds__(kKvThreads) void kv4_attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ kz, const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
    const uint8_t* __restrict__ vz, int group, int d, int T, int tcap, float scale, int chunk, int nsplit,
    float* __restrict__ part, float* __restrict__ ml, const int* __restrict__ Tk) {
    constexpr int NW = CPL / 8;                  // 32-bit code words per lane
    // Steps whose loads are issued together: one for 16-byte slices (more
    // steps in flight would hold more registers than the occupancy they cost
    // is worth: LLaMA-7B / -70B decode shapes 81.4 / 87.3 us with one, 83-86 /
    // 103-104 with two, 124 / 131 with four), four for the narrow slices.
    constexpr int U = NW == 4 ? 1 : 4;
    if constexpr (kDim != 0) d = kDim;
    __shared__ float sc[G][kKvChunkMax];
    __shared__ float red[G * 512];
    __shared__ float wred[G][4];
    const int rq = group / G;                    // workgroups per kv head and chunk
    // chunk-major order: consecutive workgroups (which the dispatcher deals
    // round-robin to the XCDs) take the same chunk of different heads, so
    // with per-head lengths the chunks that hold tokens spread over the XCDs
    const int nr = gridDim.x / nsplit;
    const int s = blockIdx.x / nr;
    const int r = blockIdx.x - s * nr;
    const int hk = r / rq;
    const int h0 = hk * group + (r - hk * rq) * G;   // first query head
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D = d / CPL;                       // lanes per token, power of two in [1, 64]
    const int TPW = 64 / D;                      // tokens per wave step
    const int j = lane & (D - 1);                // channel slice of the token
    const int sub = lane / D;                    // token slot within the wave step
    const int t0 = s * chunk;
    const int Th = head_tokens(Tk, hk, T);
    if (t0 >= Th) return;                        // a chunk past this head's tokens (whole workgroup)
    const int nt = imin(chunk, Th - t0);         // >= 1
    const int rb = d >> 1;                       // bytes per cached vector

    // the query: fp16 pairs for the dot products (32-channel slices), else
    // floats and their sum for the zero points
    constexpr bool kDot2 = NW == 4;
    float qf[G][kDot2 ? 1 : CPL], qs[G];
    uint32_t q2[G][kDot2 ? 16 : 1];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint16_t* qg = q + static_cast<size_t>(h0 + g) * d + CPL * j;
        if constexpr (kDot2) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 v = *reinterpret_cast<const uint4*>(qg + 8 * k);
                q2[g][4 * k + 0] = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);   // channels 0, 2
                q2[g][4 * k + 1] = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);   // 4, 6
                q2[g][4 * k + 2] = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);   // 1, 3
                q2[g][4 * k + 3] = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);   // 5, 7
            }
            qs[g] = 0.0f;                        // the zero points are in the code pairs
        } else {
#pragma unroll
            for (int k = 0; k < CPL / 8; ++k) unpack8(*reinterpret_cast<const uint4*>(qg + 8 * k), &qf[g][8 * k]);
            float a = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) a += qf[g][c];
            qs[g] = group_sum(a, D);
        }
    }

    const size_t base = static_cast<size_t>(hk) * tcap + t0;   // slot of the chunk's first token
    const int per_step = 4 * TPW;
    const int niter = (nt + per_step - 1) / per_step;
    const int first = wave * TPW + sub;

    // scores a_t = s_t (q . u_t - z_t sum q) / sqrt(d)
    constexpr bool kPrioForm = NW == 4 && G == 1;   // the form whose launch is one round
    const bool prio = kPrioForm && Tk == nullptr;
    const int ptotal = 2 * ((niter + U - 1) / U);   // steps of the two token loops
    for (int it0 = 0; it0 < niter; it0 += U) {
        if (prio) progress_priority(it0 / U, ptotal);
        uint32_t w[U][NW];
        float st[U];
        int zt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = (it0 + u) * per_step + first;
#pragma unroll
            for (int k = 0; k < NW; ++k) w[u][k] = 0;
            st[u] = 0.0f;
            zt[u] = 0;
            if (i < nt) {
                const size_t sl = base + i;
                load_words<NW>(kc + sl * rb + (CPL / 2) * j, w[u]);
                st[u] = h2f(ks[sl]);
                zt[u] = kz[sl];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = (it0 + u) * per_step + first;
            float dot[G];
#pragma unroll
            for (int g = 0; g < G; ++g) dot[g] = 0.0f;
            if constexpr (kDot2) {
                const uint32_t nz = static_cast<uint32_t>(0xE400 + zt[u]) * 0x00010001u;   // -(1024 + z), twice
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t x = w[u][k] & 0x0F0F0F0Fu, y = (w[u][k] >> 4) & 0x0F0F0F0Fu;
                    const uint32_t c0 = pk_add_half2(__builtin_amdgcn_perm(kCodeBias, x, 0x04010400u), nz);
                    const uint32_t c1 = pk_add_half2(__builtin_amdgcn_perm(kCodeBias, x, 0x04030402u), nz);
                    const uint32_t c2 = pk_add_half2(__builtin_amdgcn_perm(kCodeBias, y, 0x04010400u), nz);
                    const uint32_t c3 = pk_add_half2(__builtin_amdgcn_perm(kCodeBias, y, 0x04030402u), nz);
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        dot[g] = fdot2_bits(c0, q2[g][4 * k + 0], dot[g]);
                        dot[g] = fdot2_bits(c1, q2[g][4 * k + 1], dot[g]);
                        dot[g] = fdot2_bits(c2, q2[g][4 * k + 2], dot[g]);
                        dot[g] = fdot2_bits(c3, q2[g][4 * k + 3], dot[g]);
                    }
                }
            } else {
                float x[CPL];
                codes_to_float<NW>(w[u], x);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
#pragma unroll
                    for (int g = 0; g < G; ++g) dot[g] = fmaf(qf[g][c], x[c], dot[g]);
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) dot[g] = group_sum(dot[g], D);
            if (i < nt && j == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) sc[g][i] = st[u] * (dot[g] - static_cast<float>(zt[u]) * qs[g]) * scale;
            }
        }
    }
    __syncthreads();

    float m[G], l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        for (int i = threadIdx.x; i < nt; i += kKvThreads) m[g] = fmaxf(m[g], sc[g][i]);
    }
    block_reduce<G, true>(m, wred);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = 0.0f;
        for (int i = threadIdx.x; i < nt; i += kKvThreads) {
            const float p = expf(sc[g][i] - m[g]);
            sc[g][i] = p;
            l[g] += p;
        }
    }
    block_reduce<G, false>(l, wred);             // its barriers also publish sc

    // acc = sum_t p_t s_t u_t - sum_t p_t s_t z_t, the second sum once per token
    float acc[G][CPL], wz[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        wz[g] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[g][c] = 0.0f;
    }
    for (int it0 = 0; it0 < niter; it0 += U) {
        if (prio) progress_priority((niter + U - 1) / U + it0 / U, ptotal);
        uint32_t w[U][NW];
        float st[U];
        int zt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = (it0 + u) * per_step + first;
#pragma unroll
            for (int k = 0; k < NW; ++k) w[u][k] = 0;
            st[u] = 0.0f;
            zt[u] = 0;
            if (i < nt) {
                const size_t sl = base + i;
                load_words<NW>(vc + sl * rb + (CPL / 2) * j, w[u]);
                st[u] = h2f(vs[sl]);
                zt[u] = vz[sl];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = (it0 + u) * per_step + first;
            float wt[G];
            const float zf = static_cast<float>(zt[u]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                wt[g] = i < nt ? sc[g][i] * st[u] : 0.0f;
                wz[g] = fmaf(wt[g], zf, wz[g]);
            }
            // one code word (8 channels) at a time: 8 converted codes live
            // instead of CPL (the one-query 32-channel form fits 64 VGPRs,
            // eight waves per SIMD)
#pragma unroll
            for (int k = 0; k < NW; ++k) {
                float x[8];
                codes_to_float<1>(&w[u][k], x);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g][8 * k + c] = fmaf(wt[g], x[c], acc[g][8 * k + c]);
                }
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[g][c] -= wz[g];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[g][c] = stride_sum(acc[g][c], D);
    // waves in turn: ((w0 + w1) + w2) + w3, the same order on every run
    for (int wv = 0; wv < 4; ++wv) {
        if (wave == wv && sub == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int idx = g * d + CPL * j + c;
                    red[idx] = wv == 0 ? acc[g][c] : red[idx] + acc[g][c];
                }
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < G * d; i += kKvThreads) {
        const int g = i / d;
        part[(static_cast<size_t>(h0 + g) * nsplit + s) * d + (i - g * d)] = red[i];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (threadIdx.x == g) {
            const size_t row = static_cast<size_t>(h0 + g) * nsplit + s;
            ml[2 * row] = m[g];
            ml[2 * row + 1] = l[g];
        }
    }
}

// kBase2: the chunk maxima are in base-2 units (the matrix-instruction kernel).
// One workgroup per query head: the weights e^(m_c - M) of its chunks go to
// LDS 128 at a time (M and the sum L over all chunks first, by a workgroup
// reduction), then every thread adds its channels' partial outputs in chunk
// order.
template <bool kBase2>
__global__ __launch_bounds__(128) void kv4_attn_combine_kernel(const float* __restrict__ part,
                                                              const float* __restrict__ ml, int nsplit, int d,
                                                              uint16_t* __restrict__ out, const int* __restrict__ Tk,
                                                              int group, int chunk, int T) {
    __shared__ float fs[128];
    __shared__ float red2[2];
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const float* mh = ml + static_cast<size_t>(h) * nsplit * 2;
    // the chunks that hold this head's tokens (no partials exist past them)
    const int Th = head_tokens(Tk, h / group, T);
    if (Th == 0) {                               // no tokens: the output is zero
        for (int i = tid; i < d; i += 128) out[static_cast<size_t>(h) * d + i] = 0;
        return;
    }
    const int ns = (Th + chunk - 1) / chunk;
    auto ex = [](float x) { return kBase2 ? exp2f(x) : expf(x); };
    float M = -INFINITY;
    for (int s = tid; s < ns; s += 128) M = fmaxf(M, mh[2 * s]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if ((tid & 63) == 0) red2[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(red2[0], red2[1]);
    __syncthreads();
    float L = 0.0f;
    for (int s = tid; s < ns; s += 128) L += ex(mh[2 * s] - M) * mh[2 * s + 1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    if ((tid & 63) == 0) red2[tid >> 6] = L;
    __syncthreads();
    const float invL = 1.0f / (red2[0] + red2[1]);
    const float* ph = part + static_cast<size_t>(h) * nsplit * d;
    for (int i0 = 0; i0 < d; i0 += 128) {
        const int i = i0 + tid;
        float a = 0.0f;
        for (int s0 = 0; s0 < ns; s0 += 128) {
            const int n = imin(128, ns - s0);
            __syncthreads();                 // the previous batch is read
            if (tid < n) fs[tid] = ex(mh[2 * (s0 + tid)] - M);
            __syncthreads();
            if (i < d) {
                int s = 0;
                for (; s + 4 <= n; s += 4) {
                    const float p0 = ph[static_cast<size_t>(s0 + s) * d + i];
                    const float p1 = ph[static_cast<size_t>(s0 + s + 1) * d + i];
                    const float p2 = ph[static_cast<size_t>(s0 + s + 2) * d + i];
                    const float p3 = ph[static_cast<size_t>(s0 + s + 3) * d + i];
                    a += fs[s] * p0;
                    a += fs[s + 1] * p1;
                    a += fs[s + 2] * p2;
                    a += fs[s + 3] * p3;
                }
                for (; s < n; ++s) a += fs[s] * ph[static_cast<size_t>(s0 + s) * d + i];
            }
        }
        if (i < d) out[static_cast<size_t>(h) * d + i] = __half_as_ushort(__float2half_rn(a * invL));
    }
}

// ---------------------------------------------------------------------------
// Grouped-query heads on the matrix unit (d = 128). The vector-unit kernel
// above converts each code once per workgroup and then spends one
// multiply-add per code and query head; with 8 query heads per kv head that
// is most of its time. Here one workgroup takes a kv head, all of its query
// heads (up to GQ, the rows of a 16 x 16 tile past the group held at zero) and
// a chunk of CH tokens, and both products run as 16x16x32 fp16 matrix
// instructions:
//   scores  S[h][t] = s_t sum_c q_hc (u_tc - z_t) / sqrt(d): A = the queries,
//           B = the codes of 16 tokens;
//   values  acc[h][c] = sum_t w_ht (u_tc - z_t), w_ht = p_ht s_t: A = w as two
//           fp16 parts (w = hi + lo to about 2^-22, after scaling by a power of
//           two that puts the chunk's largest step near 2^14, so no weight
//           underflows), B = the codes of 32 tokens.
// Every operand value is exact: q is fp16, u - z an integer in [-15, 15]. A
// code becomes fp16 u - z in about 1.4 operations: one byte permute places
// it under the fp16 exponent of 1024 (0x64NN = 1024 + NN), one packed fp16
// add (two codes) subtracts 1024 + z exactly. The k index of a lane's 8
// operand values is a fixed permutation of the channels (scores) or the 8
// consecutive tokens (values), the same for A and B. For the values, output
// column n of tile j is channel 8 n + j, so a lane reads one 32-bit word (8
// channels) per token and the cache needs no transpose.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr uint32_t kBias64 = 0x64646464u;   // fp16 bits 0x64NN = 1024 + NN for NN < 1024

// (a + b) on packed fp16 pairs: (1024 + u) - (1024 + z), exact.
__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, uint32_t b) {
    const v2h r = __builtin_bit_cast(v2h, a) + __builtin_bit_cast(v2h, b);
    return __builtin_bit_cast(uint32_t, r);
}
// fp16 bits of -(1024 + z) in both halves.
__device__ __forceinline__ uint32_t neg_bias(int z) { return static_cast<uint32_t>(0xE400 + z) * 0x00010001u; }
__device__ __forceinline__ uint32_t neg_bias2(int z0, int z1) {
    return static_cast<uint32_t>(0xE400 + z0) | (static_cast<uint32_t>(0xE400 + z1) << 16);
}
__device__ __forceinline__ v8h as_v8h(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(v8h, v4u{a, b, c, d});
}

// Maximum and sum over the 16 lanes of a row of the wave (lanes 16 g .. 16 g + 15).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, xor_get<1>(v));
    v = fmaxf(v, xor_get<2>(v));
    v = fmaxf(v, xor_get<4>(v));
    return fmaxf(v, xor_get<8>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v = xor_add<1>(v);
    v = xor_add<2>(v);
    v = xor_add<4>(v);
    return xor_add<8>(v);
}

template <int GQ, int CH>
__global__ __launch_bounds__(kKvThreads) void kv4_attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ kz, const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
    const uint8_t* __restrict__ vz, int group, int T, int tcap, float scale, int nsplit,
    float* __restrict__ part, float* __restrict__ ml, const int* __restrict__ Tk) {
    constexpr int D = 128;         // head dimension
    constexpr int RB = D / 2;      // bytes per cached vector
    constexpr int TW = CH / 64;    // 16-token score tiles per wave
    constexpr int SW = CH / 128;   // 32-token value steps per wave
    static_assert(CH % kKvThreads == 0 && (GQ == 8 || GQ == 16), "chunk and query tile");
    __shared__ __attribute__((aligned(16))) _Float16 whi[GQ][CH];   // value weights, two fp16 parts
    __shared__ __attribute__((aligned(16))) _Float16 wlo[GQ][CH];
    __shared__ __attribute__((aligned(16))) float vst[CH];
    __shared__ __attribute__((aligned(16))) uint8_t vzt[CH];
    __shared__ __attribute__((aligned(16))) float red[4][GQ][D];
    __shared__ float wmax[4][16], wsum[4][16], wsmax[4];
    // chunk-major order (see kv4_attn_chunk_kernel)
    const int nhk = gridDim.x / nsplit;
    const int s = blockIdx.x / nhk;
    const int hk = blockIdx.x - s * nhk;
    const int h0 = hk * group;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int t0 = s * CH;
    const int Th = head_tokens(Tk, hk, T);
    if (t0 >= Th) return;                               // past this head's tokens (whole workgroup)
    const int nt = imin(CH, Th - t0);                   // >= 1
    const size_t base = static_cast<size_t>(hk) * tcap + t0;
    // buffer resources over the chunk's nt tokens: loads past them read 0
    const Rsrc rkc = make_rsrc(kc + base * RB, static_cast<uint32_t>(nt) * RB);
    const Rsrc rks = make_rsrc(ks + base, static_cast<uint32_t>(nt) * 2u);
    const Rsrc rkz = make_rsrc(kz + base, static_cast<uint32_t>(nt));
    const Rsrc rvc = make_rsrc(vc + base * RB, static_cast<uint32_t>(nt) * RB);
    const Rsrc rvs = make_rsrc(vs + base, static_cast<uint32_t>(nt) * 2u);
    const Rsrc rvz = make_rsrc(vz + base, static_cast<uint32_t>(nt));

    // Wave priority by phase, 3 for the key loads and scores down to 1 for
    // the value products: all workgroups start together, and the waves that
    // are behind go first instead of the oldest (LLaMA-70B grouped-query
    // decode shape: 28.9 to 26.6 us, its mixed-length batch 27.2 to 24.9)
    __builtin_amdgcn_s_setprio(3);
    // key slices of the wave's score tiles, then value steps and zero points
    // to LDS (their largest step by wave)
    uint4 kw[TW];
    float kst[TW];
    int kzt[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const uint32_t t = static_cast<uint32_t>((wave + 4 * i) * 16 + col);
        kw[i] = buf_load16(rkc, t * RB + 16u * g);
        kst[i] = h2f(__builtin_amdgcn_raw_buffer_load_b16(rks, 2u * t, 0, 0));
        kzt[i] = __builtin_amdgcn_raw_buffer_load_b8(rkz, t, 0, 0);
    }
    float smx = 0.0f;
#pragma unroll
    for (int k = 0; k < CH / kKvThreads; ++k) {
        const uint32_t i = threadIdx.x + k * kKvThreads;
        const float st = h2f(__builtin_amdgcn_raw_buffer_load_b16(rvs, 2u * i, 0, 0));
        vst[i] = st;
        vzt[i] = __builtin_amdgcn_raw_buffer_load_b8(rvz, i, 0, 0);
        smx = fmaxf(smx, st);
    }

    // queries as A operands: row col (query head h0 + col; zero past the
    // group), step kk: channels 32 g + 8 kk + {0, 2, 4, 6, 1, 3, 5, 7}
    v8h qa[4];
    {
        const bool real = col < group;
        const uint16_t* qr = q + static_cast<size_t>(h0 + (real ? col : 0)) * D + 32 * g;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint4 v = real ? *reinterpret_cast<const uint4*>(qr + 8 * kk) : uint4{0u, 0u, 0u, 0u};
            qa[kk] = as_v8h(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                            __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
        }
    }

    // scores: lane (col, g) holds token col of the tile, channels 32 g + 8 kk
    // + {0, 2, 4, 6, 1, 3, 5, 7} of step kk (word kk of its 16-byte slice);
    // the result holds query 4 g + r, token col. Kept in registers (-inf
    // outside the chunk and the group).
    float sr[TW][4];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        const int tile = wave + 4 * i;
        const uint32_t nz = neg_bias(kzt[i]);
        const uint32_t w4[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (tile * 16 < nt) {                            // uniform in the wave
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint32_t x = w4[kk] & 0x0F0F0F0Fu, y = (w4[kk] >> 4) & 0x0F0F0F0Fu;
                const v8h b = as_v8h(pk_add_f16(__builtin_amdgcn_perm(kBias64, x, 0x04010400u), nz),
                                     pk_add_f16(__builtin_amdgcn_perm(kBias64, x, 0x04030402u), nz),
                                     pk_add_f16(__builtin_amdgcn_perm(kBias64, y, 0x04010400u), nz),
                                     pk_add_f16(__builtin_amdgcn_perm(kBias64, y, 0x04030402u), nz));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], b, acc, 0, 0, 0);
            }
        }
        const bool tin = tile * 16 + col < nt;
#pragma unroll
        for (int r = 0; r < 4; ++r) sr[i][r] = (tin && 4 * g + r < group) ? kst[i] * acc[r] * scale : -INFINITY;
    }

    __builtin_amdgcn_s_setprio(2);
    // value words of the wave's steps: lane (col, g) reads word col (channels
    // 8 col .. 8 col + 7) of tokens 8 g + e; issued here, they arrive under
    // the softmax
    uint32_t vw[SW][8];
#pragma unroll
    for (int i = 0; i < SW; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t t = static_cast<uint32_t>((wave + 4 * i) * 32 + 8 * g + e);
            vw[i][e] = __builtin_amdgcn_raw_buffer_load_b32(rvc, t * RB + 4u * col, 0, 0);
        }

    // softmax of the chunk (scores in base-2 units: `scale` holds log2(e) /
    // sqrt(d)): row maxima by wave, then over the waves
    float mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = sr[0][r];
#pragma unroll
        for (int i = 1; i < TW; ++i) v = fmaxf(v, sr[i][r]);
        mr[r] = row16_max(v);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) smx = fmaxf(smx, __shfl_xor(smx, o));
    if (col == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) wmax[wave][4 * g + r] = mr[r];
    }
    if (lane == 0) wsmax[wave] = smx;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * g + r;
        mr[r] = fmaxf(fmaxf(wmax[0][h], wmax[1][h]), fmaxf(wmax[2][h], wmax[3][h]));
    }
    const float smax = fmaxf(fmaxf(wsmax[0], wsmax[1]), fmaxf(wsmax[2], wsmax[3]));
    int ex = 0;
    if (smax > 0.0f) frexpf(smax, &ex);
    const int k2 = 14 - ex;                              // w 2^k2 < 2^14: p <= 1, s < 2^ex
    // p = 2^(score - max) (scores are in base-2 units), and the value weight
    // w = p s 2^k2 as two fp16 parts, once per (query, token); zero past the
    // chunk and the group
    float lr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (4 * g < GQ) {
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int t = (wave + 4 * i) * 16 + col;
            const float sv = ldexpf(vst[t], k2);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool in = t < nt && 4 * g + r < group;
                const float p = in ? exp2f(sr[i][r] - mr[r]) : 0.0f;
                lr[r] += p;
                const float w = p * sv;
                const _Float16 h = static_cast<_Float16>(w);
                whi[4 * g + r][t] = h;
                wlo[4 * g + r][t] = static_cast<_Float16>(w - static_cast<float>(h));
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) lr[r] = row16_sum(lr[r]);
    if (col == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) wsum[wave][4 * g + r] = lr[r];
    }
    __syncthreads();

    __builtin_amdgcn_s_setprio(1);
    // values: lane (col, g) holds tokens 8 g + e of the step (k index e) and
    // channels 8 col + j (column col of tile j)
    v4f acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < SW; ++i) {
        const int tb = (wave + 4 * i) * 32;
        if (tb >= nt) break;                             // uniform in the wave
        const int t8 = tb + 8 * g;
        // A: the weights of query col for tokens t8 .. t8 + 7 (rows past
        // GQ are zero)
        v8h ahi = {}, alo = {};
        if (col < GQ) {
            ahi = *reinterpret_cast<const v8h*>(&whi[col < GQ ? col : 0][t8]);
            alo = *reinterpret_cast<const v8h*>(&wlo[col < GQ ? col : 0][t8]);
        }
        const uint2 zz = *reinterpret_cast<const uint2*>(&vzt[t8]);
        uint32_t nz[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t zw = p < 2 ? zz.x : zz.y;
            const int sh = 16 * (p & 1);
            nz[p] = neg_bias2(static_cast<int>((zw >> sh) & 0xFFu), static_cast<int>((zw >> (sh + 8)) & 0xFFu));
        }
        // token pairs (2p, 2p + 1) interleaved by byte: il[p][0] = low
        // nibbles of bytes 0-1, il[p][1] of bytes 2-3, il[p][2..3] the high nibbles
        uint32_t il[4][4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t xa = vw[i][2 * p] & 0x0F0F0F0Fu, xb = vw[i][2 * p + 1] & 0x0F0F0F0Fu;
            const uint32_t ya = (vw[i][2 * p] >> 4) & 0x0F0F0F0Fu, yb = (vw[i][2 * p + 1] >> 4) & 0x0F0F0F0Fu;
            il[p][0] = __builtin_amdgcn_perm(xb, xa, 0x05010400u);
            il[p][1] = __builtin_amdgcn_perm(xb, xa, 0x07030602u);
            il[p][2] = __builtin_amdgcn_perm(yb, ya, 0x05010400u);
            il[p][3] = __builtin_amdgcn_perm(yb, ya, 0x07030602u);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // channel 8 col + j: nibble j of the word, i.e. byte j / 2, low
            // nibble for even j; bytes 0-1 in il[.][0 | 2], 2-3 in il[.][1 | 3]
            const int src = (j & 1 ? 2 : 0) + (j >= 4 ? 1 : 0);
            const uint32_t sel = (j >> 1) & 1 ? 0x04030402u : 0x04010400u;
            const v8h b = as_v8h(pk_add_f16(__builtin_amdgcn_perm(kBias64, il[0][src], sel), nz[0]),
                                 pk_add_f16(__builtin_amdgcn_perm(kBias64, il[1][src], sel), nz[1]),
                                 pk_add_f16(__builtin_amdgcn_perm(kBias64, il[2][src], sel), nz[2]),
                                 pk_add_f16(__builtin_amdgcn_perm(kBias64, il[3][src], sel), nz[3]));
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, b, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, b, acc[j], 0, 0, 0);
        }
    }
    // the waves' sums in a fixed order ((w0 + w1) + w2) + w3; result: query
    // 4 g + r, channel 8 col + j
    if (4 * g < GQ) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][4 * g + r][8 * col + j] = acc[j][r];
    }
    __syncthreads();
    const float unscale = ldexpf(1.0f, -k2);
    for (int i = threadIdx.x; i < group * D; i += kKvThreads) {
        const int h = i / D, c = i - h * D;
        part[(static_cast<size_t>(h0 + h) * nsplit + s) * D + c] =
            (((red[0][h][c] + red[1][h][c]) + red[2][h][c]) + red[3][h][c]) * unscale;
    }
    if (threadIdx.x < group) {
        const int h = threadIdx.x;
        const size_t row = static_cast<size_t>(h0 + h) * nsplit + s;
        ml[2 * row] = fmaxf(fmaxf(wmax[0][h], wmax[1][h]), fmaxf(wmax[2][h], wmax[3][h]));
        ml[2 * row + 1] = ((wsum[0][h] + wsum[1][h]) + wsum[2][h]) + wsum[3][h];
    }
}

inline int imin_host(int a, int b) { return a < b ? a : b; }
constexpr unsigned kVarlenLdsPad = 17408;   // dynamic LDS of the per-length launch (see launch_kv4_attention)

}  // namespace

int launch_kv4_quantize(const uint16_t* X, int ntok, int H, int d, int ldx, int pos, int tcap, uint8_t* codes,
                        uint16_t* step, uint8_t* zero, void* stream) {
    const int nvec = ntok * H;
    const int per_block = (kKvThreads / 64) * (64 / (d >> 3));   // vectors per workgroup
    kv4_quant_kernel<<<(nvec + per_block - 1) / per_block, kKvThreads, 0, static_cast<hipStream_t>(stream)>>>(
        X, nvec, H, d, ldx, pos, tcap, codes, step, zero);
    return static_cast<int>(hipGetLastError());
}

int launch_kv4_attention(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* kz,
                         const uint8_t* vc, const uint16_t* vs, const uint8_t* vz, int Hq, int group, int d, int T,
                         int tcap, uint16_t* out, float* workspace, void* stream, const int* Tk) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // Grouped-query heads at d = 128: the matrix-instruction kernel, one
    // workgroup per (kv head, chunk) for all the group's query heads; chunks
    // of 512 tokens while that still gives 1024 workgroups (four per CU, one
    // round), else 256 (LLaMA-70B grouped-query shape: 28.5 us with 512,
    // 30.6 with 256, 31 with 1024; its value loads issued with the key loads
    // instead of after the scores: 31-34 us). Never more splits than
    // kv4_splits(T), which sizes the workspace.
    const int Hk = Hq / group;
    if (d == 128 && group >= kKvMfmaMinGroup && group <= 16 && static_cast<int64_t>(tcap) * 64 < (1ll << 31)) {
        const int ch = static_cast<int64_t>(Hk) * ((T + 511) / 512) >= 1024 ? 512 : 256;
        const int ns = (T + ch - 1) / ch;
        float* pt = workspace;
        float* mlp = workspace + static_cast<size_t>(Hq) * ns * d;
        const float sc = 1.4426950408889634f / sqrtf(static_cast<float>(d));   // log2(e) / sqrt(d)
        const int grid = Hk * ns;
        if (group <= 8) {
            if (ch == 512) kv4_attn_mfma_kernel<8, 512><<<grid, kKvThreads, 0, st>>>(q, kc, ks, kz, vc, vs, vz, group, T, tcap, sc, ns, pt, mlp, Tk);
            else kv4_attn_mfma_kernel<8, 256><<<grid, kKvThreads, 0, st>>>(q, kc, ks, kz, vc, vs, vz, group, T, tcap, sc, ns, pt, mlp, Tk);
        } else {
            if (ch == 512) kv4_attn_mfma_kernel<16, 512><<<grid, kKvThreads, 0, st>>>(q, kc, ks, kz, vc, vs, vz, group, T, tcap, sc, ns, pt, mlp, Tk);
            else kv4_attn_mfma_kernel<16, 256><<<grid, kKvThreads, 0, st>>>(q, kc, ks, kz, vc, vs, vz, group, T, tcap, sc, ns, pt, mlp, Tk);
        }
        const int e = static_cast<int>(hipGetLastError());
        if (e != 0) return e;
        kv4_attn_combine_kernel<true><<<Hq, 128, 0, st>>>(pt, mlp, ns, d, out, Tk, group, ch, T);
        return static_cast<int>(hipGetLastError());
    }
    // The vector kernel. Tokens per workgroup: 256, or 512 / 1024 when the
    // grid still has 2048 workgroups (8 per CU), to spread the fixed cost of
    // a chunk (the softmax reductions, the cross-lane sums, the partial
    // outputs) over more tokens. Query heads per workgroup: two when the
    // group allows. The kernel is bound by the vector unit per (query head,
    // code), so sharing the code conversion between two queries pays, while
    // more queries per workgroup need narrower code slices per lane
    // (registers) and more cross-lane sums per score than they save
    // (measured on the LLaMA-70B grouped-query shape: 101.6 us with two,
    // 137.0 with four, 160.7 with eight, 119.5 with one).
    const int G = group % 2 == 0 ? 2 : 1;
    int chunk = kKvChunkMax;
    while (chunk > kKvChunk && static_cast<int64_t>(Hq / G) * ((T + chunk - 1) / chunk) < 2048) chunk >>= 1;
    const int nsplit = (T + chunk - 1) / chunk;
    float* part = workspace;
    float* ml = workspace + static_cast<size_t>(Hq) * nsplit * d;
    const float scale = 1.0f / sqrtf(static_cast<float>(d));
    const int cpl = imin_host(32, d);
    const int grid = (Hq / G) * nsplit;
    // With per-head lengths, chunks past a head's tokens exit at once, and
    // with all workgroups resident in one round (the one-query 32-channel
    // form: 64 VGPRs, eight per CU) each CU keeps the live chunks it was dealt.
    // Reserving LDS so that at most six share a CU (6160 bytes static + this
    // pad = 23568; six take 141 KB of the 160, seven would need 165) leaves a
    // second round that the dispatcher hands out as slots free up (LLaMA-7B
    // decode shape, sequences of 635-3792 tokens: 43.7 against 45.6 us; the
    // uniform call keeps all eight: 61.3 us, against 74.7 for the form with
    // FP32 key products and all codes of a slice converted at once, 87 VGPRs).
    const unsigned pad = (Tk != nullptr && cpl == 32 && G == 1) ? kVarlenLdsPad : 0u;
#define COMET_KV4_CHUNK(C, GG)                                                                                 \
    do {                                                                                                       \
        if (d == 128)                                                                                          \
            kv4_attn_chunk_kernel<C, GG, 128><<<grid, kKvThreads, pad, st>>>(q, kc, ks, kz, vc, vs, vz, group, d, T, \
                                                                          tcap, scale, chunk, nsplit, part, ml, Tk); \
        else                                                                                                   \
            kv4_attn_chunk_kernel<C, GG, 0><<<grid, kKvThreads, pad, st>>>(q, kc, ks, kz, vc, vs, vz, group, d, T,   \
                                                                        tcap, scale, chunk, nsplit, part, ml, Tk); \
    } while (0)
    if (G == 2) {
        if (cpl == 32) COMET_KV4_CHUNK(32, 2); else if (cpl == 16) COMET_KV4_CHUNK(16, 2); else COMET_KV4_CHUNK(8, 2);
    } else {
        if (cpl == 32) COMET_KV4_CHUNK(32, 1); else if (cpl == 16) COMET_KV4_CHUNK(16, 1); else COMET_KV4_CHUNK(8, 1);
    }
#undef COMET_KV4_CHUNK
    const int e = static_cast<int>(hipGetLastError());
    if (e != 0) return e;
    kv4_attn_combine_kernel<false><<<Hq, 128, 0, st>>>(part, ml, nsplit, d, out, Tk, group, chunk, T);
    return static_cast<int>(hipGetLastError());
}

}  // namespace comet
