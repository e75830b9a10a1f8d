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
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "kv4_internal.h"

namespace comet {
namespace {

constexpr int kKvThreads = 256;   // 4 waves
constexpr int kKvChunkMax = 1024; // cached tokens per attention workgroup, at most


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

// One (kv head, G of its query heads, chunk of 256 tokens). A lane holds CPL
// channels of one token (d / CPL lanes share a token); each code is converted
// once and feeds the G queries, so a grouped-query cache is read once for G
// heads. Partial outputs (unnormalized),
// chunk maxima and sums go to the workspace.
template <int CPL, int G, int kDim>              // kDim: d, or 0 for any d
__global__ __launch_bounds__(kKvThreads) void kv4_attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ kz, const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
    const uint8_t* __restrict__ vz, int group, int d, int T, int tcap, float scale, int chunk, int nsplit,
    float* __restrict__ part, float* __restrict__ ml) {
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
    const int s = blockIdx.x % nsplit;
    const int r = blockIdx.x / nsplit;
    const int hk = r / rq;
    const int h0 = hk * group + (r - hk * rq) * G;   // first query head
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D = d / CPL;                       // lanes per token, power of two in [1, 64]
    const int TPW = 64 / D;                      // tokens per wave step
    const int j = lane & (D - 1);                // channel slice of the token
    const int sub = lane / D;                    // token slot within the wave step
    const int t0 = s * chunk;
    const int nt = imin(chunk, T - t0);          // >= 1
    const int rb = d >> 1;                       // bytes per cached vector

    float qf[G][CPL], qs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint16_t* qg = q + static_cast<size_t>(h0 + g) * d + CPL * j;
#pragma unroll
        for (int k = 0; k < CPL / 8; ++k) unpack8(*reinterpret_cast<const uint4*>(qg + 8 * k), &qf[g][8 * k]);
        float a = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) a += qf[g][c];
        qs[g] = group_sum(a, D);
    }

    const size_t base = static_cast<size_t>(hk) * tcap + t0;   // slot of the chunk's first token
    const int per_step = 4 * TPW;
    const int niter = (nt + per_step - 1) / per_step;
    const int first = wave * TPW + sub;

    // scores a_t = s_t (q . u_t - z_t sum q) / sqrt(d)
    for (int it0 = 0; it0 < niter; it0 += U) {
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
            float dot[G], x[CPL];
            codes_to_float<NW>(w[u], x);
#pragma unroll
            for (int g = 0; g < G; ++g) dot[g] = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
#pragma unroll
                for (int g = 0; g < G; ++g) dot[g] = fmaf(qf[g][c], x[c], dot[g]);
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
            float wt[G], x[CPL];
            codes_to_float<NW>(w[u], x);
            const float zf = static_cast<float>(zt[u]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                wt[g] = i < nt ? sc[g][i] * st[u] : 0.0f;
                wz[g] = fmaf(wt[g], zf, wz[g]);
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g][c] = fmaf(wt[g], x[c], acc[g][c]);
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

__global__ __launch_bounds__(128) void kv4_attn_combine_kernel(const float* __restrict__ part,
                                                              const float* __restrict__ ml, int nsplit, int d,
                                                              uint16_t* __restrict__ out) {
    const int h = blockIdx.x;
    const float* mh = ml + static_cast<size_t>(h) * nsplit * 2;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, mh[2 * s]);
    float L = 0.0f;
    for (int s = 0; s < nsplit; ++s) L += expf(mh[2 * s] - M) * mh[2 * s + 1];
    const float invL = 1.0f / L;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        float a = 0.0f;
        for (int s = 0; s < nsplit; ++s)
            a += expf(mh[2 * s] - M) * part[(static_cast<size_t>(h) * nsplit + s) * d + i];
        out[static_cast<size_t>(h) * d + i] = __half_as_ushort(__float2half_rn(a * invL));
    }
}

inline int imin_host(int a, int b) { return a < b ? a : b; }

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
                         int tcap, uint16_t* out, float* workspace, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // Tokens per workgroup: 256, or 512 / 1024 when the grid still has 2048
    // workgroups (8 per CU), to spread the fixed cost of a chunk (the
    // softmax reductions, the cross-lane sums, the partial outputs) over more
    // tokens. Never more splits than kv4_splits(T), which sizes the workspace.
    // Query heads per workgroup: two when the group allows. The kernel is
    // bound by the vector unit per (query head, code), so sharing the code
    // conversion between two queries pays, while more queries per workgroup
    // need narrower code slices per lane (registers) and more cross-lane sums
    // per score than they save (measured on the LLaMA-70B grouped-query
    // shape: 101.6 us with two, 137.0 with four, 160.7 with eight, 119.5 with
    // one).
    const int G = group % 2 == 0 ? 2 : 1;
    int chunk = kKvChunkMax;
    while (chunk > kKvChunk && static_cast<int64_t>(Hq / G) * ((T + chunk - 1) / chunk) < 2048) chunk >>= 1;
    const int nsplit = (T + chunk - 1) / chunk;
    float* part = workspace;
    float* ml = workspace + static_cast<size_t>(Hq) * nsplit * d;
    const float scale = 1.0f / sqrtf(static_cast<float>(d));
    const int cpl = imin_host(32, d);
    const int grid = (Hq / G) * nsplit;
#define COMET_KV4_CHUNK(C, GG)                                                                                 \
    do {                                                                                                       \
        if (d == 128)                                                                                          \
            kv4_attn_chunk_kernel<C, GG, 128><<<grid, kKvThreads, 0, st>>>(q, kc, ks, kz, vc, vs, vz, group, d, T, \
                                                                          tcap, scale, chunk, nsplit, part, ml); \
        else                                                                                                   \
            kv4_attn_chunk_kernel<C, GG, 0><<<grid, kKvThreads, 0, st>>>(q, kc, ks, kz, vc, vs, vz, group, d, T,   \
                                                                        tcap, scale, chunk, nsplit, part, ml);   \
    } while (0)
    if (G == 2) {
        if (cpl == 32) COMET_KV4_CHUNK(32, 2); else if (cpl == 16) COMET_KV4_CHUNK(16, 2); else COMET_KV4_CHUNK(8, 2);
    } else {
        if (cpl == 32) COMET_KV4_CHUNK(32, 1); else if (cpl == 16) COMET_KV4_CHUNK(16, 1); else COMET_KV4_CHUNK(8, 1);
    }
#undef COMET_KV4_CHUNK
    const int e = static_cast<int>(hipGetLastError());
    if (e != 0) return e;
    kv4_attn_combine_kernel<<<Hq, 128, 0, st>>>(part, ml, nsplit, d, out);
    return static_cast<int>(hipGetLastError());
}

}  // namespace comet
