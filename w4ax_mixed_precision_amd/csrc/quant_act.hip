// comet_quant_act: one fused pass over the fp16 activations that gathers the
// permuted channels, takes the absmax of every (token, 128-channel block) and
// writes 4-bit codes for the normal blocks and 8-bit codes for the last nb8
// (outlier) blocks, with one fp32 scale per (token, block).
//
// QUIK blog (deep-paper.org/paper/2310.09259), section "核融合": a single
// kernel reads the input, computes the statistics and quantizes, instead of a
// chain of kernels that each round-trip through memory. COMET article
// (mmssai.com/?p=43269), section "1.离群点分布规律的重定义": 8 bits for the
// outlier-dense blocks, 4 bits for the rest.
//
// Mapping on gfx950. One workgroup (4 wave64s) per token row (or per part of
// a row's blocks when there are few rows). The row is first staged into LDS
// with direct loads (buffer_load ... lds, 1 KB per wave instruction, all in
// flight at once; HBM sees one contiguous read of 2K bytes); the channel
// gather by perm then happens in LDS. A lane owns one 32-channel group of a
// block (positions 32g .. 32g+31), four lanes (one DPP quad) a block, so a
// wave covers 16 blocks per pass; the absmax is two DPP steps inside the quad.
// The perm entries of the next pass are fetched while this one computes. Codes
// leave as whole 16-byte stores:
//   * FP6 layout, 4-bit block: one v_cvt_scalef32_2xpk16_fp6_f32 (scale 1)
//     turns the lane's 32 integer values into its 192-bit FP6 E2M3 string
//     (every integer in [-7, 7] is exact in E2M3); the instruction takes its
//     two 16-value sources interleaved (code 2i from the first, 2i + 1 from
//     the second). Rows are written in the GEMM's 16-row tiles.
//   * INT4 layout, 4-bit block: zero-extended nibbles u = q + 8, byte j of the
//     group holding positions j (low) and 16 + j (high).
//   * 8-bit blocks: int8 codes in position order (FP6 layout: 16-row tiles).
//
// The same kernels optionally fuse the RMS normalization that precedes the
// quantizer in a transformer block (QoQ/QServe article,
// youleyou.com/wenzhang/3078652.html, section "运行时设计": the activation
// quantization of the QKV projection and of the first FFN layer is fused into
// the layer norm before it). The row is already staged once for the gather,
// so the statistic costs one more pass over LDS, and the normalized row never
// goes to memory: xn = fp16((x r) gamma), r = binary32(1 / sqrt(S / K + eps)),
// S the exact sum of squares rounded once to binary64. The squares are summed
// as integers (units of 2^-48) while the row is staged: the wave that loads a
// 512-channel chunk also adds its squares, so each wave's part needs no
// barrier, and the parts meet at the barrier the row needs anyway. Integer
// sums do not depend on the order, so every kernel here, and any other exact
// implementation, gets the same S, and the fused codes equal those of
// normalizing first and quantizing after.
//
// The same kernels also fuse the SwiGLU before the down projection (QoQ/QServe
// article, section "运行时设计": the quantization of the second FFN layer's
// input is fused into the activation kernel before it; QUIK blog, section
// "案例研究: 敏感的 LLaMA-2 Down-Projection 层": the down projection takes the
// element-wise product of the gate and up projections). The gate and up rows
// are both staged, and each gathered channel becomes h = fp16(silu(g) u), the
// exact value rounded once (evaluated in binary64, see silu_mul_bits), so the
// fused codes equal those of comet_swiglu followed by the quantizer.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <mutex>

#include "comet_internal.h"
#include "qoq_internal.h"
#include "device_util.h"

namespace comet {
namespace {

constexpr int kThreads = 256;                    // per-row kernel: 4 waves, 16 blocks each per pass
constexpr int kMaxLdsRowChannels = 32768;        // 64 KB of fp16 per staged row
constexpr int kSwiWaveQueue = 512;               // SwiGLU fix-up queue entries per wave

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v6i __attribute__((ext_vector_type(6)));

// Lane exchange inside a DPP quad (no LDS round trip): quad_perm [1,0,3,2]
// (xor 1) and [2,3,0,1] (xor 2).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// The 32 channels (perm entries) of group g of block b.
__device__ __forceinline__ void load_positions(const int32_t* __restrict__ perm, int b, int g, int4 (&p)[8]) {
    const int4* src = reinterpret_cast<const int4*>(perm + b * kBlock + 32 * g);
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = src[k];
}

// Row statistic S = the exact sum of x_k^2, rounded once to binary64. Every
// binary16 value is n 2^-24 with n < 2^40, so x^2 is the integer n^2 < 2^80
// in units of 2^-48; those integers add up exactly in 128 bits (two 64-bit
// words), in whatever order the lanes and waves take them, and the total is
// rounded to binary64 once at the end. Staging and reduction order therefore
// do not change a bit of S.
struct SumSq {
    uint64_t lo, hi;
};

// a += x^2 for the binary16 value with bits h (finite): |x| = s 2^(max(e,1) - 25)
// with s the significand (the implicit bit for e > 0), so x^2 = s^2 2^sh in
// units of 2^-48 with sh = 2 max(e, 1) - 2 <= 58 and s^2 < 2^22.
__device__ __forceinline__ void sumsq_add(SumSq& a, uint32_t h) {
    const uint32_t e = (h >> 10) & 31u;
    const uint32_t s = (h & 1023u) | (e != 0u ? 1024u : 0u);
    const uint32_t sh = e != 0u ? 2u * e - 2u : 0u;
    const uint64_t s2 = static_cast<uint64_t>(s * s);
    const uint64_t lo = s2 << sh;                       // the bits below 2^64
    const uint64_t hi = (s2 >> 1) >> (63u - sh);        // the bits at and above 2^64
    a.lo += lo;
    a.hi += hi + (a.lo < lo ? 1u : 0u);
}

__device__ __forceinline__ void sumsq_merge(SumSq& a, uint64_t lo, uint64_t hi) {
    a.lo += lo;
    a.hi += hi + (a.lo < lo ? 1u : 0u);
}

// binary64 value of a sum (nearest, ties to even). Below 2^64 the 64-bit
// integer converts with one rounding (two exact 32-bit conversions, one
// exact scaling, one addition); above, the 64 leading bits are kept and the
// bits shifted out are folded into the lowest kept bit (a sticky bit), which
// keeps every rounding decision of the full value.
__device__ __forceinline__ double sumsq_value(const SumSq& a) {
    if (a.hi == 0) return __builtin_ldexp(static_cast<double>(a.lo), -48);
    const int n = 64 - __clzll(static_cast<long long>(a.hi));     // 1 .. 47
    const uint64_t top = (a.hi << (64 - n)) | (a.lo >> n);
    const uint64_t sticky = (a.lo << (64 - n)) != 0 ? 1u : 0u;
    return __builtin_ldexp(static_cast<double>(top | sticky), n - 48);
}

// This lane's part of the sum over the chunks c = w, w + 8, ... (chunk c
// holds channels 512c .. 512c + 511, 8 consecutive channels per lane), then
// summed over the 64 lanes of the wave (every lane gets the total).
__device__ __forceinline__ SumSq wave_sumsq(const uint16_t* row, int K, int w, int lane) {
    SumSq s = {0u, 0u};
    const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
    const int chunks = (K + 511) / 512;
    for (int c = w; c < chunks; c += 8) {
        const int k0 = 512 * c + 8 * lane;
        if (vec && k0 + 8 <= K) {
            const uint4 q = *reinterpret_cast<const uint4*>(row + k0);
            const uint32_t h[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) sumsq_add(s, (h[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        } else {
            for (int e = 0; e < 8 && k0 + e < K; ++e) sumsq_add(s, row[k0 + e]);
        }
    }
#pragma unroll
    for (int st = 32; st >= 1; st >>= 1)
        sumsq_merge(s, static_cast<uint64_t>(__shfl_xor(static_cast<unsigned long long>(s.lo), st)),
                    static_cast<uint64_t>(__shfl_xor(static_cast<unsigned long long>(s.hi), st)));
    return s;
}

// r = binary32(1 / sqrt(S / K + eps)) from the 8 wave parts (LDS, published),
// the quotient and root in binary64.
__device__ __forceinline__ float rms_from_waves(const SumSq* red, int K, float eps) {
    SumSq s = red[0];
#pragma unroll
    for (int v = 1; v < 8; ++v) sumsq_merge(s, red[v].lo, red[v].hi);
    const double S = sumsq_value(s);
    return static_cast<float>(1.0 / __builtin_sqrt(S / static_cast<double>(K) + static_cast<double>(eps)));
}

// The 8 wave parts of a row by the T / 64 waves of a workgroup (wave i forms
// parts i, i + T / 64, ...), written to `red`; the caller publishes them with
// a barrier.
template <int T>
__device__ __forceinline__ void wave_sums(const uint16_t* row, int K, SumSq* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int v = wave; v < 8; v += T / 64) {
        const SumSq W = wave_sumsq(row, K, v, lane);
        if (lane == 0) red[v] = W;
    }
}

// binary16 nearest to a binary64 value (ties to even). The binary64 value is
// first rounded to binary32 with round-to-odd (nearest, then the odd
// neighbour if that was inexact and even): binary32 keeps 13 more significand
// bits than binary16 and the odd last bit records whether anything was cut, so
// the second rounding decides ties and near-ties as a direct one would.
__device__ __forceinline__ uint16_t half_of_double(double v) {
    float f = static_cast<float>(v);
    if (static_cast<double>(f) != v) {
        uint32_t b = __float_as_uint(f);
        if ((b & 1u) == 0u) b = __builtin_fabs(static_cast<double>(f)) < __builtin_fabs(v) ? b + 1u : b - 1u;
        f = __uint_as_float(b);
    }
    return __half_as_ushort(__float2half_rn(f));
}

// h = fp16(silu(g) u) with silu(g) = g / (1 + e^-g): sigma(g) = n / (1 + e)
// with e = e^-|g| and n = 1 (g >= 0) or e (g < 0), which never overflows; g u
// is exact in binary64 (22 significand bits). The binary64 value is within a
// few units in its last place of the exact one, far inside the binary16
// rounding margin except at an exact tie. Ties arise only when sigma rounds to
// 1 (g > 36) and g u sits on a binary16 midpoint; the true value is then just
// below |g u|, so the next binary64 value toward zero stands in for it.
__device__ __forceinline__ uint16_t silu_mul_bits(uint16_t gb, uint16_t ub) {
    const double g = h2f(gb), u = h2f(ub);
    const double e = exp(-__builtin_fabs(g));
    const double sigma = (g >= 0.0 ? 1.0 : e) / (1.0 + e);
    const double gu = g * u;
    double v = gu * sigma;
    if (sigma == 1.0 && gu != 0.0) v = __longlong_as_double(__double_as_longlong(gu) - 1);
    return half_of_double(v);
}

// The same value from binary32 arithmetic when that decides it.
//   e = e^-|g| = 2^-(n + f): n = rint(|g| log2 e), and f = |g| log2 e - n
//       from two fused multiply-adds with log2 e split into two binary32
//       parts (absolute error below 2^-25); 2^-f from v_exp_f32 (|f| <= 1/2,
//       so its result is normal), then scaled by 2^-n exactly (to 0 far out,
//       where either sigma is 1 or the product is far below the smallest
//       fp16 value);
//   sigma = (g >= 0 ? 1 : e) * rcp(1 + e), v = (g u) sigma, g u exact.
// With at most 1.2 units in the last place from e, 1 from the reciprocal and
// half a unit per rounding, v is within a relative 2^-20.4 of silu(g) u. The
// true value then lies inside [|v| (1 - 2^-19), |v| (1 + 2^-19)] with room
// for the rounding of those two bounds; if both round to the same fp16 value,
// so does the true value (rounding is monotone), and the function returns
// true with it. Otherwise (about 0.6% of inputs) the caller takes
// silu_mul_bits.
__device__ __forceinline__ bool silu_mul_fast(uint16_t gb, uint16_t ub, uint16_t& h) {
    constexpr float kLog2eHi = 1.44269502162933349609375f;       // binary32 log2(e)
    constexpr float kLog2eLo = 1.925963033500011e-08f;          // log2(e) - kLog2eHi
    const float g = h2f(gb), u = h2f(ub);
    const float a = __builtin_fabsf(g);
    const float n = __builtin_rintf(a * kLog2eHi);
    const float f = __builtin_fmaf(a, kLog2eLo, __builtin_fmaf(a, kLog2eHi, -n));
    const float e = __builtin_ldexpf(__builtin_amdgcn_exp2f(-f), -static_cast<int>(n));
    const float sigma = (g >= 0.0f ? 1.0f : e) * __builtin_amdgcn_rcpf(1.0f + e);
    const float v = (g * u) * sigma;
    const float m = __builtin_fabsf(v);
    const float w = m * 0x1p-19f;
    const uint16_t lo = __half_as_ushort(__float2half_rn(m - w));
    const uint16_t hi = __half_as_ushort(__float2half_rn(m + w));
    h = static_cast<uint16_t>(lo | (__builtin_signbit(v) ? 0x8000u : 0u));
    return lo == hi;
}

__device__ __forceinline__ uint16_t silu_mul_any(uint16_t gb, uint16_t ub) {
    uint16_t h;
    return silu_mul_fast(gb, ub, h) ? h : silu_mul_bits(gb, ub);
}

// Codes and scale of block b of row m for this lane's group g, from the row
// (LDS or global) and the lane's 32 channels `pos`. With kNorm each gathered
// value first becomes fp16((x rs) gamma), gamma in permuted order (`gperm`);
// with kSwi `row` is the gate row and each value is fp16(silu(g) u) with u
// from the up row `row_u`.
template <bool kFp6, bool kNorm = false, bool kSwi = false, bool kAsym = false>
__device__ __forceinline__ void code_block(const uint16_t* __restrict__ row, const int4 (&pos)[8], int b, int nb,
                                           int nb4, int M, int Mp, int m, int g, uint8_t* __restrict__ Xq,
                                           float* __restrict__ x_scale, float rs = 0.0f,
                                           const uint16_t* __restrict__ gperm = nullptr,
                                           const uint16_t* __restrict__ row_u = nullptr,
                                           uint8_t* __restrict__ x_zero = nullptr) {
    const bool valid = b < nb;
    const int bc = valid ? b : nb - 1;
    const bool is8 = bc >= nb4;
    float v[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int idx[4] = {pos[k].x, pos[k].y, pos[k].z, pos[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (kSwi) {
                v[4 * k + e] = h2f(silu_mul_any(row[idx[e]], row_u[idx[e]]));   // gate row, up row
                // one value at a time: interleaving 32 binary64 evaluations
                // runs out of registers
                __builtin_amdgcn_sched_barrier(0);
            } else
                v[4 * k + e] = h2f(row[idx[e]]);
        }
    }
    if constexpr (kNorm) {
        // the lane's 32 gamma values are contiguous in permuted order
        const uint4* gp = reinterpret_cast<const uint4*>(gperm + bc * kBlock + 32 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 w = gp[q];
            const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float gm = h2f(static_cast<uint16_t>(h[e >> 1] >> (16 * (e & 1))));
                const float t = v[8 * q + e] * rs;
                v[8 * q + e] = __half2float(__float2half_rn(opaque(t * gm)));
            }
        }
    }
    if constexpr (kAsym) {
        // 4-bit blocks with a scale and a zero point (the QUIK blog's
        // activation scheme, section "反量化背后的数学"): the range is the
        // block's minimum and maximum widened to include 0, step d / 15 with
        // d = hi - lo, zero point z = round(-lo * inv), code u = round(x *
        // inv) + z, both clamped to [0, 15]; inv = 15 / d and the step are
        // correctly rounded divisions. 8-bit blocks take the symmetric path.
        if (!is8) {
            float lo = 0.0f, hi = 0.0f;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                lo = fminf(lo, v[e]);
                hi = fmaxf(hi, v[e]);
            }
            lo = fminf(lo, dpp_f<0xB1>(lo));     // over the block's quad
            lo = fminf(lo, dpp_f<0x4E>(lo));
            hi = fmaxf(hi, dpp_f<0xB1>(hi));
            hi = fmaxf(hi, dpp_f<0x4E>(hi));
            float inv = 0.0f, sc = 0.0f, zf = 0.0f;
            if (lo != hi) {
                const float d = hi - lo;
                inv = 15.0f / d;
                sc = d / 15.0f;
                zf = fminf(fmaxf(__builtin_rintf(-lo * inv), 0.0f), 15.0f);
            }
            if (valid) {
                uint32_t w[4];
#pragma unroll
                for (int d4 = 0; d4 < 4; ++d4) {
                    uint32_t x = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float ul = fminf(fmaxf(__builtin_rintf(v[4 * d4 + k] * inv) + zf, 0.0f), 15.0f);
                        const float uh = fminf(fmaxf(__builtin_rintf(v[16 + 4 * d4 + k] * inv) + zf, 0.0f), 15.0f);
                        x |= (static_cast<uint32_t>(ul) | (static_cast<uint32_t>(uh) << 4)) << (8 * k);
                    }
                    w[d4] = x;
                }
                uint8_t* dst = Xq + static_cast<size_t>(bc) * M * 64 + static_cast<size_t>(m) * 64 + 16 * g;
                *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
                if (g == 0) {
                    x_scale[static_cast<size_t>(bc) * M + m] = sc;
                    x_zero[static_cast<size_t>(bc) * Mp + m] = static_cast<uint8_t>(zf);
                }
            }
            return;
        }
        if (valid && g == 0) x_zero[static_cast<size_t>(bc) * Mp + m] = 0;
    }
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) a = fmaxf(a, fabsf(v[e]));
    a = fmaxf(a, dpp_f<0xB1>(a));      // absmax over the block's quad
    a = fmaxf(a, dpp_f<0x4E>(a));

    const float qmax = is8 ? 127.0f : 7.0f;
    float inv = 0.0f, sc = 0.0f;
    if (a > 0.0f) {
        inv = qmax / a;     // correctly rounded IEEE division
        sc = a / qmax;
    }
    // q = clamp(rint(x * inv), -qmax, qmax). The clamp never acts: |x| <= a
    // and inv <= (qmax / a)(1 + 2^-24) bound |fl(x * inv)| by
    // qmax (1 + 2^-24)^2 < qmax + 1/2. Adding +0 turns a -0 into +0.
    float r[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) r[e] = __builtin_rintf(v[e] * inv) + 0.0f;

    if (valid) {
        if (!is8 && kFp6) {
            v16f even, odd;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                even[e] = r[2 * e];
                odd[e] = r[2 * e + 1];
            }
            const v6i c = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(even, odd, 1.0f);
            uint8_t* tile = Xq + static_cast<size_t>(bc) * Mp * 96 + static_cast<size_t>(m >> 4) * 1536;
            *reinterpret_cast<uint4*>(tile + tile_head(m & 15, g)) = make_uint4(c[0], c[1], c[2], c[3]);
            *reinterpret_cast<uint2*>(tile + tile_tail(m & 15, g)) = make_uint2(c[4], c[5]);
        } else if (!is8) {
            uint32_t w[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t x = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = static_cast<uint32_t>(static_cast<int>(r[4 * d + k]) + 8);
                    const uint32_t hi = static_cast<uint32_t>(static_cast<int>(r[16 + 4 * d + k]) + 8);
                    x |= (lo | (hi << 4)) << (8 * k);
                }
                w[d] = x;
            }
            uint8_t* dst = Xq + static_cast<size_t>(bc) * M * 64 + static_cast<size_t>(m) * 64 + 16 * g;
            *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            uint32_t w[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                uint32_t x = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    x |= (static_cast<uint32_t>(static_cast<int>(r[4 * d + k])) & 0xFFu) << (8 * k);
                w[d] = x;
            }
            if constexpr (kFp6) {
                // 16-row tiles of 2048 bytes: positions 32g + 16h + j of
                // row r at tile byte 1024h + tile_head(r, g) + j
                uint8_t* tile = Xq + static_cast<size_t>(nb4) * Mp * 96 +
                                static_cast<size_t>(bc - nb4) * Mp * 128 + static_cast<size_t>(m >> 4) * 2048;
                const int head = tile_head(m & 15, g);
                *reinterpret_cast<uint4*>(tile + head) = make_uint4(w[0], w[1], w[2], w[3]);
                *reinterpret_cast<uint4*>(tile + 1024 + head) = make_uint4(w[4], w[5], w[6], w[7]);
            } else {
                uint8_t* dst = Xq + static_cast<size_t>(nb4) * M * 64 +
                               static_cast<size_t>(bc - nb4) * M * 128 + static_cast<size_t>(m) * 128 + 32 * g;
                *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
                *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
            }
        }
        if (g == 0) x_scale[static_cast<size_t>(bc) * M + m] = sc;
    }
}

template <bool kRowInLds, bool kFp6, bool kNorm, bool kSwi = false, int T = kThreads, bool kAsym = false>
__global__ __launch_bounds__(T) void quant_act_kernel(
    const uint16_t* __restrict__ X, int M, int K, int ldx, const int32_t* __restrict__ perm,
    int nb, int nb4, uint8_t* __restrict__ Xq, float* __restrict__ x_scale, int rows_per_xcd,
    const uint16_t* __restrict__ gperm, float eps, const uint16_t* __restrict__ U = nullptr,
    uint8_t* __restrict__ x_zero = nullptr) {
    extern __shared__ uint16_t row_lds[];
    // Row of this workgroup. Workgroup w runs on XCD w mod 8 and each XCD has
    // its own L2; with `rows_per_xcd` > 0 every XCD takes a contiguous range
    // of rows (whole 16-row tiles), so the partial cache lines that the rows
    // of one tile write meet in one L2 instead of leaving as partial writes.
    int m = blockIdx.x;
    if (rows_per_xcd > 0) {
        m = (blockIdx.x & 7) * rows_per_xcd + (blockIdx.x >> 3);
        if (m >= M) return;
    }
    const uint16_t* xr = X + static_cast<size_t>(m) * ldx;
    const uint16_t* ur = kSwi ? U + static_cast<size_t>(m) * ldx : nullptr;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // whole 1 KB direct-load chunks of one staged row
    const size_t row_bytes = static_cast<size_t>((K + 511) / 512) * 1024;
    // the row statistic's 8 wave parts (kNorm), or the SwiGLU fix-up queue
    // (kSwi), follow the staged row
    SumSq* red = reinterpret_cast<SumSq*>(reinterpret_cast<uint8_t*>(row_lds) + (kRowInLds ? row_bytes : 0));
    bool sums_done = false;

    const int Mp = (M + 15) & ~15;        // FP6 layout: rows padded to whole 16-row tiles
    const int g = lane & 3;               // the lane's 32-channel group
    const int bl = lane >> 2;             // its block among the wave's 16
    const int stride = gridDim.y * (T / 64) * 16;
    int b0 = (blockIdx.y * (T / 64) + wave) * 16;
    int4 nxt[8];
    // the perm entries of the first pass do not depend on the row: their
    // loads go out before the row's, so the two latencies overlap (the
    // SwiGLU form, whose staging is long and register-heavy, loads them
    // after it)
    if (!kSwi && b0 < nb) load_positions(perm, imin(b0 + bl, nb - 1), g, nxt);
    if constexpr (kRowInLds && kSwi) {
        // The staged row is h itself: every thread forms 8 consecutive values
        // per step from coalesced gate and up loads with the binary32 test.
        // The channels it cannot decide go to its wave's queue (a ballot
        // gives each flagged lane its slot; once the queue is full, straight
        // to the binary64 form), which the wave then clears itself.
        int* queue = reinterpret_cast<int*>(red) + wave * kSwiWaveQueue;
        int qcount = 0;                                   // wave-uniform
        const bool vec = ((reinterpret_cast<uintptr_t>(xr) | reinterpret_cast<uintptr_t>(ur)) & 15u) == 0;
        // Every lane of a wave calls put for each step (the ballot and the
        // queue count stay wave-uniform); lanes past the row end pass
        // valid = false.
        auto put = [&](int k, uint16_t gb, uint16_t ub, bool valid) {
            uint16_t h = 0;
            const bool bad = valid && !silu_mul_fast(gb, ub, h);
            const uint64_t mask = __ballot(bad);
            if (mask) {
                const int slot = qcount + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                              static_cast<uint32_t>(mask >> 32),
                                              __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
                if (bad) {
                    if (slot < kSwiWaveQueue) queue[slot] = k;
                    else h = silu_mul_bits(gb, ub);
                }
                qcount += __popcll(mask);
            }
            if (valid) row_lds[k] = h;
        };
        auto put8 = [&](int k0, const uint4& gq, const uint4& uq, bool valid) {
            const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                put(k0 + e, static_cast<uint16_t>(gw[e >> 1] >> (16 * (e & 1))),
                    static_cast<uint16_t>(uw[e >> 1] >> (16 * (e & 1))), valid);
        };
        constexpr int kStep = 8 * T;
        if (vec) {
            // K is a multiple of 128, so every 8-channel step is whole. Two
            // register sets take turns: one step is coded while the loads of
            // the next are in flight (past the row end the loads repeat the
            // last step, in bounds, and are not used).
            auto ld = [&](int k, uint4& gq, uint4& uq) {
                const int kk = imin(k, K - 8);
                gq = *reinterpret_cast<const uint4*>(xr + kk);
                uq = *reinterpret_cast<const uint4*>(ur + kk);
            };
            const int t8 = 8 * static_cast<int>(threadIdx.x);
            uint4 ga, ua, gb, ub;
            ld(t8, ga, ua);
            for (int base = 0; base < K; base += 2 * kStep) {          // uniform trip count
                ld(base + kStep + t8, gb, ub);
                put8(base + t8, ga, ua, base + t8 < K);
                ld(base + 2 * kStep + t8, ga, ua);
                put8(base + kStep + t8, gb, ub, base + kStep + t8 < K);
            }
        } else {
            for (int base = 0; base < K; base += T) {
                const int k = base + static_cast<int>(threadIdx.x);
                const bool valid = k < K;
                put(k, valid ? xr[k] : uint16_t(0), valid ? ur[k] : uint16_t(0), valid);
            }
        }
        // this wave's undecided channels (LDS operations of one wave complete
        // in order, so these writes land after its binary32 ones)
        const int n = imin(qcount, kSwiWaveQueue);
        for (int i = lane; i < n; i += 64) {
            const int k = queue[i];
            row_lds[k] = silu_mul_bits(xr[k], ur[k]);
        }
        __syncthreads();
    } else if constexpr (kRowInLds) {
        if ((ldx & 7) == 0) {
            // direct loads of the row: 1 KB per wave instruction, all in flight
            // at once; the LDS row buffer is rounded up to whole KB and the
            // bytes past the row read as 0
            const Rsrc r = make_rsrc(xr, 2u * static_cast<uint32_t>(K));
            const int chunks = (K + 511) / 512;
            uint8_t* lds = reinterpret_cast<uint8_t*>(row_lds);
            for (int c = wave; c < chunks; c += T / 64) lds_buf16(r, 16u * lane, 1024u * c, lds + 1024 * c);
            COMET_VMCNT(0);
            // this wave's chunks have landed: its wave sums need no barrier
            if constexpr (kNorm) wave_sums<T>(row_lds, K, red);
            sums_done = true;
        } else {
            for (int c = threadIdx.x; c < K; c += T) row_lds[c] = xr[c];
        }
        __syncthreads();
    }
    float rs = 0.0f;
    if constexpr (kNorm) {
        if (!sums_done) {
            wave_sums<T>(kRowInLds ? row_lds : xr, K, red);
            __syncthreads();
        }
        rs = rms_from_waves(red, K, eps);
    }

    if (kSwi && b0 < nb) load_positions(perm, imin(b0 + bl, nb - 1), g, nxt);
    for (; b0 < nb; b0 += stride) {
        int4 pos[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pos[k] = nxt[k];
        if (b0 + stride < nb) load_positions(perm, imin(b0 + stride + bl, nb - 1), g, nxt);
        // from the staged h row, or (rows in global memory) from the gate and
        // up rows with h formed per gathered channel
        code_block<kFp6, kNorm, kSwi && !kRowInLds, kAsym>(kRowInLds ? row_lds : xr, pos, b0 + bl, nb, nb4, M, Mp,
                                                           m, g, Xq, x_scale, rs, gperm, ur, x_zero);
    }
}

// ---------------------------------------------------------------------------
// Many rows (M >= 256, K <= 32768): one persistent workgroup of 8 waves per CU
// walks its rows with two LDS row buffers, so the direct loads of row k+1 run
// while row k is coded. The 8 x 16 x 2 = 256 blocks a workgroup covers per row
// (K <= 32768) are the same for every row, so each lane loads its perm entries
// once, into registers. The rows of an XCD are a contiguous range of whole
// 16-row tiles, and its workgroups take consecutive rows of it, so the partial
// cache lines of one output tile meet in that XCD's L2.
// ---------------------------------------------------------------------------
// Two shapes: 8 waves with 2 passes (8 x 16 x 2 = 256 blocks, K <= 32768, one
// workgroup per CU), and for K <= 8192 4 waves with 1 pass (64 blocks): half
// the perm registers and a quarter of the LDS, so two workgroups share a CU
// and one's row loads and code stores overlap the other's coding.
template <int kWaves>
constexpr int row_passes() { return kWaves == 8 ? 2 : 1; }

// lds_buf16 with the non-temporal hint (data read once: the L2 keeps it only
// with low priority).
__device__ __forceinline__ void lds_buf16_nt(Rsrc r, uint32_t voff, uint32_t soff, uint8_t* lds_piece) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_piece)), 16,
        voff, soff, 0, 2);
}

template <int kWaves>
__device__ __forceinline__ void stage_row(const uint16_t* xr, int K, int wave, int lane, uint8_t* __restrict__ buf) {
    const Rsrc r = make_rsrc(xr, 2u * static_cast<uint32_t>(K));
    const int chunks = (K + 511) / 512;
    // the 8-wave form (rows of more than 8192 channels) loads its rows
    // non-temporally: they pass through once, and the hint leaves the L2 to the
    // partial cache lines of the code tiles that the rows of an XCD fill
    // together (4096 x 28672: 65 against 71 us; on the 4-wave form, 8192
    // channels, the hint cost time: 21 against 18.5 us)
    for (int c = wave; c < chunks; c += kWaves) {
        if constexpr (kWaves == 8) lds_buf16_nt(r, 16u * lane, 1024u * c, buf + 1024 * c);
        else lds_buf16(r, 16u * lane, 1024u * c, buf + 1024 * c);
    }
}

// One row: start the direct loads of the next row into `nxt_buf`, then code
// this row from `cur` (distinct buffers, restrict-qualified so that the LDS
// gathers do not wait for the loads just issued).
template <bool kFp6, bool kNorm, int kWaves>
__device__ __forceinline__ void row_step(const uint16_t* next_row, uint8_t* __restrict__ nxt_buf,
                                         const uint16_t* __restrict__ cur,
                                         const int4 (&pos)[row_passes<kWaves>()][8],
                                         int K, int nb, int nb4, int M, int Mp, int m, int wave, int lane,
                                         uint8_t* __restrict__ Xq, float* __restrict__ x_scale,
                                         const uint16_t* __restrict__ gperm, float eps, const SumSq* red_cur,
                                         SumSq* red_nxt) {
    if (next_row) stage_row<kWaves>(next_row, K, wave, lane, nxt_buf);
    float rs = 0.0f;
    if constexpr (kNorm) rs = rms_from_waves(red_cur, K, eps);
    const int g = lane & 3, bl = lane >> 2;
#pragma unroll
    for (int p = 0; p < row_passes<kWaves>(); ++p) {
        const int b0 = (p * kWaves + wave) * 16;
        if (b0 < nb) code_block<kFp6, kNorm>(cur, pos[p], b0 + bl, nb, nb4, M, Mp, m, g, Xq, x_scale, rs, gperm);
    }
    if constexpr (kNorm) {
        // the next row's chunks of this wave have landed once its loads are
        // done: its wave sum, published by the barrier that opens that row
        if (next_row) {
            COMET_VMCNT(0);
            wave_sums<64 * kWaves>(reinterpret_cast<const uint16_t*>(nxt_buf), K, red_nxt);
        }
    }
}

template <bool kFp6, bool kNorm, int kWaves = 8>
__global__ __launch_bounds__(64 * kWaves) void quant_rows_kernel(
    const uint16_t* __restrict__ X, int M, int K, int ldx, const int32_t* __restrict__ perm, int nb, int nb4,
    uint8_t* __restrict__ Xq, float* __restrict__ x_scale, int rows_per_xcd, int wgs_per_xcd,
    const uint16_t* __restrict__ gperm, float eps) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t bufs[];
    const int row_bytes = ((K + 511) / 512) * 1024;
    // the 8 wave sums of the row statistic (kNorm) follow the two row
    // buffers, alternating between two sets: row k+1's are written during row
    // k, while the waves read row k's from the other set
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int first = (blockIdx.x & 7) * rows_per_xcd + (blockIdx.x >> 3);
    const int end = imin(M, ((blockIdx.x & 7) + 1) * rows_per_xcd);
    if (first >= end) return;
    const int n = (end - first + wgs_per_xcd - 1) / wgs_per_xcd;
    const int Mp = (M + 15) & ~15;

    int4 pos[row_passes<kWaves>()][8];
#pragma unroll
    for (int p = 0; p < row_passes<kWaves>(); ++p) {
        const int b = (p * kWaves + wave) * 16 + (lane >> 2);
        load_positions(perm, imin(b, nb - 1), lane & 3, pos[p]);
    }
    SumSq* red = reinterpret_cast<SumSq*>(bufs + 2 * static_cast<size_t>(row_bytes));
    stage_row<kWaves>(X + static_cast<size_t>(first) * ldx, K, wave, lane, bufs);
    if constexpr (kNorm) {
        COMET_VMCNT(0);
        wave_sums<64 * kWaves>(reinterpret_cast<const uint16_t*>(bufs), K, red);
    }
    for (int k = 0; k < n; ++k) {
        const int m = first + k * wgs_per_xcd;
        // row k has landed (and this wave's earlier stores are done); after
        // the barrier every wave is also done with row k-1's buffer
        COMET_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        const uint16_t* next = k + 1 < n ? X + static_cast<size_t>(m + wgs_per_xcd) * ldx : nullptr;
        if (k & 1)
            row_step<kFp6, kNorm, kWaves>(next, bufs, reinterpret_cast<const uint16_t*>(bufs + row_bytes), pos, K, nb, nb4,
                                  M, Mp, m, wave, lane, Xq, x_scale, gperm, eps, red + 8 * (k & 1),
                                  red + 8 * ((k + 1) & 1));
        else
            row_step<kFp6, kNorm, kWaves>(next, bufs + row_bytes, reinterpret_cast<const uint16_t*>(bufs), pos, K, nb, nb4,
                                  M, Mp, m, wave, lane, Xq, x_scale, gperm, eps, red + 8 * (k & 1),
                                  red + 8 * ((k + 1) & 1));
    }
}

// Dynamic LDS above the 64 KB default for the kernels that need it, set once
// per kernel (one flag per kernel address).
template <auto Kern>
hipError_t allow_lds(int bytes) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [bytes] {
        attr = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                   bytes);
    });
    return attr;
}

// K: the channels of X a row stages (the gather reads any of them); kq > 0:
// only the first kq permuted channels are quantized (QUIK's split), else K.
template <bool kFp6, bool kNorm, bool kSwi = false>
int launch(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8, uint8_t* Xq,
           float* x_scale, const uint16_t* gperm, float eps, void* stream, const uint16_t* U = nullptr,
           int kq = 0) {
    const int nb = (kq > 0 ? kq : K) / kBlock;
    const int nb4 = nb - nb8;
    // Enough workgroups to cover the chip even for a handful of rows: split the
    // blocks of a row over gridDim.y workgroups (each stages the whole row).
    // the SwiGLU form stages h with 8 waves per workgroup (its evaluation
    // wants the latency cover); the others with 4
    constexpr int T = kSwi ? 512 : kThreads;
    const int per_wg = (T / 64) * 16;                       // blocks per workgroup pass
    int groups = 1;
    const int want = 1024;
    while (groups * per_wg < nb && static_cast<long>(M) * groups < want) ++groups;
    // XCD-aware row order once there are enough rows for every XCD to get
    // whole 16-row tiles
    const int rows_per_xcd = M >= 128 ? ((M + 127) / 128) * 16 : 0;
    dim3 grid(rows_per_xcd > 0 ? 8 * rows_per_xcd : M, groups);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // wave sums of the row statistic, or the SwiGLU fix-up queue and its count
    const size_t red = kNorm ? 16 * sizeof(SumSq) : kSwi ? (T / 64) * kSwiWaveQueue * sizeof(int) : 0;
    const size_t row_lds = static_cast<size_t>((K + 511) / 512) * 1024;   // whole 1 KB direct-load chunks
    const size_t buf = row_lds;
    constexpr size_t kLds = 160 * 1024;
    // (the SwiGLU form stays on the per-row kernel: with its binary64
    // evaluation on top of the perm entries held in registers, the persistent
    // kernel runs out of registers)
    if constexpr (!kSwi) {
        if (M >= 256 && K <= kMaxLdsRowChannels && 2 * buf + red <= kLds && (ldx & 7) == 0) {
            // the two row buffers (and the wave sums) may exceed the 64 KB
            // default; the kernel's 256 blocks per row cover K <= 32768
            const int rows_per_xcd = ((M + 127) / 128) * 16;
            if (nb <= 64) {
                // 4 waves, 2 workgroups per CU (2 x 2 x 16 KB of LDS at most)
                const int wgs_per_xcd = 2 * (cu_count() / 8);
                quant_rows_kernel<kFp6, kNorm, 4><<<8 * wgs_per_xcd, 256, 2 * buf + red, s>>>(
                    X, M, K, ldx, perm, nb, nb4, Xq, x_scale, rows_per_xcd, wgs_per_xcd, gperm, eps);
                return static_cast<int>(hipGetLastError());
            }
            const hipError_t attr = allow_lds<&quant_rows_kernel<kFp6, kNorm, 8>>(kLds);
            if (attr != hipSuccess) return static_cast<int>(attr);
            const int wgs_per_xcd = cu_count() / 8;
            quant_rows_kernel<kFp6, kNorm, 8><<<8 * wgs_per_xcd, 512, 2 * buf + red, s>>>(
                X, M, K, ldx, perm, nb, nb4, Xq, x_scale, rows_per_xcd, wgs_per_xcd, gperm, eps);
            return static_cast<int>(hipGetLastError());
        }
    }
    if (K <= kMaxLdsRowChannels) {
        const hipError_t attr = allow_lds<&quant_act_kernel<true, kFp6, kNorm, kSwi, T>>(kLds);
        if (attr != hipSuccess) return static_cast<int>(attr);
        quant_act_kernel<true, kFp6, kNorm, kSwi, T><<<grid, T, buf + red, s>>>(
            X, M, K, ldx, perm, nb, nb4, Xq, x_scale, rows_per_xcd, gperm, eps, U);
    } else {
        quant_act_kernel<false, kFp6, kNorm, kSwi, T><<<grid, T, kNorm ? red : 0, s>>>(
            X, M, K, ldx, perm, nb, nb4, Xq, x_scale, rows_per_xcd, gperm, eps, U);
    }
    return static_cast<int>(hipGetLastError());
}

// Standalone RMS normalization (the unfused step): one workgroup of 512
// threads per row, the same statistic as the fused kernels, fp16 out in the
// original channel order.
constexpr int kNormThreads = 512;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t* __restrict__ X, int K, int ldx,
                                                               const uint16_t* __restrict__ gamma, float eps,
                                                               uint16_t* __restrict__ Xn, int ldn) {
    __shared__ SumSq red[8];
    const int m = blockIdx.x;
    const uint16_t* xr = X + static_cast<size_t>(m) * ldx;
    wave_sums<kNormThreads>(xr, K, red);
    __syncthreads();
    const float rs = rms_from_waves(red, K, eps);
    uint16_t* out = Xn + static_cast<size_t>(m) * ldn;
    for (int k = threadIdx.x; k < K; k += kNormThreads) {
        const float t = h2f(xr[k]) * rs;
        out[k] = __half_as_ushort(__float2half_rn(opaque(t * h2f(gamma[k]))));
    }
}

// Standalone SwiGLU (the unfused step): H = fp16(silu(G) U) element-wise, one
// workgroup of 256 threads per row, 8 consecutive channels per thread when
// every row start is 16-byte aligned.
constexpr int kSwiThreads = 256;

__global__ __launch_bounds__(kSwiThreads) void swiglu_kernel(const uint16_t* __restrict__ G,
                                                             const uint16_t* __restrict__ U, int K, int ldx,
                                                             uint16_t* __restrict__ H, int ldh, int vec) {
    const size_t m = blockIdx.x;
    const uint16_t* gr = G + m * ldx;
    const uint16_t* ur = U + m * ldx;
    uint16_t* hr = H + m * ldh;
    int k0 = 0;
    if (vec) {
        for (int k = 8 * threadIdx.x; k + 8 <= K; k += 8 * kSwiThreads) {
            const uint4 gq = *reinterpret_cast<const uint4*>(gr + k);
            const uint4 uq = *reinterpret_cast<const uint4*>(ur + k);
            const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
            uint32_t hw[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t lo = silu_mul_any(static_cast<uint16_t>(gw[d]), static_cast<uint16_t>(uw[d]));
                const uint32_t hi = silu_mul_any(static_cast<uint16_t>(gw[d] >> 16), static_cast<uint16_t>(uw[d] >> 16));
                hw[d] = lo | (hi << 16);
            }
            *reinterpret_cast<uint4*>(hr + k) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        }
        k0 = K & ~7;
    }
    for (int k = k0 + threadIdx.x; k < K; k += kSwiThreads) hr[k] = silu_mul_any(gr[k], ur[k]);
}

}  // namespace

// ---------------------------------------------------------------------------
// Per-token INT8 activations of the QoQ W4A8 variant (QoQ/QServe article,
// section "运行时设计": W4A8 GEMMs take 8-bit activations): one scale per
// token over all K. One workgroup per row stages the row in LDS, takes its
// absmax (a maximum does not depend on the channel order), then each lane
// codes one 32-channel group of a block from the perm gather: q = round(x *
// inv), inv = 127 / a and s = a / 127 correctly rounded (the clamp to 127
// never acts, as for the per-block quantizer). Codes go to 8-bit slabs:
// block b, row m at byte (b M + m) 128, positions in order.
// ---------------------------------------------------------------------------
constexpr int kTokThreads = 256;

__global__ __launch_bounds__(kTokThreads) void quant_token_i8_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                                    int ldx, const int32_t* __restrict__ perm,
                                                                    int nb, uint8_t* __restrict__ Xq,
                                                                    float* __restrict__ x_scale) {
    extern __shared__ uint16_t row_lds[];
    __shared__ float wmax[kTokThreads / 64];
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint16_t* xr = X + static_cast<size_t>(m) * ldx;
    float a = 0.0f;
    if ((ldx & 7) == 0) {
        // 16-byte loads, four in flight per thread (K is a multiple of 128,
        // so the row is whole 16-byte words)
        const uint4* x4 = reinterpret_cast<const uint4*>(xr);
        uint4* l4 = reinterpret_cast<uint4*>(row_lds);
#pragma unroll 4
        for (int c = threadIdx.x; c < K / 8; c += kTokThreads) {
            const uint4 v = x4[c];
            l4[c] = v;
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(h2f(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))))));
        }
    } else {
        for (int c = threadIdx.x; c < K; c += kTokThreads) {
            const uint16_t h = xr[c];
            row_lds[c] = h;
            a = fmaxf(a, fabsf(h2f(h)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if (lane == 0) wmax[wave] = a;
    __syncthreads();
    a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    float inv = 0.0f, sc = 0.0f;
    if (a > 0.0f) {
        inv = 127.0f / a;
        sc = a / 127.0f;
    }
    for (int t = threadIdx.x; t < 4 * nb; t += kTokThreads) {
        const int b = t >> 2, g = t & 3;
        const int4* pp = reinterpret_cast<const int4*>(perm + b * kBlock + 32 * g);
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int4 pk = pp[k];
            const int idx[4] = {pk.x, pk.y, pk.z, pk.w};
            uint32_t x = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = static_cast<int>(__builtin_rintf(h2f(row_lds[idx[e]]) * inv));
                x |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * e);
            }
            w[k] = x;
        }
        uint8_t* dst = Xq + (static_cast<size_t>(b) * M + m) * 128 + 32 * g;
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
    }
    if (threadIdx.x == 0) x_scale[m] = sc;
}

int cu_count() {
    static int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 8)
            v = 256;
        return v;
    }();
    return n;
}

int launch_quant_act(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                     uint8_t* Xq, float* x_scale, void* stream) {
    return launch<false, false>(X, M, K, ldx, perm, nb8, Xq, x_scale, nullptr, 0.0f, stream);
}

// Asymmetric 4-bit blocks (INT4 layout): the per-row kernel, every M; the
// zero points go to x_zero [nb][Mp], Mp = M rounded up to a multiple of 16.
int launch_quant_act_asym(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                          uint8_t* Xq, float* x_scale, uint8_t* x_zero, void* stream) {
    const int nb = K / kBlock;
    const int nb4 = nb - nb8;
    constexpr int T = kThreads;
    const int per_wg = (T / 64) * 16;
    int groups = 1;
    while (groups * per_wg < nb && static_cast<long>(M) * groups < 1024) ++groups;
    const int rows_per_xcd = M >= 128 ? ((M + 127) / 128) * 16 : 0;
    dim3 grid(rows_per_xcd > 0 ? 8 * rows_per_xcd : M, groups);
    hipStream_t s = static_cast<hipStream_t>(stream);
    constexpr size_t kLds = 160 * 1024;
    const size_t row_lds = static_cast<size_t>((K + 511) / 512) * 1024;
    if (K <= kMaxLdsRowChannels) {
        const hipError_t attr = allow_lds<&quant_act_kernel<true, false, false, false, T, true>>(kLds);
        if (attr != hipSuccess) return static_cast<int>(attr);
        quant_act_kernel<true, false, false, false, T, true><<<grid, T, row_lds, s>>>(
            X, M, K, ldx, perm, nb, nb4, Xq, x_scale, rows_per_xcd, nullptr, 0.0f, nullptr, x_zero);
    } else {
        quant_act_kernel<false, false, false, false, T, true><<<grid, T, 0, s>>>(
            X, M, K, ldx, perm, nb, nb4, Xq, x_scale, rows_per_xcd, nullptr, 0.0f, nullptr, x_zero);
    }
    return static_cast<int>(hipGetLastError());
}

int launch_quant_act_fp6(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                         uint8_t* Xq, float* x_scale, void* stream, int kq) {
    return launch<true, false>(X, M, K, ldx, perm, nb8, Xq, x_scale, nullptr, 0.0f, stream, nullptr, kq);
}

namespace {

// QUIK's fp16 outlier channels (QUIK blog, section "第二步: 前向传播 (在线)":
// the activations split into the quantized part and the FP16 outlier
// columns): the columns perm_f[0 .. nf) of X as 16-row x 32-channel tiles in
// the operand order of the fp16 matrix instruction: tile (t, s) at half
// (t (nf / 32) + s) 512, lane slot l at + 8 l, row 16 t + l mod 16, channels
// 32 s + 8 (l / 16) .. + 7. One workgroup per row (and per padding row, which
// is written as zeros): the row is staged in LDS with coalesced 16-byte loads
// (the quantizer has just read it, so it comes from the last-level cache),
// then each thread gathers 8 consecutive outlier channels from LDS and writes
// them with one 16-byte store.
constexpr int kGatherThreads = 256;

template <bool kLds>
__global__ __launch_bounds__(kGatherThreads) void gather_outliers_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                                         int ldx, const int32_t* __restrict__ perm_f,
                                                                         int nf, uint16_t* __restrict__ Xf) {
    extern __shared__ __attribute__((aligned(16))) uint16_t row_lds[];
    const int m = blockIdx.x;
    const bool real = m < M;
    const uint16_t* xr = X + static_cast<size_t>(real ? m : 0) * ldx;
    if constexpr (kLds) {
        if (real) {
            // K and ldx are multiples of 8 on this path: whole 16-byte words
            for (int k = 8 * threadIdx.x; k < K; k += 8 * kGatherThreads)
                *reinterpret_cast<uint4*>(row_lds + k) = *reinterpret_cast<const uint4*>(xr + k);
        }
        __syncthreads();
    }
    const uint32_t steps = static_cast<uint32_t>(nf) / 32u;
    const uint32_t t = static_cast<uint32_t>(m) / 16u, r = static_cast<uint32_t>(m) & 15u;
    for (int j0 = 8 * threadIdx.x; j0 < nf; j0 += 8 * kGatherThreads) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (real) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c0 = perm_f[j0 + 2 * e], c1 = perm_f[j0 + 2 * e + 1];
                const uint16_t v0 = kLds ? row_lds[c0] : xr[c0];
                const uint16_t v1 = kLds ? row_lds[c1] : xr[c1];
                w[e] = static_cast<uint32_t>(v0) | (static_cast<uint32_t>(v1) << 16);
            }
        }
        const uint32_t st = static_cast<uint32_t>(j0) / 32u;
        const uint32_t l = r + 16u * ((static_cast<uint32_t>(j0) & 31u) / 8u);
        *reinterpret_cast<uint4*>(Xf + ((static_cast<size_t>(t) * steps + st) * 64u + l) * 8u) =
            uint4{w[0], w[1], w[2], w[3]};
    }
}

}  // namespace

int launch_gather_outliers(const uint16_t* X, int M, int K, int ldx, const int32_t* perm_f, int nf, uint16_t* Xf,
                           void* stream) {
    const int mp = (M + 15) / 16 * 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool lds = K <= kMaxLdsRowChannels && (ldx & 7) == 0 &&
                     (reinterpret_cast<uintptr_t>(X) & 15u) == 0;
    if (lds) {
        const size_t bytes = static_cast<size_t>(K) * 2u;
        if (bytes > 64 * 1024) {
            const hipError_t attr = allow_lds<&gather_outliers_kernel<true>>(160 * 1024);
            if (attr != hipSuccess) return static_cast<int>(attr);
        }
        gather_outliers_kernel<true><<<mp, kGatherThreads, bytes, s>>>(X, M, K, ldx, perm_f, nf, Xf);
    } else {
        gather_outliers_kernel<false><<<mp, kGatherThreads, 0, s>>>(X, M, K, ldx, perm_f, nf, Xf);
    }
    return static_cast<int>(hipGetLastError());
}

int launch_rmsnorm_quant_act(const uint16_t* X, int M, int K, int ldx, const uint16_t* gamma_perm, float eps,
                             const int32_t* perm, int nb8, uint8_t* Xq, float* x_scale, bool fp6, void* stream) {
    return fp6 ? launch<true, true>(X, M, K, ldx, perm, nb8, Xq, x_scale, gamma_perm, eps, stream)
               : launch<false, true>(X, M, K, ldx, perm, nb8, Xq, x_scale, gamma_perm, eps, stream);
}

int launch_swiglu_quant_act(const uint16_t* G, const uint16_t* U, int M, int K, int ldx, const int32_t* perm,
                            int nb8, uint8_t* Xq, float* x_scale, bool fp6, void* stream) {
    return fp6 ? launch<true, false, true>(G, M, K, ldx, perm, nb8, Xq, x_scale, nullptr, 0.0f, stream, U)
               : launch<false, false, true>(G, M, K, ldx, perm, nb8, Xq, x_scale, nullptr, 0.0f, stream, U);
}

int launch_swiglu(const uint16_t* G, const uint16_t* U, int M, int K, int ldx, uint16_t* H, int ldh,
                  void* stream) {
    const bool vec = ((reinterpret_cast<uintptr_t>(G) | reinterpret_cast<uintptr_t>(U) |
                       reinterpret_cast<uintptr_t>(H)) & 15u) == 0 && (ldx & 7) == 0 && (ldh & 7) == 0;
    swiglu_kernel<<<M, kSwiThreads, 0, static_cast<hipStream_t>(stream)>>>(G, U, K, ldx, H, ldh, vec ? 1 : 0);
    return static_cast<int>(hipGetLastError());
}

int launch_rmsnorm(const uint16_t* X, int M, int K, int ldx, const uint16_t* gamma, float eps, uint16_t* Xn,
                   int ldn, void* stream) {
    rmsnorm_kernel<<<M, kNormThreads, 0, static_cast<hipStream_t>(stream)>>>(X, K, ldx, gamma, eps, Xn, ldn);
    return static_cast<int>(hipGetLastError());
}

int launch_quant_act_token_i8(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, uint8_t* Xq,
                              float* x_scale, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    quant_token_i8_kernel<<<M, kTokThreads, static_cast<size_t>(K) * 2, s>>>(X, M, K, ldx, perm, K / kBlock, Xq,
                                                                           x_scale);
    return static_cast<int>(hipGetLastError());
}

}  // namespace comet
