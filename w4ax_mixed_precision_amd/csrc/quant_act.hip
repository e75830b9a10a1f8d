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
// Mapping on gfx950. One workgroup (4 wave64s) per token row. The row is first
// staged into LDS with coalesced 16-byte loads (HBM sees one contiguous read
// of 2K bytes), then the channel gather by perm happens in LDS. A wave handles
// four blocks at a time, 16 lanes per block; the absmax reduction is a 4-step
// butterfly inside the 16-lane group. Each lane quantizes 8 channels and
// writes one packed dword (4-bit block) or 8 bytes (8-bit block), so the
// stores of a block row are one coalesced 64- or 128-byte segment.
//
// The FP6 variant writes the codes of the 4-bit blocks as FP6 E2M3 values
// (every integer in [-7, 7] is exact in that format), the operand format of
// the gfx950 FP6 matrix instruction, in 16-row tiles laid out exactly as the
// GEMM reads them from LDS (each 16-lane k-group of a wave reads one
// contiguous 256-byte run). A lane codes block positions 32g + 8s .. 32g + 8s
// + 7 (g = group, s = quarter of the group), i.e. 48 bits of the group's
// 192-bit code string, and neighbouring lanes trade 16 bits so that every
// store is a whole dword.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "comet_internal.h"

namespace comet {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLdsRowChannels = 32768;     // 64 KB of fp16 per staged row

// Integer minimum by value (a reference-returning min leaves stack slots behind).
__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

__device__ inline float h2f(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

// q = clamp(rint(x * inv), -qmax, qmax); the product is a single rounded
// multiply (nothing to contract it with) and rint is round-half-even.
__device__ inline int quantize(float x, float inv, float qmax) {
    float r = __builtin_rintf(x * inv);
    r = fminf(qmax, fmaxf(-qmax, r));
    return static_cast<int>(r);
}

// FP6 E2M3 (sign, 2 exponent bits with bias 1, 3 mantissa bits) of an
// integer q in [-7, 7]: |q| = 0..7 encode as 0, 8, 16, 20, 24, 26, 28, 30.
__device__ inline uint32_t fp6_code(int q) {
    const uint32_t a = static_cast<uint32_t>(q < 0 ? -q : q);
    const uint32_t mag = static_cast<uint32_t>((0x1E1C1A1814100800ull >> (8u * a)) & 0xFFu);
    return mag | (q < 0 ? 32u : 0u);
}

template <bool kRowInLds, bool kFp6>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(
    const uint16_t* __restrict__ X, int M, int K, int ldx, const int32_t* __restrict__ perm,
    int nb, int nb4, uint8_t* __restrict__ Xq, float* __restrict__ x_scale) {
    extern __shared__ uint16_t row_lds[];
    const int m = blockIdx.x;
    const uint16_t* xr = X + static_cast<size_t>(m) * ldx;

    if constexpr (kRowInLds) {
        if ((ldx & 7) == 0) {
            for (int c = threadIdx.x * 8; c < K; c += kThreads * 8)
                *reinterpret_cast<uint4*>(row_lds + c) = *reinterpret_cast<const uint4*>(xr + c);
        } else {
            for (int c = threadIdx.x; c < K; c += kThreads) row_lds[c] = xr[c];
        }
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Mp = (M + 15) & ~15;     // FP6 layout: rows padded to whole 16-row tiles
    const int quarter = lane >> 4;    // which of the wave's four blocks
    const int i = lane & 15;          // lane within the block's 16-lane group
    const int stride = gridDim.y * 16;

    for (int b0 = (blockIdx.y * 4 + wave) * 4; b0 < nb; b0 += stride) {
        const int b = b0 + quarter;
        const bool valid = b < nb;
        const int bc = valid ? b : nb - 1;
        const bool is8 = bc >= nb4;
        const int32_t* pb = perm + bc * kBlock;

        // The 8 block positions this lane codes (see the Xq layout).
        int4 p0, p1;
        if (!is8 && kFp6) {
            const int g = i >> 2, s8 = (i & 3) * 8;
            p0 = *reinterpret_cast<const int4*>(pb + 32 * g + s8);
            p1 = *reinterpret_cast<const int4*>(pb + 32 * g + s8 + 4);
        } else if (!is8) {
            const int g = i >> 2, j0 = (i & 3) * 4;
            p0 = *reinterpret_cast<const int4*>(pb + 32 * g + j0);
            p1 = *reinterpret_cast<const int4*>(pb + 32 * g + 16 + j0);
        } else {
            p0 = *reinterpret_cast<const int4*>(pb + 8 * i);
            p1 = *reinterpret_cast<const int4*>(pb + 8 * i + 4);
        }
        const int idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        float v[8];
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[e] = h2f(kRowInLds ? row_lds[idx[e]] : xr[idx[e]]);
            a = fmaxf(a, fabsf(v[e]));
        }
        // absmax over the block's 16 lanes (xor offsets stay inside the group)
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));

        const float qmax = is8 ? 127.0f : 7.0f;
        float inv = 0.0f, s = 0.0f;
        if (a > 0.0f) {
            inv = qmax / a;     // correctly rounded IEEE division
            s = a / qmax;
        }
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = a > 0.0f ? quantize(v[e], inv, qmax) : 0;

        // FP6: this lane's 48 code bits (element e at bits 6e), and the low
        // dword of the neighbouring quarter, taken with every lane active
        uint32_t f_lo = 0, f_hi = 0, f_nlo = 0;
        if constexpr (kFp6) {
            uint64_t f = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) f |= static_cast<uint64_t>(fp6_code(q[e])) << (6 * e);
            f_lo = static_cast<uint32_t>(f);
            f_hi = static_cast<uint32_t>(f >> 32);
            f_nlo = __shfl_xor(f_lo, 1);
        }

        if (valid) {
            if (!is8 && kFp6) {
                // group string: head = bits 0..127 at tile byte 256g + 16r, tail
                // = bits 128..191 at tile byte 1024 + 128g + 8r (r = row in the
                // 16-row tile); quarter s holds bits 48s..48s+47
                const int g = i >> 2, sq = i & 3;
                uint8_t* tile = Xq + static_cast<size_t>(bc) * Mp * 96 + static_cast<size_t>(m >> 4) * 1536;
                uint8_t* head = tile + 256 * g + 16 * (m & 15);
                uint8_t* tail = tile + 1024 + 128 * g + 8 * (m & 15);
                const uint32_t joined = (f_hi & 0xFFFFu) | (f_nlo << 16);   // bits 32..47 + next 0..15
                const uint32_t upper = (f_lo >> 16) | (f_hi << 16);         // bits 16..47
                if (sq == 0) {
                    *reinterpret_cast<uint2*>(head) = make_uint2(f_lo, joined);
                } else if (sq == 1) {
                    *reinterpret_cast<uint32_t*>(head + 8) = upper;
                } else if (sq == 2) {
                    *reinterpret_cast<uint32_t*>(head + 12) = f_lo;
                    *reinterpret_cast<uint32_t*>(tail) = joined;
                } else {
                    *reinterpret_cast<uint32_t*>(tail + 4) = upper;
                }
            } else if (!is8) {
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = static_cast<uint32_t>(q[e] + 8) & 0xF;
                    const uint32_t hi = static_cast<uint32_t>(q[4 + e] + 8) & 0xF;
                    w |= (lo | (hi << 4)) << (8 * e);
                }
                uint8_t* dst = Xq + static_cast<size_t>(bc) * M * 64 + static_cast<size_t>(m) * 64;
                *reinterpret_cast<uint32_t*>(dst + 4 * i) = w;
            } else {
                uint32_t w0 = 0, w1 = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w0 |= (static_cast<uint32_t>(q[e]) & 0xFF) << (8 * e);
                    w1 |= (static_cast<uint32_t>(q[4 + e]) & 0xFF) << (8 * e);
                }
                if constexpr (kFp6) {
                    // 16-row tiles of 2048 bytes: positions 32g + 16h + j of
                    // row r at tile byte 1024h + 256g + 16r + j
                    uint8_t* tile = Xq + static_cast<size_t>(nb4) * Mp * 96 +
                                    static_cast<size_t>(bc - nb4) * Mp * 128 + static_cast<size_t>(m >> 4) * 2048;
                    const int g = i >> 2, h = (i >> 1) & 1;
                    *reinterpret_cast<uint2*>(tile + 1024 * h + 256 * g + 16 * (m & 15) + 8 * (i & 1)) =
                        make_uint2(w0, w1);
                } else {
                    uint8_t* dst = Xq + static_cast<size_t>(nb4) * M * 64 +
                                   static_cast<size_t>(bc - nb4) * M * 128 + static_cast<size_t>(m) * 128;
                    *reinterpret_cast<uint2*>(dst + 8 * i) = make_uint2(w0, w1);
                }
            }
            if (i == 0) x_scale[static_cast<size_t>(bc) * M + m] = s;
        }
    }
}

template <bool kFp6>
int launch(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8, uint8_t* Xq,
           float* x_scale, void* stream) {
    const int nb = K / kBlock;
    const int nb4 = nb - nb8;
    // Enough workgroups to cover the chip even for a handful of rows: split the
    // blocks of a row over gridDim.y workgroups (each stages the whole row).
    const int per_wg = 16;                                  // blocks per workgroup pass
    int groups = 1;
    const int want = 1024;
    while (groups * per_wg < nb && static_cast<long>(M) * groups < want) ++groups;
    dim3 grid(M, groups);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K <= kMaxLdsRowChannels) {
        const size_t lds = static_cast<size_t>(K) * sizeof(uint16_t);
        quant_act_kernel<true, kFp6><<<grid, kThreads, lds, s>>>(X, M, K, ldx, perm, nb, nb4, Xq,
                                                                 x_scale);
    } else {
        quant_act_kernel<false, kFp6><<<grid, kThreads, 0, s>>>(X, M, K, ldx, perm, nb, nb4, Xq,
                                                                x_scale);
    }
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_quant_act(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                     uint8_t* Xq, float* x_scale, void* stream) {
    return launch<false>(X, M, K, ldx, perm, nb8, Xq, x_scale, stream);
}

int launch_quant_act_fp6(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                         uint8_t* Xq, float* x_scale, void* stream) {
    return launch<true>(X, M, K, ldx, perm, nb8, Xq, x_scale, stream);
}

}  // namespace comet
