// comet_w4ax_gemm: Y = X W^T from 4/8-bit activation codes and 4-bit weight
// codes, with exact INT32 partials per 128-channel block and an FP32
// dequantization epilogue that writes fp16.
//
// The method: COMET summary (paperbot-e5f.pages.dev/papers/10460.html),
// abstract, a W4Ax kernel for mixed W4A4/W4A8 blocks; COMET article
// (mmssai.com/?p=43269), section "3.硬件指令集的极限挖掘", 4-bit values widened
// to 8 bits by zero extension with the offset compensated through the scales;
// QUIK blog (deep-paper.org/paper/2310.09259), section "反量化背后的数学", the
// weight-sum term precomputed offline, and section "核融合", dequantize while
// the integer result is still in registers.
//
// gfx950 mapping. CDNA4 has no 4-bit matrix instruction, so every block runs
// on v_mfma_i32_16x16x64_i8 (two per 128-channel block):
//   * weights: one 16-byte load per lane is exactly the lane's B fragment of
//     both MFMAs (fragment order, see comet_w4ax.h). Two-complement nibbles
//     are widened with the high-nibble trick: p & 0xF0F0F0F0 and
//     (p << 4) & 0xF0F0F0F0 give 16 q_w in each byte, sign included;
//   * 4-bit activations: the stored code is u = q + 8; p & 0x0F0F0F0F and
//     (p >> 4) & 0x0F0F0F0F give u in each byte (zero extension). The MFMA
//     accumulator starts at -128 w_sum (= -8 * 16 * w_sum), so it ends at
//     16 P exactly; 8-bit activation blocks start at 0;
//   * epilogue per block: y = fma(s_x * (s_w / 16), float(acc), y). Scaling
//     s_w by 1/16 is exact, so this is (s_x s_w) P with one fused rounding.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "comet_internal.h"

namespace comet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ inline v4i widen_weights_lo(uint4 p) {   // block positions 32g + j
    return v4i{static_cast<int>((p.x << 4) & 0xF0F0F0F0u), static_cast<int>((p.y << 4) & 0xF0F0F0F0u),
               static_cast<int>((p.z << 4) & 0xF0F0F0F0u), static_cast<int>((p.w << 4) & 0xF0F0F0F0u)};
}
__device__ inline v4i widen_weights_hi(uint4 p) {   // block positions 32g + 16 + j
    return v4i{static_cast<int>(p.x & 0xF0F0F0F0u), static_cast<int>(p.y & 0xF0F0F0F0u),
               static_cast<int>(p.z & 0xF0F0F0F0u), static_cast<int>(p.w & 0xF0F0F0F0u)};
}
__device__ inline v4i widen_act_lo(uint4 p) {
    return v4i{static_cast<int>(p.x & 0x0F0F0F0Fu), static_cast<int>(p.y & 0x0F0F0F0Fu),
               static_cast<int>(p.z & 0x0F0F0F0Fu), static_cast<int>(p.w & 0x0F0F0F0Fu)};
}
__device__ inline v4i widen_act_hi(uint4 p) {
    return v4i{static_cast<int>((p.x >> 4) & 0x0F0F0F0Fu), static_cast<int>((p.y >> 4) & 0x0F0F0F0Fu),
               static_cast<int>((p.z >> 4) & 0x0F0F0F0Fu), static_cast<int>((p.w >> 4) & 0x0F0F0F0Fu)};
}
__device__ inline v4i as_v4i(uint4 p) {
    return v4i{static_cast<int>(p.x), static_cast<int>(p.y), static_cast<int>(p.z), static_cast<int>(p.w)};
}

// One workgroup computes a (16 MR) x (64 NR) tile of Y: wave w owns columns
// [n0 + 16 NR w, n0 + 16 NR (w + 1)). MFMA 16x16 output layout: lane l holds
// rows 4 (l / 16) + i, i = 0..3, of column l mod 16.
template <int MR, int NR, bool kDump>
__global__ __launch_bounds__(kThreads) void w4ax_gemm_tile_kernel(GemmProblem p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int row_lo = kDump ? p.m_begin : 0;
    const int row_hi = kDump ? p.m_begin + p.m_count : p.M;
    const int m0 = row_lo + blockIdx.x * 16 * MR;
    const int nw = blockIdx.y * (64 * NR) + wave * (16 * NR);   // first column of this wave
    const int nb = p.nb, nb4 = p.nb4;
    const size_t slab4 = static_cast<size_t>(p.M) * 64;
    const size_t slab8 = static_cast<size_t>(p.M) * 128;
    const uint8_t* xq8 = p.Xq + static_cast<size_t>(nb4) * slab4;

    int arow[MR];          // A-operand row of this lane (clamped into [0, M))
    int orow[MR][4];       // output rows of this lane (clamped for scale loads)
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        arow[r] = min(m0 + 16 * r + l16, p.M - 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) orow[r][i] = min(m0 + 16 * r + 4 * g + i, p.M - 1);
    }

    float y[MR][NR][4];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int c = 0; c < NR; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[r][c][i] = 0.0f;

    for (int b = 0; b < nb; ++b) {
        const bool is4 = b < nb4;
        v4i B0[NR], B1[NR];
        float sw[NR];
        int corr[NR];
#pragma unroll
        for (int c = 0; c < NR; ++c) {
            const int ncol = nw + 16 * c + l16;
            const uint8_t* frag = p.Wq + (static_cast<size_t>(nw / 16 + c) * nb + b) * kFragBytes;
            const uint4 pk = *reinterpret_cast<const uint4*>(frag + 16 * lane);
            B0[c] = widen_weights_lo(pk);
            B1[c] = widen_weights_hi(pk);
            sw[c] = h2f(p.w_scale[static_cast<size_t>(ncol) * nb + b]) * 0.0625f;
            corr[c] = is4 ? -128 * static_cast<int>(p.w_sum[static_cast<size_t>(ncol) * nb + b]) : 0;
        }
        v4i A0[MR], A1[MR];
        float sa[MR][4];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            if (is4) {
                const uint4 pk = *reinterpret_cast<const uint4*>(
                    p.Xq + b * slab4 + static_cast<size_t>(arow[r]) * 64 + 16 * g);
                A0[r] = widen_act_lo(pk);
                A1[r] = widen_act_hi(pk);
            } else {
                const uint4* src = reinterpret_cast<const uint4*>(
                    xq8 + (b - nb4) * slab8 + static_cast<size_t>(arow[r]) * 128 + 32 * g);
                A0[r] = as_v4i(src[0]);
                A1[r] = as_v4i(src[1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sa[r][i] = p.x_scale[static_cast<size_t>(b) * p.M + orow[r][i]];
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) {
#pragma unroll
            for (int c = 0; c < NR; ++c) {
                v4i acc = {corr[c], corr[c], corr[c], corr[c]};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0[r], B0[c], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1[r], B1[c], acc, 0, 0, 0);
                if constexpr (kDump) {
                    const int ncol = nw + 16 * c + l16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = m0 + 16 * r + 4 * g + i;
                        if (row < row_hi)
                            p.P[(static_cast<size_t>(row - row_lo) * p.N + ncol) * nb + b] = acc[i] >> 4;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        y[r][c][i] = __builtin_fmaf(sa[r][i] * sw[c], static_cast<float>(acc[i]), y[r][c][i]);
                }
            }
        }
    }

    if constexpr (!kDump) {
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int c = 0; c < NR; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + 16 * r + 4 * g + i;
                    if (row < row_hi)
                        p.Y[static_cast<size_t>(row) * p.ldy + nw + 16 * c + l16] =
                            __half_as_ushort(__float2half_rn(y[r][c][i]));
                }
    }
}

template <int MR, int NR, bool kDump>
int launch_tile(const GemmProblem& p, int rows, hipStream_t s) {
    dim3 grid((rows + 16 * MR - 1) / (16 * MR), p.N / (64 * NR));
    w4ax_gemm_tile_kernel<MR, NR, kDump><<<grid, kThreads, 0, s>>>(p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

size_t gemm_workspace_bytes(int, int, int, int) { return 0; }

int launch_w4ax_gemm(const GemmProblem& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.P) return launch_tile<1, 2, true>(p, p.m_count, s);
    return launch_tile<2, 2, false>(p, p.M, s);
}

}  // namespace comet
