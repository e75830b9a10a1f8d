// QoQ W4A8 GEMM (QoQ/QServe article, sections "渐进式分组量化" and "W4A8
// GEMM的核心设计"): the 4-bit weight codes are dequantized to 8-bit integers
// s2 (u - z) in registers, before the matrix instruction, so the whole of K
// accumulates in one exact INT32 sum per output and only a per-(token,
// channel) scale is applied at the end: Y = fp16( fl(s_x s1) * float(P) ).
//
// gfx950 mapping (decode shapes, M <= 64). Weight-streaming kernel in the
// structure of the W4Ax register streaming kernel: a workgroup owns G = 2
// channel groups of 16 outputs, its waves split the 128-channel groups of K,
// a wave's activation words of a group feed both channel groups, and the wave
// partials are added through LDS (integer sums: exact in any order). The
// product of a group is s2 sum(q_a (u - z)); the page dequantizes the codes to
// the 8-bit s2 (u - z) in registers before the multiply. On gfx950 the two
// halves are split between the vector unit and the matrix core, which gives
// the same exact integer at a third of the VALU work: the zero point comes off
// in registers, per 32-bit word of four codes
//     (u - z) = ((u | 0x80808080) - z 0x01010101) ^ 0x80808080
// (u + 128 - z lies in [113, 143], so no byte borrows from the next), the
// INT8 matrix instruction forms sum(q_a (u - z)) (|.| <= 127 15 128), and the
// step multiplies that group sum into the running INT32 total (one 24-bit
// multiply-add per output). The multiply-per-byte form of the page would
// cost two 24-bit multiplies and a borrow-free subtraction per four codes.
#include "comet_internal.h"
#include "device_util.h"
#include "qoq_internal.h"

namespace comet {
namespace {

constexpr int kQG = 2;          // channel groups per workgroup

// The signed differences u - z of the 16 codes in one half of a lane's word.
__device__ __forceinline__ v4i minus_zero16(uint4 p, bool hi, uint32_t zrep) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
    v4i r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t u = (hi ? (w[i] >> 4) : w[i]) & 0x0F0F0F0Fu;
        r[i] = static_cast<int>(((u | 0x80808080u) - zrep) ^ 0x80808080u);
    }
    return r;
}

template <int MR>
struct QoqSlot {
    uint4 w[kQG];       // weight fragment words of the lane
    uint4 a0[MR];       // activation words (positions 32g .. 32g + 15 of the lane's row)
    uint4 a1[MR];       // positions 32g + 16 .. 32g + 31
    uint32_t sz[kQG];   // s2 | z << 8 of the lane's column
};

template <int MR>
__device__ __forceinline__ void qoq_fetch(const uint8_t* Xq, const uint8_t* Wu, const uint16_t* s2z, int M, int N,
                                          int nb, int b, int grp0, int lane, const int (&arow)[MR],
                                          QoqSlot<MR>& sl) {
    const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int j = 0; j < kQG; ++j) {
        sl.w[j] = *reinterpret_cast<const uint4*>(Wu + (static_cast<size_t>(grp0 + j) * nb + b) * kFragBytes +
                                                  16 * lane);
        sl.sz[j] = s2z[static_cast<size_t>(b) * N + (grp0 + j) * 16 + l16];
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        const uint8_t* row = Xq + (static_cast<size_t>(b) * M + arow[r]) * 128 + 32 * g;
        sl.a0[r] = *reinterpret_cast<const uint4*>(row);
        sl.a1[r] = *reinterpret_cast<const uint4*>(row + 16);
    }
}

template <int MR>
__device__ __forceinline__ void qoq_compute(const QoqSlot<MR>& sl, v4i (&acc)[kQG][MR]) {
#pragma unroll
    for (int j = 0; j < kQG; ++j) {
        const int s2 = static_cast<int>(sl.sz[j] & 0xFFu);
        const uint32_t zrep = ((sl.sz[j] >> 8) & 0xFFu) * 0x01010101u;
        const v4i B0 = minus_zero16(sl.w[j], false, zrep);
        const v4i B1 = minus_zero16(sl.w[j], true, zrep);
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            v4i g = mfma_i8(as_v4i(sl.a0[r]), B0, zero);
            g = mfma_i8(as_v4i(sl.a1[r]), B1, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][r][i] += s2 * g[i];
        }
    }
}

template <int MR, int kSplit, bool kDump>
__global__ __launch_bounds__(64 * kSplit) void qoq_gemm_kernel(const uint8_t* __restrict__ Xq,
                                                               const float* __restrict__ x_scale,
                                                               const uint8_t* __restrict__ Wu,
                                                               const uint16_t* __restrict__ s2z,
                                                               const uint16_t* __restrict__ s1, int M, int N,
                                                               int nb, uint16_t* __restrict__ Y, int ldy,
                                                               int32_t* __restrict__ P) {
    constexpr int kD = 2;
    __shared__ int red[kSplit][MR * 4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int units = N / (16 * kQG);
    const int per = (units + 7) / 8;
    const int unit = (blockIdx.x & 7) * per + (blockIdx.x >> 3);   // XCD-aware, as the W4Ax kernels
    if (unit >= units) return;                                      // whole workgroup, before any barrier
    const int grp0 = unit * kQG;
    const int bps = (nb + kSplit - 1) / kSplit;
    const int b_begin = imin(nb, wave * bps);
    const int b_end = imin(nb, b_begin + bps);
    int arow[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) arow[r] = imin(16 * r + l16, M - 1);

    v4i acc[kQG][MR];
#pragma unroll
    for (int j = 0; j < kQG; ++j)
#pragma unroll
        for (int r = 0; r < MR; ++r) acc[j][r] = v4i{0, 0, 0, 0};

    if (b_begin < b_end) {
        QoqSlot<MR> slot[kD];
#pragma unroll
        for (int u = 0; u < kD; ++u)
            if (b_begin + u < b_end) qoq_fetch<MR>(Xq, Wu, s2z, M, N, nb, b_begin + u, grp0, lane, arow, slot[u]);
        for (int b0 = b_begin; b0 < b_end; b0 += kD) {
#pragma unroll
            for (int u = 0; u < kD; ++u) {
                const int b = b0 + u;
                if (b < b_end) {
                    qoq_compute<MR>(slot[u], acc);
                    if (b + kD < b_end) qoq_fetch<MR>(Xq, Wu, s2z, M, N, nb, b + kD, grp0, lane, arow, slot[u]);
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < kQG; ++j) {
        if (j > 0) __syncthreads();       // the previous group's sums are read
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][4 * r + i][lane] = acc[j][r][i];
        __syncthreads();
        const int col = (grp0 + j) * 16 + l16;
        const float sw = h2f(s1[col]);
        for (int q = wave; q < MR * 4; q += kSplit) {
            int v = 0;
#pragma unroll
            for (int w2 = 0; w2 < kSplit; ++w2) v += red[w2][q][lane];
            const int row = 16 * (q >> 2) + 4 * g + (q & 3);
            if (row < M) {
                if constexpr (kDump) {
                    P[static_cast<size_t>(row) * N + col] = v;
                } else {
                    // binary32 product, then fp16: kept apart (opaque) so the
                    // compiler does not fold them into one mixed-precision FMA
                    // that rounds once, straight to fp16
                    const float t = x_scale[row] * sw;
                    Y[static_cast<size_t>(row) * ldy + col] =
                        __half_as_ushort(__float2half_rn(opaque(t * static_cast<float>(v))));
                }
            }
        }
    }
}

template <int MR, bool kDump>
int launch_qoq(const uint8_t* Xq, const float* x_scale, const uint8_t* Wu, const uint16_t* s2z, const uint16_t* s1,
               int M, int N, int K, uint16_t* Y, int ldy, int32_t* P, hipStream_t st) {
    const int units = N / (16 * kQG);
    const int grid = 8 * ((units + 7) / 8);
    const int nb = K / kBlock;
    // eight waves per workgroup while the workgroups alone would not fill the
    // CUs twice over, else four
    if (units < 512)
        qoq_gemm_kernel<MR, 8, kDump><<<grid, 512, 0, st>>>(Xq, x_scale, Wu, s2z, s1, M, N, nb, Y, ldy, P);
    else
        qoq_gemm_kernel<MR, 4, kDump><<<grid, 256, 0, st>>>(Xq, x_scale, Wu, s2z, s1, M, N, nb, Y, ldy, P);
    return static_cast<int>(hipGetLastError());
}

template <bool kDump>
int launch_qoq_rows(const uint8_t* Xq, const float* x_scale, const uint8_t* Wu, const uint16_t* s2z,
                    const uint16_t* s1, int M, int N, int K, uint16_t* Y, int ldy, int32_t* P, hipStream_t st) {
    const int mr = (M + 15) / 16;
    if (mr == 1) return launch_qoq<1, kDump>(Xq, x_scale, Wu, s2z, s1, M, N, K, Y, ldy, P, st);
    if (mr == 2) return launch_qoq<2, kDump>(Xq, x_scale, Wu, s2z, s1, M, N, K, Y, ldy, P, st);
    if (mr == 3) return launch_qoq<3, kDump>(Xq, x_scale, Wu, s2z, s1, M, N, K, Y, ldy, P, st);
    return launch_qoq<4, kDump>(Xq, x_scale, Wu, s2z, s1, M, N, K, Y, ldy, P, st);
}

}  // namespace

int launch_qoq_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wu, const uint16_t* s2z,
                    const uint16_t* s1, int M, int N, int K, uint16_t* Y, int ldy, int32_t* P, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (P) return launch_qoq_rows<true>(Xq, x_scale, Wu, s2z, s1, M, N, K, Y, ldy, P, s);
    return launch_qoq_rows<false>(Xq, x_scale, Wu, s2z, s1, M, N, K, Y, ldy, P, s);
}

}  // namespace comet
