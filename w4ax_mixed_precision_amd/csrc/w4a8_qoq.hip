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

// ---------------------------------------------------------------------------
// Prefill shapes (M > 64): the W4Ax tiled INT8 kernel's structure, 128 x 128
// output tile per workgroup of four waves (2 x 2, 64 x 64 per wave), two
// workgroups per CU, operands by direct loads into a three-stage LDS ring two
// groups of K ahead. Per group a wave forms B = (u - z) for its four column
// tiles in registers, the INT8 matrix instruction the group sums of its 16
// tiles, and one 24-bit multiply-add per output adds s2 times each into the
// INT32 totals; x_scale s1 is applied once at the end.
//
// LDS stage (25.6 KB): A, 16 pieces of 8 rows x 128 B, slot s = 8 r + (j ^ f)
// with f = ((r >> 1) & 3) | ((piece & 1) << 2) (the 16 lanes of one matrix
// k-group hit 16 bank groups); B, the tile's 8 fragments in lane order; each
// wave's own copy of the tile's 128 s2 | z words (one 4-byte direct load per
// lane, so every wave issues the same 7 loads per group).
// ---------------------------------------------------------------------------
constexpr int kPTM = 128, kPTN = 128;
constexpr int kPLdsA = kPTM * 128;
constexpr int kPLdsB = (kPTN / 16) * kFragBytes;
constexpr int kPLdsSz = 4 * 256;
constexpr int kPStage = kPLdsA + kPLdsB + kPLdsSz;
constexpr int kPLoads = 7;

struct QoqIssue {
    uint32_t a[4];      // 8-row A pieces 4w .. 4w+3
};

__device__ __forceinline__ QoqIssue qoq_issue_offsets(int M, int m0, int wave, int lane) {
    QoqIssue o;
    const int r = lane >> 3;
    const int j0 = (lane & 7) ^ (((r >> 1) & 3) | 0);
    const int j1 = (lane & 7) ^ (((r >> 1) & 3) | 4);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        o.a[k] = static_cast<uint32_t>(imin(m0 + 8 * (4 * wave + k) + r, M - 1)) * 128u + 16u * ((k & 1) ? j1 : j0);
    return o;
}

__device__ __forceinline__ void qoq_tiled_issue(const uint8_t* Xq, const uint8_t* Wu, const uint16_t* s2z, int M,
                                                int N, int nb, int b, int n0, int wave, int lane,
                                                const QoqIssue& o, uint8_t* st) {
    lds_load4(reinterpret_cast<const uint8_t*>(s2z + static_cast<size_t>(b) * N + n0) + 4 * lane,
              st + kPLdsA + kPLdsB + 256 * wave);
    const uint8_t* slab = Xq + static_cast<size_t>(b) * M * 128;
#pragma unroll
    for (int k = 0; k < 4; ++k) lds_load16(slab + o.a[k], st + (4 * wave + k) * kFragBytes);
    const uint8_t* frag = Wu + (static_cast<size_t>(n0 / 16 + 2 * wave) * nb + b) * kFragBytes + 16u * lane;
    lds_load16(frag, st + kPLdsA + (2 * wave) * kFragBytes);
    lds_load16(frag + static_cast<size_t>(nb) * kFragBytes, st + kPLdsA + (2 * wave + 1) * kFragBytes);
}

template <bool kDump>
__device__ __forceinline__ void qoq_tiled_block(const uint8_t* Xq, const uint8_t* Wu, const uint16_t* s2z, int M,
                                                int N, int nb, int b, int n0, int wave, int lane, const QoqIssue& io,
                                                int a8_base, const uint8_t* st, uint8_t* nxt, v4i (&acc)[4][4]) {
    const int wc = wave & 1;
    const int l16 = lane & 15;
    if (b + 2 < nb) qoq_tiled_issue(Xq, Wu, s2z, M, N, nb, b + 2, n0, wave, lane, io, nxt);
    const uint16_t* sz_l = reinterpret_cast<const uint16_t*>(st + kPLdsA + kPLdsB + 256 * wave);
    v4i A0[4], A1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        A0[r] = as_v4i(*reinterpret_cast<const uint4*>(st + a8_base + r * 2 * kFragBytes));
        A1[r] = as_v4i(*reinterpret_cast<const uint4*>(st + ((a8_base + r * 2 * kFragBytes) ^ 16)));
    }
    const v4i zero = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t sz = sz_l[64 * wc + 16 * c + l16];
        const int s2 = static_cast<int>(sz & 0xFFu);
        const uint32_t zrep = ((sz >> 8) & 0xFFu) * 0x01010101u;
        const uint4 pk = *reinterpret_cast<const uint4*>(st + kPLdsA + (4 * wc + c) * kFragBytes + 16 * lane);
        const v4i B0 = minus_zero16(pk, false, zrep);
        const v4i B1 = minus_zero16(pk, true, zrep);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v4i gs = mfma_i8(A0[r], B0, zero);
            gs = mfma_i8(A1[r], B1, gs);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r][c][i] += s2 * gs[i];
        }
    }
    // group b+1's loads are done (only b+2's may still be in flight), and
    // every wave is finished with stage `st` before it is refilled
    if (b + 2 < nb) COMET_VMCNT(kPLoads);
    else COMET_VMCNT(0);
    __builtin_amdgcn_s_barrier();
}

template <bool kDump>
__global__ __launch_bounds__(256, 2) void qoq_tiled_kernel(const uint8_t* __restrict__ Xq,
                                                           const float* __restrict__ x_scale,
                                                           const uint8_t* __restrict__ Wu,
                                                           const uint16_t* __restrict__ s2z,
                                                           const uint16_t* __restrict__ s1, int M, int N, int nb,
                                                           uint16_t* __restrict__ Y, int ldy,
                                                           int32_t* __restrict__ P) {
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[kPStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[kPStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage2[kPStage];
    const int tiles_m = (M + kPTM - 1) / kPTM;
    const int tiles_n = N / kPTN;
    int tm, tn;
    if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
    const int m0 = tm * kPTM, n0 = tn * kPTN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    const QoqIssue io = qoq_issue_offsets(M, m0, wave, lane);
    const int a8_base = (8 * wr + (l16 >> 3)) * kFragBytes +
                        16 * (8 * (l16 & 7) + ((2 * g) ^ ((((l16 & 7) >> 1) & 3) | (((l16 >> 3) & 1) << 2))));
    v4i acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = v4i{0, 0, 0, 0};

    qoq_tiled_issue(Xq, Wu, s2z, M, N, nb, 0, n0, wave, lane, io, stage0);
    if (1 < nb) {
        qoq_tiled_issue(Xq, Wu, s2z, M, N, nb, 1, n0, wave, lane, io, stage1);
        COMET_VMCNT(kPLoads);
    } else {
        COMET_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    for (int b = 0; b < nb; b += 3) {
        qoq_tiled_block<kDump>(Xq, Wu, s2z, M, N, nb, b, n0, wave, lane, io, a8_base, stage0, stage2, acc);
        if (b + 1 < nb)
            qoq_tiled_block<kDump>(Xq, Wu, s2z, M, N, nb, b + 1, n0, wave, lane, io, a8_base, stage1, stage0, acc);
        if (b + 2 < nb)
            qoq_tiled_block<kDump>(Xq, Wu, s2z, M, N, nb, b + 2, n0, wave, lane, io, a8_base, stage2, stage1, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + 64 * wr + 16 * r + 4 * g + i;
            if (row >= M) continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = n0 + 64 * wc + 16 * c + l16;
                if constexpr (kDump) {
                    P[static_cast<size_t>(row) * N + col] = acc[r][c][i];
                } else {
                    const float t = x_scale[row] * h2f(s1[col]);
                    Y[static_cast<size_t>(row) * ldy + col] =
                        __half_as_ushort(__float2half_rn(opaque(t * static_cast<float>(acc[r][c][i]))));
                }
            }
        }
}

template <bool kDump>
int launch_qoq_tiled(const uint8_t* Xq, const float* x_scale, const uint8_t* Wu, const uint16_t* s2z,
                     const uint16_t* s1, int M, int N, int K, uint16_t* Y, int ldy, int32_t* P, hipStream_t st) {
    const int tiles = ((M + kPTM - 1) / kPTM) * (N / kPTN);
    qoq_tiled_kernel<kDump><<<8 * ((tiles + 7) / 8), 256, 0, st>>>(Xq, x_scale, Wu, s2z, s1, M, N, K / kBlock, Y,
                                                                    ldy, P);
    return static_cast<int>(hipGetLastError());
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
    if (M > 64) return launch_qoq_tiled<kDump>(Xq, x_scale, Wu, s2z, s1, M, N, K, Y, ldy, P, st);
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
