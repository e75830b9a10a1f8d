// comet_w4ax_gemm: Y = X W^T from 4/8-bit activation codes and 4-bit weight
// codes, with exact INT32 partials per 128-channel block and an FP32
// dequantization epilogue that writes fp16.
//
// The method: COMET summary (paperbot-e5f.pages.dev/papers/10460.html),
// abstract, a W4Ax kernel for mixed W4A4/W4A8 blocks with a software pipeline
// that hides load and conversion latency; COMET article (mmssai.com/?p=43269),
// section "3.硬件指令集的极限挖掘", 4-bit values widened to 8 bits by zero
// extension with the offset compensated through the scales, and section
// "2.混合精度计算的动态调度", double buffering and cooperative tile scheduling;
// QUIK blog (deep-paper.org/paper/2310.09259), section "反量化背后的数学", the
// weight-sum term precomputed offline, and section "核融合", dequantize while
// the integer result is still in registers.
//
// gfx950 mapping. CDNA4 has no 4-bit matrix instruction, so every block runs
// on v_mfma_i32_16x16x64_i8, two per 16x16 output tile and 128-channel block:
//   * weights: a lane's 16-byte word of a fragment is its B operand for both
//     MFMAs. Two's-complement nibbles widen with p & 0xF0F0F0F0 and
//     (p << 4) & 0xF0F0F0F0: each byte is 16 q_w, sign included;
//   * 4-bit activations: the stored code is u = q + 8; p & 0x0F0F0F0F and
//     (p >> 4) & 0x0F0F0F0F give u per byte (zero extension). The MFMA
//     accumulator starts at -128 w_sum (= -8 * 16 * w_sum) and so ends at
//     exactly 16 P; 8-bit blocks start at 0 and also end at 16 P;
//   * epilogue per block: y = fma(t, float(acc), y) with t = s_x * (s_w / 16)
//     (scaling by 1/16 is exact).
// On CDNA4 the per-block FP32 epilogue, not the INT8 MFMA, is the binding
// cost of the compute-bound case: a 16-cycle MFMA hides only about two wave64
// VALU instructions. So the kernels keep VALU work per MAC small: the scale
// products t of four 16x16 tiles come from one v_mfma_f32_16x16x1_4b_f32
// (outer products of s_x and s_w on the matrix unit), accumulators stay in
// VGPRs, and 64x64 wave tiles amortize the widening.
#include <utility>

#include "comet_internal.h"
#include "device_util.h"

namespace comet {
namespace {

constexpr int kThreads = 256;

// Accumulator start of a 4-bit block: -16 z w_sum per output (weights enter
// as 16 q_w), so the accumulator ends at exactly 16 (sum(u q_w) - z w_sum);
// symmetric codes have z = 8 for every row, 8-bit blocks start at 0. The
// kernels form it inline from one scalar select (is4 ? -16 w_sum : 0) times
// the zero point of each row: the same value returned as a vector from a
// helper made the compiler schedule the streaming kernels' loads far ahead
// and spill.
#define COMET_ACC_START_ASYM(m, zw)                                                           \
    (v4i{(m) * static_cast<int>((zw) & 0xFFu), (m) * static_cast<int>(((zw) >> 8) & 0xFFu), \
         (m) * static_cast<int>(((zw) >> 16) & 0xFFu), (m) * static_cast<int>((zw) >> 24)})

// ---------------------------------------------------------------------------
// Tiled kernel (prefill shapes): 128 x 128 output tile per workgroup of four
// waves in a 2 x 2 arrangement, 64 x 64 per wave, one workgroup per CU.
//
// Everything a block needs goes from HBM straight into LDS with direct loads
// (global_load_lds: each lane's 16 or 4 bytes land at LDS base + lane * size,
// no registers spent on staging) into a ring of four LDS stages, issued three
// blocks ahead of the compute. Each wave issues the same number of loads per
// block (5 for a 4-bit block, 7 for an 8-bit one), so at the end of block b a
// partial wait (s_waitcnt vmcnt = loads of blocks b+2, b+3) plus a plain
// s_barrier make block b+1 visible while b+2 and b+3 stay in flight.
//
// LDS stage (25.6 KB):
//   A, 4-bit block: 8 pieces of 16 rows x 64 B. Slot s = 4 r + (j ^ ((r >> 2) & 3))
//     holds 16-byte chunk j of row r, so the 16 lanes of one MFMA k-group
//     (16 rows, same chunk) hit 16 different bank groups.
//   A, 8-bit block: 16 pieces of 8 rows x 128 B. Slot s = 8 r + (j ^ f), with
//     f = ((r >> 1) & 3) | ((piece & 1) << 2), same purpose.
//   B: 8 fragments in their stored (lane) order.
//   the block's 128 activation scales (f32), 128 weight scales (fp16 bits) and
//   128 weight sums (int16), converted when read.
// ---------------------------------------------------------------------------

// Three LDS stages (76.8 KB) and a 256-register budget let two workgroups
// share a CU, i.e. two waves per SIMD, which hides the dependency latencies
// of the widen -> MFMA -> convert -> FMA chain far better than one.
#ifndef COMET_TILED_STAGES
#define COMET_TILED_STAGES 3
#endif
#ifndef COMET_TILED_WG_PER_CU
#define COMET_TILED_WG_PER_CU 2
#endif

constexpr int kTM = 128;
constexpr int kTN = 128;
constexpr int kLdsA = kTM * 128;                 // room for an 8-bit block
constexpr int kLdsB = (kTN / 16) * kFragBytes;
constexpr int kLdsSa = kTM * 4;
constexpr int kLdsSw = kTN * 2;
constexpr int kLdsWs = kTN * 2;
constexpr int kStage = kLdsA + kLdsB + kLdsSa + kLdsSw + kLdsWs;
// asymmetric codes: each wave's own copy of the zero points of rows m0 ..
// m0 + 255 (one 4-byte direct load per lane; the tile uses the first 128)
constexpr int kLdsZ = 4 * 256;
constexpr int stage_bytes(bool asym) { return kStage + (asym ? kLdsZ : 0); }
constexpr int kStages = COMET_TILED_STAGES;
static_assert(kStages == 3 || kStages == 4, "the unrolled ring below is written for three or four stages");

// Per-lane byte offsets of the direct loads, fixed for a tile: the block only
// moves the (wave-uniform) base pointers.
struct IssueOffsets {
    uint32_t a4_0, a4_1;               // 4-bit A pieces 2w, 2w+1
    uint32_t a8_0, a8_1, a8_2, a8_3;   // 8-bit A pieces 4w .. 4w+3
    uint32_t sc;                        // scale words: wave 0/1 activation scales, 2 weight scales, 3 sums
    uint32_t z;                         // zero-point word of rows m0 + 4 lane .. + 3 (clamped into [0, Mp))
};

__device__ __forceinline__ IssueOffsets issue_offsets(int M, int m0, int wave, int lane) {
    IssueOffsets o;
    {
        const int r = lane >> 2;
        const int j = (lane & 3) ^ ((r >> 2) & 3);
        o.a4_0 = static_cast<uint32_t>(imin(m0 + 16 * (2 * wave + 0) + r, M - 1)) * 64u + 16u * j;
        o.a4_1 = static_cast<uint32_t>(imin(m0 + 16 * (2 * wave + 1) + r, M - 1)) * 64u + 16u * j;
    }
    {
        const int r = lane >> 3;
        const int j0 = (lane & 7) ^ (((r >> 1) & 3) | 0);
        const int j1 = (lane & 7) ^ (((r >> 1) & 3) | 4);
        o.a8_0 = static_cast<uint32_t>(imin(m0 + 8 * (4 * wave + 0) + r, M - 1)) * 128u + 16u * j0;
        o.a8_1 = static_cast<uint32_t>(imin(m0 + 8 * (4 * wave + 1) + r, M - 1)) * 128u + 16u * j1;
        o.a8_2 = static_cast<uint32_t>(imin(m0 + 8 * (4 * wave + 2) + r, M - 1)) * 128u + 16u * j0;
        o.a8_3 = static_cast<uint32_t>(imin(m0 + 8 * (4 * wave + 3) + r, M - 1)) * 128u + 16u * j1;
    }
    // waves 0 and 1: activation scales of rows 64w + lane (clamped into [0, M));
    // waves 2 and 3: two weight scales / sums per lane
    o.sc = wave < 2 ? static_cast<uint32_t>(imin(m0 + 64 * wave + lane, M - 1)) * 4u : 4u * lane;
    o.z = static_cast<uint32_t>(imin(m0 + 4 * lane, ((M + 15) & ~15) - 4));
    return o;
}

// Direct loads of block b into stage `st`: every wave issues 1 scale word
// load, 2 (4-bit) or 4 (8-bit) A pieces and 2 B fragments, in that order
// (asymmetric codes: first one zero-point word into the wave's own copy).
template <bool kAsym = false>
__device__ __forceinline__ void tiled_issue(const GemmProblem& p, int b, int n0, int wave, int lane,
                                            const IssueOffsets& o, uint8_t* st) {
    const int M = p.M, N = p.N, nb = p.nb, nb4 = p.nb4;
    if constexpr (kAsym)
        lds_load4(p.x_zero + static_cast<size_t>(b) * ((M + 15) & ~15) + o.z, st + kStage + 256 * wave);
    if (wave < 2) {
        lds_load4(reinterpret_cast<const uint8_t*>(p.x_scale + static_cast<size_t>(b) * M) + o.sc,
                  st + kLdsA + kLdsB + 256 * wave);
    } else if (wave == 2) {
        lds_load4(reinterpret_cast<const uint8_t*>(p.w_scale + static_cast<size_t>(b) * N + n0) + o.sc,
                  st + kLdsA + kLdsB + kLdsSa);
    } else {
        lds_load4(reinterpret_cast<const uint8_t*>(p.w_sum + static_cast<size_t>(b) * N + n0) + o.sc,
                  st + kLdsA + kLdsB + kLdsSa + kLdsSw);
    }
    if (b < nb4) {
        const uint8_t* slab = p.Xq + static_cast<size_t>(b) * M * 64;
        lds_load16(slab + o.a4_0, st + (2 * wave + 0) * kFragBytes);
        lds_load16(slab + o.a4_1, st + (2 * wave + 1) * kFragBytes);
    } else {
        const uint8_t* slab = p.Xq + static_cast<size_t>(nb4) * M * 64 + static_cast<size_t>(b - nb4) * M * 128;
        lds_load16(slab + o.a8_0, st + (4 * wave + 0) * kFragBytes);
        lds_load16(slab + o.a8_1, st + (4 * wave + 1) * kFragBytes);
        lds_load16(slab + o.a8_2, st + (4 * wave + 2) * kFragBytes);
        lds_load16(slab + o.a8_3, st + (4 * wave + 3) * kFragBytes);
    }
    const uint8_t* frag = p.Wq + (static_cast<size_t>(n0 / 16 + 2 * wave) * nb + b) * kFragBytes +
                          16u * static_cast<uint32_t>(lane);
    lds_load16(frag, st + kLdsA + (2 * wave) * kFragBytes);
    lds_load16(frag + static_cast<size_t>(nb) * kFragBytes, st + kLdsA + (2 * wave + 1) * kFragBytes);
}

// Loads one wave issues for block b (0 past the last block).
template <bool kAsym = false>
__device__ __forceinline__ int issued_loads(int b, int nb, int nb4) {
    return b >= nb ? 0 : (b < nb4 ? 5 : 7) + (kAsym ? 1 : 0);
}

// Wait until at most `younger` of this wave's direct loads are outstanding
// (the sums of one or two blocks' counts above; any other value waits for
// all, which is never too little).
__device__ __forceinline__ void wait_loads(int younger) {
    switch (younger) {
        case 5: COMET_VMCNT(5); break;
        case 6: COMET_VMCNT(6); break;
        case 7: COMET_VMCNT(7); break;
        case 8: COMET_VMCNT(8); break;
        case 10: COMET_VMCNT(10); break;
        case 12: COMET_VMCNT(12); break;
        case 13: COMET_VMCNT(13); break;
        case 14: COMET_VMCNT(14); break;
        case 16: COMET_VMCNT(16); break;
        default: COMET_VMCNT(0); break;
    }
}

// One block of the tiled kernel: issue block b+3 into `nxt`, compute block b
// from `st`, then make block b+1 visible.
template <bool kDump, bool kAsym = false>
__device__ __forceinline__ void tiled_block(const GemmProblem& p, int b, int m0, int n0, int row_lo,
                                            int row_hi, int wave, int lane, const IssueOffsets& ioff,
                                            int a4_base, int a8_base, const uint8_t* st, uint8_t* nxt,
                                            float (&y)[4][4][4]) {
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    const int nb = p.nb, nb4 = p.nb4, N = p.N;
    if (b + kStages - 1 < nb) tiled_issue<kAsym>(p, b + kStages - 1, n0, wave, lane, ioff, nxt);

    const bool is4 = b < nb4;
    const float* sa_l = reinterpret_cast<const float*>(st + kLdsA + kLdsB);
    const uint16_t* sw_l = reinterpret_cast<const uint16_t*>(st + kLdsA + kLdsB + kLdsSa);
    const int16_t* ws_l = reinterpret_cast<const int16_t*>(st + kLdsA + kLdsB + kLdsSa + kLdsSw);
    // s_x / 16 of this lane's row: the outer product then gives s_x * s_w / 16
    const float sa_lane = sa_l[64 * wr + lane] * 0.0625f;
    const int corr_factor = is4 ? -128 : 0;
    // asymmetric codes: zero points of this lane's output rows 64 wr + 16 r +
    // 4 g + i, from the wave's own copy
    uint32_t zw[4] = {0u, 0u, 0u, 0u};
    if constexpr (kAsym) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            zw[r] = *reinterpret_cast<const uint32_t*>(st + kStage + 256 * wave + 64 * wr + 16 * r + 4 * g);
    }

    // A operands of the four row tiles: row tile r is 1 KB (4-bit) or 2 KB
    // (8-bit) further into the stage; the second half of an 8-bit row is the
    // neighbouring 16-byte slot (offset ^ 16).
    v4i A0[4], A1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (is4) {
            const uint4 pk = *reinterpret_cast<const uint4*>(st + a4_base + r * kFragBytes);
            A0[r] = widen_act_lo(pk);
            A1[r] = widen_act_hi(pk);
        } else {
            A0[r] = as_v4i(*reinterpret_cast<const uint4*>(st + a8_base + r * 2 * kFragBytes));
            A1[r] = as_v4i(*reinterpret_cast<const uint4*>(st + ((a8_base + r * 2 * kFragBytes) ^ 16)));
        }
    }
    // Scale products of column tile c + 1 are formed right after column tile
    // c's epilogue, anchored there by an opaque dependency, so only one or two
    // 16-register t vectors are ever live; their latency hides under the next
    // tile's MFMAs.
    v16f t = {};
    if constexpr (!kDump)
        t = __builtin_amdgcn_mfma_f32_16x16x1f32(sa_lane, h2f(sw_l[64 * wc + l16]), t, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int col = 64 * wc + 16 * c + l16;
        float sw_next = c < 3 ? h2f(sw_l[col + 16]) : 0.0f;
        const uint4 pk = *reinterpret_cast<const uint4*>(st + kLdsA + (4 * wc + c) * kFragBytes + 16 * lane);
        const v4i B0 = widen_weights_lo(pk);
        const v4i B1 = widen_weights_hi(pk);
        const int corr = corr_factor * static_cast<int>(ws_l[col]);
        const v4i cinit = {corr, corr, corr, corr};
        const int zmul = (corr_factor >> 3) * static_cast<int>(ws_l[col]);     // is4 ? -16 w_sum : 0
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v4i acc = mfma_i8(A0[r], B0, kAsym ? COMET_ACC_START_ASYM(zmul, zw[r]) : cinit);
            acc = mfma_i8(A1[r], B1, acc);
            if constexpr (kDump) {
                const int ncol = n0 + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + 64 * wr + 16 * r + 4 * g + i;
                    if (row >= row_lo && row < row_hi)
                        p.P[(static_cast<size_t>(row - row_lo) * N + ncol) * nb + b] = acc[i] >> 4;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[r][c][i] = __builtin_fmaf(t[4 * r + i], static_cast<float>(acc[i]), y[r][c][i]);
            }
        }
        if constexpr (!kDump) {
            if (c < 3) {
                asm volatile("" : "+v"(sw_next), "+v"(y[3][c][3]));
                t = v16f{};
                t = __builtin_amdgcn_mfma_f32_16x16x1f32(sa_lane, sw_next, t, 0, 0, 0);
            }
        }
    }
    // block b+1's loads are done (only b+2 and b+3 may still be in flight),
    // and every wave is finished with stage `st` before it is refilled
    wait_loads(issued_loads<kAsym>(b + 2, nb, nb4) + (kStages == 4 ? issued_loads<kAsym>(b + 3, nb, nb4) : 0));
    __builtin_amdgcn_s_barrier();
}

template <bool kDump, bool kAsym = false>
__global__ __launch_bounds__(kThreads, COMET_TILED_WG_PER_CU) void gemm_tiled_kernel(GemmProblem p) {
    constexpr int kSt = stage_bytes(kAsym);
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[kSt];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[kSt];
    __shared__ __attribute__((aligned(1024))) uint8_t stage2[kSt];
#if COMET_TILED_STAGES == 4
    __shared__ __attribute__((aligned(1024))) uint8_t stage3[kSt];
#endif

    // the partials variant runs the tiles of the full launch (128-row tiles
    // from row 0) that hold rows of [m_begin, m_begin + m_count), and stores
    // only those rows
    const int row_lo = kDump ? p.m_begin : 0;
    const int row_hi = kDump ? p.m_begin + p.m_count : p.M;
    const int tm_lo = row_lo / kTM;
    const int tiles_m = (row_hi + kTM - 1) / kTM - tm_lo;
    const int tiles_n = p.N / kTN;
    int tm, tn;
    if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
    const int m0 = (tm_lo + tm) * kTM;
    const int n0 = tn * kTN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    const int nb = p.nb, nb4 = p.nb4;
    const IssueOffsets ioff = issue_offsets(p.M, m0, wave, lane);

    float y[4][4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[r][c][i] = 0.0f;

    // LDS read offsets of this lane's row-tile-0 A operand inside a stage (see
    // the piece layouts above); row tile r adds r KB (4-bit) or 2r KB (8-bit).
    const int a4_base = 4 * wr * kFragBytes + 16 * (4 * l16 + (g ^ ((l16 >> 2) & 3)));
    const int a8_base = (8 * wr + (l16 >> 3)) * kFragBytes +
                        16 * (8 * (l16 & 7) + ((2 * g) ^ ((((l16 & 7) >> 1) & 3) | (((l16 >> 3) & 1) << 2))));

    // prologue: blocks 0 .. kStages-2 in flight; wait for block 0
    tiled_issue<kAsym>(p, 0, n0, wave, lane, ioff, stage0);
    if (1 < nb) tiled_issue<kAsym>(p, 1, n0, wave, lane, ioff, stage1);
    if (kStages == 4 && 2 < nb) tiled_issue<kAsym>(p, 2, n0, wave, lane, ioff, stage2);
    wait_loads(issued_loads<kAsym>(1, nb, nb4) + (kStages == 4 ? issued_loads<kAsym>(2, nb, nb4) : 0));
    __builtin_amdgcn_s_barrier();

#if COMET_TILED_STAGES == 3
    for (int b = 0; b < nb; b += 3) {
        tiled_block<kDump, kAsym>(p, b, m0, n0, row_lo, row_hi, wave, lane, ioff, a4_base, a8_base, stage0, stage2, y);
        if (b + 1 < nb)
            tiled_block<kDump, kAsym>(p, b + 1, m0, n0, row_lo, row_hi, wave, lane, ioff, a4_base, a8_base, stage1, stage0, y);
        if (b + 2 < nb)
            tiled_block<kDump, kAsym>(p, b + 2, m0, n0, row_lo, row_hi, wave, lane, ioff, a4_base, a8_base, stage2, stage1, y);
    }
#else
    for (int b = 0; b < nb; b += 4) {
        tiled_block<kDump, kAsym>(p, b, m0, n0, row_lo, row_hi, wave, lane, ioff, a4_base, a8_base, stage0, stage3, y);
        if (b + 1 < nb)
            tiled_block<kDump, kAsym>(p, b + 1, m0, n0, row_lo, row_hi, wave, lane, ioff, a4_base, a8_base, stage1, stage0, y);
        if (b + 2 < nb)
            tiled_block<kDump, kAsym>(p, b + 2, m0, n0, row_lo, row_hi, wave, lane, ioff, a4_base, a8_base, stage2, stage1, y);
        if (b + 3 < nb)
            tiled_block<kDump, kAsym>(p, b + 3, m0, n0, row_lo, row_hi, wave, lane, ioff, a4_base, a8_base, stage3, stage2, y);
    }
#endif

    if constexpr (!kDump) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + 64 * wr + 16 * r + 4 * g + i;
                if (row < row_hi) {
                    uint16_t* yrow = p.Y + static_cast<size_t>(row) * p.ldy + n0 + 64 * wc + l16;
#pragma unroll
                    for (int c = 0; c < 4; ++c) yrow[16 * c] = __half_as_ushort(__float2half_rn(y[r][c][i]));
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel (decode shapes, M <= 64): weight-bandwidth bound. A
// workgroup owns one group of 16 output channels; its kSplit waves split the
// blocks (split-K inside the workgroup). Each wave keeps kD blocks in flight
// with a rolling prefetch: register slot u is consumed and immediately refilled
// with the block kD further on, everything a block needs in one slot (weight
// word, activation words, activation scale, weight scale and sum). The kSplit
// partial tiles are summed through LDS in wave order, so the result is
// deterministic, and no global atomics or device-scope fences are needed (on
// a multi-XCD part those write back and invalidate L2).
// ---------------------------------------------------------------------------

template <int MR>
struct StreamSlot {
    uint4 w;          // weight fragment word of this lane
    uint4 a0[MR];     // activation words (a1 only used by 8-bit blocks)
    uint4 a1[MR];
    float sa;         // activation scale of row `srow`
    uint32_t hs;      // weight scale bits of column `ncol`
    int32_t ws;       // weight sum of column `ncol`
    uint32_t zw[MR];  // asymmetric codes: zero points of rows 16r + 4g .. 16r + 4g + 3
};

// Zero points of the four output rows 16r + 4g + i (i = 0..3) of row tile r,
// one byte each, as one aligned word of x_zero [nb][Mp].
__device__ __forceinline__ uint32_t zero_word(const GemmProblem& p, int b, int r, int g) {
    const int Mp = (p.M + 15) & ~15;
    return *reinterpret_cast<const uint32_t*>(p.x_zero + static_cast<size_t>(b) * Mp + 16 * r + 4 * g);
}



// The partials variant of a streaming kernel: the exact P of block b for this
// lane's four outputs of row tile r (rows 16r + 4g .. 16r + 4g + 3, column
// `col`), from the accumulator (16 P), in place of the epilogue. Rows outside
// [m_begin, m_begin + m_count) are not written.
__device__ __forceinline__ void dump_tile(const GemmProblem& p, int b, int col, int r, int g, const v4i& acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * r + 4 * g + i;
        if (row >= p.m_begin && row < p.m_begin + p.m_count)
            p.P[(static_cast<size_t>(row - p.m_begin) * p.N + col) * p.nb + b] = acc[i] >> 4;
    }
}

// Everything block b needs except the weight word: activation words of the
// lane's rows, activation scale of row `srow`, weight scale and sum of its
// column. MR == 1 issues exactly five loads.
template <int MR, bool kAsym = false>
__device__ __forceinline__ void stream_fetch_aux(const GemmProblem& p, Rsrc xq, int b, int grp, int lane, int srow,
                                                 const int (&arow)[MR], StreamSlot<MR>& sl) {
    const int g = lane >> 4, l16 = lane & 15;
    const int M = p.M, N = p.N, nb4 = p.nb4;
    const int ncol = grp * 16 + l16;
    sl.sa = p.x_scale[static_cast<size_t>(b) * M + srow];
    sl.hs = p.w_scale[static_cast<size_t>(b) * N + ncol];
    sl.ws = p.w_sum[static_cast<size_t>(b) * N + ncol];
    // branch-free: 4-bit rows are 64 bytes at 16g, 8-bit rows 128 bytes at
    // 32g (+16 for the second word). A 4-bit block has no second word: its
    // load takes an offset past the buffer, which returns zeros without a
    // memory access, so the load count stays fixed at no cache traffic.
    const bool is4 = b < nb4;
    const uint32_t M32 = static_cast<uint32_t>(M), ub = static_cast<uint32_t>(b), nb4u = static_cast<uint32_t>(nb4);
    const uint32_t slab = is4 ? ub * M32 * 64u : nb4u * M32 * 64u + (ub - nb4u) * M32 * 128u;
    const uint32_t rstride = is4 ? 64u : 128u;
    const uint32_t cofs = is4 ? 16u * g : 32u * g;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        const uint32_t off = slab + static_cast<uint32_t>(arow[r]) * rstride + cofs;
        sl.a0[r] = buf_load16(xq, off);
        sl.a1[r] = buf_load16(xq, is4 ? kOutOfRange : off + 16u);
    }
    if constexpr (kAsym) {
#pragma unroll
        for (int r = 0; r < MR; ++r) sl.zw[r] = zero_word(p, b, r, g);
    }
}

template <int MR, bool kAsym = false>
__device__ __forceinline__ void stream_fetch(const GemmProblem& p, Rsrc xq, int b, int grp, int lane, int srow,
                                             const int (&arow)[MR], StreamSlot<MR>& sl) {
    sl.w = *reinterpret_cast<const uint4*>(p.Wq + (static_cast<size_t>(grp) * p.nb + b) * kFragBytes + 16 * lane);
    stream_fetch_aux<MR, kAsym>(p, xq, b, grp, lane, srow, arow, sl);
}

// Buffer resource over the INT4-layout activation codes (M rows; M <= 64 here).
__device__ __forceinline__ Rsrc stream_xq_rsrc(const GemmProblem& p) {
    const uint32_t M = static_cast<uint32_t>(p.M), nb4 = static_cast<uint32_t>(p.nb4);
    const uint32_t nb8 = static_cast<uint32_t>(p.nb) - nb4;
    return make_rsrc(p.Xq, M * (64u * nb4 + 128u * nb8));
}

// One block from a slot. `valid` is false for the clamped refetches past the
// wave's last block: they get a zero scale product, which adds exactly zero.
template <int MR, bool kAsym = false, bool kDump = false>
__device__ __forceinline__ void stream_compute(bool valid, bool is4, const StreamSlot<MR>& sl,
                                               float (&y)[MR][4], const GemmProblem& p, int b, int col) {
    const v4i B0 = widen_weights_lo(sl.w);
    const v4i B1 = widen_weights_hi(sl.w);
    const float sw = valid ? h2f(static_cast<uint16_t>(sl.hs)) * 0.0625f : 0.0f;
    const int corr = is4 ? -128 * sl.ws : 0;
    const v4i cinit = {corr, corr, corr, corr};
    const int zmul = is4 ? -16 * sl.ws : 0;
    // t[4r + i] = s_x[row 16r + 4g + i] * s_w[col] / 16 for the MR row tiles
    v16f t = {};
    t = __builtin_amdgcn_mfma_f32_16x16x1f32(sl.sa, sw, t, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        v4i A0, A1;
        if (is4) {
            A0 = widen_act_lo(sl.a0[r]);
            A1 = widen_act_hi(sl.a0[r]);
        } else {
            A0 = as_v4i(sl.a0[r]);
            A1 = as_v4i(sl.a1[r]);
        }
        v4i acc = mfma_i8(A0, B0, kAsym ? COMET_ACC_START_ASYM(zmul, sl.zw[r]) : cinit);
        acc = mfma_i8(A1, B1, acc);
        if constexpr (kDump) {
            if (valid) dump_tile(p, b, col, r, (threadIdx.x & 63) >> 4, acc);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                y[r][i] = __builtin_fmaf(t[4 * r + i], static_cast<float>(acc[i]), y[r][i]);
        }
    }
}

template <int MR, int kD, int kSplit, bool kAsym = false, bool kDump = false>
__global__ __launch_bounds__(64 * kSplit) void gemm_stream_kernel(GemmProblem p) {
    __shared__ float red[kSplit][MR * 4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // 16-channel group: workgroup w runs on XCD w mod 8, and each XCD takes a
    // contiguous range of groups, so neighbouring groups (whose weight scales
    // and sums share cache lines) are read through one L2
    const int per = (p.N / 16 + 7) / 8;
    const int grp = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (grp >= p.N / 16) return;    // whole workgroup, before any barrier
    const int nb = p.nb, nb4 = p.nb4, M = p.M;
    const int bps = (nb + kSplit - 1) / kSplit;
    const int b_begin = imin(nb, wave * bps);
    const int b_end = imin(nb, b_begin + bps);

    int arow[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) arow[r] = imin(16 * r + l16, M - 1);
    const int srow = imin(lane, M - 1);    // row whose scale this lane feeds the outer product
    const Rsrc xq = stream_xq_rsrc(p);
    float y[MR][4];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[r][i] = 0.0f;

    if (b_begin < b_end) {
        const int last = b_end - 1;
        StreamSlot<MR> slot[kD];
#pragma unroll
        for (int u = 0; u < kD; ++u)
            stream_fetch<MR, kAsym>(p, xq, imin(b_begin + u, last), grp, lane, srow, arow, slot[u]);
        for (int b0 = b_begin; b0 < b_end; b0 += kD) {
#pragma unroll
            for (int u = 0; u < kD; ++u) {
                const int b = b0 + u;
                stream_compute<MR, kAsym, kDump>(b < b_end, imin(b, last) < nb4, slot[u], y, p, b, grp * 16 + l16);
                if (b0 + kD < b_end)
                    stream_fetch<MR, kAsym>(p, xq, imin(b + kD, last), grp, lane, srow, arow, slot[u]);
            }
        }
    }
    if constexpr (kDump) return;

#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][4 * r + i][lane] = y[r][i];
    __syncthreads();
    // the (row tile, i) slots are shared out over the waves; each sums the
    // K-parts in wave order
    for (int q = wave; q < MR * 4; q += kSplit) {
        float v = red[0][q][lane];
#pragma unroll
        for (int w2 = 1; w2 < kSplit; ++w2) v += red[w2][q][lane];
        const int row = 16 * (q >> 2) + 4 * g + (q & 3);
        if (row < M) p.Y[static_cast<size_t>(row) * p.ldy + grp * 16 + l16] = __half_as_ushort(__float2half_rn(v));
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel for two to four row tiles (17 <= M <= 64): a wave's
// activation words of a block feed G channel groups. In the one-group kernel
// above every group's waves load all M rows of every block, so at M = 64 the
// activation stream out of L2 is four times the weight stream out of HBM and
// binds the kernel. Here a workgroup owns G neighbouring groups (16 G output
// channels) and its kSplit waves split the blocks as above; a wave loads the
// activation words of a block once, widens them in place, and runs them
// against the G weight fragments of the block. Per wave and block: G weight
// words, MR activation words (two for an 8-bit block), one activation scale,
// G weight scales and sums; the G partial tiles are summed through LDS one
// group after another, in wave order.
// ---------------------------------------------------------------------------

template <int MR, int G>
struct StreamSlotG {
    uint4 w[G];
    uint4 a0[MR];
    uint4 a1[MR];
    float sa;
    uint32_t hs[G];
    int32_t ws[G];
    uint32_t zw[MR];
};

template <int MR, int G, bool kAsym = false>
__device__ __forceinline__ void stream_fetch_g(const GemmProblem& p, Rsrc xq, int b, int grp0, int lane, int srow,
                                               const int (&arow)[MR], StreamSlotG<MR, G>& sl) {
    const int g = lane >> 4, l16 = lane & 15;
    const int M = p.M, N = p.N, nb4 = p.nb4;
#pragma unroll
    for (int j = 0; j < G; ++j)
        sl.w[j] = *reinterpret_cast<const uint4*>(p.Wq + (static_cast<size_t>(grp0 + j) * p.nb + b) * kFragBytes +
                                                  16 * lane);
    sl.sa = p.x_scale[static_cast<size_t>(b) * M + srow];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int ncol = (grp0 + j) * 16 + l16;
        sl.hs[j] = p.w_scale[static_cast<size_t>(b) * N + ncol];
        sl.ws[j] = p.w_sum[static_cast<size_t>(b) * N + ncol];
    }
    const bool is4 = b < nb4;
    const uint32_t M32 = static_cast<uint32_t>(M), ub = static_cast<uint32_t>(b), nb4u = static_cast<uint32_t>(nb4);
    const uint32_t slab = is4 ? ub * M32 * 64u : nb4u * M32 * 64u + (ub - nb4u) * M32 * 128u;
    const uint32_t rstride = is4 ? 64u : 128u;
    const uint32_t cofs = is4 ? 16u * g : 32u * g;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        const uint32_t off = slab + static_cast<uint32_t>(arow[r]) * rstride + cofs;
        sl.a0[r] = buf_load16(xq, off);
        sl.a1[r] = buf_load16(xq, is4 ? kOutOfRange : off + 16u);
    }
    if constexpr (kAsym) {
#pragma unroll
        for (int r = 0; r < MR; ++r) sl.zw[r] = zero_word(p, b, r, g);
    }
}

template <int MR, int G, bool kAsym = false, bool kDump = false>
__device__ __forceinline__ void stream_compute_g(bool valid, bool is4, StreamSlotG<MR, G>& sl,
                                                 float (&y)[G][MR][4], const GemmProblem& p, int b, int grp0) {
    // 4-bit rows: the one word holds both halves of the lane's 32 positions;
    // widen it in place into the two operand words an 8-bit row loads
    if (is4) {
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const v4i lo = widen_act_lo(sl.a0[r]);
            const v4i hi = widen_act_hi(sl.a0[r]);
            sl.a0[r] = uint4{static_cast<uint32_t>(lo[0]), static_cast<uint32_t>(lo[1]),
                             static_cast<uint32_t>(lo[2]), static_cast<uint32_t>(lo[3])};
            sl.a1[r] = uint4{static_cast<uint32_t>(hi[0]), static_cast<uint32_t>(hi[1]),
                             static_cast<uint32_t>(hi[2]), static_cast<uint32_t>(hi[3])};
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const v4i B0 = widen_weights_lo(sl.w[j]);
        const v4i B1 = widen_weights_hi(sl.w[j]);
        const float sw = valid ? h2f(static_cast<uint16_t>(sl.hs[j])) * 0.0625f : 0.0f;
        const int corr = is4 ? -128 * sl.ws[j] : 0;
        const v4i cinit = {corr, corr, corr, corr};
        const int zmul = is4 ? -16 * sl.ws[j] : 0;
        v16f t = {};
        t = __builtin_amdgcn_mfma_f32_16x16x1f32(sl.sa, sw, t, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            v4i acc = mfma_i8(as_v4i(sl.a0[r]), B0, kAsym ? COMET_ACC_START_ASYM(zmul, sl.zw[r]) : cinit);
            acc = mfma_i8(as_v4i(sl.a1[r]), B1, acc);
            if constexpr (kDump) {
                const int lane = threadIdx.x & 63;
                if (valid) dump_tile(p, b, (grp0 + j) * 16 + (lane & 15), r, lane >> 4, acc);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[j][r][i] = __builtin_fmaf(t[4 * r + i], static_cast<float>(acc[i]), y[j][r][i]);
            }
        }
    }
}

template <int MR, int G, int kD, int kSplit, bool kAsym = false, bool kDump = false>
__global__ __launch_bounds__(64 * kSplit) void gemm_stream_g_kernel(GemmProblem p) {
    __shared__ float red[kSplit][MR * 4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // unit of G groups, XCD-aware as in the one-group kernel
    const int units = p.N / (16 * G);
    const int per = (units + 7) / 8;
    const int unit = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (unit >= units) return;      // whole workgroup, before any barrier
    const int grp0 = unit * G;
    const int nb = p.nb, nb4 = p.nb4, M = p.M;
    const int bps = (nb + kSplit - 1) / kSplit;
    const int b_begin = imin(nb, wave * bps);
    const int b_end = imin(nb, b_begin + bps);

    int arow[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) arow[r] = imin(16 * r + l16, M - 1);
    const int srow = imin(lane, M - 1);
    const Rsrc xq = stream_xq_rsrc(p);
    float y[G][MR][4];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[j][r][i] = 0.0f;

    if (b_begin < b_end) {
        const int last = b_end - 1;
        StreamSlotG<MR, G> slot[kD];
#pragma unroll
        for (int u = 0; u < kD; ++u)
            stream_fetch_g<MR, G, kAsym>(p, xq, imin(b_begin + u, last), grp0, lane, srow, arow, slot[u]);
        for (int b0 = b_begin; b0 < b_end; b0 += kD) {
#pragma unroll
            for (int u = 0; u < kD; ++u) {
                const int b = b0 + u;
                stream_compute_g<MR, G, kAsym, kDump>(b < b_end, imin(b, last) < nb4, slot[u], y, p, b, grp0);
                if (b0 + kD < b_end)
                    stream_fetch_g<MR, G, kAsym>(p, xq, imin(b + kD, last), grp0, lane, srow, arow, slot[u]);
            }
        }
    }
    if constexpr (kDump) return;

#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (j > 0) __syncthreads();     // the previous group's sums are read
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][4 * r + i][lane] = y[j][r][i];
        __syncthreads();
        for (int q = wave; q < MR * 4; q += kSplit) {
            float v = red[0][q][lane];
#pragma unroll
            for (int w2 = 1; w2 < kSplit; ++w2) v += red[w2][q][lane];
            const int row = 16 * (q >> 2) + 4 * g + (q & 3);
            if (row < M)
                p.Y[static_cast<size_t>(row) * p.ldy + (grp0 + j) * 16 + l16] = __half_as_ushort(__float2half_rn(v));
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel with the weight fragments staged in LDS (decode, M <= 16,
// nb == NBW * kSplit). The register kernel above holds every in-flight block
// in VGPRs, which caps a CU at about 64 KB of weights in flight. Here each
// wave keeps the fragments of its next kR blocks in flight as direct loads
// into its own 8 KB LDS ring (no VGPRs held) and only the activation words
// and scales of its next kA blocks in registers, so a CU keeps twice the
// weight bytes in flight at the same occupancy. Block order, per-wave sums
// and their reduction are those of the register kernel, so Y is identical.
// The loop is unrolled at compile time: loads complete in issue order and
// the wait before block i is a constant of the issue pattern.
// ---------------------------------------------------------------------------

constexpr int kRingA = 4;   // blocks of activation words and scales in registers
constexpr int kRingR = 8;   // fragments in flight into the LDS ring
// stream_fetch_aux<1>: two activation words, three scalars (and the
// zero-point word with asymmetric codes)
constexpr int aux_loads(bool asym) { return asym ? 6 : 5; }

// Loads issued after block i's aux loads: fragment i+kR-kA, then for each
// block j in (i, i+kA) its aux loads and fragment j+kR-kA (none past nbw).
constexpr int lds_loads_after(int i, int nbw, bool asym) {
    int after = (i + kRingR - kRingA < nbw) ? 1 : 0;
    for (int j = i + 1; j < i + kRingA; ++j) {
        if (j < nbw) after += aux_loads(asym);
        if (j + kRingR - kRingA < nbw) after += 1;
    }
    return after;
}

template <class F, int... Is>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}

template <int NBW, int kSplit, bool kAsym = false, bool kDump = false>
__global__ __launch_bounds__(64 * kSplit) void gemm_stream_lds_kernel(GemmProblem p) {
    constexpr int MR = 1;
    __shared__ float red[kSplit][4][64];
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kSplit][kRingR][kFragBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int per = (p.N / 16 + 7) / 8;
    const int grp = (blockIdx.x & 7) * per + (blockIdx.x >> 3);   // as in the register kernel
    if (grp >= p.N / 16) return;
    const int nb4 = p.nb4, M = p.M;
    const int b_begin = wave * NBW;
    int arow[MR];
    arow[0] = imin(l16, M - 1);
    const int srow = imin(lane, M - 1);
    const Rsrc wq = make_rsrc(p.Wq, static_cast<uint32_t>(p.N / 16) * p.nb * kFragBytes);
    const Rsrc xq = stream_xq_rsrc(p);
    const uint32_t wbase = (static_cast<uint32_t>(grp) * p.nb + b_begin) * kFragBytes;
    uint8_t* my = &ring[wave][0][0];
    auto fragment = [&](int i) {
        lds_buf16(wq, 16u * lane, wbase + i * kFragBytes, my + (i % kRingR) * kFragBytes);
    };

    float y[MR][4] = {};
    StreamSlot<MR> slot[kRingA];
    // prologue in the steady-state order: fragments 0 .. kR-kA-1, then for
    // k < kA the aux loads of block k followed by fragment k + kR - kA
#pragma unroll
    for (int i = 0; i < kRingR - kRingA; ++i)
        if (i < NBW) fragment(i);
#pragma unroll
    for (int k = 0; k < kRingA; ++k) {
        if (k < NBW) stream_fetch_aux<MR, kAsym>(p, xq, b_begin + k, grp, lane, srow, arow, slot[k]);
        if (k + kRingR - kRingA < NBW) fragment(k + kRingR - kRingA);
    }
    unroll_seq([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        COMET_VMCNT(lds_loads_after(i, NBW, kAsym));
        StreamSlot<MR>& sl = slot[i % kRingA];
        sl.w = *reinterpret_cast<const uint4*>(my + (i % kRingR) * kFragBytes + 16 * lane);
        stream_compute<MR, kAsym, kDump>(true, b_begin + i < nb4, sl, y, p, b_begin + i, grp * 16 + l16);
        // the ring slot just read is refilled only after its word is used
        if (i + kRingA < NBW) stream_fetch_aux<MR, kAsym>(p, xq, b_begin + i + kRingA, grp, lane, srow, arow, sl);
        if (i + kRingR < NBW) fragment(i + kRingR);
    }, std::make_integer_sequence<int, NBW>{});
    if constexpr (kDump) return;

#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][i][lane] = y[0][i];
    __syncthreads();
    for (int q = wave; q < 4; q += kSplit) {
        float v = red[0][q][lane];
#pragma unroll
        for (int w2 = 1; w2 < kSplit; ++w2) v += red[w2][q][lane];
        const int row = 4 * g + q;
        if (row < M) p.Y[static_cast<size_t>(row) * p.ldy + grp * 16 + l16] = __half_as_ushort(__float2half_rn(v));
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel for two to four row tiles with the weight fragments in an
// LDS ring (nb == NBW * kSplit). At M = 64 a block's activation words take 32
// registers per wave, which leaves room for only two blocks in flight in the
// register kernels: about 4 MB of weights in flight across the chip, far too
// little to cover HBM latency. Here each wave owns G neighbouring channel
// groups (as in gemm_stream_g_kernel: its activation words feed G weight
// fragments) and keeps the fragments of its next kRR blocks in flight as
// direct loads into its own LDS ring (G KB per block, no registers held);
// activation words and scales run kRA blocks ahead in registers. Loads
// complete in issue order, so the wait before block i is a constant of the
// issue pattern, as in gemm_stream_lds_kernel.
// ---------------------------------------------------------------------------

template <int MR, int G, bool kAsym = false>
struct AuxSlotG {
    uint4 a0[MR];
    uint4 a1[MR];
    float sa;
    uint32_t hs[G];
    int32_t ws[G];
    uint32_t zw[kAsym ? MR : 1];
};

// Loads of one block's aux fetch: two activation words per row tile, the
// activation scale, G weight scales and G weight sums (and a zero-point word
// per row tile with asymmetric codes).
template <int MR, int G, bool kAsym>
constexpr int aux_loads_g() { return 2 * MR + 1 + 2 * G + (kAsym ? MR : 0); }

// Loads issued after block i's aux loads (see the issue order in the kernel).
template <int MR, int G, int kRA, int kRR, bool kAsym>
constexpr int lds_g_loads_after(int i, int nbw) {
    int after = (i + kRR - kRA < nbw) ? G : 0;
    for (int j = i + 1; j < i + kRA; ++j) {
        if (j < nbw) after += aux_loads_g<MR, G, kAsym>();
        if (j + kRR - kRA < nbw) after += G;
    }
    return after;
}

template <int MR, int G, bool kAsym = false>
__device__ __forceinline__ void stream_fetch_aux_g(const GemmProblem& p, Rsrc xq, int b, int grp0, int lane,
                                                   int srow, const int (&arow)[MR], AuxSlotG<MR, G, kAsym>& sl) {
    const int g = lane >> 4, l16 = lane & 15;
    const int M = p.M, N = p.N, nb4 = p.nb4;
    const bool is4 = b < nb4;
    const uint32_t M32 = static_cast<uint32_t>(M), ub = static_cast<uint32_t>(b), nb4u = static_cast<uint32_t>(nb4);
    const uint32_t slab = is4 ? ub * M32 * 64u : nb4u * M32 * 64u + (ub - nb4u) * M32 * 128u;
    const uint32_t rstride = is4 ? 64u : 128u;
    const uint32_t cofs = is4 ? 16u * g : 32u * g;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        const uint32_t off = slab + static_cast<uint32_t>(arow[r]) * rstride + cofs;
        sl.a0[r] = buf_load16(xq, off);
        sl.a1[r] = buf_load16(xq, is4 ? kOutOfRange : off + 16u);
    }
    sl.sa = p.x_scale[static_cast<size_t>(b) * M + srow];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const int ncol = (grp0 + j) * 16 + l16;
        sl.hs[j] = p.w_scale[static_cast<size_t>(b) * N + ncol];
        sl.ws[j] = p.w_sum[static_cast<size_t>(b) * N + ncol];
    }
    if constexpr (kAsym) {
#pragma unroll
        for (int r = 0; r < MR; ++r) sl.zw[r] = zero_word(p, b, r, g);
    }
}

// `half_j` names the group of which this workgroup owns only the channels of
// lanes with `own` set (-1: none); partials of the other half are not stored.
template <int MR, int G, bool kAsym = false, bool kDump = false>
__device__ __forceinline__ void stream_compute_lds_g(bool is4, AuxSlotG<MR, G, kAsym>& sl, const uint8_t* frags, int lane,
                                                     float (&y)[G][MR][4], const GemmProblem& p, int b, int grp0,
                                                     int half_j = -1, bool own = true) {
    // branch-free operand words (a branch on the block kind splits the
    // straight-line block sequence, and the compiler then waits for every
    // outstanding load before the next LDS read): a 4-bit row's second word
    // was loaded as zero, so ((a0 >> 4) & hi4) | a1 (a shift and one and-or)
    // is the high nibbles of a0 for a 4-bit block and a1 for an 8-bit one
    // (three operations per word pair instead of five: LLaMA-70B decode,
    // M = 64, 256 fewer vector instructions per wave)
    const uint32_t mask = is4 ? 0x0F0F0F0Fu : 0xFFFFFFFFu;
    const uint32_t hi4 = is4 ? 0x0F0F0F0Fu : 0u;
    v4i A0[MR], A1[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        const uint4 a = sl.a0[r], c = sl.a1[r];
        A0[r] = v4i{static_cast<int>(a.x & mask), static_cast<int>(a.y & mask), static_cast<int>(a.z & mask),
                    static_cast<int>(a.w & mask)};
        A1[r] = v4i{static_cast<int>(((a.x >> 4) & hi4) | c.x), static_cast<int>(((a.y >> 4) & hi4) | c.y),
                    static_cast<int>(((a.z >> 4) & hi4) | c.z), static_cast<int>(((a.w >> 4) & hi4) | c.w)};
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(frags + j * kFragBytes + 16 * lane);
        const v4i B0 = widen_weights_lo(w);
        const v4i B1 = widen_weights_hi(w);
        const float sw = h2f(static_cast<uint16_t>(sl.hs[j])) * 0.0625f;
        const int corr = is4 ? -128 * sl.ws[j] : 0;
        const v4i cinit = {corr, corr, corr, corr};
        const int zmul = is4 ? -16 * sl.ws[j] : 0;
        v16f t = {};
        t = __builtin_amdgcn_mfma_f32_16x16x1f32(sl.sa, sw, t, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            v4i acc = mfma_i8(A0[r], B0, kAsym ? COMET_ACC_START_ASYM(zmul, sl.zw[r]) : cinit);
            acc = mfma_i8(A1[r], B1, acc);
            if constexpr (kDump) {
                if (j != half_j || own) dump_tile(p, b, (grp0 + j) * 16 + (lane & 15), r, lane >> 4, acc);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[j][r][i] = __builtin_fmaf(t[4 * r + i], static_cast<float>(acc[i]), y[j][r][i]);
            }
        }
    }
}

// H > 0: half-group units. Unit u owns the half-groups [H u, H u + H) (H odd,
// half-group h = channels 8 (h mod 2) .. + 8 of group h / 2), so 2 N / (16 H)
// units split the channels evenly over that many CUs where whole groups would
// not (N = 10240: 640 groups are 2.5 per CU; 256 units of five halves). The
// unit's G = (H + 1) / 2 groups are whole but one, whose other half belongs to
// the neighbouring unit: its lanes of the other half load nothing (an offset
// past the buffer reads zeros, no memory access) and store nothing. A group's
// columns depend only on its own weight columns, so the owned half is exact.
template <int MR, int G, int NBW, int kSplit, int kRA, int kRR, bool kAsym = false, bool kDump = false, int H = 0>
__global__ __launch_bounds__(64 * kSplit) __attribute__((amdgpu_waves_per_eu(2))) void gemm_stream_lds_g_kernel(GemmProblem p) {
    static_assert(H == 0 || (H % 2 == 1 && G == (H + 1) / 2), "a unit of H half-groups spans (H + 1) / 2 groups");
    // two LDS objects: the compiler can then tell ring reads from other LDS
    // accesses and waits only for the direct loads a read depends on (with
    // one object it waits for every outstanding load before each read)
    // the wait before block i counts the loads issued after block i's aux
    // loads, so block i's fragments must have gone out before them
    static_assert(kRR > kRA, "the fragments of a block are issued before its aux loads");
    // at most 63 loads may be outstanding behind a wait
    static_assert(lds_g_loads_after<MR, G, kRA, kRR, kAsym>(0, NBW) <= 63, "vmcnt range");
    __shared__ float red[kSplit][MR * 4][64];
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kSplit][kRR * G][kFragBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int units = H > 0 ? p.N / (8 * H) : p.N / (16 * G);
    const int per = (units + 7) / 8;
    const int unit = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (unit >= units) return;      // whole workgroup, before any barrier
    const int grp0 = H > 0 ? (H * unit) / 2 : unit * G;
    // the shared group: first of the unit when it starts on a second half,
    // else its last (first half)
    const int hh = H > 0 ? (H * unit) & 1 : 0;
    const int half_j = H > 0 ? (hh ? 0 : G - 1) : -1;
    const bool own = ((lane & 15) >> 3) == hh;
    const int nb4 = p.nb4, M = p.M;
    const int b_begin = wave * NBW;
    int arow[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) arow[r] = imin(16 * r + l16, M - 1);
    const int srow = imin(lane, M - 1);
    const Rsrc wq = make_rsrc(p.Wq, static_cast<uint32_t>(p.N / 16) * p.nb * kFragBytes);
    const Rsrc xq = stream_xq_rsrc(p);
    uint8_t* my = &ring[wave][0][0];
    // the G fragments of block i (channel groups grp0 .. grp0 + G - 1) into
    // ring slot i mod kRR
    auto fragments = [&](int i) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t off = (static_cast<uint32_t>(grp0 + j) * p.nb + b_begin + i) * kFragBytes;
            if constexpr (H > 0)
                lds_buf16(wq, j != half_j || own ? 16u * lane + off : kOutOfRange, 0u,
                          my + ((i % kRR) * G + j) * kFragBytes);
            else
                lds_buf16(wq, 16u * lane, off, my + ((i % kRR) * G + j) * kFragBytes);
        }
    };

    float y[G][MR][4];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[j][r][i] = 0.0f;
    AuxSlotG<MR, G, kAsym> slot[kRA];
    // issue order: fragments of blocks 0 .. kRR-kRA-1; then for k < kRA the
    // aux loads of block k followed by the fragments of block k + kRR - kRA;
    // in the loop, after block i: aux of i + kRA, fragments of i + kRR
#pragma unroll
    for (int i = 0; i < kRR - kRA; ++i)
        if (i < NBW) fragments(i);
#pragma unroll
    for (int k = 0; k < kRA; ++k) {
        if (k < NBW) stream_fetch_aux_g<MR, G, kAsym>(p, xq, b_begin + k, grp0, lane, srow, arow, slot[k]);
        if (k + kRR - kRA < NBW) fragments(k + kRR - kRA);
    }
    unroll_seq([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        // wave priority from progress through the wave's blocks (3 in the
        // first quarter down to 0): the workgroup waits for its slowest wave
        // at the split-K sum, and with equal priorities the oldest waves win
        // the issue arbitration. Measured to pay for the half-group units and
        // four row tiles (LLaMA-70B decode, N = 10240: 12.1 to 11.8 us at
        // M = 1, 19.3 to 18.3 at M = 64; N = 28672, M = 64: 39.8 to 37.7), not
        // for the one-tile whole-group forms (N = 28672, M = 1: 24.9 to 26.5)
        if constexpr ((H > 0 || MR == 4) && (i == 0 || 4 * i / NBW != 4 * (i - 1) / NBW))
            __builtin_amdgcn_s_setprio(3 - (4 * i) / NBW);
        COMET_VMCNT((lds_g_loads_after<MR, G, kRA, kRR, kAsym>(i, NBW)));
        AuxSlotG<MR, G, kAsym>& sl = slot[i % kRA];
        stream_compute_lds_g<MR, G, kAsym, kDump>(b_begin + i < nb4, sl, my + (i % kRR) * G * kFragBytes, lane, y,
                                                  p, b_begin + i, grp0, half_j, own);
        if (i + kRA < NBW) stream_fetch_aux_g<MR, G, kAsym>(p, xq, b_begin + i + kRA, grp0, lane, srow, arow, sl);
        // the ring slot just read is refilled only after its words are used
        if (i + kRR < NBW) fragments(i + kRR);
    }, std::make_integer_sequence<int, NBW>{});
    if constexpr (kDump) return;

#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (j > 0) __syncthreads();     // the previous group's sums are read
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][4 * r + i][lane] = y[j][r][i];
        __syncthreads();
        for (int q = wave; q < MR * 4; q += kSplit) {
            float v = red[0][q][lane];
#pragma unroll
            for (int w2 = 1; w2 < kSplit; ++w2) v += red[w2][q][lane];
            const int row = 16 * (q >> 2) + 4 * g + (q & 3);
            if (row < M && (j != half_j || own))
                p.Y[static_cast<size_t>(row) * p.ldy + (grp0 + j) * 16 + l16] = __half_as_ushort(__float2half_rn(v));
        }
    }
}

bool use_stream(int M) { return M <= 64; }

#ifndef COMET_STREAM_TARGET_WAVES
#define COMET_STREAM_TARGET_WAVES 4096
#endif
#ifndef COMET_STREAM_DEPTH
#define COMET_STREAM_DEPTH 4
#endif

// One row tile (M <= 16): at 64 blocks mostly the multi-group LDS-ring
// kernel (below); otherwise one channel group per workgroup, its blocks split
// over the waves: the LDS-ring kernel for 32, 64 and 128 blocks, the register
// kernel (four blocks in flight, 120 VGPRs) otherwise.
template <int MR, int G, int kSplit, int kRR, int kRA, bool kAsym, bool kDump>
int launch_stream_lds_g_cfg(const GemmProblem& p, hipStream_t st);

// Half-group units (see gemm_stream_lds_g_kernel) where N = 2048 H, H = 5 or
// 7: 256 units of H half-groups, one per CU, every CU the same load, where
// whole groups leave some CUs a third more work than others. Measured at K =
// 8192 against the whole-group kernels (60 back-to-back calls, medians): N =
// 10240, M = 1 / 4 / 16 11.8 / 11.5 / 11.6 against 12.8 / 12.7 / 13.3 us,
// M = 32 / 48 / 64 13.5 / 15.9 / 18.6 against 16.6 / 17.4 / 20.1 us; N =
// 14336, M = 1 / 4 / 16 15.2 / 15.2 / 14.7 against 16.8 / 16.6 / 17.2 us.
// Not used where it was not faster: H = 3 (N = 6144, equal), and H = 7 above
// 16 rows (M = 48 / 64 19.0 / 22.2 against 18.8 / 21.9 us).
template <int MR, int H, int kSplit, int kRR, int kRA, bool kAsym, bool kDump>
int launch_stream_lds_half_cfg(const GemmProblem& p, hipStream_t st) {
    constexpr int G = (H + 1) / 2;
    const int units = p.N / (8 * H);
    const int grid = 8 * ((units + 7) / 8);
    gemm_stream_lds_g_kernel<MR, G, 64 / kSplit, kSplit, kRA, kRR, kAsym, kDump, H><<<grid, 64 * kSplit, 0, st>>>(p);
    return static_cast<int>(hipGetLastError());
}

bool half_units(const GemmProblem& p, int mr) {
    const int h = p.N / 2048;
    return p.nb == 64 && p.N % 2048 == 0 && (h == 5 || (h == 7 && mr == 1));
}

template <int MR, bool kAsym, bool kDump>
int launch_stream_lds_half(const GemmProblem& p, hipStream_t st) {
    if constexpr (MR == 1)
        if (p.N == 7 * 2048) return launch_stream_lds_half_cfg<1, 7, 8, 4, 2, kAsym, kDump>(p, st);
    return launch_stream_lds_half_cfg<MR, 5, 8, 4, 2, kAsym, kDump>(p, st);
}

template <bool kAsym, bool kDump>
int launch_stream1(const GemmProblem& p, hipStream_t st) {
    if (half_units(p, 1)) return launch_stream_lds_half<1, kAsym, kDump>(p, st);
    // 64 blocks: the multi-group LDS-ring kernel in its narrow form (two
    // groups per wave, eight waves of 8 blocks), except where its grid of
    // N / 32 workgroups falls between one and two per CU and leaves the CUs
    // unevenly loaded. Measured at K = 8192, M = 1..16 against the one-group
    // kernels below: N = 8192 9.3-9.5 against 10.8-11.2 us, N = 28672
    // 24.7-26.5 against 29.1-31.8 us; N = 10240 (320 workgroups) 13.1-13.5
    // against 12.8-13.4 us. N = 10240 and 14336 now take the half-group
    // units above; other such grids stay on the one-group kernel.
    const int narrow_units = p.N / 32;
    if (p.nb == 64 && !(narrow_units > 256 && narrow_units < 512))
        return launch_stream_lds_g_cfg<1, 2, 8, 4, 2, kAsym, kDump>(p, st);
    constexpr int kD = COMET_STREAM_DEPTH;
    const int groups = p.N / 16;
    const int grid = 8 * ((groups + 7) / 8);     // XCD-aware order; surplus workgroups exit
    if (p.nb == 32) {
        gemm_stream_lds_kernel<8, 4, kAsym, kDump><<<grid, 256, 0, st>>>(p);
    } else if (p.nb == 64 && groups * 8 < 2 * COMET_STREAM_TARGET_WAVES) {
        gemm_stream_lds_kernel<8, 8, kAsym, kDump><<<grid, 512, 0, st>>>(p);
    } else if (p.nb == 64) {
        gemm_stream_lds_kernel<16, 4, kAsym, kDump><<<grid, 256, 0, st>>>(p);
    } else if (p.nb == 128) {
        gemm_stream_lds_kernel<16, 8, kAsym, kDump><<<grid, 512, 0, st>>>(p);
    } else if (groups * 4 >= COMET_STREAM_TARGET_WAVES || p.nb < 8 * kD) {
        // split the blocks of a channel group over enough waves to keep
        // many weight fragments in flight across the chip
        gemm_stream_kernel<1, kD, 4, kAsym, kDump><<<grid, 256, 0, st>>>(p);
    } else if (groups * 8 >= COMET_STREAM_TARGET_WAVES || p.nb < 16 * kD) {
        gemm_stream_kernel<1, kD, 8, kAsym, kDump><<<grid, 512, 0, st>>>(p);
    } else {
        gemm_stream_kernel<1, kD, 16, kAsym, kDump><<<grid, 1024, 0, st>>>(p);
    }
    return static_cast<int>(hipGetLastError());
}

// Register multi-group kernel, any block count. Measured against the
// one-group kernel on the K = 8192 decode shapes it is faster in 11 of 12
// (N = 10240, M = 64: 34 against 32 us).
template <int MR, int G, int kSplit, bool kAsym, bool kDump>
int launch_stream_g_cfg(const GemmProblem& p, hipStream_t st) {
    constexpr int kD = 2;
    const int units = p.N / (16 * G);
    const int grid = 8 * ((units + 7) / 8);
    gemm_stream_g_kernel<MR, G, kD, kSplit, kAsym, kDump><<<grid, 64 * kSplit, 0, st>>>(p);
    return static_cast<int>(hipGetLastError());
}

template <int MR, bool kAsym, bool kDump>
int launch_stream_g(const GemmProblem& p, hipStream_t st) {
    const int groups = p.N / 16;
    // four groups per workgroup while that still leaves about two four-wave
    // workgroups per CU; else two groups, with eight waves per workgroup when
    // four-wave workgroups alone would not cover the CUs
    if (groups / 4 >= 384) return launch_stream_g_cfg<MR, 4, 4, kAsym, kDump>(p, st);
    if (groups / 2 >= 384) return launch_stream_g_cfg<MR, 2, 4, kAsym, kDump>(p, st);
    return launch_stream_g_cfg<MR, 2, 8, kAsym, kDump>(p, st);
}

// LDS-ring multi-group kernel, 64 blocks. Three configurations, chosen by
// measurement on the LLaMA-70B decode shapes (K = 8192; N = 8192, 10240,
// 28672; M = 17 .. 64):
//   wide:   G = 4, four waves of 16 blocks, 4-block ring (64 KB, plus 16 KB
//           for the reduction: two workgroups per CU);
//   narrow: G = 2, eight waves of 8 blocks, 4-block ring (64 KB + 32 KB).
//   wide8:  G = 4, eight waves of 8 blocks, 3-block ring (96 KB + up to
//           32 KB), one workgroup per CU.
// The wide form reads each activation word for twice the channels and is
// faster when it still yields about 1.5 workgroups per CU (N >= 24576), and
// at M > 32 from 160 workgroups on (N = 10240, M = 64: 23 against 26 us); the
// narrow one has twice the waves and wins on the smaller grids. A wide grid
// of fewer workgroups than CUs leaves one wave per SIMD on the CUs it uses;
// there the eight-wave form hides more latency (N = 10240, M = 33 / 48 / 64:
// 16.8 / 17.3 / 19.9 against 18.9 / 19.2 / 22.4 us), while on grids of more
// workgroups than CUs it is slower (N = 28672, M = 64: 41.9 against 37.3 us).
// (N = 10240 itself has since moved to the half-group units.)
template <int MR, int G, int kSplit, int kRR, int kRA, bool kAsym, bool kDump>
int launch_stream_lds_g_cfg(const GemmProblem& p, hipStream_t st) {
    const int units = p.N / (16 * G);
    const int grid = 8 * ((units + 7) / 8);
    gemm_stream_lds_g_kernel<MR, G, 64 / kSplit, kSplit, kRA, kRR, kAsym, kDump><<<grid, 64 * kSplit, 0, st>>>(p);
    return static_cast<int>(hipGetLastError());
}

template <int MR, bool kAsym, bool kDump>
int launch_stream_lds_g(const GemmProblem& p, hipStream_t st) {
    const int wide_units = p.N / 64;
    const bool wide = wide_units >= 384 || (p.M > 32 && wide_units >= 160);
    if (wide && wide_units < 256) return launch_stream_lds_g_cfg<MR, 4, 8, 3, 2, kAsym, kDump>(p, st);
    if (wide) return launch_stream_lds_g_cfg<MR, 4, 4, 4, 2, kAsym, kDump>(p, st);
    return launch_stream_lds_g_cfg<MR, 2, 8, 4, 2, kAsym, kDump>(p, st);
}

// Two to four row tiles (16 < M <= 64): several channel groups per wave.
template <int MR, bool kAsym, bool kDump>
int launch_stream(const GemmProblem& p, hipStream_t st) {
    if (half_units(p, MR)) return launch_stream_lds_half<MR, kAsym, kDump>(p, st);
    if (p.nb == 64) return launch_stream_lds_g<MR, kAsym, kDump>(p, st);
    return launch_stream_g<MR, kAsym, kDump>(p, st);
}

// One kernel choice for both variants: the partials entry points (kDump)
// launch exactly the kernel, launch shape and block split that produce Y for
// the same (M, N, K), with the epilogue replaced by stores of P.
template <bool kAsym, bool kDump>
int launch_gemm(const GemmProblem& p, hipStream_t s) {
    if (use_stream(p.M)) {
        const int mr = (p.M + 15) / 16;
        if (mr == 1) return launch_stream1<kAsym, kDump>(p, s);
        if (mr == 2) return launch_stream<2, kAsym, kDump>(p, s);
        if (mr == 3) return launch_stream<3, kAsym, kDump>(p, s);
        return launch_stream<4, kAsym, kDump>(p, s);
    }
    // the tiles of the full launch that hold rows of the partials' range
    const int tm_lo = kDump ? p.m_begin / kTM : 0;
    const int tm_hi = kDump ? (p.m_begin + p.m_count + kTM - 1) / kTM : (p.M + kTM - 1) / kTM;
    const int tiles = (tm_hi - tm_lo) * (p.N / kTN);
    gemm_tiled_kernel<kDump, kAsym><<<8 * ((tiles + 7) / 8), kThreads, 0, s>>>(p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

size_t gemm_workspace_bytes(int, int, int, int) { return 0; }

int launch_w4ax_gemm(const GemmProblem& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.P) return p.x_zero ? launch_gemm<true, true>(p, s) : launch_gemm<false, true>(p, s);
    return p.x_zero ? launch_gemm<true, false>(p, s) : launch_gemm<false, false>(p, s);
}

}  // namespace comet
