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
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "comet_internal.h"

namespace comet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// Integer minimum by value (a reference-returning min leaves stack slots behind).
__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

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

__device__ inline v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Tiled kernel (prefill shapes): 128 x 128 output tile per workgroup of four
// waves in a 2 x 2 arrangement, 64 x 64 per wave. The packed A and B tiles of
// a block go from HBM straight into LDS (global_load_lds_dwordx4: each lane's
// 16 bytes land at LDS base + 16 * lane, so one wave instruction fills one
// 1 KB piece and no registers are spent on staging). Two LDS stages: the
// loads of block b+1 are in flight while block b computes; one barrier per
// block.
//
// LDS pieces (1 KB each) of a stage:
//   A, 4-bit block: 8 pieces of 16 rows x 64 B. Slot s = 4 r + (j ^ ((r >> 2) & 3))
//     holds 16-byte chunk j of row r, so the 16 lanes of one MFMA k-group
//     (16 rows, same chunk) hit 16 different bank groups.
//   A, 8-bit block: 16 pieces of 8 rows x 128 B. Slot s = 8 r + (j ^ f), with
//     f = ((r >> 1) & 3) | ((piece & 1) << 2), same purpose.
//   B: 8 fragments in their stored (lane) order.
// plus the block's 128 activation scales, 128 weight scales (pre-divided by
// 16) and 128 weight-sum corrections.
// ---------------------------------------------------------------------------

#ifndef COMET_TILED_WG_PER_CU
#define COMET_TILED_WG_PER_CU 1   // workgroups per CU the register budget is sized for
#endif

constexpr int kTM = 128;
constexpr int kTN = 128;
constexpr int kLdsA = kTM * 128;                 // room for an 8-bit block
constexpr int kLdsB = (kTN / 16) * kFragBytes;
constexpr int kLdsSa = kTM * 4;
constexpr int kLdsSw = kTN * 4;
constexpr int kLdsCorr = kTN * 4;
constexpr int kStage = kLdsA + kLdsB + kLdsSa + kLdsSw + kLdsCorr;

// Tile of a workgroup. Workgroups are dispatched round-robin over the eight
// XCDs (workgroup w runs on XCD w mod 8); each XCD gets a contiguous range of
// the tile order, and the tile order walks 8-row-tile groups column by
// column, so the ~64 workgroups an XCD runs at once cover about an 8 x 8 patch
// and share their A and B stripes in that XCD's L2.
__device__ inline bool tile_of(int w, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int t = (w & 7) * per_xcd + (w >> 3);
    if (t >= total) return false;
    constexpr int G = 8;
    const int group = t / (G * tiles_n);
    const int first = group * G;
    const int gh = imin(G, tiles_m - first);
    const int in = t - group * G * tiles_n;
    tn = in / gh;
    tm = first + in % gh;
    return true;
}

__device__ __forceinline__ void lds_load16(const void* g, uint8_t* lds_piece) {
    __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                            reinterpret_cast<uintptr_t>(lds_piece)),
                                     16, 0, 0);
}

// Per-lane byte offsets of the direct-to-LDS loads, fixed for a tile: the
// block only moves the (wave-uniform) base pointers.
struct IssueOffsets {
    uint32_t a4[2];   // 4-bit A pieces 2w, 2w+1: row * 64 + 16 * swizzled chunk
    uint32_t a8[4];   // 8-bit A pieces 4w .. 4w+3: row * 128 + 16 * swizzled piece
    uint32_t sa;      // activation-scale row (threads 0..127)
};

__device__ __forceinline__ IssueOffsets issue_offsets(int M, int m0, int wave, int lane, int tid) {
    IssueOffsets o;
    {
        const int r = lane >> 2;
        const int j = (lane & 3) ^ ((r >> 2) & 3);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int row = imin(m0 + 16 * (2 * wave + k) + r, M - 1);
            o.a4[k] = static_cast<uint32_t>(row) * 64u + 16u * j;
        }
    }
    {
        const int r = lane >> 3;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int piece = 4 * wave + k;
            const int j = (lane & 7) ^ (((r >> 1) & 3) | ((piece & 1) << 2));
            const int row = imin(m0 + 8 * piece + r, M - 1);
            o.a8[k] = static_cast<uint32_t>(row) * 128u + 16u * j;
        }
    }
    o.sa = static_cast<uint32_t>(imin(m0 + (tid & (kTM - 1)), M - 1));
    return o;
}

// Issue the direct-to-LDS loads of block b's A and B pieces (wave `wave`, a
// wave-uniform value, loads its share) and fetch this thread's scale words.
__device__ __forceinline__ void tiled_issue(const GemmProblem& p, int b, int n0, int wave, int lane,
                                            int tid, const IssueOffsets& o, uint8_t* st, float& sa,
                                            uint32_t& hs, int32_t& ws) {
    const int M = p.M, N = p.N, nb = p.nb, nb4 = p.nb4;
    // Scale words first (every thread, no branch), all 32-bit: threads 0..127
    // take an activation scale, 128..191 two weight scales, 192..255 two weight
    // sums. Waiting for them later then leaves the younger LDS loads in flight.
    {
        sa = (p.x_scale + static_cast<size_t>(b) * M)[o.sa];
        const uint32_t* wsc = reinterpret_cast<const uint32_t*>(p.w_scale + static_cast<size_t>(b) * N + n0);
        const uint32_t* wsm = reinterpret_cast<const uint32_t*>(p.w_sum + static_cast<size_t>(b) * N + n0);
        hs = wsc[tid & 63];
        ws = static_cast<int32_t>(wsm[tid & 63]);
    }
    // (written out: an array indexed in a loop would be left on the stack)
    if (b < nb4) {
        const uint8_t* slab = p.Xq + static_cast<size_t>(b) * M * 64;
        lds_load16(slab + o.a4[0], st + (2 * wave + 0) * kFragBytes);
        lds_load16(slab + o.a4[1], st + (2 * wave + 1) * kFragBytes);
    } else {
        const uint8_t* slab = p.Xq + static_cast<size_t>(nb4) * M * 64 + static_cast<size_t>(b - nb4) * M * 128;
        lds_load16(slab + o.a8[0], st + (4 * wave + 0) * kFragBytes);
        lds_load16(slab + o.a8[1], st + (4 * wave + 1) * kFragBytes);
        lds_load16(slab + o.a8[2], st + (4 * wave + 2) * kFragBytes);
        lds_load16(slab + o.a8[3], st + (4 * wave + 3) * kFragBytes);
    }
    const uint8_t* frag = p.Wq + (static_cast<size_t>(n0 / 16 + 2 * wave) * nb + b) * kFragBytes +
                          16u * static_cast<uint32_t>(lane);
    lds_load16(frag, st + kLdsA + (2 * wave) * kFragBytes);
    lds_load16(frag + static_cast<size_t>(nb) * kFragBytes, st + kLdsA + (2 * wave + 1) * kFragBytes);
}

// Scales of a staged block into LDS: s_w / 16 as f32 and the weight-sum
// correction -128 w_sum (4-bit blocks) or 0 (8-bit blocks) as int32.
__device__ __forceinline__ void tiled_store_scales(uint8_t* st, int tid, bool is4, float sa,
                                                   uint32_t hs, int32_t ws) {
    // Opaque redefinition: keeps the compiler from hoisting the conversions
    // (and so the wait for these loads, which would also wait for the
    // in-flight LDS loads) up to where the loads are issued.
    asm volatile("" : "+v"(sa), "+v"(hs), "+v"(ws));
    float* sa_l = reinterpret_cast<float*>(st + kLdsA + kLdsB);
    float* sw_l = reinterpret_cast<float*>(st + kLdsA + kLdsB + kLdsSa);
    int* corr_l = reinterpret_cast<int*>(st + kLdsA + kLdsB + kLdsSa + kLdsSw);
    if (tid < kTM) {
        sa_l[tid] = sa;
    } else if (tid < kTM + 64) {
        const int c = 2 * (tid - kTM);
        sw_l[c] = h2f(static_cast<uint16_t>(hs & 0xFFFFu)) * 0.0625f;
        sw_l[c + 1] = h2f(static_cast<uint16_t>(hs >> 16)) * 0.0625f;
    } else {
        const int c = 2 * (tid - kTM - 64);
        const int lo = static_cast<int16_t>(static_cast<uint32_t>(ws) & 0xFFFFu);
        const int hi = ws >> 16;
        corr_l[c] = is4 ? -128 * lo : 0;
        corr_l[c + 1] = is4 ? -128 * hi : 0;
    }
}

// One block of the tiled kernel: compute from stage `st` while block b+1
// streams into stage `nxt`.
template <bool kDump>
__device__ __forceinline__ void tiled_block(const GemmProblem& p, int b, int m0, int n0, int row_lo,
                                            int row_hi, int wave, int lane, int tid,
                                            const IssueOffsets& ioff, int a4_base, int a8_base,
                                            const uint8_t* st, uint8_t* nxt, float (&y)[4][4][4]) {
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    const int nb = p.nb, nb4 = p.nb4, N = p.N;
    float gsa = 0.0f;
    uint32_t ghs = 0;
    int32_t gws = 0;
    if (b + 1 < nb) tiled_issue(p, b + 1, n0, wave, lane, tid, ioff, nxt, gsa, ghs, gws);

    const bool is4 = b < nb4;
    const float* sa_l = reinterpret_cast<const float*>(st + kLdsA + kLdsB);
    const float* sw_l = reinterpret_cast<const float*>(st + kLdsA + kLdsB + kLdsSa);
    const int* corr_l = reinterpret_cast<const int*>(st + kLdsA + kLdsB + kLdsSa + kLdsSw);
    const float sa_lane = sa_l[64 * wr + lane];

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
    if constexpr (!kDump) t = __builtin_amdgcn_mfma_f32_16x16x1f32(sa_lane, sw_l[64 * wc + l16], t, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int col = 64 * wc + 16 * c + l16;
        float sw_next = c < 3 ? sw_l[col + 16] : 0.0f;
        const uint4 pk = *reinterpret_cast<const uint4*>(st + kLdsA + (4 * wc + c) * kFragBytes + 16 * lane);
        const v4i B0 = widen_weights_lo(pk);
        const v4i B1 = widen_weights_hi(pk);
        const int corr = corr_l[col];
        const v4i cinit = {corr, corr, corr, corr};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v4i acc = mfma_i8(A0[r], B0, cinit);
            acc = mfma_i8(A1[r], B1, acc);
            if constexpr (kDump) {
                const int ncol = n0 + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + 64 * wr + 16 * r + 4 * g + i;
                    if (row < row_hi)
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
        __builtin_amdgcn_sched_barrier(0);
    }
    if (b + 1 < nb) tiled_store_scales(nxt, tid, b + 1 < nb4, gsa, ghs, gws);
    __syncthreads();    // this thread's direct-to-LDS loads have landed, and everyone is done with st
}

template <bool kDump>
__global__ __launch_bounds__(kThreads, COMET_TILED_WG_PER_CU) void gemm_tiled_kernel(GemmProblem p) {
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStage];

    const int row_lo = kDump ? p.m_begin : 0;
    const int row_hi = kDump ? p.m_begin + p.m_count : p.M;
    const int tiles_m = (row_hi - row_lo + kTM - 1) / kTM;
    const int tiles_n = p.N / kTN;
    int tm, tn;
    if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
    const int m0 = row_lo + tm * kTM;
    const int n0 = tn * kTN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    const int nb = p.nb;
    const IssueOffsets ioff = issue_offsets(p.M, m0, wave, lane, tid);

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

    {
        float sa = 0.0f;
        uint32_t hs = 0;
        int32_t ws = 0;
        tiled_issue(p, 0, n0, wave, lane, tid, ioff, stage0, sa, hs, ws);
        tiled_store_scales(stage0, tid, 0 < p.nb4, sa, hs, ws);
        __syncthreads();
    }
    for (int b = 0; b < nb; b += 2) {
        tiled_block<kDump>(p, b, m0, n0, row_lo, row_hi, wave, lane, tid, ioff, a4_base, a8_base, stage0,
                           stage1, y);
        if (b + 1 < nb)
            tiled_block<kDump>(p, b + 1, m0, n0, row_lo, row_hi, wave, lane, tid, ioff, a4_base, a8_base,
                               stage1, stage0, y);
    }

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
// workgroup owns one group of 16 output channels; its four waves split the
// blocks four ways (split-K inside the workgroup) and stream their weight
// fragments with everything else a block needs (activation codes, activation
// scale, weight scale and sum) fetched a batch of kU blocks ahead, double
// buffered. The four partial tiles are summed through LDS in wave order, so
// the result is deterministic, and no global atomics or device-scope fences
// are needed (on a multi-XCD part those write back and invalidate L2).
// ---------------------------------------------------------------------------

constexpr int kSplitWaves = 4;

// One batch of kU blocks in registers: weight word, activation words (the
// second only for 8-bit blocks), activation scale, weight scale bits, weight sum.
template <int MR, int kU>
struct StreamBatch {
    uint4 w[kU];
    uint4 a0[kU][MR];
    uint4 a1[kU][MR];
    float sa[kU];
    uint32_t hs[kU];
    int32_t ws[kU];
};

template <int MR, int kU>
__device__ __forceinline__ void stream_fetch(const GemmProblem& p, int b0, int b_end, int grp, int lane,
                                             int srow, const int (&arow)[MR], StreamBatch<MR, kU>& sb) {
    const int g = lane >> 4, l16 = lane & 15;
    const int M = p.M, N = p.N, nb = p.nb, nb4 = p.nb4;
    const int ncol = grp * 16 + l16;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int b = imin(b0 + u, b_end - 1);
        sb.w[u] = *reinterpret_cast<const uint4*>(p.Wq + (static_cast<size_t>(grp) * nb + b) * kFragBytes +
                                                  16 * lane);
        sb.sa[u] = p.x_scale[static_cast<size_t>(b) * M + srow];
        sb.hs[u] = p.w_scale[static_cast<size_t>(b) * N + ncol];
        sb.ws[u] = p.w_sum[static_cast<size_t>(b) * N + ncol];
        // branch-free: 4-bit rows are 64 bytes at 16g, 8-bit rows 128 bytes at
        // 32g (+16 for the second word); a 4-bit block reloads its one word
        const bool is4 = b < nb4;
        const uint8_t* slab = is4 ? p.Xq + static_cast<size_t>(b) * M * 64
                                  : p.Xq + static_cast<size_t>(nb4) * M * 64 + static_cast<size_t>(b - nb4) * M * 128;
        const uint32_t rstride = is4 ? 64u : 128u;
        const uint32_t cofs = is4 ? 16u * g : 32u * g;
        const uint32_t second = is4 ? 0u : 16u;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const uint8_t* src = slab + static_cast<uint32_t>(arow[r]) * rstride + cofs;
            sb.a0[u][r] = *reinterpret_cast<const uint4*>(src);
            sb.a1[u][r] = *reinterpret_cast<const uint4*>(src + second);
        }
    }
}

// Blocks past b_end (the tail of the last batch) were fetched clamped to a
// valid block; they get a zero scale product, which adds exactly zero.
template <int MR, int kU>
__device__ __forceinline__ void stream_compute(int b0, int b_end, int nb4, const StreamBatch<MR, kU>& sb,
                                               float (&y)[MR][4]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int b = b0 + u;
        const bool valid = b < b_end;
        const bool is4 = imin(b, b_end - 1) < nb4;
        const v4i B0 = widen_weights_lo(sb.w[u]);
        const v4i B1 = widen_weights_hi(sb.w[u]);
        const float sw = valid ? h2f(static_cast<uint16_t>(sb.hs[u])) * 0.0625f : 0.0f;
        const int corr = is4 ? -128 * sb.ws[u] : 0;
        const v4i cinit = {corr, corr, corr, corr};
        // t[4r + i] = s_x[row 16r + 4g + i] * s_w[col] / 16 for the MR row tiles
        v16f t = {};
        t = __builtin_amdgcn_mfma_f32_16x16x1f32(sb.sa[u], sw, t, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            v4i A0, A1;
            if (is4) {
                A0 = widen_act_lo(sb.a0[u][r]);
                A1 = widen_act_hi(sb.a0[u][r]);
            } else {
                A0 = as_v4i(sb.a0[u][r]);
                A1 = as_v4i(sb.a1[u][r]);
            }
            v4i acc = mfma_i8(A0, B0, cinit);
            acc = mfma_i8(A1, B1, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) y[r][i] = __builtin_fmaf(t[4 * r + i], static_cast<float>(acc[i]), y[r][i]);
        }
    }
}

template <int MR, int kU>
__global__ __launch_bounds__(kThreads) void gemm_stream_kernel(GemmProblem p) {
    __shared__ float red[kSplitWaves][MR * 4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    const int grp = blockIdx.x;                    // 16-channel group
    const int nb = p.nb, M = p.M;
    const int bps = (nb + kSplitWaves - 1) / kSplitWaves;
    const int b_begin = imin(nb, wave * bps);
    const int b_end = imin(nb, b_begin + bps);

    int arow[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) arow[r] = imin(16 * r + l16, M - 1);
    const int srow = imin(lane, M - 1);    // row whose scale this lane feeds the outer product
    float y[MR][4];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[r][i] = 0.0f;

    if (b_begin < b_end) {
        StreamBatch<MR, kU> s0, s1;
        stream_fetch<MR, kU>(p, b_begin, b_end, grp, lane, srow, arow, s0);
        for (int b0 = b_begin; b0 < b_end; b0 += 2 * kU) {
            stream_fetch<MR, kU>(p, b0 + kU, b_end, grp, lane, srow, arow, s1);
            stream_compute<MR, kU>(b0, b_end, p.nb4, s0, y);
            stream_fetch<MR, kU>(p, b0 + 2 * kU, b_end, grp, lane, srow, arow, s0);
            stream_compute<MR, kU>(b0 + kU, b_end, p.nb4, s1, y);
        }
    }

#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][4 * r + i][lane] = y[r][i];
    __syncthreads();
    // each wave finishes MR*4/4 of the (row tile, i) slots, summing the four
    // K-quarters in wave order
    for (int q = wave; q < MR * 4; q += kSplitWaves) {
        const float v = ((red[0][q][lane] + red[1][q][lane]) + red[2][q][lane]) + red[3][q][lane];
        const int row = 16 * (q >> 2) + 4 * g + (q & 3);
        if (row < M) p.Y[static_cast<size_t>(row) * p.ldy + grp * 16 + l16] = __half_as_ushort(__float2half_rn(v));
    }
}

bool use_stream(int M) { return M <= 64; }

template <int MR>
int launch_stream(const GemmProblem& p, hipStream_t st) {
    constexpr int kU = MR <= 1 ? 4 : 2;
    gemm_stream_kernel<MR, kU><<<p.N / 16, kThreads, 0, st>>>(p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

size_t gemm_workspace_bytes(int, int, int, int) { return 0; }

int launch_w4ax_gemm(const GemmProblem& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.P) {
        const int tiles = ((p.m_count + kTM - 1) / kTM) * (p.N / kTN);
        gemm_tiled_kernel<true><<<8 * ((tiles + 7) / 8), kThreads, 0, s>>>(p);
        return static_cast<int>(hipGetLastError());
    }
    if (use_stream(p.M)) {
        const int mr = (p.M + 15) / 16;
        if (mr == 1) return launch_stream<1>(p, s);
        if (mr == 2) return launch_stream<2>(p, s);
        if (mr == 3) return launch_stream<3>(p, s);
        return launch_stream<4>(p, s);
    }
    const int tiles = ((p.M + kTM - 1) / kTM) * (p.N / kTN);
    gemm_tiled_kernel<false><<<8 * ((tiles + 7) / 8), kThreads, 0, s>>>(p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace comet
