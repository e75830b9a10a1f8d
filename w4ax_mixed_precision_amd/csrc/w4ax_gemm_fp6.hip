// comet_w4ax_gemm_fp6: the W4Ax GEMM for prefill shapes on the FP6 operand
// layout. Same result as comet_w4ax_gemm: exact integer partials per
// 128-channel block and the FP32 dequantization epilogue, fp16 out.
//
// The method: COMET summary (paperbot-e5f.pages.dev/papers/10460.html),
// abstract, a W4Ax kernel for mixed W4A4/W4A8 blocks whose software pipeline
// hides load and conversion latency; QUIK blog (deep-paper.org/paper/2310.09259),
// section "核融合", dequantize while the integer result is still in registers.
//
// Why FP6 on gfx950. CDNA4 has no 4-bit integer matrix instruction, but it has
// a 16x16x128 FP6 one at twice the INT8 rate, and FP6 E2M3 represents every
// 4-bit code in [-7, 7] exactly. Products of two codes are integers of
// magnitude at most 49 and every partial sum of a 128-channel block is an
// integer below 2^13, so the FP32 result of the instruction is the block's
// INT32 partial P, exactly, whatever the order of accumulation inside the
// unit. One instruction covers a whole 16x16 tile of a 4-bit block, its result
// is already a float (no integer-to-float conversion in the epilogue) and the
// codes arrive in the operand format (no widening), so the per-block VALU work
// drops to one FMA per output. 8-bit blocks (INT8 activations, INT4 weights)
// keep the v_mfma_i32_16x16x64_i8 path: weights widened to 16 q_w in
// registers, accumulator 16 P, scale product divided by 16.
//
// Tiling: 128 x 128 output tile per workgroup of four waves (2 x 2, 64 x 64
// per wave), two workgroups per CU. Every operand of a block goes from HBM
// straight into LDS with direct loads (global_load_lds, each lane's 16 or 4
// bytes at LDS base + lane * size) into a ring of three 25.6 KB stages, two
// blocks ahead of the compute. Each wave issues 7 loads per block of either
// kind, so at the end of block b a partial wait (vmcnt <= 7: block b+2 may
// still be in flight) and a plain s_barrier publish block b+1.
//
// LDS stage:
//   4-bit block: A heads 8 KB at 0 (8 pieces of 16 rows; slot
//     4r + (g ^ ((r >> 2) & 3)) holds row r's 16-byte head of group g, so the
//     16 lanes of one MFMA k-group read 16 different bank groups); A tails
//     4 KB at 8192 (per piece: the (g0, g1) tail pairs of rows 0..15, then the
//     (g2, g3) pairs, conflict-free for 8-byte reads); B 12 KB at 12288, the
//     tile's 8 FP6 fragments as stored.
//   8-bit block: A 16 KB at 0 (16 pieces of 8 rows x 128 B, slot
//     8r + (j ^ f), f = ((r >> 1) & 3) | ((piece & 1) << 2)); B 8 KB at 16384,
//     the tile's 8 INT4 fragments as stored.
//   then the block's 128 activation scales (f32) and 128 weight scales (fp16).
#include "comet_internal.h"
#include "device_util.h"

namespace comet {
namespace {

constexpr int kThreads = 256;
constexpr int kTM = 128;
constexpr int kTN = 128;
constexpr int kFragF = 1536;                 // FP6 fragment: 16 channels x 128 positions x 6 bits
constexpr int kATail = 8192;                 // FP6 A tails
constexpr int kOffB6 = 12288;                // B of a 4-bit block
constexpr int kOffB8 = 16384;                // B of an 8-bit block
constexpr int kOffSa = 24576;
constexpr int kOffSw = kOffSa + kTM * 4;
constexpr int kOffPad = kOffSw + kTN * 2;    // target of wave 3's balancing load
constexpr int kStage = kOffPad + 256;
constexpr int kLoadsPerBlock = 7;

// Per-lane byte offsets of the direct loads inside a block's activation slab,
// fixed for a tile.
struct IssueOffsets {
    uint32_t h0, h1, t;                 // FP6 A: head pieces 2w, 2w+1; tails of pieces 2w, 2w+1
    uint32_t a8_0, a8_1, a8_2, a8_3;    // INT8 A pieces 4w .. 4w+3
    uint32_t sc;                        // scale words
};

__device__ __forceinline__ IssueOffsets issue_offsets(int M, int m0, int wave, int lane) {
    IssueOffsets o;
    {
        const int r = lane >> 2;
        const int g = (lane & 3) ^ ((r >> 2) & 3);
        o.h0 = static_cast<uint32_t>(imin(m0 + 16 * (2 * wave + 0) + r, M - 1)) * 96u + 16u * g;
        o.h1 = static_cast<uint32_t>(imin(m0 + 16 * (2 * wave + 1) + r, M - 1)) * 96u + 16u * g;
        const int piece = 2 * wave + (lane >> 5);
        const int rt = lane & 15, chunk = (lane >> 4) & 1;
        o.t = static_cast<uint32_t>(imin(m0 + 16 * piece + rt, M - 1)) * 96u + 64u + 16u * chunk;
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
    // waves 2 and 3: two weight scales per lane
    o.sc = wave < 2 ? static_cast<uint32_t>(imin(m0 + 64 * wave + lane, M - 1)) * 4u : 4u * lane;
    return o;
}

// Buffer resources of the four inputs, built once per workgroup (SGPRs).
struct Inputs {
    Rsrc xq, xs, wq, ws;
};

__device__ __forceinline__ Inputs make_inputs(const GemmProblem& p) {
    const uint32_t nb8 = static_cast<uint32_t>(p.nb - p.nb4);
    Inputs in;
    in.xq = make_rsrc(p.Xq, static_cast<uint32_t>(p.M) * (96u * p.nb4 + 128u * nb8));
    in.xs = make_rsrc(p.x_scale, static_cast<uint32_t>(p.M) * p.nb * 4u);
    in.wq = make_rsrc(p.Wq, static_cast<uint32_t>(p.N) * (96u * p.nb4 + 64u * nb8));
    in.ws = make_rsrc(p.w_scale, static_cast<uint32_t>(p.N) * p.nb * 2u);
    return in;
}

// Direct loads of block b into stage `st`: one scale word, then A and B
// (3 + 3 for a 4-bit block, 4 + 2 for an 8-bit block), 7 per wave either way.
// Block and tile bases are wave-uniform (scalar offsets); the per-lane parts
// are the fixed offsets of `o`.
__device__ __forceinline__ void fp6_issue(const GemmProblem& p, const Inputs& in, int b, int n0, int wave,
                                          int lane, const IssueOffsets& o, uint8_t* st) {
    const uint32_t M = p.M, N = p.N, nb4 = p.nb4;
    const uint32_t ub = static_cast<uint32_t>(b);
    if (wave < 2)
        lds_buf4(in.xs, o.sc, ub * M * 4u, st + kOffSa + 256 * wave);
    else
        lds_buf4(in.ws, o.sc, (ub * N + n0) * 2u, st + (wave == 2 ? kOffSw : kOffPad));
    const uint32_t groups = N / 16;
    const uint32_t lane16 = 16u * static_cast<uint32_t>(lane);
    if (b < p.nb4) {
        const uint32_t slab = ub * M * 96u;
        lds_buf16(in.xq, o.h0, slab, st + (2 * wave + 0) * 1024);
        lds_buf16(in.xq, o.h1, slab, st + (2 * wave + 1) * 1024);
        lds_buf16(in.xq, o.t, slab, st + kATail + 1024 * wave);
        const uint32_t wbase = (ub * groups + n0 / 16) * kFragF + 3072u * wave;
        lds_buf16(in.wq, lane16, wbase, st + kOffB6 + 3072 * wave);
        lds_buf16(in.wq, lane16, wbase + 1024, st + kOffB6 + 3072 * wave + 1024);
        lds_buf16(in.wq, lane16, wbase + 2048, st + kOffB6 + 3072 * wave + 2048);
    } else {
        const uint32_t slab = nb4 * M * 96u + (ub - nb4) * M * 128u;
        lds_buf16(in.xq, o.a8_0, slab, st + (4 * wave + 0) * 1024);
        lds_buf16(in.xq, o.a8_1, slab, st + (4 * wave + 1) * 1024);
        lds_buf16(in.xq, o.a8_2, slab, st + (4 * wave + 2) * 1024);
        lds_buf16(in.xq, o.a8_3, slab, st + (4 * wave + 3) * 1024);
        const uint32_t wbase = groups * (kFragF * nb4 + kFragBytes * (ub - nb4)) + (n0 / 16) * kFragBytes + 2048u * wave;
        lds_buf16(in.wq, lane16, wbase, st + kOffB8 + 2048 * wave);
        lds_buf16(in.wq, lane16, wbase + 1024, st + kOffB8 + 2048 * wave + 1024);
    }
}

__device__ __forceinline__ v8i fp6_operand(const uint8_t* head, const uint8_t* tail) {
    const uint4 h = *reinterpret_cast<const uint4*>(head);
    const uint2 t = *reinterpret_cast<const uint2*>(tail);
    return v8i{static_cast<int>(h.x), static_cast<int>(h.y), static_cast<int>(h.z), static_cast<int>(h.w),
               static_cast<int>(t.x), static_cast<int>(t.y), 0, 0};
}

// Per-lane LDS read offsets of row tile 0 (row tile r adds r KB to a head,
// r * 512 to a tail, 2r KB to an INT8 row).
struct ReadOffsets {
    int ah, at, a8;
};

// Output (row tile r, column tile c, element i) of this lane, or its partial.
template <bool kDump>
__device__ __forceinline__ void emit(const GemmProblem& p, float t, float P, int b, int row, int col,
                                     int row_lo, int row_hi, float& y) {
    if constexpr (kDump) {
        if (row < row_hi)
            p.P[(static_cast<size_t>(row - row_lo) * p.N + col) * p.nb + b] = static_cast<int>(P);
    } else {
        y = __builtin_fmaf(t, P, y);
    }
}

// Wait at the end of block b: block b+1's loads are done (only block b+2's may
// still be in flight), and every wave is finished with block b's stage before
// it is refilled.
__device__ __forceinline__ void end_block(int b, int nb) {
    if (b + 2 < nb) COMET_VMCNT(kLoadsPerBlock);
    else COMET_VMCNT(0);
    __builtin_amdgcn_s_barrier();
}

// One 4-bit block: issue block b+2 into `nxt`, compute block b from `st` on
// the FP6 matrix instruction.
template <bool kDump>
__device__ __forceinline__ void block_fp6(const GemmProblem& p, int b, int m0, int n0, int row_lo, int row_hi,
                                          int wave, int lane, const Inputs& in, const IssueOffsets& ioff,
                                          const ReadOffsets& ro, const uint8_t* __restrict__ st,
                                          uint8_t* __restrict__ nxt,
                                          float (&y)[4][4][4]) {
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    if (b + 2 < p.nb) fp6_issue(p, in, b + 2, n0, wave, lane, ioff, nxt);
    const float* sa_l = reinterpret_cast<const float*>(st + kOffSa);
    const uint16_t* sw_l = reinterpret_cast<const uint16_t*>(st + kOffSw);
    const float sa_lane = sa_l[64 * wr + lane];
    const int row0 = m0 + 64 * wr + 4 * g;
    const int col0 = n0 + 64 * wc + l16;

    v16f t = {};
    if constexpr (!kDump)
        t = __builtin_amdgcn_mfma_f32_16x16x1f32(sa_lane, h2f(sw_l[64 * wc + l16]), t, 0, 0, 0);
    v8i A[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) A[r] = fp6_operand(st + ro.ah + r * 1024, st + ro.at + r * 512);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float sw_next = c < 3 ? h2f(sw_l[64 * wc + 16 * (c + 1) + l16]) : 0.0f;
        const uint8_t* frag = st + kOffB6 + (4 * wc + c) * kFragF;
        const v8i B = fp6_operand(frag + 16 * lane, frag + 1024 + 8 * lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const v4f D = mfma_fp6(A[r], B);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                emit<kDump>(p, t[4 * r + i], D[i], b, row0 + 16 * r + i, col0 + 16 * c, row_lo, row_hi,
                            y[r][c][i]);
        }
        if constexpr (!kDump) {
            if (c < 3) {
                // the next scale product is formed after this tile's epilogue
                // (opaque dependency), so one t vector is live
                asm volatile("" : "+v"(sw_next), "+v"(y[3][c][3]));
                t = v16f{};
                t = __builtin_amdgcn_mfma_f32_16x16x1f32(sa_lane, sw_next, t, 0, 0, 0);
            }
        }
    }
    end_block(b, p.nb);
}

// One 8-bit block on the INT8 matrix instruction (weights widened to 16 q_w,
// so the accumulator holds 16 P and the scale product is divided by 16).
template <bool kDump>
__device__ __forceinline__ void block_int8(const GemmProblem& p, int b, int m0, int n0, int row_lo, int row_hi,
                                           int wave, int lane, const Inputs& in, const IssueOffsets& ioff,
                                           const ReadOffsets& ro, const uint8_t* __restrict__ st,
                                          uint8_t* __restrict__ nxt,
                                           float (&y)[4][4][4]) {
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    if (b + 2 < p.nb) fp6_issue(p, in, b + 2, n0, wave, lane, ioff, nxt);
    const float* sa_l = reinterpret_cast<const float*>(st + kOffSa);
    const uint16_t* sw_l = reinterpret_cast<const uint16_t*>(st + kOffSw);
    const float sa_lane = sa_l[64 * wr + lane] * 0.0625f;
    const int row0 = m0 + 64 * wr + 4 * g;
    const int col0 = n0 + 64 * wc + l16;

    v16f t = {};
    if constexpr (!kDump)
        t = __builtin_amdgcn_mfma_f32_16x16x1f32(sa_lane, h2f(sw_l[64 * wc + l16]), t, 0, 0, 0);
    v4i A0[4], A1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        A0[r] = as_v4i(*reinterpret_cast<const uint4*>(st + ro.a8 + r * 2048));
        A1[r] = as_v4i(*reinterpret_cast<const uint4*>(st + ((ro.a8 + r * 2048) ^ 16)));
    }
    const v4i zero = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float sw_next = c < 3 ? h2f(sw_l[64 * wc + 16 * (c + 1) + l16]) : 0.0f;
        const uint4 pk = *reinterpret_cast<const uint4*>(st + kOffB8 + (4 * wc + c) * kFragBytes + 16 * lane);
        const v4i B0 = widen_weights_lo(pk);
        const v4i B1 = widen_weights_hi(pk);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v4i acc = mfma_i8(A0[r], B0, zero);
            acc = mfma_i8(A1[r], B1, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float Pf = kDump ? static_cast<float>(acc[i] >> 4) : static_cast<float>(acc[i]);
                emit<kDump>(p, t[4 * r + i], Pf, b, row0 + 16 * r + i, col0 + 16 * c, row_lo, row_hi,
                            y[r][c][i]);
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
    end_block(b, p.nb);
}

template <bool kDump>
__global__ __launch_bounds__(kThreads, 2) void gemm_fp6_kernel(GemmProblem p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * kStage];

    const int row_lo = kDump ? p.m_begin : 0;
    const int row_hi = kDump ? p.m_begin + p.m_count : p.M;
    const int tiles_m = (row_hi - row_lo + kTM - 1) / kTM;
    const int tiles_n = p.N / kTN;
    int tm, tn;
    if (!tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn)) return;
    const int m0 = row_lo + tm * kTM;
    const int n0 = tn * kTN;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, l16 = lane & 15;
    const int nb = p.nb, nb4 = p.nb4;
    const IssueOffsets ioff = issue_offsets(p.M, m0, wave, lane);
    const Inputs in = make_inputs(p);
    ReadOffsets ro;
    ro.ah = 4 * wr * 1024 + 16 * (4 * l16 + (g ^ ((l16 >> 2) & 3)));
    ro.at = kATail + 4 * wr * 512 + 256 * (g >> 1) + 16 * l16 + 8 * (g & 1);
    ro.a8 = (8 * wr + (l16 >> 3)) * 1024 +
            16 * (8 * (l16 & 7) + ((2 * g) ^ ((((l16 & 7) >> 1) & 3) | (((l16 >> 3) & 1) << 2))));

    float y[4][4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[r][c][i] = 0.0f;

    // prologue: blocks 0 and 1 in flight; wait for block 0
    fp6_issue(p, in, 0, n0, wave, lane, ioff, smem);
    if (1 < nb) {
        fp6_issue(p, in, 1, n0, wave, lane, ioff, smem + kStage);
        COMET_VMCNT(kLoadsPerBlock);
    } else {
        COMET_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();

    // Block b lives in stage b mod 3 and block b+2 is loaded into stage
    // (b + 2) mod 3. The 4-bit blocks come first in the permuted order, the
    // 8-bit ones last.
    int cur = 0;
    for (int b = 0; b < nb4; ++b) {
        const int nxt = cur == 0 ? 2 : cur - 1;
        block_fp6<kDump>(p, b, m0, n0, row_lo, row_hi, wave, lane, in, ioff, ro, smem + cur * kStage,
                         smem + nxt * kStage, y);
        cur = cur == 2 ? 0 : cur + 1;
    }
    for (int b = nb4; b < nb; ++b) {
        const int nxt = cur == 0 ? 2 : cur - 1;
        block_int8<kDump>(p, b, m0, n0, row_lo, row_hi, wave, lane, in, ioff, ro, smem + cur * kStage,
                          smem + nxt * kStage, y);
        cur = cur == 2 ? 0 : cur + 1;
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

}  // namespace

int launch_w4ax_gemm_fp6(const GemmProblem& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool dump = p.P != nullptr;
    const int rows = dump ? p.m_count : p.M;
    const int tiles = ((rows + kTM - 1) / kTM) * (p.N / kTN);
    const int grid = 8 * ((tiles + 7) / 8);
    if (dump)
        gemm_fp6_kernel<true><<<grid, kThreads, 0, s>>>(p);
    else
        gemm_fp6_kernel<false><<<grid, kThreads, 0, s>>>(p);
    return static_cast<int>(hipGetLastError());
}

}  // namespace comet
