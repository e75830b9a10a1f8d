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
// Tiling: four waves per workgroup (2 x 2), two workgroups per CU; a wave
// computes 64 rows x 16 kWC columns. kWC = 8 (128 x 256 per workgroup) reads
// a quarter fewer LDS and HBM bytes per output than kWC = 4 (128 x 128), at
// the register limit (255 VGPRs), and is used when the grid is large. Operands
// travel HBM -> LDS by direct loads (buffer_load ... lds: each lane's 16 or 4
// bytes land at LDS base + lane * size) into a ring of stages ahead of the
// compute: three stages two blocks ahead for kWC = 4, two stages one block
// ahead for kWC = 8 (whose stage is half again as large and whose block takes
// twice as long). Both operand layouts are 16-row (16-channel) tiles, so
// every direct load is a contiguous copy. The weight tiles are in the order a
// wave reads them (every LDS read of a 16-lane k-group one contiguous 256-byte
// run); the activation tiles keep each row's bytes together for the
// quantizer's stores, with a per-row slot permutation that keeps the reads
// free of bank conflicts (tile_head, tile_tail). Each wave issues the same number of direct loads per block of
// either kind (one scale word, then A and B, plus a balancing load where the
// kinds differ), so a single partial wait at the end of a block publishes the
// next one.
//
// Epilogue. Per block every output needs y += (s_x s_w) P. On gfx950 the
// matrix unit and the VALU barely overlap, so the epilogue is kept to one FMA
// per output and the scale products t = s_x s_w of a 64 x 16 column tile come
// from one v_mfma_f32_16x16x1_4b_f32 (an outer product of the lane's row
// scale and column scale, exact in FP32, cheaper than 16 VALU multiplies per
// lane). The epilogue of column tile c is issued after the matrix
// instructions of tile c+1, so it never waits on a result just produced.
//
// LDS stage (kWC = 4: 25.6 KB, kWC = 8: 38 KB):
//   4-bit block: A at 0, eight 16-row tiles of 1536 bytes (row-contiguous:
//     heads at tile_head(r, g), tails at tile_tail(r, g)); B at 12288, the
//     tile's 2 kWC FP6 fragments (lane order: 16 lane, 1024 + 8 lane).
//   8-bit block: A at 0, eight 16-row tiles of 2048 bytes (1024h +
//     tile_head(r, g) for positions 32g + 16h ..); B at 16384, the tile's
//     2 kWC INT4 fragments.
//   then the block's 128 activation scales (f32) and 32 kWC weight scales
//   (fp16), and a pad that receives the balancing loads.
#include <mutex>

#include "comet_internal.h"
#include "device_util.h"

namespace comet {
namespace {

constexpr int kThreads = 256;
constexpr int kTM = 128;
constexpr int kTileF6 = 1536;                // 16 rows / channels x 128 positions of FP6 codes
constexpr int kTileI8 = 2048;                // 16 rows x 128 positions of INT8 codes
constexpr int kOffB6 = 12288;                // B of a 4-bit block
constexpr int kOffB8 = 16384;                // B of an 8-bit block

// Shape of the workgroup tile for kWC column tiles per wave.
template <int kWC>
struct Cfg {
    static constexpr int kTN = 32 * kWC;                                   // columns per workgroup
    static constexpr int kOffSa = kOffB6 + 3072 * kWC > kOffB8 + 2048 * kWC ? kOffB6 + 3072 * kWC
                                                                            : kOffB8 + 2048 * kWC;
    static constexpr int kOffSw = kOffSa + kTM * 4;
    static constexpr int kOffPad = kOffSw + kTN * 2;
    static constexpr int kStage = kOffPad + (kWC == 4 ? 256 : 1024);
    static constexpr int kStages = kWC == 4 ? 3 : 2;
    static constexpr int kAhead = kStages - 1;                             // blocks in flight ahead
    static constexpr int kLoads = kWC == 4 ? 7 : 10;                       // direct loads per wave and block
};

// Buffer resources of the four inputs, built once per workgroup (SGPRs).
struct Inputs {
    Rsrc xq, xs, wq, ws;
    uint32_t mp;                        // rows padded to whole 16-row tiles
};

__device__ __forceinline__ Inputs make_inputs(const GemmProblem& p) {
    const uint32_t nb8 = static_cast<uint32_t>(p.nb - p.nb4);
    Inputs in;
    in.mp = (static_cast<uint32_t>(p.M) + 15u) & ~15u;
    in.xq = make_rsrc(p.Xq, in.mp * (96u * p.nb4 + 128u * nb8));
    in.xs = make_rsrc(p.x_scale, static_cast<uint32_t>(p.M) * p.nb * 4u);
    in.wq = make_rsrc(p.Wq, static_cast<uint32_t>(p.N) * (96u * p.nb4 + 64u * nb8));
    in.ws = make_rsrc(p.w_scale, static_cast<uint32_t>(p.N) * p.nb * 2u);
    return in;
}

// Direct loads of block b into stage `st` for the tile at rows m0 (a multiple
// of 16) and columns n0. `sc` is this lane's scale-word offset: waves 0 and 1
// load the activation scales of rows 64w + lane (clamped into [0, M)), the
// other waves two weight scales per lane (kWC = 4: wave 2; kWC = 8: waves 2
// and 3, 128 columns each).
template <int kWC>
__device__ __forceinline__ void issue(const GemmProblem& p, const Inputs& in, int b, int m0, int n0, int wave,
                                      int lane, uint32_t sc, uint8_t* st) {
    using C = Cfg<kWC>;
    const uint32_t M = p.M, N = p.N, nb4 = p.nb4, mp = in.mp;
    const uint32_t ub = static_cast<uint32_t>(b);
    if (wave < 2)
        lds_buf4(in.xs, sc, ub * M * 4u, st + C::kOffSa + 256 * wave);
    else if (kWC == 8)
        lds_buf4(in.ws, sc, (ub * N + n0) * 2u + 256u * (wave - 2), st + C::kOffSw + 256 * (wave - 2));
    else
        lds_buf4(in.ws, sc, (ub * N + n0) * 2u, st + (wave == 2 ? C::kOffSw : C::kOffPad));
    const uint32_t groups = N / 16;
    const uint32_t lane16 = 16u * static_cast<uint32_t>(lane);
    const uint32_t tile = static_cast<uint32_t>(m0) / 16;
    // 1 KB pieces of B per wave: 2 kWC tiles of 1536 (4-bit) or 1024 (8-bit)
    // bytes shared by four waves
    constexpr int kB6 = 3 * kWC / 4;
    constexpr int kB8 = kWC / 2;
    static_assert(1 + 3 + kB6 == C::kLoads && 1 + 4 + kB8 + (kWC == 8 ? 1 : 0) == C::kLoads,
                  "one partial wait needs equal load counts for both block kinds");
    static_assert(kOffB6 + 4 * 1024 * kB6 <= C::kOffSa && kOffB8 + 4 * 1024 * kB8 <= C::kOffSa &&
                      4 * 3072 <= kOffB6 && 4 * 4096 <= kOffB8,
                  "operands overlap in the stage");
    static_assert(C::kOffSw == C::kOffSa + 2 * 256 && C::kOffPad + (kWC == 8 ? 4 : 1) * 256 <= C::kStage,
                  "scale words or balancing loads outside the stage");
    if (b < p.nb4) {
        const uint32_t a = ub * mp * 96u + tile * kTileF6 + 3072u * wave;
#pragma unroll
        for (int k = 0; k < 3; ++k) lds_buf16(in.xq, lane16, a + 1024 * k, st + 3072 * wave + 1024 * k);
        const uint32_t w = (ub * groups + n0 / 16) * kTileF6 + 1024u * kB6 * wave;
#pragma unroll
        for (int k = 0; k < kB6; ++k)
            lds_buf16(in.wq, lane16, w + 1024 * k, st + kOffB6 + 1024 * kB6 * wave + 1024 * k);
    } else {
        const uint32_t a = nb4 * mp * 96u + (ub - nb4) * mp * 128u + tile * kTileI8 + 4096u * wave;
#pragma unroll
        for (int k = 0; k < 4; ++k) lds_buf16(in.xq, lane16, a + 1024 * k, st + 4096 * wave + 1024 * k);
        const uint32_t w = groups * (kTileF6 * nb4 + kFragBytes * (ub - nb4)) + (n0 / 16) * kFragBytes +
                           1024u * kB8 * wave;
#pragma unroll
        for (int k = 0; k < kB8; ++k)
            lds_buf16(in.wq, lane16, w + 1024 * k, st + kOffB8 + 1024 * kB8 * wave + 1024 * k);
        if (kWC == 8) lds_buf4(in.xs, sc, ub * M * 4u, st + C::kOffPad + 256 * wave);   // balancing load
    }
}

// End of block b (of a run of blocks ending before b_end): block b+1 has
// landed once only the loads of the blocks issued after it may still be in
// flight; the barrier publishes it and frees block b's stage.
template <int kWC>
__device__ __forceinline__ void end_block(int b, int b_end) {
    using C = Cfg<kWC>;
    if (C::kAhead == 2 && b + 2 < b_end) COMET_VMCNT(C::kLoads);
    else COMET_VMCNT(0);
    __builtin_amdgcn_s_barrier();
}

// Scales of a block for this lane: s_x of its row in the wave's 64 (the A
// input of the outer products, divided by 16 on the INT8 path) and s_w of its
// column in each of the kWC column tiles.
template <int kWC>
struct Scales {
    float sa;
    float sw[kWC];
};

template <int kWC>
__device__ __forceinline__ void read_scales(const uint8_t* __restrict__ st, int wr, int wc, int lane, float mul,
                                            Scales<kWC>& s) {
    const float* sa_l = reinterpret_cast<const float*>(st + Cfg<kWC>::kOffSa);
    const uint16_t* sw_l = reinterpret_cast<const uint16_t*>(st + Cfg<kWC>::kOffSw);
    s.sa = sa_l[64 * wr + lane] * mul;
#pragma unroll
    for (int c = 0; c < kWC; ++c) s.sw[c] = h2f(sw_l[16 * kWC * wc + 16 * c + (lane & 15)]);
}

// t of column tile c: element 4r + i is s_x(row 16r + 4g + i) * s_w(column).
template <int kWC>
__device__ __forceinline__ v16f scale_products(const Scales<kWC>& s, int c) {
    v16f t = {};
    return __builtin_amdgcn_mfma_f32_16x16x1f32(s.sa, s.sw[c], t, 0, 0, 0);
}

__device__ __forceinline__ v8i fp6_operand(const uint8_t* tile, int lane) {
    const uint4 h = *reinterpret_cast<const uint4*>(tile + 16 * lane);
    const uint2 t = *reinterpret_cast<const uint2*>(tile + 1024 + 8 * lane);
    return v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)t.x, (int)t.y, 0, 0};
}

// The activation operand of lane 16 g + r from a row-contiguous tile
// (tile_head / tile_tail).
__device__ __forceinline__ v8i fp6_operand_rows(const uint8_t* tile, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const uint4 h = *reinterpret_cast<const uint4*>(tile + tile_head(r, g));
    const uint2 t = *reinterpret_cast<const uint2*>(tile + tile_tail(r, g));
    return v8i{(int)h.x, (int)h.y, (int)h.z, (int)h.w, (int)t.x, (int)t.y, 0, 0};
}

// Epilogue of column tile c: y += t P, or the partials themselves.
template <bool kDump, int kWC>
__device__ __forceinline__ void epilogue(const GemmProblem& p, const v16f& t, const v4f (&D)[4], int c, int b,
                                         int row0, int col0, int row_lo, int row_hi, float (&y)[4][kWC][4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (kDump) {
                const int row = row0 + 16 * r + i;
                if (row >= row_lo && row < row_hi)
                    p.P[(static_cast<size_t>(row - row_lo) * p.N + col0 + 16 * c) * p.nb + b] =
                        static_cast<int>(D[r][i]);
            } else {
                y[r][c][i] = __builtin_fmaf(t[4 * r + i], D[r][i], y[r][c][i]);
            }
        }
}

// One 4-bit block from stage `st`: issue the block kAhead further on into
// `nxt`, then the matrix work of column tile c followed by the epilogue of
// tile c-1.
template <bool kDump, int kWC>
__device__ __forceinline__ void block_fp6(const GemmProblem& p, const Inputs& in, int b, int b_end, int m0, int n0,
                                          int row_lo, int row_hi, int wave, int lane, uint32_t sc,
                                          const uint8_t* __restrict__ st, uint8_t* __restrict__ nxt,
                                          float (&y)[4][kWC][4]) {
    constexpr int kAhead = Cfg<kWC>::kAhead;
    const int wr = wave >> 1, wc = wave & 1;
    if (b + kAhead < b_end) issue<kWC>(p, in, b + kAhead, m0, n0, wave, lane, sc, nxt);
    const int row0 = m0 + 64 * wr + 4 * (lane >> 4);
    const int col0 = n0 + 16 * kWC * wc + (lane & 15);
    Scales<kWC> s;
    read_scales<kWC>(st, wr, wc, lane, 1.0f, s);
    v8i A[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) A[r] = fp6_operand_rows(st + (4 * wr + r) * kTileF6, lane);
    v4f Dp[4], Dc[4];
    v16f tp = {}, tc = {};
    if constexpr (!kDump) tp = scale_products<kWC>(s, 0);
    {
        const v8i B = fp6_operand(st + kOffB6 + (kWC * wc) * kTileF6, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) Dp[r] = mfma_fp6(A[r], B);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 1; c < kWC; ++c) {
        if constexpr (!kDump) tc = scale_products<kWC>(s, c);
        const v8i B = fp6_operand(st + kOffB6 + (kWC * wc + c) * kTileF6, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) Dc[r] = mfma_fp6(A[r], B);
        epilogue<kDump, kWC>(p, tp, Dp, c - 1, b, row0, col0, row_lo, row_hi, y);
#pragma unroll
        for (int r = 0; r < 4; ++r) Dp[r] = Dc[r];
        tp = tc;
        __builtin_amdgcn_sched_barrier(0);
    }
    epilogue<kDump, kWC>(p, tp, Dp, kWC - 1, b, row0, col0, row_lo, row_hi, y);
    end_block<kWC>(b, b_end);
}

// One 8-bit block: INT8 matrix instruction, weights widened to 16 q_w, so the
// accumulator holds 16 P; the row scales are divided by 16 (exactly).
template <bool kDump, int kWC>
__device__ __forceinline__ void block_int8(const GemmProblem& p, const Inputs& in, int b, int b_end, int m0, int n0,
                                           int row_lo, int row_hi, int wave, int lane, uint32_t sc,
                                           const uint8_t* __restrict__ st, uint8_t* __restrict__ nxt,
                                           float (&y)[4][kWC][4]) {
    constexpr int kAhead = Cfg<kWC>::kAhead;
    const int wr = wave >> 1, wc = wave & 1;
    if (b + kAhead < b_end) issue<kWC>(p, in, b + kAhead, m0, n0, wave, lane, sc, nxt);
    const int row0 = m0 + 64 * wr + 4 * (lane >> 4);
    const int col0 = n0 + 16 * kWC * wc + (lane & 15);
    Scales<kWC> s;
    read_scales<kWC>(st, wr, wc, lane, kDump ? 1.0f : 0.0625f, s);
    v4i A0[4], A1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint8_t* t = st + (4 * wr + r) * kTileI8 + tile_head(lane & 15, lane >> 4);
        A0[r] = as_v4i(*reinterpret_cast<const uint4*>(t));
        A1[r] = as_v4i(*reinterpret_cast<const uint4*>(t + 1024));
    }
    const v4i zero = {0, 0, 0, 0};
    v4f Dp[4], Dc[4];
    v16f tp = {}, tc = {};
#pragma unroll
    for (int c = 0; c < kWC; ++c) {
        if constexpr (!kDump) tc = scale_products<kWC>(s, c);
        const uint4 pk = *reinterpret_cast<const uint4*>(st + kOffB8 + (kWC * wc + c) * kFragBytes + 16 * lane);
        const v4i B0 = widen_weights_lo(pk);
        const v4i B1 = widen_weights_hi(pk);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v4i acc = mfma_i8(A0[r], B0, zero);
            acc = mfma_i8(A1[r], B1, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Dc[r][i] = kDump ? static_cast<float>(acc[i] >> 4) : static_cast<float>(acc[i]);
        }
        if (c > 0) epilogue<kDump, kWC>(p, tp, Dp, c - 1, b, row0, col0, row_lo, row_hi, y);
#pragma unroll
        for (int r = 0; r < 4; ++r) Dp[r] = Dc[r];
        tp = tc;
    }
    epilogue<kDump, kWC>(p, tp, Dp, kWC - 1, b, row0, col0, row_lo, row_hi, y);
    end_block<kWC>(b, b_end);
}

// QUIK's fp16 outlier channels (QUIK blog, section "第二步: 前向传播 (在线)":
// the outlier columns are multiplied in FP16 on their own path and the two
// results added). Here the two paths meet in the tile's FP32 accumulators:
// after the quantized blocks, each 32-channel step of the outlier part is one
// 16x16x32 fp16 matrix instruction per 16x16 tile, accumulating straight into
// y (the products of two fp16 values are exact in FP32). A step's operands
// are the workgroup's 8 row-tile pieces and 2 kWC column-tile pieces of 1 KB;
// the waves share them out of LDS (the main loop's ring, free by now), two
// steps in flight, each piece one direct load by one wave. Row tiles past the
// padded rows read 0 through the buffer's range check.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

template <int kWC>
__device__ __forceinline__ void fp16_tail(const GemmProblem& p, int m0, int n0, int wave, int lane,
                                          uint8_t* smem, float (&y)[4][kWC][4]) {
    constexpr int kRowPieces = kTM / 16;
    constexpr int kPieces = kRowPieces + 2 * kWC;
    constexpr int kPerWave = kPieces / 4;                 // direct loads per wave and step
    static_assert(kPieces % 4 == 0 && 2 * kPieces * 1024 <= Cfg<kWC>::kStages * Cfg<kWC>::kStage, "tail stages");
    const int wr = wave >> 1, wc = wave & 1;
    const uint32_t steps = static_cast<uint32_t>(p.nf) / 32u;
    const uint32_t mp = (static_cast<uint32_t>(p.M) + 15u) & ~15u;
    const Rsrc rx = make_rsrc(p.xf, mp * static_cast<uint32_t>(p.nf) * 2u);
    const Rsrc rw = make_rsrc(p.wf, static_cast<uint32_t>(p.N) * static_cast<uint32_t>(p.nf) * 2u);
    const uint32_t tr0 = static_cast<uint32_t>(m0) / 16u, tc0 = static_cast<uint32_t>(n0) / 16u;
    auto issue = [&](uint32_t s, uint8_t* st) {
#pragma unroll
        for (int k = 0; k < kPerWave; ++k) {
            const int q = wave + 4 * k;                   // piece q: row tiles first, then column tiles
            if (q < kRowPieces)
                lds_buf16(rx, 16u * lane, ((tr0 + q) * steps + s) * 1024u, st + q * 1024);
            else
                lds_buf16(rw, 16u * lane, ((tc0 + q - kRowPieces) * steps + s) * 1024u, st + q * 1024);
        }
    };
    COMET_VMCNT(0);
    __syncthreads();                                      // the last block's LDS reads are done
    issue(0, smem);
    for (uint32_t s = 0; s < steps; ++s) {
        uint8_t* cur = smem + (s & 1u) * kPieces * 1024;
        if (s + 1 < steps) {
            issue(s + 1, smem + ((s + 1) & 1u) * kPieces * 1024);
            COMET_VMCNT(kPerWave);                        // this wave's pieces of step s
        } else {
            COMET_VMCNT(0);
        }
        __syncthreads();                                  // every wave's pieces of step s
        v8h a[4], b[kWC];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            a[r] = *reinterpret_cast<const v8h*>(cur + (4 * wr + r) * 1024 + 16 * lane);
#pragma unroll
        for (int c = 0; c < kWC; ++c)
            b[c] = *reinterpret_cast<const v8h*>(cur + (kRowPieces + kWC * wc + c) * 1024 + 16 * lane);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < kWC; ++c) {
                v4f acc = {y[r][c][0], y[r][c][1], y[r][c][2], y[r][c][3]};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], b[c], acc, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[r][c][i] = acc[i];
            }
        __syncthreads();                                  // step s read before its buffer is refilled
    }
}

// ---------------------------------------------------------------------------
// Tile scheduling (COMET article, mmssai.com/?p=43269, section
// "2.混合精度计算的动态调度": tiles are not bound to compute units; work is
// balanced between units even though 8-bit blocks cost more than 4-bit ones).
//
// A grid of at least one wave of 128-row tiles (two workgroups per CU) runs as
// it is: one tile per workgroup, XCD-aware order (tile_of). A smaller grid
// cannot fill 256 CUs with whole tiles, so each tile's blocks are split into
// S runs of equal cost (an 8-bit block costs twice a 4-bit one: twice the
// matrix instructions, plus widening and conversion), S chosen by the cost
// model of make_plan, and the runs are the work items of a persistent grid:
//   * the items are dealt in the XCD-aware tile order into 8 contiguous
//     ranges, one per XCD (workgroup w runs on XCD w mod 8); workgroup j of an
//     XCD starts on item j of its range without any atomic, and a range
//     longer than its XCD's workgroups hands out the rest with an atomic
//     counter (the workgroups that finish first take them);
//   * each run stores its FP32 partial tile in the workspace; a second kernel
//     adds the runs of every tile in split order, y_0 + y_1 + ... + y_{S-1},
//     writes Y and clears the counters for the next call. The kernel
//     boundary publishes the partial tiles: no device-scope fence, no
//     floating-point atomics, no workgroup waiting for another, and Y does
//     not depend on timing.
// Measured on MI355X and kept out: a fix-up inside the kernel by the last
// run to finish (its device-scope fences write back and invalidate L2:
// down_7b 256 us against 64), idle workgroups taking items from other XCDs'
// ranges (the cross-XCD takes doubled the time of every grid that used them:
// up_gate_7b split 101 us against 64 without), and splitting grids of one
// wave or more (up_gate_7b, 688 tiles: whole tiles 58 us, the tiles past the
// first wave split 64 us).
// ---------------------------------------------------------------------------

constexpr int kMaxSplits = 8;
#ifndef COMET_FP6_SPLITS_CAP
#define COMET_FP6_SPLITS_CAP kMaxSplits
#endif

struct Sched {
    uint32_t* queue;       // [0..7] per-XCD counters; nullptr: one tile per workgroup
    float* partials;       // [tiles][splits][kTM * 32 kWC] FP32 partial tiles
    int tiles_m, tiles_n, tm0;   // tiles launched (row tiles tm0 .. tm0 + tiles_m - 1)
    int splits;
    int items, per_xcd;    // runs in all, and per XCD range (rounded up)
    int wg_per_xcd;        // workgroups per XCD: the first that many items of a range are
                           // dealt one per workgroup, the rest by the range's counter
    int bounds[kMaxSplits + 1];  // run s covers blocks [bounds[s], bounds[s + 1])
};

// Workspace: the 8 queue counters in the first kCtrlBytes (the same place for
// every shape, zero between calls), then the partial tiles.
constexpr size_t kCtrlBytes = 256;

// Row and column tile of tile t in the XCD-aware order of tile_of (8-row-tile
// groups walked column by column).
__host__ __device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
    constexpr int G = 8;
    const int group = t / (G * tiles_n);
    const int first = group * G;
    const int gh = imin(G, tiles_m - first);
    const int in = t - group * G * tiles_n;
    tn = in / gh;
    tm = first + in % gh;
}

// The range counters are taken and cleared at system scope: the take is then
// coherent whichever XCD a workgroup actually runs on, so every item goes to
// exactly one workgroup.
__device__ __forceinline__ uint32_t take_counter(uint32_t* a) {
    return __hip_atomic_fetch_add(a, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Number of items in XCD x's range: [x per_xcd, x per_xcd + count).
__device__ __forceinline__ int range_count(const Sched& sc, int x) {
    return imax(0, imin(sc.per_xcd, sc.items - x * sc.per_xcd));
}

// Next item for a workgroup of XCD x after its first, or -1: the range's
// items past the first wg_per_xcd go out in order of the counter (one thread
// calls this).
__device__ __forceinline__ int next_item(const Sched& sc, int x) {
    const int n = range_count(sc, x) - sc.wg_per_xcd;
    if (n <= 0) return -1;
    const int h = static_cast<int>(take_counter(&sc.queue[x]));
    return h < n ? x * sc.per_xcd + sc.wg_per_xcd + h : -1;
}

// The blocks [b_begin, b_end) of the tile at rows m0, columns n0, into y (or
// the partials of those blocks, kDump). Stages are used from stage 0 on; at
// the end every wave is past the last barrier, so the stages are free again.
template <bool kDump, int kWC>
__device__ __forceinline__ void run_blocks(const GemmProblem& p, const Inputs& in, int b_begin, int b_end, int m0,
                                           int n0, int row_lo, int row_hi, int wave, int lane, uint32_t sc,
                                           uint8_t* smem, float (&y)[4][kWC][4]) {
    using C = Cfg<kWC>;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < kWC; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) y[r][c][i] = 0.0f;
    if (b_begin >= b_end) return;

    // prologue: blocks b_begin .. b_begin + kAhead - 1 in flight; wait for the first
    issue<kWC>(p, in, b_begin, m0, n0, wave, lane, sc, smem);
    if (C::kAhead == 2 && b_begin + 1 < b_end) {
        issue<kWC>(p, in, b_begin + 1, m0, n0, wave, lane, sc, smem + C::kStage);
        COMET_VMCNT(C::kLoads);
    } else {
        COMET_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();

    // Block b lives in stage (b - b_begin) mod kStages and block b+kAhead is
    // loaded into the stage after it. The stage pointers are restrict-qualified
    // in the block functions: an LDS read of one stage does not wait for the
    // direct loads in flight into another. The 4-bit blocks come first in the
    // permuted order, the 8-bit ones last.
    int cur = 0;
    const int end4 = imin(b_end, p.nb4);
    for (int b = b_begin; b < end4; ++b) {
        const int nxt = cur == 0 ? C::kStages - 1 : cur - 1;
        block_fp6<kDump, kWC>(p, in, b, b_end, m0, n0, row_lo, row_hi, wave, lane, sc, smem + cur * C::kStage,
                              smem + nxt * C::kStage, y);
        cur = cur == C::kStages - 1 ? 0 : cur + 1;
    }
    for (int b = imax(b_begin, p.nb4); b < b_end; ++b) {
        const int nxt = cur == 0 ? C::kStages - 1 : cur - 1;
        block_int8<kDump, kWC>(p, in, b, b_end, m0, n0, row_lo, row_hi, wave, lane, sc, smem + cur * C::kStage,
                               smem + nxt * C::kStage, y);
        cur = cur == C::kStages - 1 ? 0 : cur + 1;
    }
}

// Y of the tile from y (rows below row_hi).
template <int kWC>
__device__ __forceinline__ void store_y(const GemmProblem& p, int m0, int n0, int row_hi, int wave, int lane,
                                        const float (&y)[4][kWC][4]) {
    const int wr = wave >> 1, wc = wave & 1, g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + 64 * wr + 16 * r + 4 * g + i;
            if (row < row_hi) {
                uint16_t* yrow = p.Y + static_cast<size_t>(row) * p.ldy + n0 + 16 * kWC * wc + l16;
#pragma unroll
                for (int c = 0; c < kWC; ++c) yrow[16 * c] = __half_as_ushort(__float2half_rn(y[r][c][i]));
            }
        }
}

// Partial tile of run s of a tile: the float4 y[r][c][0..3] of thread t at
// index (r kWC + c) 256 + t, so each float4 store or load of a workgroup is
// one contiguous 4 KB run.
template <int kWC>
__host__ __device__ __forceinline__ size_t slot_offset(int tile, int splits, int s) {
    return (static_cast<size_t>(tile) * splits + s) * (kTM * 32 * kWC / 4);
}

template <int kWC>
__device__ __forceinline__ void store_partial(const Sched& sc, int tile, int s, const float (&y)[4][kWC][4]) {
    float4* own = reinterpret_cast<float4*>(sc.partials) + slot_offset<kWC>(tile, sc.splits, s);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < kWC; ++c)
            own[(r * kWC + c) * kThreads + threadIdx.x] = make_float4(y[r][c][0], y[r][c][1], y[r][c][2], y[r][c][3]);
}

template <bool kDump, int kWC>
__global__ __launch_bounds__(kThreads, 2) void gemm_fp6_kernel(GemmProblem p, Sched sc) {
    using C = Cfg<kWC>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kStages * C::kStage];
    __shared__ int item_lds;

    // the partials variant runs the tiles of the full launch (128-row tiles
    // from row 0) that hold rows of [m_begin, m_begin + m_count), and stores
    // only those rows
    const int row_lo = kDump ? p.m_begin : 0;
    const int row_hi = kDump ? p.m_begin + p.m_count : p.M;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Inputs in = make_inputs(p);
    float y[4][kWC][4];

    if (kWC != 4 || sc.queue == nullptr) {
        // one tile per workgroup, all blocks (the work queue serves the
        // 128 x 128 tiles only: the wide tile is chosen for large grids)
        int tm, tn;
        if (!tile_of(blockIdx.x, sc.tiles_m, sc.tiles_n, tm, tn)) return;
        const int m0 = (sc.tm0 + tm) * kTM;
        const int n0 = tn * C::kTN;
        const uint32_t scw = wave < 2 ? static_cast<uint32_t>(imin(m0 + 64 * wave + lane, p.M - 1)) * 4u : 4u * lane;
        run_blocks<kDump, kWC>(p, in, 0, p.nb, m0, n0, row_lo, row_hi, wave, lane, scw, smem, y);
        if constexpr (!kDump) {
            if (p.nf > 0) fp16_tail<kWC>(p, m0, n0, wave, lane, smem, y);
            store_y<kWC>(p, m0, n0, row_hi, wave, lane, y);
        }
        return;
    }

    // persistent: item j of the XCD's range to its workgroup j, then (when
    // the range is longer than the XCD's workgroups) items from the counter
    const int xcd = blockIdx.x & 7;
    const bool queued = sc.per_xcd > sc.wg_per_xcd;
    int item = static_cast<int>(blockIdx.x >> 3) < range_count(sc, xcd) ? xcd * sc.per_xcd + (blockIdx.x >> 3) : -1;
    while (item >= 0) {
        const int tile = item / sc.splits, s = item - tile * sc.splits;
        int tm, tn;
        tile_coords(tile, sc.tiles_m, sc.tiles_n, tm, tn);
        const int m0 = (sc.tm0 + tm) * kTM;
        const int n0 = tn * C::kTN;
        const uint32_t scw = wave < 2 ? static_cast<uint32_t>(imin(m0 + 64 * wave + lane, p.M - 1)) * 4u : 4u * lane;
        run_blocks<kDump, kWC>(p, in, sc.bounds[s], sc.bounds[s + 1], m0, n0, row_lo, row_hi, wave, lane, scw, smem, y);
        if constexpr (!kDump) {
            if (p.nf > 0 && s == sc.splits - 1) fp16_tail<kWC>(p, m0, n0, wave, lane, smem, y);   // the last run
            store_partial<kWC>(sc, tile, s, y);
        }
        if (!queued) break;
        if (threadIdx.x == 0) item_lds = next_item(sc, xcd);
        __syncthreads();
        item = item_lds;
        __syncthreads();         // every wave has the item before thread 0 may overwrite it
    }
}

// The second kernel of a split grid: four workgroups per tile (one per row
// tile r of each wave's 64 rows) add the tile's partial tiles in split order
// and write Y. Threads are numbered as in the GEMM's workgroup, so thread t
// reads what thread t stored; each thread first issues the loads of every
// run (kWC float4 per run, all in flight at once), then adds them in order.
// Workgroup 0 also clears the queue counters. With `tiles` = 0 it only clears
// them (the partials variant, which stores no partial tiles).
template <int kWC>
__global__ __launch_bounds__(kThreads) void gemm_fp6_splits_kernel(GemmProblem p, Sched sc, int tiles) {
    if (blockIdx.x == 0 && threadIdx.x < 8) sc.queue[threadIdx.x] = 0u;
    const int tile = blockIdx.x >> 2, r = blockIdx.x & 3;
    if (tile >= tiles) return;
    int tm, tn;
    tile_coords(tile, sc.tiles_m, sc.tiles_n, tm, tn);
    const int t = threadIdx.x;
    const float4* base = reinterpret_cast<const float4*>(sc.partials);
    float4 v[kMaxSplits][kWC];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
        if (s < sc.splits)
#pragma unroll
            for (int c = 0; c < kWC; ++c) v[s][c] = base[slot_offset<kWC>(tile, sc.splits, s) + (r * kWC + c) * kThreads + t];
    float y[kWC][4];
#pragma unroll
    for (int c = 0; c < kWC; ++c) {
        float4 a = v[0][c];
#pragma unroll
        for (int s = 1; s < kMaxSplits; ++s)
            if (s < sc.splits) {
                a.x += v[s][c].x;
                a.y += v[s][c].y;
                a.z += v[s][c].z;
                a.w += v[s][c].w;
            }
        y[c][0] = a.x;
        y[c][1] = a.y;
        y[c][2] = a.z;
        y[c][3] = a.w;
    }
    const int wave = t >> 6, lane = t & 63;
    const int wr = wave >> 1, wc = wave & 1, g = lane >> 4, l16 = lane & 15;
    const int m0 = (sc.tm0 + tm) * kTM, n0 = tn * Cfg<kWC>::kTN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + 64 * wr + 16 * r + 4 * g + i;
        if (row < p.M) {
            uint16_t* yrow = p.Y + static_cast<size_t>(row) * p.ldy + n0 + 16 * kWC * wc + l16;
#pragma unroll
            for (int c = 0; c < kWC; ++c) yrow[16 * c] = __half_as_ushort(__float2half_rn(y[c][i]));
        }
    }
}

// Launch plan of a shape; the same for both variants (Y and the partials).
struct Plan {
    int wc;                  // column tiles per wave: 8 (128 x 256 tiles) or 4 (128 x 128)
    int tiles_m, tiles_n;    // of the full launch
    int splits;              // runs per tile; 1: one tile per workgroup, no workspace
    int bounds[kMaxSplits + 1];
    size_t ws_bytes;         // workspace the plan needs
};

// The plan (and so the workspace size) depends on the shape only: it is made
// for the 256 CUs of an MI355X, so a workspace query needs no device. The
// persistent grid itself is sized from the device's CU count.
constexpr int kPlanCUs = 256;

Plan make_plan(int M, int N, int K, int nb8) {
    Plan pl{};
    const int nb = K / kBlock, nb4 = nb - nb8;
    pl.tiles_m = (M + kTM - 1) / kTM;
    const int slots = 2 * kPlanCUs;      // two workgroups per CU
    const int wide_tiles = N % Cfg<8>::kTN == 0 ? pl.tiles_m * (N / Cfg<8>::kTN) : 0;
    pl.wc = wide_tiles >= 2 * slots ? 8 : 4;
    pl.tiles_n = N / (32 * pl.wc);
    const int tiles = pl.tiles_m * pl.tiles_n;
    pl.splits = 1;
    // Split only where the cost model says it pays: time in block-steps of
    // a 4-bit block with two workgroups per CU (an 8-bit block costs 2), a
    // workgroup alone on its CU about 1.3x faster, each run paying about 2
    // block-steps of its own (pipeline start, partial tile store) and a split
    // plan about 15 more for the second kernel, and at most two waves of
    // runs. Calibrated on the 7B layers (whole tiles against runs): q_proj_7b
    // 24 against 16 us (8 runs), down_7b 72 against 63 us (2 runs); a
    // 300-tile grid of 8 blocks 14 against 28 us (2 runs: it stays whole).
    if (pl.wc == 4 && tiles < slots) {
        const double c = nb4 + 2.0 * nb8;
        auto run_cost = [&](int items, double per_item) {
            if (items <= kPlanCUs) return per_item / 1.3;
            return per_item * ((items + slots - 1) / slots);
        };
        double best = run_cost(tiles, c);
        for (int sp = 2; sp <= imin(COMET_FP6_SPLITS_CAP, nb / 2) && tiles * sp <= 2 * slots; ++sp) {
            const double t = run_cost(tiles * sp, c / sp + 2.0) + 15.0;
            if (t < best) {
                best = t;
                pl.splits = sp;
            }
        }
    }
    // runs of about equal cost: a 4-bit block 1, an 8-bit block 2 (the 8-bit
    // blocks are the last nb8); every run holds at least one block
    auto cost_to = [nb4](int b) { return imin(b, nb4) + 2 * imax(0, b - nb4); };
    const int cost = cost_to(nb);
    pl.bounds[0] = 0;
    for (int s = 1; s < pl.splits; ++s) {
        const int goal = (cost * s + pl.splits / 2) / pl.splits;
        int b = pl.bounds[s - 1] + 1;
        while (b < nb && cost_to(b + 1) <= goal) ++b;
        pl.bounds[s] = imin(b, nb - (pl.splits - s));
    }
    pl.bounds[pl.splits] = nb;
    if (pl.splits > 1)
        pl.ws_bytes = kCtrlBytes + static_cast<size_t>(tiles) * pl.splits * kTM * 32 * pl.wc * 4;
    return pl;
}

template <bool kDump, int kWC>
int launch_plan(const GemmProblem& p, const Plan& pl, hipStream_t s) {
    Sched sc{};
    sc.splits = pl.splits;
    for (int i = 0; i <= pl.splits; ++i) sc.bounds[i] = pl.bounds[i];
    sc.tiles_n = pl.tiles_n;
    // the partials variant: the row tiles that hold [m_begin, m_begin + m_count)
    sc.tm0 = kDump ? p.m_begin / kTM : 0;
    sc.tiles_m = kDump ? (p.m_begin + p.m_count + kTM - 1) / kTM - sc.tm0 : pl.tiles_m;
    const int tiles = sc.tiles_m * sc.tiles_n;
    if (pl.splits == 1) {
        gemm_fp6_kernel<kDump, kWC><<<8 * ((tiles + 7) / 8), kThreads, 0, s>>>(p, sc);
        return static_cast<int>(hipGetLastError());
    }
    uint8_t* ws = static_cast<uint8_t*>(p.workspace);
    sc.queue = reinterpret_cast<uint32_t*>(ws);
    sc.partials = reinterpret_cast<float*>(ws + kCtrlBytes);
    sc.items = tiles * sc.splits;
    sc.per_xcd = (sc.items + 7) / 8;
    sc.wg_per_xcd = imin(sc.per_xcd, imax(1, 2 * cu_count() / 8));
    if (kDump && p.max_wg > 0) sc.wg_per_xcd = imin(sc.wg_per_xcd, imax(1, p.max_wg / 8));
    gemm_fp6_kernel<kDump, kWC><<<8 * sc.wg_per_xcd, kThreads, 0, s>>>(p, sc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
    gemm_fp6_splits_kernel<kWC><<<kDump ? 1 : 4 * tiles, kThreads, 0, s>>>(p, sc, kDump ? 0 : tiles);
    return static_cast<int>(hipGetLastError());
}

template <bool kDump>
int launch_fp6(const GemmProblem& p, hipStream_t s) {
    const Plan pl = make_plan(p.M, p.N, p.K, p.nb - p.nb4);
    return pl.wc == 8 ? launch_plan<kDump, 8>(p, pl, s) : launch_plan<kDump, 4>(p, pl, s);
}

}  // namespace

size_t gemm_fp6_workspace_bytes(int M, int N, int K, int nb8) {
    return make_plan(M, N, K, nb8).ws_bytes;
}

int launch_w4ax_gemm_fp6(const GemmProblem& p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    return p.P != nullptr ? launch_fp6<true>(p, s) : launch_fp6<false>(p, s);
}

// ---------------------------------------------------------------------------
// Allocation-free form of the FP6 GEMM, for callers that cannot allocate
// (code under HIP graph capture, serving loops, harnesses that forbid
// allocation): the workspace is a fixed array in device memory, one per GPU,
// held until the process ends. In host code the array's name is only a
// host-side stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// passed on. Calls on one GPU share the array: calls that may overlap on one
// GPU race. The queue counters at its start are zero when the code object is
// loaded, each call leaves them zero, and the first call on a device clears
// them again with a small kernel (no memset node, should that call be
// captured).
// ---------------------------------------------------------------------------

namespace {

static __device__ __align__(256) uint8_t scratch[COMET_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_cleared[kMaxDevices] = {};

__global__ void clear_words_kernel(uint32_t* w, int n) {
    if (static_cast<int>(threadIdx.x) < n) w[threadIdx.x] = 0u;
}

}  // namespace

int launch_w4ax_gemm_fp6_noalloc(GemmProblem p, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
    bool clear = false;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch_ptr[dev] == nullptr) {
            void* ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return static_cast<int>(e);
            g_scratch_ptr[dev] = ptr;
        }
        if (!g_scratch_cleared[dev]) {
            g_scratch_cleared[dev] = true;
            clear = true;
        }
        p.workspace = g_scratch_ptr[dev];
    }
    p.workspace_bytes = COMET_NOALLOC_SCRATCH_BYTES;
    if (clear) {
        clear_words_kernel<<<1, 64, 0, s>>>(static_cast<uint32_t*>(p.workspace), static_cast<int>(kCtrlBytes / 4));
        e = hipGetLastError();
        if (e != hipSuccess) return static_cast<int>(e);
    }
    return launch_w4ax_gemm_fp6(p, stream);
}

}  // namespace comet
