/*
 * comet_w4ax.h -- C ABI of the W4Ax fine-grained mixed-precision GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (COMET, ASPLOS 2025; FMPQ quantization plus the W4Ax kernel):
 *   - the input channels of a linear layer are split into 128-channel blocks;
 *     activation outliers concentrate in about a tenth of the channels, so a
 *     channel permutation gathers them into a few blocks, which are quantized
 *     to 8 bits while every other block is quantized to 4 bits
 *     (COMET article, mmssai.com/?p=43269, section "1.离群点分布规律的重定义");
 *   - weights are quantized to symmetric INT4 per output channel per block,
 *     offline (QUIK blog, deep-paper.org/paper/2310.09259, section
 *     "反量化背后的数学"); activations are quantized online, per token and per
 *     block, in one fused pass (QUIK blog, section "核融合");
 *   - the GEMM forms exact integer partial sums per block on the matrix
 *     units and dequantizes them in an FP32 epilogue that writes fp16
 *     (COMET summary, paperbot-e5f.pages.dev/papers/10460.html, abstract;
 *     QUIK blog, section "核融合").
 *
 * Three calls follow that statement of the problem: comet_pack_weights
 * (offline, host memory), comet_quant_act and comet_w4ax_gemm (online,
 * device memory, asynchronous on a HIP stream). The *_fp6 calls are the same
 * three steps on a second operand layout (FP6-encoded 4-bit codes) that the
 * prefill GEMM kernel consumes directly; the INT4 layout is the smaller one
 * and serves the weight-bandwidth-bound decode shapes. Further down: the
 * quantizer fused into the RMSNorm or SwiGLU before it, QUIK's asymmetric
 * 4-bit activations, QoQ's W4A8 variant, and a 4-bit KV cache with decode
 * attention over it.
 *
 * Shared rules
 *   - Every function returns a comet_status. Nothing throws across the ABI.
 *   - The caller owns every buffer. The online calls never allocate; the GEMM
 *     and the KV4 attention use only the workspace the caller passes.
 *   - All argument checks run before any HIP call, so a rejected call has no
 *     effect on the device and needs no GPU.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream. The
 *     online calls are asynchronous on it and never synchronize; errors of the
 *     kernels themselves surface at the caller's next synchronization.
 *   - Calls on different streams with disjoint outputs may run concurrently.
 *     Two GEMM calls that share one workspace must be ordered by the caller.
 *   - Device pointers must be 16-byte aligned, except where a call states
 *     2 bytes (comet_rmsnorm, comet_swiglu, the output of comet_kv4_attention).
 *
 * Notation: nb = K / 128 blocks; nb8 = n_int8_blocks; nb4 = nb - nb8. The
 * 8-bit blocks are always the LAST nb8 blocks of the permuted channel order
 * (comet_pack_weights ranks channels by ascending score, so the outlier
 * channels fill the highest blocks).
 *
 * Layouts (all little-endian):
 *   Xq, activation codes, device, M * (64 * nb4 + 128 * nb8) bytes,
 *     block-major. 4-bit block b (b < nb4) lives at byte b*M*64, row m at
 *     + m*64; byte 16g + j (g in 0..3, j in 0..15) of a row holds the code of
 *     block position 32g + j in its low nibble and of position 32g + 16 + j
 *     in its high nibble. A 4-bit code is the zero-extended value u = q + 8,
 *     q in [-7, 7]. 8-bit block b (b >= nb4) lives at byte
 *     nb4*M*64 + (b - nb4)*M*128, row m at + m*128, byte k = int8 code q of
 *     block position k, q in [-127, 127].
 *   x_scale, activation scales, device, float [nb][M] (block-major).
 *   Wq, weight codes, N * K / 2 bytes, fragment-ordered: the 16 output
 *     channels 16c .. 16c+15 and block b form the 1024-byte fragment at byte
 *     (c*nb + b) * 1024. Byte 16l + j of a fragment (l in 0..63, j in 0..15)
 *     belongs to channel 16c + (l mod 16) and holds, as 4-bit two's
 *     complement, q_w of block position 32(l/16) + j in its low nibble and of
 *     position 32(l/16) + 16 + j in its high nibble.
 *   w_scale, fp16 bit patterns [nb][N]; w_sum, int16 [nb][N] (sum of the
 *     group's q_w, in [-896, 896]); block-major like x_scale, so the scales of
 *     one block are one contiguous row.
 *   Block position p of block b is permuted channel 128b + p, i.e. original
 *   channel perm[128b + p].
 *
 * FP6 layout (the *_fp6 calls; the same codes, stored as the gfx950 FP6 matrix
 * instruction consumes them). A 4-bit code q in [-7, 7] is stored as FP6 E2M3
 * (bit 5 sign, bits 4..3 exponent with bias 1, bits 2..0 mantissa; |q| = 0..7
 * encode as 0, 8, 16, 20, 24, 26, 28, 30), which represents it exactly. The 32
 * codes of block positions 32g .. 32g+31 form a 192-bit little-endian string,
 * code j at bits 6j .. 6j+5; its bytes 0..15 are the group's head, bytes
 * 16..23 its tail.
 *   Xq_fp6, device, Mp * (96 * nb4 + 128 * nb8) bytes with Mp = M rounded up
 *     to a multiple of 16, block-major, in 16-row tiles (rows M .. Mp-1 are
 *     padding, never written and never used). 4-bit block b lives at byte
 *     b*Mp*96; its tile t (rows 16t .. 16t+15) at + t*1536 holds the head of
 *     group g of row 16t + r at byte H(r, g) = 64r + 16(g ^ h(r)) and its
 *     tail at 1024 + 32r + 8(g ^ u(r)), with h(r) = (r >> 1) & 3
 *     and u(r) = (r >> 2) & 3 (a row's bytes contiguous; the slot
 *     permutation keeps the kernel's LDS reads free of bank conflicts).
 *     8-bit block b lives at byte nb4*Mp*96 + (b - nb4)*Mp*128; its tile t at
 *     + t*2048 holds the int8 codes of block positions 32g + 16h' .. 32g +
 *     16h' + 15 of row 16t + r at byte 1024h' + H(r, g).
 *   Wq_fp6, N * (96 * nb4 + 64 * nb8) bytes, block-major: for a 4-bit block b
 *     the N/16 fragments of 1536 bytes start at byte b*(N/16)*1536; fragment c
 *     (channels 16c .. 16c+15) holds, for lane l in 0..63 (channel
 *     16c + (l mod 16), group l/16), the head at byte 16l and the tail at
 *     1024 + 8l. For an 8-bit block b the N/16 INT4 fragments of 1024 bytes
 *     (the Wq fragment format) start at byte (N/16)*(1536*nb4 + 1024*(b - nb4)).
 *   x_scale and w_scale as above; no weight sums (the codes are signed).
 */
#ifndef COMET_W4AX_H
#define COMET_W4AX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    COMET_OK = 0,
    COMET_ERR_NULL = 1,        /* a required pointer is NULL */
    COMET_ERR_SHAPE = 2,       /* M < 1, N < 1, K < 128, K % 128 != 0, ldx < K or ldy < N */
    COMET_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
    COMET_ERR_ARG = 4,         /* n_int8_blocks outside [0, K/128]; non-finite score or weight */
    COMET_ERR_WORKSPACE = 5,   /* workspace smaller than comet_w4ax_gemm_workspace_bytes() */
    COMET_ERR_HIP = 6,         /* a HIP launch or query failed */
    COMET_ERR_UNSUPPORTED = 7  /* N % 128 != 0, or a size beyond the 32-bit index range */
} comet_status;

/*
 * Offline: rank channels, quantize W to INT4 and pack it. Host memory only;
 * touches no device.
 *
 * Channel order (COMET article, section "1.离群点分布规律的重定义", channel
 * permutation; QUIK blog, section "第一步: 识别与重排", outlier columns moved
 * to the end; QoQ/QServe article, youleyou.com/wenzhang/3078652.html,
 * section "通用量化优化技巧", item 3): perm sorts the channels by ascending
 * chan_score, ties in original order; block_is_int8[b] = (b >= nb - nb8).
 * chan_score is a per-channel outlier statistic from calibration, e.g. the
 * per-channel absmax of a calibration batch.
 *
 * Weights (QUIK blog, section "反量化背后的数学", symmetric weights; QoQ/QServe
 * article, section "背景", fp16 group scales): for output channel n and block
 * b with absmax a over the block's permuted channels, s = fp16(a / 7)
 * (the smallest fp16 subnormal if that rounds to 0; 0 if a = 0) and
 * q_w = clamp(round_half_even(w / s), -7, 7); w_sum = sum of the block's q_w.
 *
 *   W_fp16        in   [N][K] row-major fp16 bit patterns
 *   chan_score    in   [K] float, finite
 *   n_int8_blocks in   nb8, 0 <= nb8 <= K/128
 *   perm          out  int32 [K]
 *   block_is_int8 out  uint8 [K/128]
 *   Wq_packed     out  N*K/2 bytes, layout above
 *   w_scale_fp16  out  uint16 [K/128][N]
 *   w_sum         out  int16 [K/128][N]
 * Errors: NULL, SHAPE (N < 1, K % 128 != 0), UNSUPPORTED (N % 128 != 0),
 * ARG (nb8 range, non-finite score or weight).
 */
int comet_pack_weights(const uint16_t* W_fp16, int N, int K, const float* chan_score,
                       int n_int8_blocks, int32_t* perm, uint8_t* block_is_int8,
                       uint8_t* Wq_packed, uint16_t* w_scale_fp16, int16_t* w_sum);

/*
 * Online, one kernel: gather the permuted channels of X, take the absmax of
 * every (token, block), and write INT4 codes for the 4-bit blocks and INT8
 * codes for the last nb8 blocks, with their scales (QUIK blog, section
 * "核融合": one fused pass reads the input, takes the statistics and
 * quantizes; COMET article, section "1.离群点分布规律的重定义": 8 bits for
 * the outlier blocks, 4 bits elsewhere).
 * For a (token, block) with absmax a > 0 and qmax = 7 or 127:
 *   inv = qmax / a, s = a / qmax (IEEE float divisions),
 *   q = clamp(round_half_even(x * inv), -qmax, qmax);
 * an all-zero block gets s = 0 and q = 0.
 *
 *   X_fp16        in   device, [M][ldx] fp16, ldx >= K (elements)
 *   perm          in   device, int32 [K], a permutation of 0..K-1
 *   n_int8_blocks in   nb8
 *   Xq            out  device, M * (64 nb4 + 128 nb8) bytes, layout above
 *   x_scale       out  device, float [nb][M]
 * Errors: NULL, SHAPE, ALIGN, ARG, HIP. perm must be a permutation and X
 * finite; neither is checked (the result is then unspecified).
 */
int comet_quant_act(const void* X_fp16, int M, int K, int ldx, const int32_t* perm,
                    int n_int8_blocks, void* Xq, float* x_scale, void* stream);

/*
 * Online: Y = X W^T from the quantized operands. For every output (m, n) and
 * block b the exact INT32 partial P = sum over the block of q_a q_w is formed
 * on INT8 matrix cores (4-bit operands are widened to 8 bits in registers;
 * 4-bit activation codes enter zero-extended, u = q + 8, and the offset is
 * removed through the precomputed weight sum: COMET article, section
 * "3.硬件指令集的极限挖掘"; QUIK blog, section "反量化背后的数学"), then
 *   y = sum over blocks of (x_scale[b][m] * w_scale[b][n]) * P   in FP32,
 *   Y[m][n] = fp16(y) (round to nearest even; overflow gives +-Inf).
 * Summation order over blocks is not fixed (split-K reorders it), but the
 * result of one configuration is deterministic: no floating-point atomics.
 *
 *   Xq, x_scale       in   from comet_quant_act
 *   Wq_packed, w_scale_fp16, w_sum  in  from comet_pack_weights, on device
 *   n_int8_blocks     in   nb8, the same value as for the other two calls
 *   Y_fp16            out  device, [M][ldy] fp16, ldy >= N (elements)
 *   workspace         in/out device scratch of workspace_bytes bytes; may be
 *                     NULL when comet_w4ax_gemm_workspace_bytes() is 0
 * Errors: NULL, SHAPE, ALIGN, ARG, WORKSPACE, UNSUPPORTED, HIP.
 */
int comet_w4ax_gemm(const void* Xq, const float* x_scale, const void* Wq_packed,
                     const uint16_t* w_scale_fp16, const int16_t* w_sum, int n_int8_blocks,
                     int M, int N, int K, void* Y_fp16, int ldy, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Workspace bytes comet_w4ax_gemm needs for this shape (0 if none). */
size_t comet_w4ax_gemm_workspace_bytes(int M, int N, int K, int n_int8_blocks);

/*
 * Debug variant of the GEMM: writes the exact INT32 block partials of rows
 * [m_begin, m_begin + m_count) instead of Y, as P[m - m_begin][n][b] (int32,
 * [m_count][N][K/128], device). It launches the kernel that comet_w4ax_gemm
 * launches for the same (M, N, K), with the same tile shape, block split and
 * pipeline, over the tiles that hold those rows; only the epilogue is
 * replaced by the stores of P. Same inputs and errors as comet_w4ax_gemm (no
 * workspace); SHAPE also covers a row range outside [0, M).
 */
int comet_w4ax_gemm_partials(const void* Xq, const float* x_scale, const void* Wq_packed,
                             const uint16_t* w_scale_fp16, const int16_t* w_sum,
                             int n_int8_blocks, int M, int N, int K, int m_begin, int m_count,
                             int32_t* P, void* stream);

/*
 * Asymmetric 4-bit activation blocks (the QUIK blog's scheme, section
 * "反量化背后的数学": activations with a scale and a zero point, weights with
 * a scale only; the zero-point term z * sum(w) needs only the zero point and
 * the offline weight sum). On the INT4 layout only: the FP6 format cannot hold
 * the codes 8..15.
 *
 * comet_quant_act_asym: as comet_quant_act, but every 4-bit (token, block)
 * takes its range [lo, hi] = [min(0, min x), max(0, max x)] and, if hi > lo,
 *   d = hi - lo, inv = 15 / d, s = d / 15 (IEEE float operations),
 *   z = clamp(round_half_even(-lo * inv), 0, 15),
 *   u = clamp(round_half_even(x * inv) + z, 0, 15);
 * an all-zero block gets s = 0, z = 0, u = 0. The nibble stores u (same
 * positions as comet_quant_act's u = q + 8); the value represented is
 * s (u - z). 8-bit blocks are coded exactly as by comet_quant_act, z = 0.
 *   x_zero  out  device, uint8 [nb][Mp], Mp = M rounded up to a multiple of
 *                16 (comet_x_zero_bytes); rows M .. Mp-1 are not written
 * Errors: as comet_quant_act (NULL and ALIGN also for x_zero).
 */
int comet_quant_act_asym(const void* X_fp16, int M, int K, int ldx, const int32_t* perm,
                         int n_int8_blocks, void* Xq, float* x_scale, uint8_t* x_zero, void* stream);

/* Bytes of x_zero for M rows and K channels (0 for an invalid shape). */
size_t comet_x_zero_bytes(int M, int K);

/*
 * comet_w4ax_gemm on asymmetric codes: on a 4-bit block the exact partial is
 *   P = sum over the block of u q_w - z w_sum = sum of (u - z) q_w,
 * formed on the matrix cores from the stored u with the accumulator starting
 * at the zero-point term; then Y as comet_w4ax_gemm. Arguments and errors as
 * comet_w4ax_gemm, plus x_zero (in, from comet_quant_act_asym; NULL, ALIGN).
 */
int comet_w4ax_gemm_asym(const void* Xq, const float* x_scale, const uint8_t* x_zero, const void* Wq_packed,
                         const uint16_t* w_scale_fp16, const int16_t* w_sum, int n_int8_blocks, int M, int N,
                         int K, void* Y_fp16, int ldy, void* workspace, size_t workspace_bytes, void* stream);

/* Debug variant: the partials P above of rows [m_begin, m_begin + m_count), as
 * comet_w4ax_gemm_partials. */
int comet_w4ax_gemm_asym_partials(const void* Xq, const float* x_scale, const uint8_t* x_zero,
                                  const void* Wq_packed, const uint16_t* w_scale_fp16, const int16_t* w_sum,
                                  int n_int8_blocks, int M, int N, int K, int m_begin, int m_count, int32_t* P,
                                  void* stream);

/*
 * QoQ W4A8 variant: progressive group quantization (QoQ/QServe article,
 * sections "渐进式分组量化" and "W4A8 GEMM的核心设计"). Weights: per output
 * channel symmetric INT8 in the protected range [-119, 119] with an fp16 scale
 * s1 = fp16(max |W[n, :]| / 119), w8 = clamp(round(W / s1), -119, 119); then per
 * 128-channel group of the permuted order (perm as comet_pack_weights, ascending
 * score) over the range [lo, hi] = [min(0, min w8), max(0, max w8)]: integer
 * step s2 = max(1, ceil((hi - lo) / 15)), zero point z = round(-lo / s2),
 * code u = clamp(round(w8 / s2) + z, 0, 15) (exact integer rounding, ties to
 * even), so that s2 (u - z) is an 8-bit integer. Activations: one symmetric
 * INT8 scale per token over all K. Product: P = sum over K of q_a s2 (u - z),
 * one exact INT32 sum; Y = fp16( fl(x_scale * s1) * float(P) ).
 *
 * comet_pack_weights_qoq (host): perm int32 [K]; Wu_packed N*K/2 bytes in the
 * Wq fragment order of comet_pack_weights, unsigned codes u; s1_fp16 [N];
 * s2z uint16 [K/128][N] = s2 | z << 8. Errors: NULL, SHAPE, ARG (non-finite
 * score or weight), UNSUPPORTED (N % 128).
 */
int comet_pack_weights_qoq(const uint16_t* W_fp16, int N, int K, const float* chan_score, int32_t* perm,
                           uint8_t* Wu_packed, uint16_t* s1_fp16, uint16_t* s2z);

/* Per-token INT8 codes in 8-bit slabs (block b, row m at byte (b M + m) 128,
 * positions in order; M*K bytes) and x_scale float [M]: a = max |x| over the
 * row, inv = 127 / a, s = a / 127, q = round(x * inv). Errors: NULL, SHAPE,
 * ALIGN, UNSUPPORTED (K > 32768), HIP. */
int comet_quant_act_token_i8(const void* X_fp16, int M, int K, int ldx, const int32_t* perm, void* Xq,
                             float* x_scale, void* stream);

/* The QoQ GEMM: Y fp16 [M][ldy] = fp16(fl(x_scale s1) float(P)). Per group of
 * K the zero point comes off the codes in registers, the INT8 matrix
 * instruction forms sum(q_a (u - z)), and s2 multiplies that group sum into
 * the INT32 total (the same exact P as the page's dequantization to
 * s2 (u - z) before the multiply). M <= 64: weight-streaming kernel; above: a
 * 128 x 128 tiled kernel. Errors: NULL, SHAPE, ALIGN, UNSUPPORTED (N % 128,
 * K > 32768, M N beyond int32), HIP. */
int comet_w4a8_qoq_gemm(const void* Xq, const float* x_scale, const void* Wu_packed, const uint16_t* s2z,
                        const uint16_t* s1_fp16, int M, int N, int K, void* Y_fp16, int ldy, void* stream);

/* Debug variant: the exact products P int32 [M][N] instead of Y. */
int comet_w4a8_qoq_gemm_products(const void* Xq, const float* x_scale, const void* Wu_packed, const uint16_t* s2z,
                                 const uint16_t* s1_fp16, int M, int N, int K, int32_t* P, void* stream);

/*
 * KV4 cache (QoQ/QServe article, section "KV4注意力Kernel优化": keys and values
 * quantized per head to 4 bits at run time, an fp16 scale and a zero point
 * stored with the codes; COMET article: KV cache at 4 bits). For each (token,
 * head) vector x of d channels: lo = min(0, min x), hi = max(0, max x),
 * inv = 15 / (hi - lo) and step = fp16((hi - lo) / 15) (binary32 divisions; the
 * smallest fp16 subnormal if the step rounds to 0), z = clamp(round(-lo inv)),
 * u = clamp(round(x inv) + z), clamps to [0, 15], ties to even; value
 * step (u - z). An all-zero vector stores step 0, z 0, codes 0.
 *
 * Cache layout per kv head h and slot t < tcap: codes [h][t][d/2] bytes
 * (channel 2i in the low nibble of byte i, 2i+1 in the high nibble),
 * step [h][t] fp16 bits, zero [h][t] bytes.
 *
 *   X_fp16     in   [ntok, ldx] fp16, device, 16-byte aligned, ldx % 8 == 0:
 *                   row = token, head h at columns [h d, h d + d)
 *   pos        in   cache slot of the first token (tokens go to pos .. pos+ntok-1)
 *   tcap       in   slots per head in the cache
 *   codes, step_fp16, zero   out (slots outside the range are untouched)
 * Errors: NULL, SHAPE (ntok, H < 1, ldx < H d, pos < 0, pos + ntok > tcap),
 * UNSUPPORTED (d not a power of two in [8, 512]), ALIGN, HIP.
 */
int comet_kv4_quantize(const void* X_fp16, int ntok, int H, int d, int ldx, int pos, int tcap, void* codes,
                       uint16_t* step_fp16, uint8_t* zero, void* stream);

/* Workspace bytes of comet_kv4_attention (0 for an invalid shape). */
size_t comet_kv4_attention_workspace_bytes(int Hq, int d, int T);

/*
 * Decode attention over the KV4 cache (QoQ/QServe article, section
 * "KV4注意力Kernel优化"): for each query head h, with kv head g = h / group,
 * over the first T slots of g's cache, k_t and v_t the dequantized vectors,
 *   a_t = q_h . k_t / sqrt(d),  p = softmax(a),  out_h = fp16(sum_t p_t v_t),
 * in FP32 (a split over 256-token chunks, combined exactly as a softmax over
 * the whole; the order of the sums differs from a plain loop).
 *
 *   q_fp16     in   [Hq][d] fp16, device, 16-byte aligned
 *   k_*, v_*   in   caches of Hq / group kv heads, layout as comet_kv4_quantize
 *   group      in   query heads per kv head (1 for multi-head attention)
 *   T, tcap    in   tokens to attend (1 <= T <= tcap) and the cache's slots per head
 *   out_fp16   out  [Hq][d] fp16, device, 2-byte aligned
 *   workspace  in   device, 16-byte aligned, comet_kv4_attention_workspace_bytes()
 * Errors: NULL, SHAPE (Hq < 1, group < 1, Hq % group, T < 1, tcap < T),
 * UNSUPPORTED (d not a power of two in [8, 512]; Hq ceil(T / 256) beyond
 * int32), WORKSPACE, ALIGN, HIP.
 */
int comet_kv4_attention(const void* q_fp16, const void* k_codes, const uint16_t* k_step, const uint8_t* k_zero,
                        const void* v_codes, const uint16_t* v_step, const uint8_t* v_zero, int Hq, int group, int d,
                        int T, int tcap, void* out_fp16, void* workspace, size_t workspace_bytes, void* stream);

/*
 * comet_kv4_attention over sequences of different lengths in one call (a
 * decode batch: each sequence its own kv heads, each at its own position; the
 * serving KV cache of QoQ/QServe article, section "运行时设计", holds many
 * sequences, each with its own length):
 * kv head g attends to its first T_kv[g] slots, the same formula as
 * comet_kv4_attention with T = T_kv[g].
 *
 *   T_kv       in   device, 4-byte aligned, int32 [Hq / group]: tokens of each kv
 *                   head; values are clamped to [0, T_max] on the device, and
 *                   a head with 0 tokens gives an all-zero output
 *   T_max      in   the largest T_kv (1 <= T_max <= tcap): it sizes the split
 *                   and the workspace, comet_kv4_attention_workspace_bytes(Hq, d,
 *                   T_max); chunks past a head's tokens exit at once
 * Other arguments, layouts and errors as comet_kv4_attention (T_max in the
 * place of T); NULL also for a null T_kv, ALIGN for a misaligned one. With
 * every T_kv[g] = T_max the output is bit for bit that of comet_kv4_attention.
 */
int comet_kv4_attention_varlen(const void* q_fp16, const void* k_codes, const uint16_t* k_step,
                               const uint8_t* k_zero, const void* v_codes, const uint16_t* v_step,
                               const uint8_t* v_zero, int Hq, int group, int d, const int32_t* T_kv, int T_max,
                               int tcap, void* out_fp16, void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP6 layout, sizes: bytes of Xq_fp6 for M rows (padded to a multiple of 16)
 * and of Wq_fp6 for N output channels (0 for an invalid shape).
 */
size_t comet_xq_fp6_bytes(int M, int K, int n_int8_blocks);
size_t comet_wq_fp6_bytes(int N, int K, int n_int8_blocks);

/*
 * Offline, host memory: re-encode comet_pack_weights' Wq into the FP6 layout
 * (4-bit blocks as FP6 E2M3 fragments, 8-bit blocks copied). The codes are
 * unchanged, so w_scale applies as is.
 *
 *   Wq_packed      in   N*K/2 bytes from comet_pack_weights
 *   n_int8_blocks  in   nb8 of that call
 *   Wq_fp6         out  comet_wq_fp6_bytes(N, K, nb8) bytes, layout above
 * Errors: NULL, SHAPE (N < 1, K % 128 != 0), ARG (nb8 range), UNSUPPORTED
 * (N % 128 != 0).
 */
int comet_repack_weights_fp6(const uint8_t* Wq_packed, int N, int K, int n_int8_blocks,
                             uint8_t* Wq_fp6);

/*
 * comet_quant_act writing the FP6 layout: the same codes and scales (QUIK
 * blog, section "核融合"; COMET article, section "1.离群点分布规律的重定义"),
 * 4-bit codes as FP6 E2M3. Arguments and errors as comet_quant_act; Xq_fp6
 * has comet_xq_fp6_bytes(M, K, nb8) bytes.
 */
int comet_quant_act_fp6(const void* X_fp16, int M, int K, int ldx, const int32_t* perm,
                        int n_int8_blocks, void* Xq_fp6, float* x_scale, void* stream);

/*
 * comet_w4ax_gemm on the FP6 layout, for prefill shapes (any M >= 1 is
 * valid; it pays off from a few hundred rows). The same result definition
 * (COMET summary, abstract; QUIK blog, section "核融合"): exact block
 * partials P (4-bit blocks on the FP6 matrix instruction, whose FP32 result
 * is exact for these integer products; 8-bit blocks on the INT8 one), then
 * y = sum over blocks of (x_scale * w_scale) * P in FP32 and Y = fp16(y).
 * No weight sums (the codes are signed). UNSUPPORTED also covers
 * Mp * K > 2^31 - 1 (the kernel's 32-bit offsets into Xq_fp6).
 *
 * Scheduling (COMET article, section "2.混合精度计算的动态调度": tiles are
 * not bound to compute units; idle units take over their neighbours' work).
 * A grid of at least one wave of whole output tiles (two per CU) runs one
 * tile per workgroup and needs no workspace. A smaller grid splits each
 * tile's blocks into runs of about equal cost (an 8-bit block counts twice)
 * and runs them as the work items of a persistent grid with per-XCD work
 * queues (atomic counters; an idle workgroup takes from the fullest queue);
 * each run stores its FP32 partial tile, and a second kernel adds them in
 * split order and writes Y. Y is deterministic: the same inputs give the same
 * bits whatever the timing (no floating-point atomics); the sum over blocks
 * is then grouped by runs, which is one of the orders the definition allows.
 *
 *   Xq_fp6, x_scale   in   from comet_quant_act_fp6
 *   Wq_fp6            in   from comet_repack_weights_fp6, on device
 *   w_scale_fp16      in   from comet_pack_weights, on device
 *   Y_fp16            out  device, [M][ldy] fp16, ldy >= N
 *   workspace         in/out  device, 16-byte aligned, at least
 *                     comet_w4ax_gemm_fp6_workspace_bytes(M, N, K, nb8) bytes
 *                     (may be NULL when that is 0). Its first 256 bytes (the
 *                     queue counters) must be zero before its first use (e.g.
 *                     allocated zeroed); every call returns them to zero before
 *                     it ends, so calls of any shape ordered on one stream can
 *                     share the workspace. Calls that may run at the same time
 *                     need workspaces of their own.
 * Errors: NULL, SHAPE, ALIGN, ARG, WORKSPACE, UNSUPPORTED, HIP.
 */
int comet_w4ax_gemm_fp6(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                        const uint16_t* w_scale_fp16, int n_int8_blocks, int M, int N, int K,
                        void* Y_fp16, int ldy, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes comet_w4ax_gemm_fp6 (and its partials variant) needs for
 * this shape: 0 for grids of a wave of tiles or more; otherwise the work
 * queue's counters and the runs' FP32 partial tiles. A function of the shape
 * only (no device is queried); 0 for an invalid shape. */
size_t comet_w4ax_gemm_fp6_workspace_bytes(int M, int N, int K, int n_int8_blocks);

/*
 * comet_w4ax_gemm_fp6 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a fixed array of
 * COMET_NOALLOC_SCRATCH_BYTES in device memory inside the library, one per
 * GPU, held until the process ends; this call allocates nothing. Calls on one
 * GPU share that array, so calls that may overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller. Same result, kernels
 * and errors as comet_w4ax_gemm_fp6; WORKSPACE when the shape needs more than
 * COMET_NOALLOC_SCRATCH_BYTES (comet_w4ax_gemm_fp6_workspace_bytes tells).
 */
#define COMET_NOALLOC_SCRATCH_BYTES (36u << 20)
int comet_w4ax_gemm_fp6_noalloc(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                                const uint16_t* w_scale_fp16, int n_int8_blocks, int M, int N, int K,
                                void* Y_fp16, int ldy, void* stream);

/*
 * Debug variant of comet_w4ax_gemm_fp6: the exact INT32 block partials of rows
 * [m_begin, m_begin + m_count) as P[m - m_begin][n][b], from the kernel, tile
 * shape, block runs and work queue comet_w4ax_gemm_fp6 uses for the same
 * (M, N, K), over the tiles that hold those rows; each run stores the
 * partials of its own blocks (no fix-up). Workspace as comet_w4ax_gemm_fp6.
 * max_workgroups: 0 runs the grid the Y call runs; n > 0 caps a split plan's
 * persistent grid at about n workgroups (8 at least, one per XCD), so that
 * the work-queue counters deal most items (a check of the queue, which on a
 * full MI355X only deals the items a plan has beyond its resident grid).
 * Errors as comet_w4ax_gemm_fp6, plus SHAPE (row range), ARG (max_workgroups < 0).
 */
int comet_w4ax_gemm_fp6_partials(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                                 const uint16_t* w_scale_fp16, int n_int8_blocks, int M, int N,
                                 int K, int m_begin, int m_count, int32_t* P, int max_workgroups,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * QUIK's fp16 outlier columns on the FP6 layout (QUIK blog,
 * deep-paper.org/paper/2310.09259, section "第一步: 识别与重排": the outlier
 * columns, found offline from calibration, are moved to the end of W; section
 * "第二步: 前向传播 (在线)": the activations split into a quantized part and
 * the fp16 outlier part, each multiplied on its own path, and the results are
 * added). With the channel order of comet_pack_weights (ascending score), the
 * last n_fp16 channels (the highest scores) keep their fp16 values in X and
 * W; the first K - n_fp16 are the quantized channels of the three calls
 * above (their last nb8 blocks 8-bit). Then
 *   y = (the FP32 block sum of comet_w4ax_gemm over the quantized channels)
 *       + sum over the fp16 channels j of x_j * w_j     in FP32
 * (a product of two fp16 values is exact in FP32), Y = fp16(y). The two
 * parts are summed in the same FP32 accumulators inside the GEMM kernel.
 * n_fp16 is a multiple of 128 with K - n_fp16 >= 128 (0 gives the plain
 * FP6 path).
 *
 * Fp16 operand layouts (fp16 bits, 1 KB pieces = 16 rows or output channels
 * x 32 channels, the operand order of the 16x16x32 fp16 matrix instruction):
 *   Xf  [Mp/16][n_fp16/32] tiles (Mp = M rounded up to 16): tile (t, s) at
 *       half (t * (n_fp16/32) + s) * 512; half 8l + e (l in 0..63, e in 0..7)
 *       is row 16t + (l mod 16), outlier channel 32s + 8(l/16) + e; rows
 *       past M are zero. comet_xf_bytes(M, n_fp16) bytes.
 *   Wf  [N/16][n_fp16/32] fragments: fragment (c, s) at half
 *       (c * (n_fp16/32) + s) * 512; half 8l + e is output channel
 *       16c + (l mod 16), outlier channel 32s + 8(l/16) + e. N * n_fp16 * 2
 *       bytes.
 * Outlier channel j is original channel perm[K - n_fp16 + j].
 */

/*
 * Offline, host memory: channel order, quantized pack of the first K - n_fp16
 * permuted channels (exactly comet_pack_weights' Wq, w_scale and w_sum for
 * them; repack Wq to the FP6 layout with comet_repack_weights_fp6(Wq, N,
 * K - n_fp16, nb8)) and the fp16 fragments of the rest.
 *   perm        out  int32 [K]
 *   Wq_packed   out  N*(K - n_fp16)/2 bytes;  w_scale_fp16, w_sum  out  [(K - n_fp16)/128][N]
 *   Wf_fp16     out  N * n_fp16 halves, layout above (may be NULL if n_fp16 = 0)
 * Errors: NULL, SHAPE (N < 1, K % 128 != 0), UNSUPPORTED (N % 128 != 0),
 * ARG (n_fp16 not a multiple of 128 or above K - 128; non-finite score or weight).
 */
int comet_pack_weights_quik(const uint16_t* W_fp16, int N, int K, const float* chan_score, int n_fp16,
                            int32_t* perm, uint8_t* Wq_packed, uint16_t* w_scale_fp16, int16_t* w_sum,
                            uint16_t* Wf_fp16);

/* Bytes of Xf for M rows (0 for an invalid argument). */
size_t comet_xf_bytes(int M, int n_fp16);

/*
 * Online: comet_quant_act_fp6 over the quantized channels perm[0 .. K - n_fp16)
 * (Xq_fp6 and x_scale of K - n_fp16 channels), and Xf, the fp16 values of the
 * outlier channels perm[K - n_fp16 .. K).
 * Errors: NULL, SHAPE (M < 1, K % 128 != 0, ldx < K), ARG (n_fp16 or nb8
 * range), ALIGN, HIP.
 */
int comet_quant_act_quik_fp6(const void* X_fp16, int M, int K, int ldx, const int32_t* perm, int n_int8_blocks,
                             int n_fp16, void* Xq_fp6, float* x_scale, void* Xf_fp16, void* stream);

/*
 * Online: Y of the QUIK split (above) from the FP6-layout quantized operands
 * (K - n_fp16 channels) and the fp16 outlier operands. K is the full channel
 * count. workspace as comet_w4ax_gemm_fp6 with K - n_fp16 channels
 * (comet_w4ax_gemm_fp6_workspace_bytes(M, N, K - n_fp16, nb8) bytes).
 * Errors: NULL, SHAPE, ARG (n_fp16 or nb8 range), ALIGN, WORKSPACE,
 * UNSUPPORTED (as comet_w4ax_gemm_fp6, or Xf / Wf of 2 GB or more), HIP.
 */
int comet_w4ax_gemm_quik_fp6(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                             const uint16_t* w_scale_fp16, int n_int8_blocks, const void* Xf_fp16,
                             const void* Wf_fp16, int n_fp16, int M, int N, int K, void* Y_fp16, int ldy,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * RMS normalization fused into the activation quantizer. QoQ/QServe article
 * (youleyou.com/wenzhang/3078652.html), section "运行时设计": the activation
 * quantization of the QKV projection and of the first FFN layer is fused into
 * the layer norm before it; QUIK blog (deep-paper.org/paper/2310.09259),
 * section "核融合": one kernel reads the input, takes its statistics and
 * quantizes. The normalization (RMSNorm, as in the LLaMA models the pages
 * evaluate) of row m:
 *   S  = sum over k of x_k^2, the exact real sum rounded once to binary64
 *        (nearest, ties to even); no summation order enters it;
 *   r  = binary32( 1 / sqrt(S / K + eps) ), the root and quotient in binary64;
 *   xn_k = fp16( (x_k * r) * gamma_k ), two binary32 products, nearest-even.
 * Every kernel of the library forms this S, so the fused calls give exactly
 * the codes and scales of comet_rmsnorm followed by comet_quant_act.
 * Normalized values must stay finite (|gamma| sqrt(K) < 65504); eps must be a
 * positive finite float.
 * ------------------------------------------------------------------------ */

/*
 * comet_quant_act of the RMS-normalized rows: the normalized row is formed in
 * the quantizer and never stored.
 *
 *   X_fp16           in   [M, ldx] fp16, device, 16-byte aligned, rows NOT normalized
 *   gamma_perm_fp16  in   [K] fp16, device, 16-byte aligned: the RMSNorm weight in the
 *                         permuted channel order, gamma_perm[k] = gamma[perm[k]]
 *                         (comet_permute_channels)
 *   eps              in   > 0, finite
 *   perm, n_int8_blocks, Xq, x_scale, stream: as comet_quant_act
 * Errors: as comet_quant_act, plus NULL (gamma_perm), ARG (eps), ALIGN (gamma_perm).
 */
int comet_rmsnorm_quant_act(const void* X_fp16, int M, int K, int ldx, const void* gamma_perm_fp16, float eps,
                            const int32_t* perm, int n_int8_blocks, void* Xq, float* x_scale, void* stream);

/* The same on the FP6 layout (comet_quant_act_fp6's output). */
int comet_rmsnorm_quant_act_fp6(const void* X_fp16, int M, int K, int ldx, const void* gamma_perm_fp16, float eps,
                                const int32_t* perm, int n_int8_blocks, void* Xq_fp6, float* x_scale,
                                void* stream);

/*
 * The normalization on its own (the unfused step, for comparison):
 * Xn[m][k] = xn_k of row m, original channel order.
 *
 *   X_fp16      in   [M, ldx] fp16, device (2-byte aligned), ldx >= K
 *   gamma_fp16  in   [K] fp16, device, original channel order
 *   eps         in   > 0, finite
 *   Xn_fp16     out  [M, ldn] fp16, device, ldn >= K (columns past K untouched)
 * Errors: NULL, SHAPE (M < 1, K < 1, ldx < K, ldn < K), ARG (eps), ALIGN (odd
 * addresses), HIP.
 */
int comet_rmsnorm(const void* X_fp16, int M, int K, int ldx, const void* gamma_fp16, float eps, void* Xn_fp16,
                  int ldn, void* stream);

/* ------------------------------------------------------------------------
 * SwiGLU fused into the activation quantizer of the down projection.
 * QoQ/QServe article (youleyou.com/wenzhang/3078652.html), section
 * "运行时设计": the second FFN layer's activation quantization is fused into
 * the activation kernel before it; QUIK blog (deep-paper.org/paper/2310.09259),
 * section "案例研究: 敏感的 LLaMA-2 Down-Projection 层": LLaMA's MLP uses
 * SwiGLU, and the down projection takes the element-wise product of the gate
 * and up projections' outputs. With the standard SiLU, element k of row m is
 *   h = fp16( silu(g) u ),  silu(g) = g / (1 + e^-g),
 * the exact real value rounded once to binary16 (nearest, ties to even): the
 * pages give no precision for this step, and the exact rounding is what makes
 * the fused codes reproducible. g and u must be finite and the product must
 * not overflow binary16 (|h| <= 65504); otherwise the result is unspecified.
 * ------------------------------------------------------------------------ */

/*
 * comet_quant_act of the SwiGLU rows: h is formed in the quantizer and never
 * stored.
 *
 *   gate_fp16, up_fp16  in  [M, ldx] fp16 each, device, 16-byte aligned: the gate and
 *                           up projections' outputs in the original channel order
 *                           (e.g. the two halves of one [M, 2K] output: up = gate + K,
 *                           ldx = 2K)
 *   perm, n_int8_blocks, Xq, x_scale, stream: as comet_quant_act
 * Errors: as comet_quant_act (NULL and ALIGN also for up_fp16).
 */
int comet_swiglu_quant_act(const void* gate_fp16, const void* up_fp16, int M, int K, int ldx, const int32_t* perm,
                           int n_int8_blocks, void* Xq, float* x_scale, void* stream);

/* The same for the FP6 layout (Xq_fp6 and x_scale as comet_quant_act_fp6). */
int comet_swiglu_quant_act_fp6(const void* gate_fp16, const void* up_fp16, int M, int K, int ldx,
                               const int32_t* perm, int n_int8_blocks, void* Xq_fp6, float* x_scale,
                               void* stream);

/*
 * The unfused step: H[m][k] = fp16(silu(gate[m][k]) up[m][k]) as defined above,
 * original channel order.
 *
 *   gate_fp16, up_fp16  in   [M, ldx] fp16, device, 2-byte aligned
 *   H_fp16              out  [M, ldh] fp16, device, 2-byte aligned (columns >= K untouched)
 * Errors: NULL, SHAPE (M < 1, K < 1, ldx < K, ldh < K), ALIGN, HIP.
 */
int comet_swiglu(const void* gate_fp16, const void* up_fp16, int M, int K, int ldx, void* H_fp16, int ldh,
                 void* stream);

/*
 * Offline, host memory: out[k] = v[perm[k]] for k < K (for example the
 * RMSNorm weight into the permuted order the fused calls take).
 * Errors: NULL, SHAPE (K < 1), ARG (a perm entry outside [0, K)).
 */
int comet_permute_channels(const uint16_t* v, const int32_t* perm, int K, uint16_t* out);

/* Static description of a status code. */
const char* comet_status_string(int status);

/* Library version string. */
const char* comet_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COMET_W4AX_H */
