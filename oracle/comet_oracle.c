/*
 * CPU oracle for the W4Ax fine-grained mixed-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
 * CPU-baseline leg are the only code that may load or call this library. The
 * product library never links, loads or calls it, and shares no code with it.
 *
 * What it computes, step by step, in the order the pages describe it:
 *
 *  1. Channel order (offline). Channels are ranked by a calibration score and
 *     permuted so that the outlier channels share 128-channel blocks; the
 *     highest-scoring blocks are stored in 8 bits, the rest in 4 bits.
 *     COMET article (mmssai.com/?p=43269), section "1.离群点分布规律的重定义";
 *     QUIK blog (deep-paper.org/paper/2310.09259), section "第一步: 识别与重排"
 *     (outlier columns go to the end of W); QoQ/QServe article
 *     (youleyou.com/wenzhang/3078652.html), section "通用量化优化技巧", item 3
 *     (channels of similar saliency share a quantization group).
 *  2. Weight quantization (offline). Symmetric INT4 per output channel per
 *     128-channel group, with an fp16 scale per group (QUIK blog, section
 *     "反量化背后的数学": weights are quantized symmetrically; QoQ/QServe
 *     article, section "背景": an fp16 scale shared per group). The per-group
 *     weight sum is precomputed here (QUIK blog, same section: the term that
 *     involves the sum of the weights depends on the weights only).
 *  3. Activation quantization (online). Per token and per block, absmax
 *     scaling to INT4 ([-7, 7]) or INT8 ([-127, 127]); QoQ/QServe article,
 *     section "保护量化范围", names the symmetric 8-bit range [-127, 127].
 *  3b. Asymmetric 4-bit activations (a variant of step 3, the outlier-handling
 *     scheme of the QUIK blog, section "反量化背后的数学": activations carry a
 *     scale and a zero point, weights a scale only, and the zero point enters
 *     the result through a term that needs only the zero point and the
 *     offline sum of the weights). On a 4-bit block the range [lo, hi] is the
 *     block's minimum and maximum widened to include 0, the step is
 *     s = (hi - lo) / 15, the zero point z = round(-lo / s) in [0, 15] and the
 *     stored code u = round(x / s) + z in [0, 15]; the value represented is
 *     s (u - z). 8-bit blocks stay symmetric (step 3). The signed code q =
 *     u - z then enters steps 4 and 5 unchanged.
 *  4. Block partials. The exact INT32 dot product of each 128-channel block.
 *     A second form uses the zero-extended 4-bit code u = q + 8 and removes
 *     the offset with the precomputed weight sum (COMET article, section
 *     "3.硬件指令集的极限挖掘": zero extension instead of sign extension,
 *     compensated through the scales).
 *  5. Epilogue. Y = fp16( sum over blocks of (s_x * s_w) * P ), in FP32, in
 *     block order (QUIK blog, section "核融合": the integer result is
 *     dequantized to fp16 while still in registers).
 *
 *  8. QoQ's progressive group quantization (W4A8; QoQ/QServe article, section
 *     "渐进式分组量化" and "W4A8 GEMM的核心设计"), a variant of steps 2-5 kept
 *     apart from them: weights first to per-channel symmetric INT8 in the
 *     protected range [-119, 119] with an fp16 scale s1, then each
 *     128-channel group of those INT8 values to asymmetric UINT4 with an
 *     integer step s2 and zero point z, so that s2 (u - z) is again an 8-bit
 *     integer; activations per token symmetric INT8; the product is one exact
 *     integer accumulation over all of K (the dequantization to 8 bits happens
 *     before the multiply), and only a per-(token, channel) scale remains:
 *     Y = fp16( (s_x s1) * P ).
 *
 *  9. KV4 decode attention (QoQ/QServe article, section "KV4注意力Kernel优化",
 *     and section "运行时设计": per-head dynamic 4-bit KV quantization with an
 *     fp16 scale and zero point stored beside the codes; COMET article: the
 *     KV cache compressed to 4 bits). Each cached key and value vector of one
 *     head (d channels of one token) is coded as asymmetric 4-bit codes with
 *     the range widened to include 0 (as step 3b), its step kept in fp16;
 *     decode attention then computes, per head, softmax(q . k / sqrt(d)) over
 *     the cached tokens and the weighted sum of the values, on the
 *     dequantized vectors s (u - z).
 *
 * 10. QUIK's FP16 outlier columns (QUIK blog, section "第一步: 识别与重排":
 *     the outlier columns, chosen offline from calibration, go to the end of
 *     W; section "第二步: 前向传播 (在线)": the activations split into a
 *     quantized part and the FP16 outlier part, the two are multiplied on
 *     their own paths and the results are added). The last nf channels of
 *     the permuted order (step 1's ascending-score order, so the
 *     highest-scoring ones) keep their fp16 values in both X and W; the first
 *     K - nf channels go through steps 2-5 (their last nb8 blocks 8-bit).
 *     y = (step 5's FP32 sum over the blocks) + the FP32 sum of the fp16
 *     products x_j w_j in channel order; a product of two fp16 values is
 *     exact in FP32. Y = fp16(y).
 *
 *  6. RMS normalization before the quantizer (the next step the quantization
 *     fuses into). QoQ/QServe article, section "运行时设计": the activation
 *     quantization of the QKV projection and of the first FFN layer is fused
 *     into the layer norm that precedes it; QUIK blog, section "核融合": one
 *     kernel reads the input, takes its statistics and quantizes. The LLaMA
 *     models the pages evaluate normalize with RMSNorm. The normalized row is
 *     the block's FP16 activation (QoQ/QServe, same section: FP16 block inputs
 *     and outputs), which step 3 then quantizes.
 *
 *  7. SwiGLU before the quantizer of the second FFN layer. QoQ/QServe
 *     article, section "运行时设计": the activation quantization of the second
 *     FFN layer is fused into the activation kernel before it; QUIK blog,
 *     section "案例研究: 敏感的 LLaMA-2 Down-Projection 层": LLaMA's MLP uses
 *     SwiGLU, and the down projection takes the element-wise product of the
 *     gate and up projections' outputs. With the standard SiLU, the down
 *     projection's fp16 input is h = fp16( silu(g) u ), silu(g) = g / (1 +
 *     e^-g), and step 3 quantizes it.
 *
 * Readings of points the pages leave open (INT4 range, rounding mode, scale
 * form, all-zero blocks, tie-breaking of the channel sort) are listed with the
 * design notes at the repository root; each is stated where it is used below.
 *
 * Precision. Built with -O2 -ffp-contract=off and without fast-math, so every
 * float operation below is a single IEEE-754 binary32 operation rounded to
 * nearest-even, and rintf() rounds half-way cases to even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLOCK 128

enum { ORC_OK = 0, ORC_ERR_ARG = 1, ORC_ERR_NONFINITE = 2 };

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16, written from the format's definition.                 */
/* ------------------------------------------------------------------------ */

/* Exact conversion of a binary16 bit pattern to binary32. */
float orc_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);                 /* zero / subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even; overflow gives +-Inf. */
uint16_t orc_float_to_half(float f)
{
    if (isnan(f))
        return 0x7E00;
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);                    /* exact */
    if (isinf(f))
        return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {
        /* Subnormal range: the quantum is 2^-24. A result of 1024 quanta is
         * the smallest normal number, whose bit pattern is also 1024. */
        double q = nearbyint(a * 16777216.0);
        return sign | (uint16_t)q;
    }
    int e2;
    frexp(a, &e2);                                 /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;                                /* unbiased exponent */
    double q = nearbyint(ldexp(a, 10 - E));        /* significand in quanta, [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)q - 1024);
}

/* Array forms of the two conversions (used by the exhaustive checks). */
void orc_half_to_float_array(const uint16_t *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_half_to_float(in[i]);
}

void orc_float_to_half_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_float_to_half(in[i]);
}

/* ------------------------------------------------------------------------ */
/* 1. Channel order                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
    float score;
    int32_t index;
} orc_ranked;

/* Ascending score; equal scores keep the original channel order. */
static int orc_rank_cmp(const void *pa, const void *pb)
{
    const orc_ranked *a = (const orc_ranked *)pa, *b = (const orc_ranked *)pb;
    if (a->score < b->score) return -1;
    if (a->score > b->score) return 1;
    return (a->index > b->index) - (a->index < b->index);
}

/* perm[k'] = original channel stored at permuted position k'; block b holds
 * positions [128 b, 128 b + 128). The nb8 highest-scoring blocks, which are the
 * last ones, are the 8-bit blocks: is_int8[b] = (b >= nb - nb8). */
int orc_channel_order(int K, const float *score, int nb8, int32_t *perm, uint8_t *is_int8)
{
    if (K <= 0 || K % ORC_BLOCK != 0)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
    if (nb8 < 0 || nb8 > nb)
        return ORC_ERR_ARG;
    orc_ranked *r = (orc_ranked *)malloc(sizeof(orc_ranked) * (size_t)K);
    if (!r)
        return ORC_ERR_ARG;
    for (int k = 0; k < K; ++k) {
        if (!isfinite(score[k])) {
            free(r);
            return ORC_ERR_NONFINITE;
        }
        r[k].score = score[k];
        r[k].index = k;
    }
    qsort(r, (size_t)K, sizeof(orc_ranked), orc_rank_cmp);
    for (int k = 0; k < K; ++k)
        perm[k] = r[k].index;
    for (int b = 0; b < nb; ++b)
        is_int8[b] = (uint8_t)(b >= nb - nb8);
    free(r);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Shared element rule: round half to even, then clamp to [-qmax, qmax].     */
/* ------------------------------------------------------------------------ */

static int orc_round_clamp(float v, int qmax)
{
    float r = rintf(v);
    if (r > (float)qmax) r = (float)qmax;
    if (r < (float)-qmax) r = (float)-qmax;
    return (int)r;
}

/* ------------------------------------------------------------------------ */
/* 2. Weight quantization: symmetric INT4, fp16 scale per (channel, group)   */
/* ------------------------------------------------------------------------ */

/* Scale of one weight group with absmax a > 0: fp16(a / 7). A scale that
 * rounds to zero (a below 3.5 * 2^-24) becomes the smallest fp16 subnormal,
 * 2^-24, so that the division below stays finite. Returns the fp16 bits. */
uint16_t orc_weight_scale(float a)
{
    float s = a / 7.0f;
    uint16_t h = orc_float_to_half(s);
    if (h == 0)
        h = 1;
    return h;
}

/* qw: [N][K] in permuted channel order, values in [-7, 7].
 * sw16: [N][nb] fp16 bits. wsum: [N][nb], sum of the group's qw. */
int orc_quantize_weights(const uint16_t *W, int N, int K, const int32_t *perm,
                         int8_t *qw, uint16_t *sw16, int32_t *wsum)
{
    if (N <= 0 || K <= 0 || K % ORC_BLOCK != 0)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int n = 0; n < N; ++n) {
        const uint16_t *wrow = W + (size_t)n * K;
        for (int b = 0; b < nb; ++b) {
            float a = 0.0f;
            for (int k = 0; k < ORC_BLOCK; ++k) {
                float v = orc_half_to_float(wrow[perm[b * ORC_BLOCK + k]]);
                if (!isfinite(v))
                    bad = 1;
                float av = fabsf(v);
                if (av > a)
                    a = av;
            }
            int32_t sum = 0;
            int8_t *q = qw + (size_t)n * K + (size_t)b * ORC_BLOCK;
            if (a == 0.0f) {
                sw16[(size_t)n * nb + b] = 0;
                for (int k = 0; k < ORC_BLOCK; ++k)
                    q[k] = 0;
            } else {
                uint16_t h = orc_weight_scale(a);
                float s = orc_half_to_float(h);
                sw16[(size_t)n * nb + b] = h;
                for (int k = 0; k < ORC_BLOCK; ++k) {
                    float v = orc_half_to_float(wrow[perm[b * ORC_BLOCK + k]]);
                    float d = v / s;
                    q[k] = (int8_t)orc_round_clamp(d, 7);
                    sum += q[k];
                }
            }
            wsum[(size_t)n * nb + b] = sum;
        }
    }
    return bad ? ORC_ERR_NONFINITE : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 3. Activation quantization: per token, per block, symmetric absmax        */
/* ------------------------------------------------------------------------ */

/* Reciprocal and scale of one (token, block) with absmax a > 0:
 * inv = qmax / a and s = a / qmax, each one correctly rounded division. */
void orc_act_scale(float a, int qmax, float *inv, float *s)
{
    *inv = (float)qmax / a;
    *s = a / (float)qmax;
}

/* One element: round(x * inv) clamped to [-qmax, qmax]; the product is a
 * single rounded multiply, never fused with anything. */
int orc_act_quantize_value(float x, float inv, int qmax)
{
    float p = x * inv;
    return orc_round_clamp(p, qmax);
}

/* qa: [M][K] in permuted channel order. sa: [M][nb].
 * An all-zero block gets scale 0 and codes 0. */
int orc_quantize_activations(const uint16_t *X, int M, int K, int ldx, const int32_t *perm,
                             const uint8_t *is_int8, int8_t *qa, float *sa)
{
    if (M <= 0 || K <= 0 || K % ORC_BLOCK != 0 || ldx < K)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int m = 0; m < M; ++m) {
        const uint16_t *xrow = X + (size_t)m * ldx;
        for (int b = 0; b < nb; ++b) {
            int qmax = is_int8[b] ? 127 : 7;
            float a = 0.0f;
            for (int k = 0; k < ORC_BLOCK; ++k) {
                float v = orc_half_to_float(xrow[perm[b * ORC_BLOCK + k]]);
                if (!isfinite(v))
                    bad = 1;
                float av = fabsf(v);
                if (av > a)
                    a = av;
            }
            int8_t *q = qa + (size_t)m * K + (size_t)b * ORC_BLOCK;
            if (a == 0.0f) {
                sa[(size_t)m * nb + b] = 0.0f;
                for (int k = 0; k < ORC_BLOCK; ++k)
                    q[k] = 0;
                continue;
            }
            float inv, s;
            orc_act_scale(a, qmax, &inv, &s);
            sa[(size_t)m * nb + b] = s;
            for (int k = 0; k < ORC_BLOCK; ++k) {
                float v = orc_half_to_float(xrow[perm[b * ORC_BLOCK + k]]);
                q[k] = (int8_t)orc_act_quantize_value(v, inv, qmax);
            }
        }
    }
    return bad ? ORC_ERR_NONFINITE : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 3b. Activation quantization, asymmetric 4-bit blocks                      */
/* ------------------------------------------------------------------------ */

/* Step, reciprocal and zero point of one 4-bit (token, block) with range
 * [lo, hi], lo <= 0 <= hi, lo < hi:
 *   d = hi - lo (one binary32 subtraction), inv = 15 / d, s = d / 15 (each one
 *   correctly rounded division), z = round(-lo * inv) clamped to [0, 15]. */
void orc_act_asym_params(float lo, float hi, float *inv, float *s, int *z)
{
    float d = hi - lo;
    *inv = 15.0f / d;
    *s = d / 15.0f;
    float t = -lo * *inv;
    int zz = (int)rintf(t);
    *z = zz < 0 ? 0 : (zz > 15 ? 15 : zz);
}

/* One element's stored code: u = round(x * inv) + z clamped to [0, 15] (the
 * product is a single rounded multiply). */
int orc_act_asym_code(float x, float inv, int z)
{
    float p = x * inv;
    int u = (int)rintf(p) + z;
    return u < 0 ? 0 : (u > 15 ? 15 : u);
}

/* qa: [M][K] signed codes in permuted channel order (4-bit blocks: u - z in
 * [-15, 15]; 8-bit blocks: step 3's symmetric codes). u4: [M][K] the stored
 * 4-bit codes u (0 on 8-bit blocks). sa: [M][nb] steps. za: [M][nb] zero
 * points (0 on 8-bit blocks). A 4-bit block whose range is [0, 0] (all zero)
 * gets step 0, zero point 0 and codes 0. */
int orc_quantize_activations_asym(const uint16_t *X, int M, int K, int ldx, const int32_t *perm,
                                  const uint8_t *is_int8, int8_t *qa, uint8_t *u4, float *sa,
                                  uint8_t *za)
{
    if (M <= 0 || K <= 0 || K % ORC_BLOCK != 0 || ldx < K)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int m = 0; m < M; ++m) {
        const uint16_t *xrow = X + (size_t)m * ldx;
        for (int b = 0; b < nb; ++b) {
            int8_t *q = qa + (size_t)m * K + (size_t)b * ORC_BLOCK;
            uint8_t *u = u4 + (size_t)m * K + (size_t)b * ORC_BLOCK;
            if (is_int8[b]) {
                /* step 3, unchanged */
                float a = 0.0f;
                for (int k = 0; k < ORC_BLOCK; ++k) {
                    float v = orc_half_to_float(xrow[perm[b * ORC_BLOCK + k]]);
                    if (!isfinite(v))
                        bad = 1;
                    if (fabsf(v) > a)
                        a = fabsf(v);
                }
                float inv = 0.0f, s = 0.0f;
                if (a > 0.0f)
                    orc_act_scale(a, 127, &inv, &s);
                sa[(size_t)m * nb + b] = s;
                za[(size_t)m * nb + b] = 0;
                for (int k = 0; k < ORC_BLOCK; ++k) {
                    float v = orc_half_to_float(xrow[perm[b * ORC_BLOCK + k]]);
                    q[k] = a > 0.0f ? (int8_t)orc_act_quantize_value(v, inv, 127) : 0;
                    u[k] = 0;
                }
                continue;
            }
            float lo = 0.0f, hi = 0.0f;     /* the range always holds 0 */
            for (int k = 0; k < ORC_BLOCK; ++k) {
                float v = orc_half_to_float(xrow[perm[b * ORC_BLOCK + k]]);
                if (!isfinite(v))
                    bad = 1;
                if (v < lo)
                    lo = v;
                if (v > hi)
                    hi = v;
            }
            if (lo == hi) {                 /* all zero */
                sa[(size_t)m * nb + b] = 0.0f;
                za[(size_t)m * nb + b] = 0;
                for (int k = 0; k < ORC_BLOCK; ++k) {
                    q[k] = 0;
                    u[k] = 0;
                }
                continue;
            }
            float inv, s;
            int z;
            orc_act_asym_params(lo, hi, &inv, &s, &z);
            sa[(size_t)m * nb + b] = s;
            za[(size_t)m * nb + b] = (uint8_t)z;
            for (int k = 0; k < ORC_BLOCK; ++k) {
                float v = orc_half_to_float(xrow[perm[b * ORC_BLOCK + k]]);
                int uu = orc_act_asym_code(v, inv, z);
                u[k] = (uint8_t)uu;
                q[k] = (int8_t)(uu - z);
            }
        }
    }
    return bad ? ORC_ERR_NONFINITE : ORC_OK;
}

/* The asymmetric partials through the stored code and the zero point: on a
 * 4-bit block P = sum(u * qw) - z * wsum (QUIK blog, section "反量化背后的数学":
 * the zero-point term needs only z and the offline weight sum); 8-bit blocks
 * take the signed codes. */
int orc_block_partials_zero_point(const int8_t *qa, const uint8_t *u4, const uint8_t *za,
                                  const int8_t *qw, const int32_t *wsum, const uint8_t *is_int8,
                                  int M, int N, int K, int m0, int m1, int32_t *P)
{
    if (N <= 0 || K <= 0 || K % ORC_BLOCK != 0 || m0 < 0 || m1 > M || m0 >= m1)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int m = m0; m < m1; ++m) {
        for (int n = 0; n < N; ++n) {
            const int8_t *w = qw + (size_t)n * K;
            int32_t *out = P + ((size_t)(m - m0) * N + n) * nb;
            for (int b = 0; b < nb; ++b) {
                int32_t acc = 0;
                if (is_int8[b]) {
                    const int8_t *a = qa + (size_t)m * K;
                    for (int k = b * ORC_BLOCK; k < (b + 1) * ORC_BLOCK; ++k)
                        acc += (int32_t)a[k] * (int32_t)w[k];
                } else {
                    const uint8_t *u = u4 + (size_t)m * K;
                    for (int k = b * ORC_BLOCK; k < (b + 1) * ORC_BLOCK; ++k)
                        acc += (int32_t)u[k] * (int32_t)w[k];
                    acc -= (int32_t)za[(size_t)m * nb + b] * wsum[(size_t)n * nb + b];
                }
                out[b] = acc;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 4. Block partials                                                         */
/* ------------------------------------------------------------------------ */

/* P[m - m0][n][b] = sum over the block of qa[m][k'] * qw[n][k'], exact. */
int orc_block_partials(const int8_t *qa, const int8_t *qw, int M, int N, int K, int m0, int m1,
                       int32_t *P)
{
    if (N <= 0 || K <= 0 || K % ORC_BLOCK != 0 || m0 < 0 || m1 > M || m0 >= m1)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int m = m0; m < m1; ++m) {
        const int8_t *a = qa + (size_t)m * K;
        for (int n = 0; n < N; ++n) {
            const int8_t *w = qw + (size_t)n * K;
            int32_t *out = P + ((size_t)(m - m0) * N + n) * nb;
            for (int b = 0; b < nb; ++b) {
                int32_t acc = 0;
                for (int k = b * ORC_BLOCK; k < (b + 1) * ORC_BLOCK; ++k)
                    acc += (int32_t)a[k] * (int32_t)w[k];
                out[b] = acc;
            }
        }
    }
    return ORC_OK;
}

/* The same partials through the zero-extended 4-bit code: on a 4-bit block the
 * activation enters as u = q + 8 in [1, 15] and the offset is removed with the
 * precomputed weight sum, P = sum(u * qw) - 8 * wsum. 8-bit blocks are signed. */
int orc_block_partials_zero_extend(const int8_t *qa, const int8_t *qw, const int32_t *wsum,
                                   const uint8_t *is_int8, int M, int N, int K, int m0, int m1,
                                   int32_t *P)
{
    if (N <= 0 || K <= 0 || K % ORC_BLOCK != 0 || m0 < 0 || m1 > M || m0 >= m1)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int m = m0; m < m1; ++m) {
        const int8_t *a = qa + (size_t)m * K;
        for (int n = 0; n < N; ++n) {
            const int8_t *w = qw + (size_t)n * K;
            int32_t *out = P + ((size_t)(m - m0) * N + n) * nb;
            for (int b = 0; b < nb; ++b) {
                int32_t acc = 0;
                if (is_int8[b]) {
                    for (int k = b * ORC_BLOCK; k < (b + 1) * ORC_BLOCK; ++k)
                        acc += (int32_t)a[k] * (int32_t)w[k];
                } else {
                    for (int k = b * ORC_BLOCK; k < (b + 1) * ORC_BLOCK; ++k) {
                        uint32_t u = (uint32_t)(a[k] + 8);          /* 1 .. 15 */
                        acc += (int32_t)u * (int32_t)w[k];
                    }
                    acc -= 8 * wsum[(size_t)n * nb + b];
                }
                out[b] = acc;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 5. Epilogue                                                               */
/* ------------------------------------------------------------------------ */

/* For rows r of P ([rows][N][nb]) with scales sa ([rows][nb]) and sw16
 * ([N][nb]):
 *   y32 = 0;  for b in order:  y32 = y32 + (sa * sw) * float(P)
 *   Y16 = fp16(y32)
 * and, in double, yexact = sum_b sa * sw * P (each product is exact in
 * double: 24 + 11 + 17 significant bits). Any output pointer may be NULL. */
int orc_epilogue(const int32_t *P, const float *sa, const uint16_t *sw16, int rows, int N, int nb,
                 float *y32, uint16_t *Y16, double *yexact)
{
    if (rows <= 0 || N <= 0 || nb <= 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        for (int n = 0; n < N; ++n) {
            const int32_t *p = P + ((size_t)r * N + n) * nb;
            float y = 0.0f;
            double ye = 0.0;
            for (int b = 0; b < nb; ++b) {
                float s_x = sa[(size_t)r * nb + b];
                float s_w = orc_half_to_float(sw16[(size_t)n * nb + b]);
                float t = s_x * s_w;
                float u = t * (float)p[b];
                y = y + u;
                ye += (double)s_x * (double)s_w * (double)p[b];
            }
            size_t o = (size_t)r * N + n;
            if (y32) y32[o] = y;
            if (Y16) Y16[o] = orc_float_to_half(y);
            if (yexact) yexact[o] = ye;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 6. RMS normalization (the step before the quantizer)                      */
/* ------------------------------------------------------------------------ */

/* binary64 nearest to a non-negative 128-bit integer, ties to even: keep the
 * 53 leading bits, look at the bits cut off (above, at or below half a unit
 * of the kept last bit) and round the kept part up where the rule says so. */
static double orc_u128_to_double(unsigned __int128 v)
{
    if ((v >> 53) == 0)
        return (double)(uint64_t)v; /* fits the significand: exact */
    int n = 0; /* bit length of v */
    for (unsigned __int128 t = v; t != 0; t >>= 1)
        ++n;
    int cut = n - 53;
    unsigned __int128 kept = v >> cut;
    unsigned __int128 rest = v - (kept << cut);
    unsigned __int128 half = (unsigned __int128)1 << (cut - 1);
    if (rest > half || (rest == half && (kept & 1)))
        kept += 1; /* may reach 2^53: still exact in binary64 */
    return ldexp((double)(uint64_t)kept, cut);
}

/* Row statistic S = sum over k of x_k^2, the exact real sum rounded once to
 * binary64 (nearest, ties to even). The pages fix no precision or order for
 * it; the exact sum is the one value that needs neither. Every binary16 value
 * is an integer multiple of 2^-24 (|x| = n 2^-24 with n < 2^40), so every
 * square is n^2 2^-48 with n^2 < 2^80, and the integers n^2 add up exactly in
 * 128 bits for any row this library accepts (K < 2^47). */
double orc_rms_sumsq(const uint16_t *x, int K)
{
    unsigned __int128 acc = 0;
    for (int k = 0; k < K; ++k) {
        double v = fabs((double)orc_half_to_float(x[k])); /* exact */
        uint64_t n = (uint64_t)ldexp(v, 24);              /* exact integer */
        acc += (unsigned __int128)n * n;
    }
    return ldexp(orc_u128_to_double(acc), -48); /* a power-of-two scaling: exact */
}

/* Xn[m][k] = fp16( (x * r) * gamma_k ) with r = binary32( 1 / sqrt(S / K +
 * eps) ), S the row statistic above, the reciprocal square root taken in
 * binary64 and rounded once to binary32, the two products in binary32, and
 * the result rounded to binary16 (nearest, ties to even). Channels stay in
 * their original order; gamma is fp16 [K]. Non-finite inputs are rejected. */
int orc_rmsnorm_rows(const uint16_t *X, int M, int K, int ldx, const uint16_t *gamma, float eps,
                     uint16_t *Xn, int ldn)
{
    if (M <= 0 || K <= 0 || ldx < K || ldn < K || !(eps > 0.0f) || !isfinite(eps))
        return ORC_ERR_ARG;
    for (int k = 0; k < K; ++k)
        if (!isfinite(orc_half_to_float(gamma[k])))
            return ORC_ERR_NONFINITE;
    int rc = ORC_OK;
    for (int m = 0; m < M; ++m) {
        const uint16_t *x = X + (size_t)m * ldx;
        for (int k = 0; k < K; ++k)
            if (!isfinite(orc_half_to_float(x[k])))
                rc = ORC_ERR_NONFINITE;
        if (rc != ORC_OK)
            return rc;
        double S = orc_rms_sumsq(x, K);
        double r64 = 1.0 / sqrt(S / (double)K + (double)eps);
        float r = (float)r64;
        for (int k = 0; k < K; ++k) {
            float t = orc_half_to_float(x[k]) * r;
            float u = t * orc_half_to_float(gamma[k]);
            Xn[(size_t)m * ldn + k] = orc_float_to_half(u);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 7. SwiGLU (the step before the down projection's quantizer)               */
/* ------------------------------------------------------------------------ */

/* binary16 nearest to a binary64 value, ties to even; overflow gives an
 * infinity. The value is scaled by a power of two so that its binary16
 * quantum becomes 1, rounded there with rint(), and scaled back; every step
 * but the rint() is exact. */
uint16_t orc_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00u;
    if (a >= 65520.0) /* at or past the midpoint between 65504 and 2^16 */
        return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int q = e - 11; /* binary16 quantum of that binade */
    if (q < -24)
        q = -24; /* subnormal quantum */
    double r = ldexp(rint(ldexp(a, -q)), q);
    return (uint16_t)(sign | orc_float_to_half((float)r)); /* r is a binary16 value */
}

/* h = silu(g) u = g u / (1 + e^-g), the exact real value rounded once to
 * binary16 (ties to even); this library's reading of a step whose precision
 * the pages do not state. Evaluated in binary64: sigma = 1 / (1 + e^-g) for
 * g >= 0 and e^g / (1 + e^g) below (no overflow), g u exact (two binary16
 * significands fit in 22 bits). When sigma rounds to exactly 1 (g > 36) the
 * true product lies strictly between g u and the next binary64 value toward
 * zero, so that value stands in for it: a tie of g u on the binary16 grid
 * then resolves toward zero, as it must. */
uint16_t orc_silu_mul(uint16_t g16, uint16_t u16)
{
    double g = (double)orc_half_to_float(g16);
    double u = (double)orc_half_to_float(u16);
    double sigma;
    if (g >= 0.0) {
        sigma = 1.0 / (1.0 + exp(-g));
    } else {
        double e = exp(g);
        sigma = e / (1.0 + e);
    }
    double gu = g * u;
    double v = gu * sigma;
    if (sigma == 1.0 && gu != 0.0)
        v = nextafter(gu, 0.0);
    return orc_double_to_half(v);
}

/* H[m][k] = orc_silu_mul(G[m][k], U[m][k]) for the gate and up rows (row
 * stride ldx, both) into H (row stride ldh). Non-finite inputs are rejected,
 * and so is a product that overflows binary16. */
int orc_swiglu_rows(const uint16_t *G, const uint16_t *U, int M, int K, int ldx, uint16_t *H, int ldh)
{
    if (M <= 0 || K <= 0 || ldx < K || ldh < K)
        return ORC_ERR_ARG;
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) {
            uint16_t g = G[(size_t)m * ldx + k], u = U[(size_t)m * ldx + k];
            if (!isfinite(orc_half_to_float(g)) || !isfinite(orc_half_to_float(u)))
                return ORC_ERR_NONFINITE;
            uint16_t h = orc_silu_mul(g, u);
            if (!isfinite(orc_half_to_float(h)))
                return ORC_ERR_NONFINITE;
            H[(size_t)m * ldh + k] = h;
        }
    return ORC_OK;
}

/* Element-wise form for the pins: h[i] = orc_silu_mul(g[i], u[i]). */
void orc_silu_mul_array(const uint16_t *g, const uint16_t *u, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = orc_silu_mul(g[i], u[i]);
}

/* ------------------------------------------------------------------------ */
/* Online forward for a row range (steps 3-5), for timing on the host        */
/* ------------------------------------------------------------------------ */

/* Quantizes rows [m0, m1) of X, forms their block partials against the
 * already-quantized weights and applies the epilogue. Y16 and yexact are
 * [(m1-m0)][N]; either may be NULL. */
int orc_forward_rows(const uint16_t *X, int M, int K, int ldx, const int32_t *perm,
                     const uint8_t *is_int8, const int8_t *qw, const uint16_t *sw16, int N,
                     int m0, int m1, uint16_t *Y16, double *yexact)
{
    if (M <= 0 || K <= 0 || K % ORC_BLOCK != 0 || m0 < 0 || m1 > M || m0 >= m1 || N <= 0)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
    int rows = m1 - m0;
    int8_t *qa = (int8_t *)malloc((size_t)rows * K);
    float *sa = (float *)malloc(sizeof(float) * (size_t)rows * nb);
    int32_t *P = (int32_t *)malloc(sizeof(int32_t) * (size_t)rows * N * nb);
    int rc = ORC_ERR_ARG;
    if (qa && sa && P) {
        rc = orc_quantize_activations(X + (size_t)m0 * ldx, rows, K, ldx, perm, is_int8, qa, sa);
        if (rc == ORC_OK)
            rc = orc_block_partials(qa, qw, rows, N, K, 0, rows, P);
        if (rc == ORC_OK)
            rc = orc_epilogue(P, sa, sw16, rows, N, nb, NULL, Y16, yexact);
    }
    free(qa);
    free(sa);
    free(P);
    return rc;
}

/* Threads an OpenMP parallel region of this library uses. */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the OpenMP loops use from now on (for timing on one core). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* 8. QoQ progressive group quantization (W4A8)                             */
/* ------------------------------------------------------------------------ */

/* Nearest integer of the rational num / den (den > 0), ties to even. */
static int orc_div_round_even(int num, int den)
{
    int q = num / den, r = num % den;          /* C division truncates toward 0 */
    if (r < 0) {                                /* make the remainder non-negative */
        q -= 1;
        r += den;
    }
    /* num / den = q + r / den with 0 <= r < den */
    if (2 * r > den || (2 * r == den && (q & 1)))
        q += 1;
    return q;
}

/* Second level of one group of 8-bit weights w8[0..n): range [lo, hi] =
 * [min(0, min w8), max(0, max w8)], integer step s2 = max(1, ceil((hi - lo)
 * / 15)), zero point z = round(-lo / s2), code u = clamp(round(w8 / s2) + z,
 * 0, 15), all in exact integer arithmetic, ties to even. Returns s2; z and u
 * through the pointers. */
int orc_qoq_group(const int8_t *w8, int n, int *z, uint8_t *u)
{
    int lo = 0, hi = 0;
    for (int k = 0; k < n; ++k) {
        if (w8[k] < lo) lo = w8[k];
        if (w8[k] > hi) hi = w8[k];
    }
    int s2 = (hi - lo + 14) / 15;
    if (s2 < 1)
        s2 = 1;
    int zz = orc_div_round_even(-lo, s2);
    *z = zz;
    for (int k = 0; k < n; ++k) {
        int v = orc_div_round_even(w8[k], s2) + zz;
        u[k] = (uint8_t)(v < 0 ? 0 : (v > 15 ? 15 : v));
    }
    return s2;
}

/* Weights [N][K] (original channel order) with channel order perm:
 *   s1[n] = fp16(a / 119) with a = max |W[n, :]| (the smallest fp16 subnormal
 *   if that rounds to 0; 0 for an all-zero row), w8 = clamp(round(W / s1),
 *   -119, 119) (binary32 division, ties to even);
 *   per 128-channel group g of permuted positions: s2[n][g], z[n][g] and the
 *   codes u[n][k'] by orc_qoq_group.
 * w8 is also returned ([N][K], permuted order). */
int orc_qoq_quantize_weights(const uint16_t *W, int N, int K, const int32_t *perm, uint16_t *s1,
                             int8_t *w8, uint8_t *s2, uint8_t *z, uint8_t *u)
{
    if (N <= 0 || K <= 0 || K % ORC_BLOCK != 0)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int n = 0; n < N; ++n) {
        const uint16_t *wrow = W + (size_t)n * K;
        float a = 0.0f;
        for (int k = 0; k < K; ++k) {
            float v = orc_half_to_float(wrow[k]);
            if (!isfinite(v))
                bad = 1;
            if (fabsf(v) > a)
                a = fabsf(v);
        }
        uint16_t h = 0;
        if (a > 0.0f) {
            h = orc_float_to_half(a / 119.0f);
            if (h == 0)
                h = 1;
        }
        s1[n] = h;
        float s = orc_half_to_float(h);
        int8_t *wq = w8 + (size_t)n * K;
        for (int k = 0; k < K; ++k) {
            if (h == 0) {
                wq[k] = 0;
                continue;
            }
            float v = orc_half_to_float(wrow[perm[k]]);
            int q = (int)rintf(v / s);
            wq[k] = (int8_t)(q < -119 ? -119 : (q > 119 ? 119 : q));
        }
        for (int b = 0; b < nb; ++b) {
            int zz;
            s2[(size_t)n * nb + b] = (uint8_t)orc_qoq_group(wq + (size_t)b * ORC_BLOCK, ORC_BLOCK, &zz,
                                                             u + (size_t)n * K + (size_t)b * ORC_BLOCK);
            z[(size_t)n * nb + b] = (uint8_t)zz;
        }
    }
    return bad ? ORC_ERR_NONFINITE : ORC_OK;
}

/* Activations [M][ldx], per token over all K in permuted order: a = max |x|,
 * inv = 127 / a and s = a / 127 (binary32 divisions), q = clamp(round(x *
 * inv), -127, 127); an all-zero token gets s = 0 and q = 0. */
int orc_qoq_quantize_activations(const uint16_t *X, int M, int K, int ldx, const int32_t *perm, int8_t *qa,
                                 float *sa)
{
    if (M <= 0 || K <= 0 || K % ORC_BLOCK != 0 || ldx < K)
        return ORC_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int m = 0; m < M; ++m) {
        const uint16_t *xrow = X + (size_t)m * ldx;
        float a = 0.0f;
        for (int k = 0; k < K; ++k) {
            float v = orc_half_to_float(xrow[perm[k]]);
            if (!isfinite(v))
                bad = 1;
            if (fabsf(v) > a)
                a = fabsf(v);
        }
        int8_t *q = qa + (size_t)m * K;
        if (a == 0.0f) {
            sa[m] = 0.0f;
            memset(q, 0, (size_t)K);
            continue;
        }
        float inv, s;
        orc_act_scale(a, 127, &inv, &s);
        sa[m] = s;
        for (int k = 0; k < K; ++k)
            q[k] = (int8_t)orc_act_quantize_value(orc_half_to_float(xrow[perm[k]]), inv, 127);
    }
    return bad ? ORC_ERR_NONFINITE : ORC_OK;
}

/* Rows [m0, m1): P[m - m0][n] = sum over groups of s2 * (sum_k qa u - z sum_k
 * qa) (the zero point subtracted after the multiplication, as the page puts
 * it), exact in 64-bit and returned as int32 (|P| <= 127 * 128 * K < 2^31 for
 * K <= 131072); then y32 = fl(s_x s1) * (float)P, Y16 = fp16(y32), and
 * yexact = s_x s1 P in double. Any output pointer may be NULL. */
int orc_qoq_gemm(const int8_t *qa, const float *sa, const uint8_t *u, const uint8_t *s2, const uint8_t *z,
                 const uint16_t *s1, int M, int N, int K, int m0, int m1, int32_t *P, float *y32,
                 uint16_t *Y16, double *yexact)
{
    if (N <= 0 || K <= 0 || K % ORC_BLOCK != 0 || K > 131072 || m0 < 0 || m1 > M || m0 >= m1)
        return ORC_ERR_ARG;
    int nb = K / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int m = m0; m < m1; ++m) {
        const int8_t *a = qa + (size_t)m * K;
        for (int n = 0; n < N; ++n) {
            const uint8_t *w = u + (size_t)n * K;
            int64_t acc = 0;
            for (int b = 0; b < nb; ++b) {
                int64_t dot = 0, asum = 0;
                for (int k = b * ORC_BLOCK; k < (b + 1) * ORC_BLOCK; ++k) {
                    dot += (int64_t)a[k] * (int64_t)w[k];
                    asum += a[k];
                }
                int64_t st = s2[(size_t)n * nb + b];
                acc += st * dot - st * (int64_t)z[(size_t)n * nb + b] * asum;
            }
            size_t o = (size_t)(m - m0) * N + n;
            if (P) P[o] = (int32_t)acc;
            float sw = orc_half_to_float(s1[n]);
            float t = sa[m] * sw;
            float y = t * (float)acc;
            if (y32) y32[o] = y;
            if (Y16) Y16[o] = orc_float_to_half(y);
            if (yexact) yexact[o] = (double)sa[m] * (double)sw * (double)acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 9. KV4 decode attention                                                   */
/* ------------------------------------------------------------------------ */

/* One vector v[0..d) of one (token, head): range [lo, hi] = [min(0, min v),
 * max(0, max v)]; if hi > lo: step s16 = fp16(d_ / 15) with d_ = hi - lo (the
 * smallest fp16 subnormal if that rounds to 0), inv = 15 / d_ (binary32), z =
 * clamp(round(-lo * inv), 0, 15), u = clamp(round(v * inv) + z, 0, 15); an
 * all-zero vector gets s16 = 0, z = 0, u = 0. The value represented is
 * float(s16) (u - z). */
void orc_kv4_code_vector(const uint16_t *v, int d, uint8_t *u, uint16_t *s16, uint8_t *z)
{
    float lo = 0.0f, hi = 0.0f;
    for (int i = 0; i < d; ++i) {
        float x = orc_half_to_float(v[i]);
        if (x < lo) lo = x;
        if (x > hi) hi = x;
    }
    if (lo == hi) {
        *s16 = 0;
        *z = 0;
        memset(u, 0, (size_t)d);
        return;
    }
    float dd = hi - lo;
    float inv = 15.0f / dd;
    uint16_t h = orc_float_to_half(dd / 15.0f);
    if (h == 0)
        h = 1;
    *s16 = h;
    int zz = (int)rintf(-lo * inv);
    zz = zz < 0 ? 0 : (zz > 15 ? 15 : zz);
    *z = (uint8_t)zz;
    for (int i = 0; i < d; ++i) {
        int c = (int)rintf(orc_half_to_float(v[i]) * inv) + zz;
        u[i] = (uint8_t)(c < 0 ? 0 : (c > 15 ? 15 : c));
    }
}

/* A cache [n][d] of n vectors (one head's keys or values): codes [n][d],
 * steps [n] (fp16 bits), zero points [n]. */
int orc_kv4_quantize(const uint16_t *V, int n, int d, uint8_t *u, uint16_t *s16, uint8_t *z)
{
    if (n <= 0 || d <= 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n; ++t)
        orc_kv4_code_vector(V + (size_t)t * d, d, u + (size_t)t * d, s16 + t, z + t);
    return ORC_OK;
}

/* Decode attention for H heads (one query each) over T cached tokens, in
 * double precision on the dequantized cache:
 *   k_t = s_k[t] (uk[t] - zk[t]),  v_t = s_v[t] (uv[t] - zv[t]),
 *   a_t = (q . k_t) / sqrt(d),  p_t = exp(a_t - max a) / sum exp(. - max a),
 *   out = sum_t p_t v_t.
 * q: fp16 [H][d]; codes [H][T][d]; steps fp16 [H][T]; zero points [H][T];
 * out: double [H][d]. */
int orc_kv4_attention(const uint16_t *q, const uint8_t *uk, const uint16_t *sk, const uint8_t *zk,
                      const uint8_t *uv, const uint16_t *sv, const uint8_t *zv, int H, int T, int d,
                      double *out)
{
    if (H <= 0 || T <= 0 || d <= 0)
        return ORC_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int h = 0; h < H; ++h) {
        double *a = (double *)malloc(sizeof(double) * (size_t)T);
        if (!a) {
            bad = 1;
            continue;
        }
        const uint16_t *qh = q + (size_t)h * d;
        double amax = -INFINITY;
        for (int t = 0; t < T; ++t) {
            size_t o = ((size_t)h * T + t);
            double sk_t = orc_half_to_float(sk[o]);
            double dot = 0.0;
            for (int i = 0; i < d; ++i)
                dot += (double)orc_half_to_float(qh[i]) * sk_t * ((double)uk[o * d + i] - (double)zk[o]);
            a[t] = dot / sqrt((double)d);
            if (a[t] > amax)
                amax = a[t];
        }
        double denom = 0.0;
        for (int t = 0; t < T; ++t) {
            a[t] = exp(a[t] - amax);
            denom += a[t];
        }
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int t = 0; t < T; ++t) {
                size_t o = ((size_t)h * T + t);
                acc += a[t] * (double)orc_half_to_float(sv[o]) * ((double)uv[o * d + i] - (double)zv[o]);
            }
            out[(size_t)h * d + i] = acc / denom;
        }
        free(a);
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 10. QUIK's FP16 outlier columns                                          */
/* ------------------------------------------------------------------------ */

/* Add the FP16 outlier part to step 5's results for `rows` rows: Xf [rows][nf]
 * and Wf [N][nf] hold the fp16 bits of the last nf permuted channels; y32 and
 * yexact come from orc_epilogue over the quantized channels and are updated in
 * place (y32 in channel order, one FP32 addition per channel of the exact
 * product), Y16 = fp16(y32). */
int orc_quik_outlier_add(const uint16_t *Xf, const uint16_t *Wf, int rows, int N, int nf, float *y32,
                         uint16_t *Y16, double *yexact)
{
    if (rows <= 0 || N <= 0 || nf < 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        for (int n = 0; n < N; ++n) {
            size_t o = (size_t)r * N + n;
            float y = y32[o];
            double ye = yexact[o];
            for (int j = 0; j < nf; ++j) {
                float x = orc_half_to_float(Xf[(size_t)r * nf + j]);
                float w = orc_half_to_float(Wf[(size_t)n * nf + j]);
                y = y + x * w;
                ye += (double)x * (double)w;
            }
            y32[o] = y;
            yexact[o] = ye;
            if (Y16) Y16[o] = orc_float_to_half(y);
        }
    }
    return ORC_OK;
}
