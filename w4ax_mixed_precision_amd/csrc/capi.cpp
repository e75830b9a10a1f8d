// The C entry points: argument validation (before any HIP call, so a rejected
// call needs no GPU and has no device effect), then the launchers.
#include <cstdint>
#include <limits>

#include "comet_internal.h"
#include "kv4_internal.h"
#include "qoq_internal.h"

namespace {

using comet::kBlock;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common shape checks of the online calls. Sizes must keep every byte offset
// the kernels form inside size_t and every element index of one buffer
// inside int32 where the kernels use 32-bit products.
int check_online_shape(int M, int N, int K, int nb8) {
    if (M < 1 || N < 1 || K < kBlock || K % kBlock != 0) return COMET_ERR_SHAPE;
    if (nb8 < 0 || nb8 > K / kBlock) return COMET_ERR_ARG;
    if (N % 128 != 0) return COMET_ERR_UNSUPPORTED;
    const int64_t mk = static_cast<int64_t>(M) * K;
    const int64_t nk = static_cast<int64_t>(N) * K;
    const int64_t mn = static_cast<int64_t>(M) * N;
    const int64_t lim = std::numeric_limits<int32_t>::max();
    if (mk > lim || nk > lim || mn > lim) return COMET_ERR_UNSUPPORTED;
    return COMET_OK;
}

int hip_status(int e) { return e == 0 ? COMET_OK : COMET_ERR_HIP; }

// The FP6 GEMM addresses its activation buffer (rows padded to 16) with
// 32-bit byte offsets: at most 128 bytes per (padded row, block).
bool fp6_offsets_fit(int M, int K) {
    const int64_t mp = (static_cast<int64_t>(M) + 15) & ~static_cast<int64_t>(15);
    return mp * K <= std::numeric_limits<int32_t>::max();
}

// Shared checks of the two fused normalization + quantization calls.
int check_rmsnorm_quant(const void* X, int M, int K, int ldx, const void* gamma_perm, float eps,
                        const int32_t* perm, int nb8, const void* Xq, const float* x_scale) {
    if (!X || !gamma_perm || !perm || !Xq || !x_scale) return COMET_ERR_NULL;
    if (M < 1 || K < kBlock || K % kBlock != 0 || ldx < K) return COMET_ERR_SHAPE;
    if (nb8 < 0 || nb8 > K / kBlock) return COMET_ERR_ARG;
    if (!(eps > 0.0f) || !(eps <= std::numeric_limits<float>::max())) return COMET_ERR_ARG;
    if (!aligned16(X) || !aligned16(gamma_perm) || !aligned16(perm) || !aligned16(Xq) || !aligned16(x_scale))
        return COMET_ERR_ALIGN;
    return COMET_OK;
}

int check_swiglu_quant(const void* G, const void* U, int M, int K, int ldx, const int32_t* perm, int nb8,
                       const void* Xq, const float* x_scale) {
    if (!G || !U || !perm || !Xq || !x_scale) return COMET_ERR_NULL;
    if (M < 1 || K < kBlock || K % kBlock != 0 || ldx < K) return COMET_ERR_SHAPE;
    if (nb8 < 0 || nb8 > K / kBlock) return COMET_ERR_ARG;
    if (!aligned16(G) || !aligned16(U) || !aligned16(perm) || !aligned16(Xq) || !aligned16(x_scale))
        return COMET_ERR_ALIGN;
    return COMET_OK;
}

}  // namespace

extern "C" {

int comet_pack_weights(const uint16_t* W_fp16, int N, int K, const float* chan_score,
                       int n_int8_blocks, int32_t* perm, uint8_t* block_is_int8,
                       uint8_t* Wq_packed, uint16_t* w_scale_fp16, int16_t* w_sum) {
    if (!W_fp16 || !chan_score || !perm || !block_is_int8 || !Wq_packed || !w_scale_fp16 || !w_sum)
        return COMET_ERR_NULL;
    if (N < 1 || K < kBlock || K % kBlock != 0) return COMET_ERR_SHAPE;
    if (n_int8_blocks < 0 || n_int8_blocks > K / kBlock) return COMET_ERR_ARG;
    if (N % 128 != 0) return COMET_ERR_UNSUPPORTED;
    return comet::pack_weights(W_fp16, N, K, chan_score, n_int8_blocks, perm, block_is_int8,
                               Wq_packed, w_scale_fp16, w_sum);
}

int comet_quant_act(const void* X_fp16, int M, int K, int ldx, const int32_t* perm,
                    int n_int8_blocks, void* Xq, float* x_scale, void* stream) {
    if (!X_fp16 || !perm || !Xq || !x_scale) return COMET_ERR_NULL;
    if (M < 1 || K < kBlock || K % kBlock != 0 || ldx < K) return COMET_ERR_SHAPE;
    if (n_int8_blocks < 0 || n_int8_blocks > K / kBlock) return COMET_ERR_ARG;
    if (!aligned16(X_fp16) || !aligned16(perm) || !aligned16(Xq) || !aligned16(x_scale))
        return COMET_ERR_ALIGN;
    return hip_status(comet::launch_quant_act(static_cast<const uint16_t*>(X_fp16), M, K, ldx, perm,
                                              n_int8_blocks, static_cast<uint8_t*>(Xq), x_scale,
                                              stream));
}

size_t comet_w4ax_gemm_workspace_bytes(int M, int N, int K, int n_int8_blocks) {
    if (check_online_shape(M, N, K, n_int8_blocks) != COMET_OK) return 0;
    return comet::gemm_workspace_bytes(M, N, K, n_int8_blocks);
}

int comet_quant_act_asym(const void* X_fp16, int M, int K, int ldx, const int32_t* perm,
                         int n_int8_blocks, void* Xq, float* x_scale, uint8_t* x_zero, void* stream) {
    if (!X_fp16 || !perm || !Xq || !x_scale || !x_zero) return COMET_ERR_NULL;
    if (M < 1 || K < kBlock || K % kBlock != 0 || ldx < K) return COMET_ERR_SHAPE;
    if (n_int8_blocks < 0 || n_int8_blocks > K / kBlock) return COMET_ERR_ARG;
    if (!aligned16(X_fp16) || !aligned16(perm) || !aligned16(Xq) || !aligned16(x_scale) || !aligned16(x_zero))
        return COMET_ERR_ALIGN;
    return hip_status(comet::launch_quant_act_asym(static_cast<const uint16_t*>(X_fp16), M, K, ldx, perm,
                                                   n_int8_blocks, static_cast<uint8_t*>(Xq), x_scale, x_zero,
                                                   stream));
}

int comet_pack_weights_qoq(const uint16_t* W_fp16, int N, int K, const float* chan_score, int32_t* perm,
                           uint8_t* Wu_packed, uint16_t* s1_fp16, uint16_t* s2z) {
    if (!W_fp16 || !chan_score || !perm || !Wu_packed || !s1_fp16 || !s2z) return COMET_ERR_NULL;
    if (N < 1 || K < kBlock || K % kBlock != 0) return COMET_ERR_SHAPE;
    if (N % 128 != 0) return COMET_ERR_UNSUPPORTED;
    return comet::pack_weights_qoq(W_fp16, N, K, chan_score, perm, Wu_packed, s1_fp16, s2z);
}

int comet_quant_act_token_i8(const void* X_fp16, int M, int K, int ldx, const int32_t* perm, void* Xq,
                             float* x_scale, void* stream) {
    if (!X_fp16 || !perm || !Xq || !x_scale) return COMET_ERR_NULL;
    if (M < 1 || K < kBlock || K % kBlock != 0 || ldx < K) return COMET_ERR_SHAPE;
    if (K > 32768) return COMET_ERR_UNSUPPORTED;
    if (!aligned16(X_fp16) || !aligned16(perm) || !aligned16(Xq) || !aligned16(x_scale)) return COMET_ERR_ALIGN;
    return hip_status(comet::launch_quant_act_token_i8(static_cast<const uint16_t*>(X_fp16), M, K, ldx, perm,
                                                       static_cast<uint8_t*>(Xq), x_scale, stream));
}

namespace {

int qoq_check(const void* Xq, const float* x_scale, const void* Wu_packed, const uint16_t* s2z,
              const uint16_t* s1_fp16, int M, int N, int K) {
    if (!Xq || !x_scale || !Wu_packed || !s2z || !s1_fp16) return COMET_ERR_NULL;
    if (M < 1 || N < 1 || K < kBlock || K % kBlock != 0) return COMET_ERR_SHAPE;
    if (N % 128 != 0 || K > 32768) return COMET_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(M) * N > std::numeric_limits<int32_t>::max()) return COMET_ERR_UNSUPPORTED;
    if (!aligned16(Xq) || !aligned16(x_scale) || !aligned16(Wu_packed) || !aligned16(s2z) || !aligned16(s1_fp16))
        return COMET_ERR_ALIGN;
    return COMET_OK;
}

}  // namespace

int comet_w4a8_qoq_gemm(const void* Xq, const float* x_scale, const void* Wu_packed, const uint16_t* s2z,
                        const uint16_t* s1_fp16, int M, int N, int K, void* Y_fp16, int ldy, void* stream) {
    if (!Y_fp16) return COMET_ERR_NULL;
    const int st = qoq_check(Xq, x_scale, Wu_packed, s2z, s1_fp16, M, N, K);
    if (st != COMET_OK) return st;
    if (ldy < N) return COMET_ERR_SHAPE;
    if (!aligned16(Y_fp16)) return COMET_ERR_ALIGN;
    return hip_status(comet::launch_qoq_gemm(static_cast<const uint8_t*>(Xq), x_scale,
                                             static_cast<const uint8_t*>(Wu_packed), s2z, s1_fp16, M, N, K,
                                             static_cast<uint16_t*>(Y_fp16), ldy, nullptr, stream));
}

int comet_w4a8_qoq_gemm_products(const void* Xq, const float* x_scale, const void* Wu_packed, const uint16_t* s2z,
                                 const uint16_t* s1_fp16, int M, int N, int K, int32_t* P, void* stream) {
    if (!P) return COMET_ERR_NULL;
    const int st = qoq_check(Xq, x_scale, Wu_packed, s2z, s1_fp16, M, N, K);
    if (st != COMET_OK) return st;
    if (!aligned16(P)) return COMET_ERR_ALIGN;
    return hip_status(comet::launch_qoq_gemm(static_cast<const uint8_t*>(Xq), x_scale,
                                             static_cast<const uint8_t*>(Wu_packed), s2z, s1_fp16, M, N, K,
                                             nullptr, N, P, stream));
}

namespace {

bool kv4_dim_ok(int d) { return d >= 8 && d <= 512 && (d & (d - 1)) == 0; }

}  // namespace

int comet_kv4_quantize(const void* X_fp16, int ntok, int H, int d, int ldx, int pos, int tcap, void* codes,
                       uint16_t* step_fp16, uint8_t* zero, void* stream) {
    if (!X_fp16 || !codes || !step_fp16 || !zero) return COMET_ERR_NULL;
    if (ntok < 1 || H < 1 || d < 1 || pos < 0 || tcap < 1 || static_cast<int64_t>(ldx) < static_cast<int64_t>(H) * d)
        return COMET_ERR_SHAPE;
    if (static_cast<int64_t>(pos) + ntok > tcap) return COMET_ERR_SHAPE;
    if (!kv4_dim_ok(d)) return COMET_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(ntok) * H > std::numeric_limits<int32_t>::max() - 256) return COMET_ERR_UNSUPPORTED;
    if (!aligned16(X_fp16) || ldx % 8 != 0 || !aligned16(codes) || !aligned16(step_fp16) || !aligned16(zero))
        return COMET_ERR_ALIGN;
    return hip_status(comet::launch_kv4_quantize(static_cast<const uint16_t*>(X_fp16), ntok, H, d, ldx, pos, tcap,
                                                 static_cast<uint8_t*>(codes), step_fp16, zero, stream));
}

size_t comet_kv4_attention_workspace_bytes(int Hq, int d, int T) {
    if (Hq < 1 || T < 1 || !kv4_dim_ok(d)) return 0;
    return comet::kv4_workspace_bytes(Hq, d, T);
}

namespace {

int kv4_attention_impl(const void* q_fp16, const void* k_codes, const uint16_t* k_step, const uint8_t* k_zero,
                       const void* v_codes, const uint16_t* v_step, const uint8_t* v_zero, int Hq, int group, int d,
                       int T, int tcap, void* out_fp16, void* workspace, size_t workspace_bytes, void* stream,
                       const int32_t* T_kv) {
    if (!q_fp16 || !k_codes || !k_step || !k_zero || !v_codes || !v_step || !v_zero || !out_fp16 || !workspace)
        return COMET_ERR_NULL;
    if (Hq < 1 || group < 1 || Hq % group != 0 || d < 1 || T < 1 || tcap < T) return COMET_ERR_SHAPE;
    if (!kv4_dim_ok(d)) return COMET_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(Hq) * comet::kv4_splits(T) > std::numeric_limits<int32_t>::max()) return COMET_ERR_UNSUPPORTED;
    if (workspace_bytes < comet::kv4_workspace_bytes(Hq, d, T)) return COMET_ERR_WORKSPACE;
    if (!aligned16(q_fp16) || !aligned16(k_codes) || !aligned16(k_step) || !aligned16(k_zero) ||
        !aligned16(v_codes) || !aligned16(v_step) || !aligned16(v_zero) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(out_fp16) & 1u) != 0 || (reinterpret_cast<uintptr_t>(T_kv) & 3u) != 0)
        return COMET_ERR_ALIGN;
    return hip_status(comet::launch_kv4_attention(
        static_cast<const uint16_t*>(q_fp16), static_cast<const uint8_t*>(k_codes), k_step, k_zero,
        static_cast<const uint8_t*>(v_codes), v_step, v_zero, Hq, group, d, T, tcap,
        static_cast<uint16_t*>(out_fp16), static_cast<float*>(workspace), stream, T_kv));
}

}  // namespace

int comet_kv4_attention(const void* q_fp16, const void* k_codes, const uint16_t* k_step, const uint8_t* k_zero,
                        const void* v_codes, const uint16_t* v_step, const uint8_t* v_zero, int Hq, int group, int d,
                        int T, int tcap, void* out_fp16, void* workspace, size_t workspace_bytes, void* stream) {
    return kv4_attention_impl(q_fp16, k_codes, k_step, k_zero, v_codes, v_step, v_zero, Hq, group, d, T, tcap,
                              out_fp16, workspace, workspace_bytes, stream, nullptr);
}

int comet_kv4_attention_varlen(const void* q_fp16, const void* k_codes, const uint16_t* k_step,
                               const uint8_t* k_zero, const void* v_codes, const uint16_t* v_step,
                               const uint8_t* v_zero, int Hq, int group, int d, const int32_t* T_kv, int T_max,
                               int tcap, void* out_fp16, void* workspace, size_t workspace_bytes, void* stream) {
    if (!T_kv) return COMET_ERR_NULL;
    return kv4_attention_impl(q_fp16, k_codes, k_step, k_zero, v_codes, v_step, v_zero, Hq, group, d, T_max, tcap,
                              out_fp16, workspace, workspace_bytes, stream, T_kv);
}

size_t comet_x_zero_bytes(int M, int K) {
    if (M < 1 || K < kBlock || K % kBlock != 0) return 0;
    return static_cast<size_t>(K / kBlock) * ((static_cast<size_t>(M) + 15u) & ~static_cast<size_t>(15));
}

namespace {

int gemm_impl(const void* Xq, const float* x_scale, const uint8_t* x_zero, const void* Wq_packed,
              const uint16_t* w_scale_fp16, const int16_t* w_sum, int n_int8_blocks, int M, int N, int K,
              void* Y_fp16, int ldy, void* workspace, size_t workspace_bytes, void* stream) {
    if (!Xq || !x_scale || !Wq_packed || !w_scale_fp16 || !w_sum || !Y_fp16) return COMET_ERR_NULL;
    int st = check_online_shape(M, N, K, n_int8_blocks);
    if (st != COMET_OK) return st;
    if (ldy < N) return COMET_ERR_SHAPE;
    if (static_cast<int64_t>(M) * ldy > std::numeric_limits<int32_t>::max())
        return COMET_ERR_UNSUPPORTED;
    if (!aligned16(Xq) || !aligned16(x_scale) || !aligned16(Wq_packed) || !aligned16(w_scale_fp16) ||
        !aligned16(w_sum) || !aligned16(Y_fp16))
        return COMET_ERR_ALIGN;
    const size_t need = comet::gemm_workspace_bytes(M, N, K, n_int8_blocks);
    if (need > 0) {
        if (!workspace) return COMET_ERR_NULL;
        if (workspace_bytes < need) return COMET_ERR_WORKSPACE;
        if (!aligned16(workspace)) return COMET_ERR_ALIGN;
    }
    comet::GemmProblem p{};
    p.Xq = static_cast<const uint8_t*>(Xq);
    p.x_scale = x_scale;
    p.x_zero = x_zero;
    p.Wq = static_cast<const uint8_t*>(Wq_packed);
    p.w_scale = w_scale_fp16;
    p.w_sum = w_sum;
    p.M = M;
    p.N = N;
    p.K = K;
    p.nb = K / kBlock;
    p.nb4 = p.nb - n_int8_blocks;
    p.Y = static_cast<uint16_t*>(Y_fp16);
    p.ldy = ldy;
    p.P = nullptr;
    p.m_begin = 0;
    p.m_count = M;
    p.workspace = workspace;
    p.workspace_bytes = workspace_bytes;
    return hip_status(comet::launch_w4ax_gemm(p, stream));
}

int partials_impl(const void* Xq, const float* x_scale, const uint8_t* x_zero, const void* Wq_packed,
                  const uint16_t* w_scale_fp16, const int16_t* w_sum, int n_int8_blocks, int M, int N, int K,
                  int m_begin, int m_count, int32_t* P, void* stream) {
    if (!Xq || !x_scale || !Wq_packed || !w_scale_fp16 || !w_sum || !P) return COMET_ERR_NULL;
    int st = check_online_shape(M, N, K, n_int8_blocks);
    if (st != COMET_OK) return st;
    if (m_begin < 0 || m_count < 1 || m_begin > M - m_count) return COMET_ERR_SHAPE;
    if (static_cast<int64_t>(m_count) * N * (K / kBlock) > std::numeric_limits<int32_t>::max())
        return COMET_ERR_UNSUPPORTED;
    if (!aligned16(Xq) || !aligned16(x_scale) || !aligned16(Wq_packed) || !aligned16(w_scale_fp16) ||
        !aligned16(w_sum) || !aligned16(P))
        return COMET_ERR_ALIGN;
    comet::GemmProblem p{};
    p.Xq = static_cast<const uint8_t*>(Xq);
    p.x_scale = x_scale;
    p.x_zero = x_zero;
    p.Wq = static_cast<const uint8_t*>(Wq_packed);
    p.w_scale = w_scale_fp16;
    p.w_sum = w_sum;
    p.M = M;
    p.N = N;
    p.K = K;
    p.nb = K / kBlock;
    p.nb4 = p.nb - n_int8_blocks;
    p.Y = nullptr;
    p.ldy = N;
    p.P = P;
    p.m_begin = m_begin;
    p.m_count = m_count;
    return hip_status(comet::launch_w4ax_gemm(p, stream));
}

}  // namespace

int comet_w4ax_gemm(const void* Xq, const float* x_scale, const void* Wq_packed,
                     const uint16_t* w_scale_fp16, const int16_t* w_sum, int n_int8_blocks,
                     int M, int N, int K, void* Y_fp16, int ldy, void* workspace,
                     size_t workspace_bytes, void* stream) {
    return gemm_impl(Xq, x_scale, nullptr, Wq_packed, w_scale_fp16, w_sum, n_int8_blocks, M, N, K, Y_fp16, ldy,
                     workspace, workspace_bytes, stream);
}

int comet_w4ax_gemm_partials(const void* Xq, const float* x_scale, const void* Wq_packed,
                             const uint16_t* w_scale_fp16, const int16_t* w_sum,
                             int n_int8_blocks, int M, int N, int K, int m_begin, int m_count,
                             int32_t* P, void* stream) {
    return partials_impl(Xq, x_scale, nullptr, Wq_packed, w_scale_fp16, w_sum, n_int8_blocks, M, N, K, m_begin,
                         m_count, P, stream);
}

int comet_w4ax_gemm_asym(const void* Xq, const float* x_scale, const uint8_t* x_zero, const void* Wq_packed,
                         const uint16_t* w_scale_fp16, const int16_t* w_sum, int n_int8_blocks, int M, int N,
                         int K, void* Y_fp16, int ldy, void* workspace, size_t workspace_bytes, void* stream) {
    if (!x_zero) return COMET_ERR_NULL;
    if (!aligned16(x_zero)) return COMET_ERR_ALIGN;
    return gemm_impl(Xq, x_scale, x_zero, Wq_packed, w_scale_fp16, w_sum, n_int8_blocks, M, N, K, Y_fp16, ldy,
                     workspace, workspace_bytes, stream);
}

int comet_w4ax_gemm_asym_partials(const void* Xq, const float* x_scale, const uint8_t* x_zero,
                                  const void* Wq_packed, const uint16_t* w_scale_fp16, const int16_t* w_sum,
                                  int n_int8_blocks, int M, int N, int K, int m_begin, int m_count, int32_t* P,
                                  void* stream) {
    if (!x_zero) return COMET_ERR_NULL;
    if (!aligned16(x_zero)) return COMET_ERR_ALIGN;
    return partials_impl(Xq, x_scale, x_zero, Wq_packed, w_scale_fp16, w_sum, n_int8_blocks, M, N, K, m_begin,
                         m_count, P, stream);
}

size_t comet_xq_fp6_bytes(int M, int K, int n_int8_blocks) {
    if (M < 1 || K < kBlock || K % kBlock != 0 || n_int8_blocks < 0 || n_int8_blocks > K / kBlock) return 0;
    return comet::xq_fp6_bytes(M, K / kBlock - n_int8_blocks, n_int8_blocks);
}

size_t comet_wq_fp6_bytes(int N, int K, int n_int8_blocks) {
    if (N < 1 || K < kBlock || K % kBlock != 0 || n_int8_blocks < 0 || n_int8_blocks > K / kBlock) return 0;
    return comet::wq_fp6_bytes(N, K / kBlock - n_int8_blocks, n_int8_blocks);
}

int comet_repack_weights_fp6(const uint8_t* Wq_packed, int N, int K, int n_int8_blocks, uint8_t* Wq_fp6) {
    if (!Wq_packed || !Wq_fp6) return COMET_ERR_NULL;
    if (N < 1 || K < kBlock || K % kBlock != 0) return COMET_ERR_SHAPE;
    if (n_int8_blocks < 0 || n_int8_blocks > K / kBlock) return COMET_ERR_ARG;
    if (N % 128 != 0) return COMET_ERR_UNSUPPORTED;
    comet::repack_fp6(Wq_packed, N, K, n_int8_blocks, Wq_fp6);
    return COMET_OK;
}

int comet_quant_act_fp6(const void* X_fp16, int M, int K, int ldx, const int32_t* perm,
                        int n_int8_blocks, void* Xq_fp6, float* x_scale, void* stream) {
    if (!X_fp16 || !perm || !Xq_fp6 || !x_scale) return COMET_ERR_NULL;
    if (M < 1 || K < kBlock || K % kBlock != 0 || ldx < K) return COMET_ERR_SHAPE;
    if (n_int8_blocks < 0 || n_int8_blocks > K / kBlock) return COMET_ERR_ARG;
    if (!aligned16(X_fp16) || !aligned16(perm) || !aligned16(Xq_fp6) || !aligned16(x_scale))
        return COMET_ERR_ALIGN;
    return hip_status(comet::launch_quant_act_fp6(static_cast<const uint16_t*>(X_fp16), M, K, ldx, perm,
                                                  n_int8_blocks, static_cast<uint8_t*>(Xq_fp6), x_scale,
                                                  stream));
}

int comet_rmsnorm_quant_act(const void* X_fp16, int M, int K, int ldx, const void* gamma_perm_fp16, float eps,
                            const int32_t* perm, int n_int8_blocks, void* Xq, float* x_scale, void* stream) {
    const int st = check_rmsnorm_quant(X_fp16, M, K, ldx, gamma_perm_fp16, eps, perm, n_int8_blocks, Xq, x_scale);
    if (st != COMET_OK) return st;
    return hip_status(comet::launch_rmsnorm_quant_act(static_cast<const uint16_t*>(X_fp16), M, K, ldx,
                                                      static_cast<const uint16_t*>(gamma_perm_fp16), eps, perm,
                                                      n_int8_blocks, static_cast<uint8_t*>(Xq), x_scale, false,
                                                      stream));
}

int comet_rmsnorm_quant_act_fp6(const void* X_fp16, int M, int K, int ldx, const void* gamma_perm_fp16, float eps,
                                const int32_t* perm, int n_int8_blocks, void* Xq_fp6, float* x_scale,
                                void* stream) {
    const int st =
        check_rmsnorm_quant(X_fp16, M, K, ldx, gamma_perm_fp16, eps, perm, n_int8_blocks, Xq_fp6, x_scale);
    if (st != COMET_OK) return st;
    return hip_status(comet::launch_rmsnorm_quant_act(static_cast<const uint16_t*>(X_fp16), M, K, ldx,
                                                      static_cast<const uint16_t*>(gamma_perm_fp16), eps, perm,
                                                      n_int8_blocks, static_cast<uint8_t*>(Xq_fp6), x_scale, true,
                                                      stream));
}

int comet_rmsnorm(const void* X_fp16, int M, int K, int ldx, const void* gamma_fp16, float eps, void* Xn_fp16,
                  int ldn, void* stream) {
    if (!X_fp16 || !gamma_fp16 || !Xn_fp16) return COMET_ERR_NULL;
    if (M < 1 || K < 1 || ldx < K || ldn < K) return COMET_ERR_SHAPE;
    if (!(eps > 0.0f) || !(eps <= std::numeric_limits<float>::max())) return COMET_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(X_fp16) | reinterpret_cast<uintptr_t>(gamma_fp16) |
         reinterpret_cast<uintptr_t>(Xn_fp16)) & 1u)
        return COMET_ERR_ALIGN;
    return hip_status(comet::launch_rmsnorm(static_cast<const uint16_t*>(X_fp16), M, K, ldx,
                                            static_cast<const uint16_t*>(gamma_fp16), eps,
                                            static_cast<uint16_t*>(Xn_fp16), ldn, stream));
}

int comet_swiglu_quant_act(const void* gate_fp16, const void* up_fp16, int M, int K, int ldx, const int32_t* perm,
                           int n_int8_blocks, void* Xq, float* x_scale, void* stream) {
    const int st = check_swiglu_quant(gate_fp16, up_fp16, M, K, ldx, perm, n_int8_blocks, Xq, x_scale);
    if (st != COMET_OK) return st;
    return hip_status(comet::launch_swiglu_quant_act(static_cast<const uint16_t*>(gate_fp16),
                                                     static_cast<const uint16_t*>(up_fp16), M, K, ldx, perm,
                                                     n_int8_blocks, static_cast<uint8_t*>(Xq), x_scale, false,
                                                     stream));
}

int comet_swiglu_quant_act_fp6(const void* gate_fp16, const void* up_fp16, int M, int K, int ldx,
                               const int32_t* perm, int n_int8_blocks, void* Xq_fp6, float* x_scale,
                               void* stream) {
    const int st = check_swiglu_quant(gate_fp16, up_fp16, M, K, ldx, perm, n_int8_blocks, Xq_fp6, x_scale);
    if (st != COMET_OK) return st;
    return hip_status(comet::launch_swiglu_quant_act(static_cast<const uint16_t*>(gate_fp16),
                                                     static_cast<const uint16_t*>(up_fp16), M, K, ldx, perm,
                                                     n_int8_blocks, static_cast<uint8_t*>(Xq_fp6), x_scale, true,
                                                     stream));
}

int comet_swiglu(const void* gate_fp16, const void* up_fp16, int M, int K, int ldx, void* H_fp16, int ldh,
                 void* stream) {
    if (!gate_fp16 || !up_fp16 || !H_fp16) return COMET_ERR_NULL;
    if (M < 1 || K < 1 || ldx < K || ldh < K) return COMET_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(gate_fp16) | reinterpret_cast<uintptr_t>(up_fp16) |
         reinterpret_cast<uintptr_t>(H_fp16)) & 1u)
        return COMET_ERR_ALIGN;
    return hip_status(comet::launch_swiglu(static_cast<const uint16_t*>(gate_fp16),
                                           static_cast<const uint16_t*>(up_fp16), M, K, ldx,
                                           static_cast<uint16_t*>(H_fp16), ldh, stream));
}

int comet_permute_channels(const uint16_t* v, const int32_t* perm, int K, uint16_t* out) {
    if (!v || !perm || !out) return COMET_ERR_NULL;
    if (K < 1) return COMET_ERR_SHAPE;
    for (int k = 0; k < K; ++k)
        if (perm[k] < 0 || perm[k] >= K) return COMET_ERR_ARG;
    for (int k = 0; k < K; ++k) out[k] = v[perm[k]];
    return COMET_OK;
}

size_t comet_w4ax_gemm_fp6_workspace_bytes(int M, int N, int K, int n_int8_blocks) {
    if (check_online_shape(M, N, K, n_int8_blocks) != COMET_OK) return 0;
    return comet::gemm_fp6_workspace_bytes(M, N, K, n_int8_blocks);
}

namespace {

// Checks shared by the FP6 GEMM and its partials variant (workspace included).
int check_fp6_gemm(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6, const uint16_t* w_scale_fp16,
                   int n_int8_blocks, int M, int N, int K, void* workspace, size_t workspace_bytes) {
    if (!Xq_fp6 || !x_scale || !Wq_fp6 || !w_scale_fp16) return COMET_ERR_NULL;
    int st = check_online_shape(M, N, K, n_int8_blocks);
    if (st != COMET_OK) return st;
    if (!fp6_offsets_fit(M, K)) return COMET_ERR_UNSUPPORTED;
    const size_t need = comet::gemm_fp6_workspace_bytes(M, N, K, n_int8_blocks);
    if (need > 0) {
        if (!workspace) return COMET_ERR_NULL;
        if (workspace_bytes < need) return COMET_ERR_WORKSPACE;
        if (!aligned16(workspace)) return COMET_ERR_ALIGN;
    }
    if (!aligned16(Xq_fp6) || !aligned16(x_scale) || !aligned16(Wq_fp6) || !aligned16(w_scale_fp16))
        return COMET_ERR_ALIGN;
    return COMET_OK;
}

comet::GemmProblem fp6_problem(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                               const uint16_t* w_scale_fp16, int n_int8_blocks, int M, int N, int K,
                               void* workspace, size_t workspace_bytes) {
    comet::GemmProblem p{};
    p.Xq = static_cast<const uint8_t*>(Xq_fp6);
    p.x_scale = x_scale;
    p.Wq = static_cast<const uint8_t*>(Wq_fp6);
    p.w_scale = w_scale_fp16;
    p.w_sum = nullptr;
    p.M = M;
    p.N = N;
    p.K = K;
    p.nb = K / kBlock;
    p.nb4 = p.nb - n_int8_blocks;
    p.workspace = workspace;
    p.workspace_bytes = workspace_bytes;
    return p;
}

}  // namespace

int comet_w4ax_gemm_fp6(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                        const uint16_t* w_scale_fp16, int n_int8_blocks, int M, int N, int K,
                        void* Y_fp16, int ldy, void* workspace, size_t workspace_bytes, void* stream) {
    if (!Y_fp16) return COMET_ERR_NULL;
    int st = check_fp6_gemm(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, K, workspace,
                            workspace_bytes);
    if (st != COMET_OK) return st;
    if (ldy < N) return COMET_ERR_SHAPE;
    if (static_cast<int64_t>(M) * ldy > std::numeric_limits<int32_t>::max())
        return COMET_ERR_UNSUPPORTED;
    if (!aligned16(Y_fp16)) return COMET_ERR_ALIGN;
    comet::GemmProblem p =
        fp6_problem(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, K, workspace, workspace_bytes);
    p.Y = static_cast<uint16_t*>(Y_fp16);
    p.ldy = ldy;
    p.P = nullptr;
    p.m_begin = 0;
    p.m_count = M;
    return hip_status(comet::launch_w4ax_gemm_fp6(p, stream));
}

int comet_w4ax_gemm_fp6_noalloc(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                                const uint16_t* w_scale_fp16, int n_int8_blocks, int M, int N, int K,
                                void* Y_fp16, int ldy, void* stream) {
    if (!Y_fp16) return COMET_ERR_NULL;
    // the fixed scratch array stands in for the workspace (16-byte aligned)
    static uint8_t* const kScratchStandIn = reinterpret_cast<uint8_t*>(static_cast<uintptr_t>(256));
    int st = check_fp6_gemm(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, K, kScratchStandIn,
                            COMET_NOALLOC_SCRATCH_BYTES);
    if (st != COMET_OK) return st;
    if (ldy < N) return COMET_ERR_SHAPE;
    if (static_cast<int64_t>(M) * ldy > std::numeric_limits<int32_t>::max())
        return COMET_ERR_UNSUPPORTED;
    if (!aligned16(Y_fp16)) return COMET_ERR_ALIGN;
    comet::GemmProblem p =
        fp6_problem(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, K, nullptr, 0);
    p.Y = static_cast<uint16_t*>(Y_fp16);
    p.ldy = ldy;
    p.P = nullptr;
    p.m_begin = 0;
    p.m_count = M;
    return hip_status(comet::launch_w4ax_gemm_fp6_noalloc(p, stream));
}

int comet_w4ax_gemm_fp6_partials(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                                 const uint16_t* w_scale_fp16, int n_int8_blocks, int M, int N, int K,
                                 int m_begin, int m_count, int32_t* P, int max_workgroups, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    if (!P) return COMET_ERR_NULL;
    int st = check_fp6_gemm(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, K, workspace,
                            workspace_bytes);
    if (st != COMET_OK) return st;
    if (m_begin < 0 || m_count < 1 || m_begin > M - m_count) return COMET_ERR_SHAPE;
    if (max_workgroups < 0) return COMET_ERR_ARG;
    if (static_cast<int64_t>(m_count) * N * (K / kBlock) > std::numeric_limits<int32_t>::max())
        return COMET_ERR_UNSUPPORTED;
    if (!aligned16(P)) return COMET_ERR_ALIGN;
    comet::GemmProblem p =
        fp6_problem(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, K, workspace, workspace_bytes);
    p.max_wg = max_workgroups;
    p.Y = nullptr;
    p.ldy = N;
    p.P = P;
    p.m_begin = m_begin;
    p.m_count = m_count;
    return hip_status(comet::launch_w4ax_gemm_fp6(p, stream));
}

// QUIK's fp16 outlier channels: n_fp16 a multiple of 128 leaving at least one
// quantized block, nb8 within the quantized blocks.
static bool quik_split_ok(int K, int n_fp16, int n_int8_blocks) {
    return n_fp16 >= 0 && n_fp16 % kBlock == 0 && n_fp16 <= K - kBlock && n_int8_blocks >= 0 &&
           n_int8_blocks <= (K - n_fp16) / kBlock;
}

int comet_pack_weights_quik(const uint16_t* W_fp16, int N, int K, const float* chan_score, int n_fp16,
                            int32_t* perm, uint8_t* Wq_packed, uint16_t* w_scale_fp16, int16_t* w_sum,
                            uint16_t* Wf_fp16) {
    if (!W_fp16 || !chan_score || !perm || !Wq_packed || !w_scale_fp16 || !w_sum || (n_fp16 > 0 && !Wf_fp16))
        return COMET_ERR_NULL;
    if (N < 1 || K < kBlock || K % kBlock != 0) return COMET_ERR_SHAPE;
    if (!quik_split_ok(K, n_fp16, 0)) return COMET_ERR_ARG;
    if (N % 128 != 0) return COMET_ERR_UNSUPPORTED;
    return comet::pack_weights_quik(W_fp16, N, K, chan_score, n_fp16, perm, Wq_packed, w_scale_fp16, w_sum,
                                    Wf_fp16);
}

size_t comet_xf_bytes(int M, int n_fp16) {
    if (M < 1 || n_fp16 < 0 || n_fp16 % kBlock != 0) return 0;
    return comet::xf_bytes(M, n_fp16);
}

int comet_quant_act_quik_fp6(const void* X_fp16, int M, int K, int ldx, const int32_t* perm, int n_int8_blocks,
                             int n_fp16, void* Xq_fp6, float* x_scale, void* Xf_fp16, void* stream) {
    if (!X_fp16 || !perm || !Xq_fp6 || !x_scale || (n_fp16 > 0 && !Xf_fp16)) return COMET_ERR_NULL;
    if (M < 1 || K < kBlock || K % kBlock != 0 || ldx < K) return COMET_ERR_SHAPE;
    if (!quik_split_ok(K, n_fp16, n_int8_blocks)) return COMET_ERR_ARG;
    if (!aligned16(X_fp16) || !aligned16(perm) || !aligned16(Xq_fp6) || !aligned16(x_scale) ||
        (n_fp16 > 0 && !aligned16(Xf_fp16)))
        return COMET_ERR_ALIGN;
    const int Kq = K - n_fp16;
    int e = comet::launch_quant_act_fp6(static_cast<const uint16_t*>(X_fp16), M, K, ldx, perm, n_int8_blocks,
                                        static_cast<uint8_t*>(Xq_fp6), x_scale, stream, Kq);
    if (e != 0 || n_fp16 == 0) return hip_status(e);
    return hip_status(comet::launch_gather_outliers(static_cast<const uint16_t*>(X_fp16), M, K, ldx, perm + Kq,
                                                    n_fp16, static_cast<uint16_t*>(Xf_fp16), stream));
}

int comet_w4ax_gemm_quik_fp6(const void* Xq_fp6, const float* x_scale, const void* Wq_fp6,
                             const uint16_t* w_scale_fp16, int n_int8_blocks, const void* Xf_fp16,
                             const void* Wf_fp16, int n_fp16, int M, int N, int K, void* Y_fp16, int ldy,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!Y_fp16 || (n_fp16 > 0 && (!Xf_fp16 || !Wf_fp16))) return COMET_ERR_NULL;
    if (K < kBlock || K % kBlock != 0) return COMET_ERR_SHAPE;
    if (!quik_split_ok(K, n_fp16, n_int8_blocks)) return COMET_ERR_ARG;
    const int Kq = K - n_fp16;
    int st = check_fp6_gemm(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, Kq, workspace,
                            workspace_bytes);
    if (st != COMET_OK) return st;
    if (ldy < N) return COMET_ERR_SHAPE;
    if (static_cast<int64_t>(M) * ldy > std::numeric_limits<int32_t>::max()) return COMET_ERR_UNSUPPORTED;
    // the fp16 operands are read through 32-bit buffer offsets
    if (comet::xf_bytes(M, n_fp16) >= (1ull << 31) ||
        static_cast<uint64_t>(N) * static_cast<uint64_t>(n_fp16) * 2u >= (1ull << 31))
        return COMET_ERR_UNSUPPORTED;
    if (!aligned16(Y_fp16) || (n_fp16 > 0 && (!aligned16(Xf_fp16) || !aligned16(Wf_fp16))))
        return COMET_ERR_ALIGN;
    comet::GemmProblem p =
        fp6_problem(Xq_fp6, x_scale, Wq_fp6, w_scale_fp16, n_int8_blocks, M, N, Kq, workspace, workspace_bytes);
    p.Y = static_cast<uint16_t*>(Y_fp16);
    p.ldy = ldy;
    p.P = nullptr;
    p.m_begin = 0;
    p.m_count = M;
    p.xf = static_cast<const uint16_t*>(Xf_fp16);
    p.wf = static_cast<const uint16_t*>(Wf_fp16);
    p.nf = n_fp16;
    return hip_status(comet::launch_w4ax_gemm_fp6(p, stream));
}

const char* comet_status_string(int status) {
    switch (status) {
        case COMET_OK: return "ok";
        case COMET_ERR_NULL: return "a required pointer is NULL";
        case COMET_ERR_SHAPE: return "invalid shape or leading dimension";
        case COMET_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case COMET_ERR_ARG: return "invalid argument (n_int8_blocks range or non-finite input)";
        case COMET_ERR_WORKSPACE: return "workspace too small";
        case COMET_ERR_HIP: return "HIP launch or query failed";
        case COMET_ERR_UNSUPPORTED: return "unsupported shape (N % 128 != 0 or size beyond 32-bit indexing)";
        default: return "unknown status";
    }
}

const char* comet_version(void) { return "comet-w4ax-gfx950 0.1"; }

}  // extern "C"
