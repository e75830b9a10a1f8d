// Host-side check under AddressSanitizer and UndefinedBehaviorSanitizer: runs
// every oracle step and the library's host packers on small seeded layers
// (including one-block rows, all-4-bit and all-8-bit block sets, ragged row
// counts) and compares the packers' perm, scales and sums with the oracle's.
// Built and run by tests/test_sanitizers.py; exits non-zero on a mismatch,
// and the sanitizers abort on any invalid access or undefined operation.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../../w4ax_mixed_precision_amd/csrc/comet_internal.h"
#include "../../w4ax_mixed_precision_amd/csrc/qoq_internal.h"

extern "C" {
uint16_t orc_float_to_half(float f);
float orc_half_to_float(uint16_t h);
int orc_channel_order(int K, const float* score, int nb8, int32_t* perm, uint8_t* is_int8);
int orc_quantize_weights(const uint16_t* W, int N, int K, const int32_t* perm, int8_t* qw, uint16_t* sw16,
                         int32_t* wsum);
int orc_quantize_activations(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, const uint8_t* is_int8,
                             int8_t* qa, float* sa);
int orc_quantize_activations_asym(const uint16_t* X, int M, int K, int ldx, const int32_t* perm,
                                  const uint8_t* is_int8, int8_t* qa, uint8_t* u4, float* sa, uint8_t* za);
int orc_block_partials_zero_point(const int8_t* qa, const uint8_t* u4, const uint8_t* za, const int8_t* qw,
                                  const int32_t* wsum, const uint8_t* is_int8, int M, int N, int K, int m0, int m1,
                                  int32_t* P);
int orc_block_partials(const int8_t* qa, const int8_t* qw, int M, int N, int K, int m0, int m1, int32_t* P);
int orc_block_partials_zero_extend(const int8_t* qa, const int8_t* qw, const int32_t* wsum, const uint8_t* is_int8,
                                   int M, int N, int K, int m0, int m1, int32_t* P);
int orc_epilogue(const int32_t* P, const float* sa, const uint16_t* sw16, int rows, int N, int nb, float* y32,
                 uint16_t* Y16, double* yexact);
double orc_rms_sumsq(const uint16_t* x, int K);
int orc_rmsnorm_rows(const uint16_t* X, int M, int K, int ldx, const uint16_t* gamma, float eps, uint16_t* Xn,
                     int ldn);
int orc_swiglu_rows(const uint16_t* G, const uint16_t* U, int M, int K, int ldx, uint16_t* H, int ldh);
int orc_forward_rows(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, const uint8_t* is_int8,
                     const int8_t* qw, const uint16_t* sw16, int N, int m0, int m1, uint16_t* Y16, double* yexact);
int orc_qoq_quantize_weights(const uint16_t* W, int N, int K, const int32_t* perm, uint16_t* s1, int8_t* w8,
                             uint8_t* s2, uint8_t* z, uint8_t* u);
int orc_qoq_quantize_activations(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int8_t* qa,
                                 float* sa);
int orc_qoq_gemm(const int8_t* qa, const float* sa, const uint8_t* u, const uint8_t* s2, const uint8_t* z,
                 const uint16_t* s1, int M, int N, int K, int m0, int m1, int32_t* P, float* y32, uint16_t* Y16,
                 double* yexact);
int orc_kv4_quantize(const uint16_t* V, int n, int d, uint8_t* u, uint16_t* s16, uint8_t* z);
int orc_kv4_attention(const uint16_t* q, const uint8_t* uk, const uint16_t* sk, const uint8_t* zk, const uint8_t* uv,
                      const uint16_t* sv, const uint8_t* zv, int H, int T, int d, double* out);
}

namespace {

int failures = 0;

void expect(bool ok, const char* what, int M, int N, int K, int nb8) {
    if (!ok) {
        std::printf("MISMATCH %s (M=%d N=%d K=%d nb8=%d)\n", what, M, N, K, nb8);
        ++failures;
    }
}

std::vector<uint16_t> halves(std::mt19937& g, size_t n, float scale) {
    std::normal_distribution<float> d(0.0f, scale);
    std::vector<uint16_t> v(n);
    for (auto& x : v) x = orc_float_to_half(d(g));
    return v;
}

void layer(int M, int N, int K, int nb8, unsigned seed) {
    std::mt19937 g(seed);
    const int nb = K / 128;
    auto X = halves(g, static_cast<size_t>(M) * K, 1.0f);
    auto W = halves(g, static_cast<size_t>(N) * K, 0.02f);
    std::vector<float> score(K);
    std::uniform_real_distribution<float> u01(0.0f, 1.0f);
    for (auto& s : score) s = u01(g);
    for (int i = 0; i < K / 10; ++i) X[static_cast<size_t>(g() % M) * K + g() % K] = orc_float_to_half(60.0f);

    std::vector<int32_t> perm(K), lperm(K);
    std::vector<uint8_t> flags(nb), lflags(nb);
    orc_channel_order(K, score.data(), nb8, perm.data(), flags.data());
    std::vector<int8_t> qw(static_cast<size_t>(N) * K);
    std::vector<uint16_t> sw16(static_cast<size_t>(N) * nb);
    std::vector<int32_t> wsum(static_cast<size_t>(N) * nb);
    orc_quantize_weights(W.data(), N, K, perm.data(), qw.data(), sw16.data(), wsum.data());
    std::vector<int8_t> qa(static_cast<size_t>(M) * K);
    std::vector<float> sa(static_cast<size_t>(M) * nb);
    orc_quantize_activations(X.data(), M, K, K, perm.data(), flags.data(), qa.data(), sa.data());
    std::vector<int8_t> qa2(static_cast<size_t>(M) * K);
    std::vector<uint8_t> u4(static_cast<size_t>(M) * K), za(static_cast<size_t>(M) * nb);
    std::vector<float> sa2(static_cast<size_t>(M) * nb);
    orc_quantize_activations_asym(X.data(), M, K, K, perm.data(), flags.data(), qa2.data(), u4.data(), sa2.data(),
                                  za.data());
    std::vector<int32_t> P(static_cast<size_t>(M) * N * nb), P2(P.size()), P3(P.size());
    orc_block_partials(qa.data(), qw.data(), M, N, K, 0, M, P.data());
    orc_block_partials_zero_extend(qa.data(), qw.data(), wsum.data(), flags.data(), M, N, K, 0, M, P2.data());
    orc_block_partials_zero_point(qa2.data(), u4.data(), za.data(), qw.data(), wsum.data(), flags.data(), M, N, K,
                                  0, M, P3.data());
    expect(P == P2, "zero-extended partials", M, N, K, nb8);
    std::vector<float> y32(static_cast<size_t>(M) * N);
    std::vector<uint16_t> Y16(static_cast<size_t>(M) * N), Y16b(Y16.size());
    std::vector<double> ye(static_cast<size_t>(M) * N), ye2(ye.size());
    orc_epilogue(P.data(), sa.data(), sw16.data(), M, N, nb, y32.data(), Y16.data(), ye.data());
    orc_forward_rows(X.data(), M, K, K, perm.data(), flags.data(), qw.data(), sw16.data(), N, 0, M, Y16b.data(),
                     ye2.data());
    expect(Y16 == Y16b, "forward rows", M, N, K, nb8);

    std::vector<uint16_t> gamma = halves(g, K, 1.0f), Xn(static_cast<size_t>(M) * K), H(Xn.size());
    orc_rmsnorm_rows(X.data(), M, K, K, gamma.data(), 1e-5f, Xn.data(), K);
    (void)orc_rms_sumsq(X.data(), K);
    orc_swiglu_rows(X.data(), Xn.data(), M, K, K, H.data(), K);

    // QoQ: oracle and the library's packer
    std::vector<uint16_t> s1(N), ls1(N), ls2z(static_cast<size_t>(N) * nb);
    std::vector<int8_t> w8(static_cast<size_t>(N) * K);
    std::vector<uint8_t> s2(static_cast<size_t>(N) * nb), z(static_cast<size_t>(N) * nb), uq(static_cast<size_t>(N) * K);
    orc_qoq_quantize_weights(W.data(), N, K, perm.data(), s1.data(), w8.data(), s2.data(), z.data(), uq.data());
    std::vector<int8_t> qa8(static_cast<size_t>(M) * K);
    std::vector<float> sa8(M);
    orc_qoq_quantize_activations(X.data(), M, K, K, perm.data(), qa8.data(), sa8.data());
    std::vector<int32_t> Pq(static_cast<size_t>(M) * N);
    orc_qoq_gemm(qa8.data(), sa8.data(), uq.data(), s2.data(), z.data(), s1.data(), M, N, K, 0, M, Pq.data(),
                 y32.data(), Y16.data(), ye.data());
    std::vector<uint8_t> Wu(static_cast<size_t>(N) * K / 2);
    comet::pack_weights_qoq(W.data(), N, K, score.data(), lperm.data(), Wu.data(), ls1.data(), ls2z.data());
    expect(lperm == perm && ls1 == s1, "QoQ pack", M, N, K, nb8);

    // the library's INT4 packer and FP6 repack
    std::vector<uint8_t> Wq(static_cast<size_t>(N) * K / 2);
    std::vector<uint16_t> lsw(static_cast<size_t>(N) * nb);
    std::vector<int16_t> lws(static_cast<size_t>(N) * nb);
    comet::pack_weights(W.data(), N, K, score.data(), nb8, lperm.data(), lflags.data(), Wq.data(), lsw.data(),
                        lws.data());
    bool same = lperm == perm && lflags == flags;
    for (int n = 0; n < N && same; ++n)
        for (int b = 0; b < nb; ++b)
            same = same && lsw[static_cast<size_t>(b) * N + n] == sw16[static_cast<size_t>(n) * nb + b] &&
                   lws[static_cast<size_t>(b) * N + n] == wsum[static_cast<size_t>(n) * nb + b];
    expect(same, "INT4 pack", M, N, K, nb8);
    std::vector<uint8_t> WqF(comet::wq_fp6_bytes(N, nb - nb8, nb8));
    comet::repack_fp6(Wq.data(), N, K, nb8, WqF.data());
}

void kv4(int H, int T, int d, unsigned seed) {
    std::mt19937 g(seed);
    auto q = halves(g, static_cast<size_t>(H) * d, 1.0f);
    auto K = halves(g, static_cast<size_t>(H) * T * d, 1.0f);
    auto V = halves(g, static_cast<size_t>(H) * T * d, 1.0f);
    std::vector<uint8_t> uk(K.size()), uv(V.size()), zk(static_cast<size_t>(H) * T), zv(zk.size());
    std::vector<uint16_t> sk(zk.size()), sv(zk.size());
    orc_kv4_quantize(K.data(), H * T, d, uk.data(), sk.data(), zk.data());
    orc_kv4_quantize(V.data(), H * T, d, uv.data(), sv.data(), zv.data());
    std::vector<double> out(static_cast<size_t>(H) * d);
    orc_kv4_attention(q.data(), uk.data(), sk.data(), zk.data(), uv.data(), sv.data(), zv.data(), H, T, d, out.data());
}

}  // namespace

int main() {
    const int shapes[][4] = {{3, 128, 128, 0}, {3, 128, 128, 1}, {5, 256, 512, 1}, {17, 384, 640, 5},
                             {2, 128, 1024, 8}, {9, 256, 384, 0}};
    unsigned seed = 1;
    for (const auto& s : shapes) layer(s[0], s[1], s[2], s[3], seed++);
    kv4(2, 17, 8, 99);
    kv4(3, 40, 128, 100);
    std::printf("%s (%d mismatches)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
