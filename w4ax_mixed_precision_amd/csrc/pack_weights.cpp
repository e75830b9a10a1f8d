// Offline weight preparation: channel ranking, symmetric INT4 quantization per
// (output channel, 128-channel block) with an fp16 scale, the per-block weight
// sums, and the nibble pack in MFMA fragment order.
//
// Channel ranking: COMET article (mmssai.com/?p=43269), section
// "1.离群点分布规律的重定义" (permute so that outlier channels share blocks);
// QUIK blog (deep-paper.org/paper/2310.09259), section "第一步: 识别与重排"
// (outlier columns go to the end of W); QoQ/QServe article
// (youleyou.com/wenzhang/3078652.html), section "通用量化优化技巧", item 3.
// Quantization: QUIK blog, section "反量化背后的数学" (symmetric weights, the
// weight sum is a weight-only quantity computed offline); QoQ/QServe article,
// section "背景" (fp16 scale per group).
// Fragment order: QoQ/QServe article, section "W4A8 GEMM的核心设计" (store the
// weights in the order the matrix instructions consume them, one wide load per
// lane); here the consumer is the gfx950 16x16x64 INT8 MFMA, see the Wq layout
// in comet_w4ax.h.
#include <algorithm>
#include <cmath>
#include <numeric>
#include <thread>
#include <vector>

#include "comet_internal.h"
#include "qoq_internal.h"

namespace comet {
namespace {

inline float half_bits_to_float(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return static_cast<float>(v);
}

inline uint16_t float_to_half_bits(float f) {
    _Float16 v = static_cast<_Float16>(f);   // IEEE round to nearest even
    uint16_t h;
    __builtin_memcpy(&h, &v, 2);
    return h;
}

// One output channel: quantize every block and scatter its nibbles into the
// channel's lane of each fragment. Returns false on a non-finite weight.
bool pack_row(const uint16_t* wrow, int N, int K, const int32_t* perm, int n, uint8_t* Wq,
              uint16_t* w_scale, int16_t* w_sum) {
    const int nb = K / kBlock;
    const int frag_col = n / 16;
    const int lane_col = n % 16;
    int8_t q[kBlock];
    for (int b = 0; b < nb; ++b) {
        float v[kBlock];
        float a = 0.0f;
        for (int p = 0; p < kBlock; ++p) {
            v[p] = half_bits_to_float(wrow[perm[b * kBlock + p]]);
            if (!std::isfinite(v[p])) return false;
            a = std::max(a, std::fabs(v[p]));
        }
        int sum = 0;
        if (a == 0.0f) {
            w_scale[static_cast<size_t>(b) * N + n] = 0;
            std::fill(q, q + kBlock, 0);
        } else {
            uint16_t hs = float_to_half_bits(a / 7.0f);
            if (hs == 0) hs = 1;                      // keep the divisor nonzero
            const float s = half_bits_to_float(hs);
            w_scale[static_cast<size_t>(b) * N + n] = hs;
            for (int p = 0; p < kBlock; ++p) {
                float r = std::rint(v[p] / s);
                r = std::min(7.0f, std::max(-7.0f, r));
                q[p] = static_cast<int8_t>(r);
                sum += q[p];
            }
        }
        w_sum[static_cast<size_t>(b) * N + n] = static_cast<int16_t>(sum);
        uint8_t* frag = Wq + (static_cast<size_t>(frag_col) * nb + b) * kFragBytes;
        for (int g = 0; g < 4; ++g) {
            uint8_t* dst = frag + 16 * (16 * g + lane_col);
            for (int j = 0; j < 16; ++j) {
                const uint8_t lo = static_cast<uint8_t>(q[32 * g + j]) & 0xF;
                const uint8_t hi = static_cast<uint8_t>(q[32 * g + 16 + j]) & 0xF;
                dst[j] = static_cast<uint8_t>(lo | (hi << 4));
            }
        }
    }
    return true;
}

// FP6 E2M3 bits of an integer code q in [-7, 7] (sign bit 5, exponent bits
// 4..3 with bias 1, mantissa bits 2..0): |q| = 0..7 -> 0, 8, 16, 20, 24, 26, 28, 30.
inline uint8_t fp6_code(int q) {
    static const uint8_t mag[8] = {0, 8, 16, 20, 24, 26, 28, 30};
    return static_cast<uint8_t>(mag[q < 0 ? -q : q] | (q < 0 ? 32 : 0));
}

inline int sext4(int v) { return v >= 8 ? v - 16 : v; }

// One INT4 fragment (1024 B) of a 4-bit block to its FP6 fragment (1536 B):
// lane l's 32 codes (positions 32(l/16) + j) become a 192-bit string, code j
// at bits 6j; bytes 0..15 go to the head at 16l, bytes 16..23 to the tail at
// 1024 + 8l.
void fragment_to_fp6(const uint8_t* src, uint8_t* dst) {
    for (int l = 0; l < 64; ++l) {
        uint8_t bits[24] = {};
        for (int j = 0; j < 32; ++j) {
            const uint8_t byte = src[16 * l + (j & 15)];
            const int q = sext4(j < 16 ? (byte & 0xF) : (byte >> 4));
            const uint32_t code = fp6_code(q);
            const int bit = 6 * j;
            bits[bit / 8] |= static_cast<uint8_t>(code << (bit % 8));
            if (bit % 8 > 2) bits[bit / 8 + 1] |= static_cast<uint8_t>(code >> (8 - bit % 8));
        }
        std::copy(bits, bits + 16, dst + 16 * l);
        std::copy(bits + 16, bits + 24, dst + 1024 + 8 * l);
    }
}

}  // namespace

void repack_fp6(const uint8_t* Wq, int N, int K, int nb8, uint8_t* WqF) {
    const int nb = K / kBlock;
    const int nb4 = nb - nb8;
    const int groups = N / 16;
    unsigned hw = std::thread::hardware_concurrency();
    const int threads = static_cast<int>(std::max(1u, std::min(hw ? hw : 1u, 32u)));
    const int per = (groups + threads - 1) / threads;
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) {
        const int f0 = t * per, f1 = std::min(groups, f0 + per);
        if (f0 >= f1) break;
        pool.emplace_back([=] {
            for (int f = f0; f < f1; ++f)
                for (int b = 0; b < nb; ++b) {
                    const uint8_t* src = Wq + (static_cast<size_t>(f) * nb + b) * kFragBytes;
                    if (b < nb4) {
                        uint8_t* dst = WqF + static_cast<size_t>(b) * groups * 1536 + static_cast<size_t>(f) * 1536;
                        fragment_to_fp6(src, dst);
                    } else {
                        uint8_t* dst = WqF + static_cast<size_t>(groups) * (1536u * static_cast<size_t>(nb4) +
                                                                            1024u * static_cast<size_t>(b - nb4)) +
                                       static_cast<size_t>(f) * kFragBytes;
                        std::copy(src, src + kFragBytes, dst);
                    }
                }
        });
    }
    for (auto& th : pool) th.join();
}

namespace {

// Channel order: stable ascending sort by score (the highest-scoring channels
// last). False on a non-finite score.
bool channel_order(const float* score, int K, int32_t* perm) {
    for (int k = 0; k < K; ++k)
        if (!std::isfinite(score[k])) return false;
    std::vector<int32_t> order(K);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [score](int32_t x, int32_t y) { return score[x] < score[y]; });
    std::copy(order.begin(), order.end(), perm);
    return true;
}

// Quantize and pack the channels perm[0 .. Kq) of every row of W ([N][K]),
// threaded over rows. False on a non-finite weight.
bool pack_rows(const uint16_t* W, int N, int K, int Kq, const int32_t* perm, uint8_t* Wq, uint16_t* w_scale,
               int16_t* w_sum) {
    unsigned hw = std::thread::hardware_concurrency();
    const int threads = static_cast<int>(std::max(1u, std::min(hw ? hw : 1u, 32u)));
    const int per = (N + threads - 1) / threads;
    std::vector<char> ok(threads, 1);
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) {
        const int n0 = t * per, n1 = std::min(N, n0 + per);
        if (n0 >= n1) break;
        pool.emplace_back([=, &ok] {
            for (int n = n0; n < n1; ++n)
                if (!pack_row(W + static_cast<size_t>(n) * K, N, Kq, perm, n, Wq, w_scale, w_sum)) {
                    ok[t] = 0;
                    return;
                }
        });
    }
    for (auto& th : pool) th.join();
    for (char c : ok)
        if (!c) return false;
    return true;
}

}  // namespace

int pack_weights(const uint16_t* W, int N, int K, const float* score, int nb8, int32_t* perm,
                 uint8_t* flags, uint8_t* Wq, uint16_t* w_scale, int16_t* w_sum) {
    const int nb = K / kBlock;
    if (!channel_order(score, K, perm)) return COMET_ERR_ARG;
    for (int b = 0; b < nb; ++b) flags[b] = static_cast<uint8_t>(b >= nb - nb8);
    return pack_rows(W, N, K, K, perm, Wq, w_scale, w_sum) ? COMET_OK : COMET_ERR_ARG;
}

// QUIK's outlier columns (QUIK blog, sections "第一步: 识别与重排" and "第二步:
// 前向传播 (在线)"): the same channel order; the first K - nf channels are
// quantized and packed as by pack_weights (their last nb8 blocks 8-bit), the
// last nf (the highest scores) keep their fp16 values in 1 KB fragments of
// 16 output channels x 32 channels, the operand order of the fp16 matrix
// instruction: fragment (c, s) at half (c * (nf / 32) + s) * 512 holds, at
// half 8 l + e, W[16 c + l mod 16][perm[K - nf + 32 s + 8 (l / 16) + e]].
int pack_weights_quik(const uint16_t* W, int N, int K, const float* score, int nf, int32_t* perm, uint8_t* Wq,
                      uint16_t* w_scale, int16_t* w_sum, uint16_t* Wf) {
    if (!channel_order(score, K, perm)) return COMET_ERR_ARG;
    const int Kq = K - nf;
    if (!pack_rows(W, N, K, Kq, perm, Wq, w_scale, w_sum)) return COMET_ERR_ARG;
    const int steps = nf / 32;
    for (int c = 0; c < N / 16; ++c)
        for (int s = 0; s < steps; ++s) {
            uint16_t* frag = Wf + (static_cast<size_t>(c) * steps + s) * 512;
            for (int l = 0; l < 64; ++l)
                for (int e = 0; e < 8; ++e) {
                    const int n = 16 * c + (l & 15);
                    const uint16_t w = W[static_cast<size_t>(n) * K + perm[Kq + 32 * s + 8 * (l >> 4) + e]];
                    if (!std::isfinite(half_bits_to_float(w))) return COMET_ERR_ARG;
                    frag[8 * l + e] = w;
                }
        }
    return COMET_OK;
}

// ---------------------------------------------------------------------------
// QoQ progressive group quantization (QoQ/QServe article, sections
// "渐进式分组量化" and "W4A8 GEMM的核心设计"): per output channel symmetric
// INT8 in the protected range [-119, 119] with an fp16 scale s1; then per
// 128-channel group of the permuted order an integer step s2 and zero point z
// over the group's range widened to include 0, codes u in [0, 15], so that
// s2 (u - z) is an 8-bit integer again. The codes go into the same fragment
// order as the INT4 pack (unsigned nibbles); s2 and z of (channel, group) are
// one 16-bit word s2 | z << 8.
// ---------------------------------------------------------------------------
namespace {

// Nearest integer of num / den (den > 0), ties to even, in integers.
inline int round_div_even(int num, int den) {
    int q = num / den, r = num % den;
    if (r < 0) {
        q -= 1;
        r += den;
    }
    if (2 * r > den || (2 * r == den && (q & 1))) ++q;
    return q;
}

bool pack_row_qoq(const uint16_t* wrow, int N, int K, const int32_t* perm, int n, uint8_t* Wu, uint16_t* s1,
                  uint16_t* s2z) {
    const int nb = K / kBlock;
    float a = 0.0f;
    for (int k = 0; k < K; ++k) {
        const float v = half_bits_to_float(wrow[k]);
        if (!std::isfinite(v)) return false;
        a = std::max(a, std::fabs(v));
    }
    uint16_t hs = 0;
    if (a > 0.0f) {
        hs = float_to_half_bits(a / 119.0f);
        if (hs == 0) hs = 1;
    }
    s1[n] = hs;
    const float s = half_bits_to_float(hs);
    const int frag_col = n / 16, lane_col = n % 16;
    int w8[kBlock];
    uint8_t u[kBlock];
    for (int b = 0; b < nb; ++b) {
        int lo = 0, hi = 0;
        for (int p = 0; p < kBlock; ++p) {
            int q = 0;
            if (hs != 0) {
                const float r = std::rint(half_bits_to_float(wrow[perm[b * kBlock + p]]) / s);
                q = static_cast<int>(std::min(119.0f, std::max(-119.0f, r)));
            }
            w8[p] = q;
            lo = std::min(lo, q);
            hi = std::max(hi, q);
        }
        const int st = std::max(1, (hi - lo + 14) / 15);
        const int z = round_div_even(-lo, st);
        for (int p = 0; p < kBlock; ++p)
            u[p] = static_cast<uint8_t>(std::min(15, std::max(0, round_div_even(w8[p], st) + z)));
        s2z[static_cast<size_t>(b) * N + n] = static_cast<uint16_t>(st | (z << 8));
        uint8_t* frag = Wu + (static_cast<size_t>(frag_col) * nb + b) * kFragBytes;
        for (int g = 0; g < 4; ++g) {
            uint8_t* dst = frag + 16 * (16 * g + lane_col);
            for (int j = 0; j < 16; ++j) dst[j] = static_cast<uint8_t>(u[32 * g + j] | (u[32 * g + 16 + j] << 4));
        }
    }
    return true;
}

}  // namespace

int pack_weights_qoq(const uint16_t* W, int N, int K, const float* score, int32_t* perm, uint8_t* Wu,
                     uint16_t* s1, uint16_t* s2z) {
    for (int k = 0; k < K; ++k)
        if (!std::isfinite(score[k])) return COMET_ERR_ARG;
    std::vector<int32_t> order(K);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [score](int32_t x, int32_t y) { return score[x] < score[y]; });
    std::copy(order.begin(), order.end(), perm);
    unsigned hw = std::thread::hardware_concurrency();
    const int threads = static_cast<int>(std::max(1u, std::min(hw ? hw : 1u, 32u)));
    const int per = (N + threads - 1) / threads;
    std::vector<char> ok(threads, 1);
    std::vector<std::thread> pool;
    for (int t = 0; t < threads; ++t) {
        const int n0 = t * per, n1 = std::min(N, n0 + per);
        if (n0 >= n1) break;
        pool.emplace_back([=, &ok] {
            for (int n = n0; n < n1; ++n)
                if (!pack_row_qoq(W + static_cast<size_t>(n) * K, N, K, perm, n, Wu, s1, s2z)) {
                    ok[t] = 0;
                    return;
                }
        });
    }
    for (auto& th : pool) th.join();
    for (char c : ok)
        if (!c) return COMET_ERR_ARG;
    return COMET_OK;
}

}  // namespace comet
