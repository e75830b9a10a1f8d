// Internal declarations shared by the library's translation units.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/comet_w4ax.h"

namespace comet {

constexpr int kBlock = 128;          // channels per quantization block
constexpr int kFragBytes = 1024;     // packed weight fragment: 16 channels x 128 positions

// Bytes of the activation code buffer for M rows.
inline size_t xq_bytes(int M, int nb4, int nb8) {
    return static_cast<size_t>(M) * (64u * static_cast<size_t>(nb4) + 128u * static_cast<size_t>(nb8));
}

// Bytes of the FP6-layout activation and weight buffers.
inline size_t xq_fp6_bytes(int M, int nb4, int nb8) {     // rows padded to 16-row tiles
    const size_t mp = (static_cast<size_t>(M) + 15u) & ~static_cast<size_t>(15);
    return mp * (96u * static_cast<size_t>(nb4) + 128u * static_cast<size_t>(nb8));
}
inline size_t wq_fp6_bytes(int N, int nb4, int nb8) {
    return static_cast<size_t>(N) * (96u * static_cast<size_t>(nb4) + 64u * static_cast<size_t>(nb8));
}

// Launchers (device code lives in the .hip files). Arguments were validated by
// the C entry points; each returns a hipError_t value as int.
int launch_quant_act(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                     uint8_t* Xq, float* x_scale, void* stream);

// Asymmetric 4-bit blocks (INT4 layout); x_zero [nb][Mp], Mp = M rounded up to 16.
int launch_quant_act_asym(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                          uint8_t* Xq, float* x_scale, uint8_t* x_zero, void* stream);

// kq > 0: quantize only the first kq permuted channels (QUIK's split; the
// rows are still staged K channels wide, since perm reaches any of them).
int launch_quant_act_fp6(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, int nb8,
                         uint8_t* Xq, float* x_scale, void* stream, int kq = 0);
// QUIK's fp16 outlier channels: Xf tiles (GemmProblem::xf layout) of columns
// perm_f[0 .. nf) of X (rows of K channels), rows past M zero.
int launch_gather_outliers(const uint16_t* X, int M, int K, int ldx, const int32_t* perm_f, int nf, uint16_t* Xf,
                           void* stream);

// Bytes of the QUIK fp16 outlier tiles of M rows.
inline size_t xf_bytes(int M, int nf) {
    const size_t mp = (static_cast<size_t>(M) + 15u) & ~static_cast<size_t>(15);
    return mp * static_cast<size_t>(nf) * 2u;
}

// RMS normalization fused into the quantizer (either layout), and on its own.
int launch_rmsnorm_quant_act(const uint16_t* X, int M, int K, int ldx, const uint16_t* gamma_perm, float eps,
                             const int32_t* perm, int nb8, uint8_t* Xq, float* x_scale, bool fp6, void* stream);
// SwiGLU before the quantizer (fused) and on its own: H = fp16(silu(G) U).
int launch_swiglu_quant_act(const uint16_t* G, const uint16_t* U, int M, int K, int ldx, const int32_t* perm,
                            int nb8, uint8_t* Xq, float* x_scale, bool fp6, void* stream);
int launch_swiglu(const uint16_t* G, const uint16_t* U, int M, int K, int ldx, uint16_t* H, int ldh,
                  void* stream);
int launch_rmsnorm(const uint16_t* X, int M, int K, int ldx, const uint16_t* gamma, float eps, uint16_t* Xn,
                   int ldn, void* stream);

struct GemmProblem {
    const uint8_t* Xq;
    const float* x_scale;
    const uint8_t* Wq;
    const uint16_t* w_scale;
    const int16_t* w_sum;
    int M, N, K, nb, nb4;
    uint16_t* Y;
    int ldy;
    const uint8_t* x_zero;   // zero points of asymmetric 4-bit blocks [nb][Mp] (Mp = M rounded
                             // up to 16), or nullptr for symmetric codes
    int32_t* P;              // debug partials output, or nullptr
    int m_begin, m_count;    // row range of the partials output
    void* workspace;
    size_t workspace_bytes;
    int max_wg;              // FP6 partials only: cap on the persistent grid (0: none)
    // FP6 layout only: QUIK's fp16 outlier channels after the K quantized ones
    // (nf = 0: none). xf: [Mp/16][nf/32] 1 KB tiles (16 rows x 32 channels, Mp
    // = M rounded up to 16); wf: [N/16][nf/32] 1 KB fragments.
    const uint16_t* xf;
    const uint16_t* wf;
    int nf;
};

size_t gemm_workspace_bytes(int M, int N, int K, int nb8);
int launch_w4ax_gemm(const GemmProblem& p, void* stream);
int launch_w4ax_gemm_fp6(const GemmProblem& p, void* stream);   // FP6 layout; w_sum unused
// Workspace of the FP6 GEMM (work queue, tile counts, split partial tiles);
// a function of the shape only (no device query).
size_t gemm_fp6_workspace_bytes(int M, int N, int K, int nb8);
// The FP6 GEMM with the library's fixed per-device scratch array as its
// workspace (p.workspace is ignored); the shape's workspace must fit it.
int launch_w4ax_gemm_fp6_noalloc(GemmProblem p, void* stream);

// Compute units of the current device (quant_act.hip; read once per process).
int cu_count();

// Host packer (pack_weights.cpp).
int pack_weights(const uint16_t* W, int N, int K, const float* score, int nb8, int32_t* perm,
                 uint8_t* flags, uint8_t* Wq, uint16_t* w_scale, int16_t* w_sum);
int pack_weights_quik(const uint16_t* W, int N, int K, const float* score, int nf, int32_t* perm, uint8_t* Wq,
                      uint16_t* w_scale, int16_t* w_sum, uint16_t* Wf);
// INT4 fragments to the FP6 layout (pack_weights.cpp).
void repack_fp6(const uint8_t* Wq, int N, int K, int nb8, uint8_t* WqF);

}  // namespace comet
