// Internal declarations of the QoQ W4A8 variant (progressive group
// quantization): the host packer, the per-token INT8 quantizer and the GEMM.
#pragma once

#include <cstddef>
#include <cstdint>

namespace comet {

// pack_weights.cpp: perm, unsigned 4-bit codes in fragment order, s1 fp16 [N],
// s2 | z << 8 [nb][N].
int pack_weights_qoq(const uint16_t* W, int N, int K, const float* score, int32_t* perm, uint8_t* Wu,
                     uint16_t* s1, uint16_t* s2z);

// quant_act.hip: per-token INT8 codes in 8-bit slabs ([nb][M][128] bytes) and
// one scale per token.
int launch_quant_act_token_i8(const uint16_t* X, int M, int K, int ldx, const int32_t* perm, uint8_t* Xq,
                              float* x_scale, void* stream);

// w4a8_qoq.hip: Y (fp16 [M][ldy]) or, when P is non-null, the exact products
// P (int32 [M][N]); M <= 64.
int launch_qoq_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wu, const uint16_t* s2z,
                    const uint16_t* s1, int M, int N, int K, uint16_t* Y, int ldy, int32_t* P, void* stream);

}  // namespace comet
