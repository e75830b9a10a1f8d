// Internal declarations of the KV4 decode attention: the cache quantizer and
// the split attention with its combine step.
#pragma once

#include <cstddef>
#include <cstdint>

namespace comet {

constexpr int kKvChunk = 256;   // cached tokens per attention workgroup, at least

inline int kv4_splits(int T) { return (T + kKvChunk - 1) / kKvChunk; }

// FP32 workspace of the split attention: partial outputs [Hq][splits][d], then
// the running maximum and sum [Hq][splits][2].
inline size_t kv4_workspace_bytes(int Hq, int d, int T) {
    return static_cast<size_t>(Hq) * static_cast<size_t>(kv4_splits(T)) * (static_cast<size_t>(d) + 2u) * 4u;
}

// X fp16: ntok rows of ldx, H heads of d channels each; vector (tok, h) goes to
// cache slot h * tcap + pos + tok.
int launch_kv4_quantize(const uint16_t* X, int ntok, int H, int d, int ldx, int pos, int tcap, uint8_t* codes,
                        uint16_t* step, uint8_t* zero, void* stream);

// q fp16 [Hq][d]; out fp16 [Hq][d]; query head h reads kv head h / group.
// Tk (device, Hq / group int32) or null: kv head g attends to its first
// min(max(Tk[g], 0), T) slots (an empty head gives zeros), else all T.
int launch_kv4_attention(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* kz,
                         const uint8_t* vc, const uint16_t* vs, const uint8_t* vz, int Hq, int group, int d, int T,
                         int tcap, uint16_t* out, float* workspace, void* stream, const int* Tk = nullptr);

}  // namespace comet
