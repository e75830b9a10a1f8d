// Device helpers shared by the GEMM kernels: operand widening, matrix-core
// wrappers, direct global-to-LDS loads, partial load waits and the XCD-aware
// tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdint>

namespace comet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Integer minimum and maximum by value (a reference-returning min leaves stack
// slots behind).
__host__ __device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Byte offsets inside a 16-row activation tile of the FP6 layout. Row r keeps
// its bytes together: the 16-byte pieces of its four 32-channel groups g (the
// FP6 heads, or an 8-bit block's half-group) at 64 r + 16 (g ^ h(r)), the
// 8-byte FP6 tails at 1024 + 32 r + 8 (g ^ t(r)). The quantizer, which codes
// one row at a time, then writes a row's groups as one 64-byte and one
// 32-byte run. The slot permutations h(r) = (r >> 1) & 3 and t(r) =
// (r >> 2) & 3 were chosen by measurement (LDS bank-conflict counter of a
// probe that reads candidate layouts in the matrix-operand lane order, lane
// 16 g + r): with them the 16-byte and 8-byte operand reads run without bank
// conflicts, as the lane-order layout does; the other permutations tried
// (no permutation, r & 3, r >> 2, ...) cost a second cycle per read.
__host__ __device__ constexpr int tile_head(int r, int g) { return 64 * r + 16 * (g ^ ((r >> 1) & 3)); }
__host__ __device__ constexpr int tile_tail(int r, int g) { return 1024 + 32 * r + 8 * (g ^ ((r >> 2) & 3)); }

// The value unchanged but opaque to the optimizer. A binary32 product that is
// then rounded to fp16 must stay a product: otherwise the compiler folds the
// two into one mixed-precision FMA (v_fma_mixlo_f16) that rounds once,
// directly to fp16, instead of to binary32 and then to fp16, and a value on
// an fp16 tie after the first rounding comes out one step away.
__device__ __forceinline__ float opaque(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// 4-bit two's-complement weight nibbles to bytes holding 16 q_w (sign kept).
__device__ __forceinline__ v4i widen_weights_lo(uint4 p) {   // block positions 32g + j
    return v4i{static_cast<int>((p.x << 4) & 0xF0F0F0F0u), static_cast<int>((p.y << 4) & 0xF0F0F0F0u),
               static_cast<int>((p.z << 4) & 0xF0F0F0F0u), static_cast<int>((p.w << 4) & 0xF0F0F0F0u)};
}
__device__ __forceinline__ v4i widen_weights_hi(uint4 p) {   // block positions 32g + 16 + j
    return v4i{static_cast<int>(p.x & 0xF0F0F0F0u), static_cast<int>(p.y & 0xF0F0F0F0u),
               static_cast<int>(p.z & 0xF0F0F0F0u), static_cast<int>(p.w & 0xF0F0F0F0u)};
}
// Zero-extended 4-bit activation codes u = q + 8 to bytes.
__device__ __forceinline__ v4i widen_act_lo(uint4 p) {
    return v4i{static_cast<int>(p.x & 0x0F0F0F0Fu), static_cast<int>(p.y & 0x0F0F0F0Fu),
               static_cast<int>(p.z & 0x0F0F0F0Fu), static_cast<int>(p.w & 0x0F0F0F0Fu)};
}
__device__ __forceinline__ v4i widen_act_hi(uint4 p) {
    return v4i{static_cast<int>((p.x >> 4) & 0x0F0F0F0Fu), static_cast<int>((p.y >> 4) & 0x0F0F0F0Fu),
               static_cast<int>((p.z >> 4) & 0x0F0F0F0Fu), static_cast<int>((p.w >> 4) & 0x0F0F0F0Fu)};
}
__device__ __forceinline__ v4i as_v4i(uint4 p) {
    return v4i{static_cast<int>(p.x), static_cast<int>(p.y), static_cast<int>(p.z), static_cast<int>(p.w)};
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16x16x128 product of FP6 (E2M3) operands with an FP32 result; unit block
// scales (E8M0 127 = 2^0). A and B carry 32 codes per lane in the low six
// dwords.
__device__ __forceinline__ v4f mfma_fp6(v8i a, v8i b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 2, 2, 0, 127, 0, 127);
}

// Direct loads: each lane's 16 or 4 bytes from global memory land at LDS
// address (base + lane * size); `lds_piece` is the wave-uniform base.
__device__ __forceinline__ void lds_load16(const void* g, uint8_t* lds_piece) {
    __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                            reinterpret_cast<uintptr_t>(lds_piece)),
                                     16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, uint8_t* lds_piece) {
    __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                            reinterpret_cast<uintptr_t>(lds_piece)),
                                     4, 0, 0);
}

// Buffer-resource form of the direct loads: a raw buffer over `bytes` bytes at
// `base` (gfx9 descriptor word 3: 32-bit data format), a per-lane 32-bit
// offset in a VGPR and a wave-uniform offset in an SGPR, so a load costs no
// address arithmetic on the vector unit. Offsets at or past `bytes` read 0.
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void lds_buf16(Rsrc r, uint32_t voff, uint32_t soff, uint8_t* lds_piece) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_piece)), 16,
        voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_buf4(Rsrc r, uint32_t voff, uint32_t soff, uint8_t* lds_piece) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_piece)), 4,
        voff, soff, 0, 0);
}

// 16-byte load through a raw buffer resource. An offset at or past the
// buffer's size (the range check covers the per-lane offset) returns zeros
// and touches no memory: kOutOfRange, with buffers below 2 GB, is such an
// offset.
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ uint4 buf_load16(Rsrc r, uint32_t voff) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    return uint4{v.x, v.y, v.z, v.w};
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define COMET_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Tile of a workgroup. Workgroups are dispatched round-robin over the eight
// XCDs (workgroup w runs on XCD w mod 8); each XCD gets a contiguous range of
// the tile order, and the tile order walks 8-row-tile groups column by
// column, so the workgroups an XCD runs at once cover a compact patch and
// share their A and B stripes in that XCD's L2.
__device__ __forceinline__ bool tile_of(int w, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int t = (w & 7) * per_xcd + (w >> 3);
    if (t >= total) return false;
    constexpr int G = 8;
    const int group = t / (G * tiles_n);
    const int first = group * G;
    const int gh = imin(G, tiles_m - first);
    const int in = t - group * G * tiles_n;
    tn = in / gh;
    tm = first + in % gh;
    return true;
}

}  // namespace comet
