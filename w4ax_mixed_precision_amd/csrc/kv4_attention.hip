// KV4 decode attention (QoQ/QServe article, section "KV4注意力Kernel优化", and
// section "运行时设计"; COMET article: the KV cache held at 4 bits). Keys and
// values are cached per (head, token) as d unsigned 4-bit codes with an fp16
// step and an 8-bit zero point beside them, chosen at run time from each
// vector's own range; a decode step attends one query per head over the
// cached tokens.
//
// Cache layout in HBM, per kv head h and token slot t (capacity tcap):
//   codes  [h][t][d/2] bytes, channel 2i in the low nibble of byte i and 2i+1
//          in the high nibble (one 32-bit word = 8 consecutive channels);
//   step   [h][t] fp16 bits, zero [h][t] bytes.
//
// Quantizer: one wave per vector; a lane holds 8 channels (one 16-byte load,
// one 32-bit code store), the range comes from two wave reductions.
//
// Attention: the page's point is that decode attention is memory bound, so
// dequantization must cost few operations per code. Here a workgroup (4
// waves) takes one query head and a chunk of 256 cached tokens; d/8 lanes
// share a token, each reading one 32-bit word of its codes, so a wave load
// covers 256 contiguous bytes of the cache. The zero point is taken out of
// the key product as a whole, s (q.u - z sum(q)), so a key code costs one
// conversion and one multiply-add; the value codes are weighted by p s and the
// zero point subtracted per code. The chunk keeps its own maximum and sum, and
// a second kernel combines the chunks (the split-softmax identity:
// out = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "kv4_internal.h"

namespace comet {
namespace {

constexpr int kKvThreads = 256;   // 4 waves

__device__ __forceinline__ void unpack8(uint4 p, float* x) {
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
        x[2 * i + 1] = h2f(static_cast<uint16_t>(w[i] >> 16));
    }
}

__global__ __launch_bounds__(kKvThreads) void kv4_quant_kernel(const uint16_t* __restrict__ X, int nvec, int H,
                                                               int d, int ldx, int pos, int tcap,
                                                               uint8_t* __restrict__ codes,
                                                               uint16_t* __restrict__ step,
                                                               uint8_t* __restrict__ zero) {
    const int lane = threadIdx.x & 63;
    const int v = blockIdx.x * (kKvThreads / 64) + (threadIdx.x >> 6);
    if (v >= nvec) return;                               // whole wave
    const int tok = v / H, h = v - tok * H;
    const int D = d >> 3;                                // 32-bit code words per vector
    const bool act = lane < D;
    float x[8];
    if (act) {
        unpack8(*reinterpret_cast<const uint4*>(X + static_cast<size_t>(tok) * ldx + static_cast<size_t>(h) * d +
                                                8 * lane),
                x);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = 0.0f;
    }
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        lo = fminf(lo, x[c]);
        hi = fmaxf(hi, x[c]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, o));
        hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    const size_t slot = static_cast<size_t>(h) * tcap + pos + tok;
    uint32_t word = 0;
    uint16_t s16 = 0;
    int z = 0;
    if (lo != hi) {
        const float dd = hi - lo;
        const float inv = 15.0f / dd;
        s16 = __half_as_ushort(__float2half_rn(opaque(dd / 15.0f)));
        if (s16 == 0) s16 = 1;                           // smallest fp16 subnormal
        z = static_cast<int>(rintf(-lo * inv));
        z = z < 0 ? 0 : (z > 15 ? 15 : z);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            int u = static_cast<int>(rintf(x[c] * inv)) + z;
            u = u < 0 ? 0 : (u > 15 ? 15 : u);
            word |= static_cast<uint32_t>(u) << (4 * c);
        }
    }
    if (act) *reinterpret_cast<uint32_t*>(codes + slot * static_cast<size_t>(d >> 1) + 4 * lane) = word;
    if (lane == 0) {
        step[slot] = s16;
        zero[slot] = static_cast<uint8_t>(z);
    }
}

__device__ __forceinline__ float block_max(float v, float* wred) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    __syncthreads();
    return v;
}

__device__ __forceinline__ float block_sum(float v, float* wred) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = v;
    __syncthreads();
    v = (wred[0] + wred[1]) + (wred[2] + wred[3]);
    __syncthreads();
    return v;
}

// One (query head, chunk of 256 tokens). Partial output (unnormalized), chunk
// maximum and sum go to the workspace.
__global__ __launch_bounds__(kKvThreads) void kv4_attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
    const uint8_t* __restrict__ kz, const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
    const uint8_t* __restrict__ vz, int group, int d, int T, int tcap, float scale, int nsplit,
    float* __restrict__ part, float* __restrict__ ml) {
    __shared__ float sc[kKvChunk];
    __shared__ float red[4][512];
    __shared__ float wred[4];
    const int h = blockIdx.x / nsplit;
    const int s = blockIdx.x - h * nsplit;
    const int hk = h / group;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D = d >> 3;                        // lanes per token, power of two in [1, 64]
    const int TPW = 64 / D;                      // tokens per wave step
    const int j = lane & (D - 1);                // code word of the token
    const int sub = lane / D;                    // token slot within the wave step
    const int t0 = s * kKvChunk;
    const int nt = imin(kKvChunk, T - t0);       // >= 1
    const int rb = d >> 1;                       // bytes per cached vector

    float qf[8];
    unpack8(*reinterpret_cast<const uint4*>(q + static_cast<size_t>(h) * d + 8 * j), qf);
    float qs = ((qf[0] + qf[1]) + (qf[2] + qf[3])) + ((qf[4] + qf[5]) + (qf[6] + qf[7]));
    for (int o = 1; o < D; o <<= 1) qs += __shfl_xor(qs, o);

    const size_t base = static_cast<size_t>(hk) * tcap + t0;   // slot of the chunk's first token
    const int per_step = 4 * TPW;
    const int niter = (nt + per_step - 1) / per_step;

    // scores a_t = s_t (q . u_t - z_t sum q) / sqrt(d)
#pragma unroll 2
    for (int it = 0; it < niter; ++it) {
        const int i = it * per_step + wave * TPW + sub;
        const bool ok = i < nt;
        uint32_t w = 0;
        float st = 0.0f;
        int zt = 0;
        if (ok) {
            const size_t sl = base + i;
            w = *reinterpret_cast<const uint32_t*>(kc + sl * rb + 4 * j);
            st = h2f(ks[sl]);
            zt = kz[sl];
        }
        float dot = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) dot += qf[c] * static_cast<float>((w >> (4 * c)) & 15u);
        for (int o = 1; o < D; o <<= 1) dot += __shfl_xor(dot, o);
        if (ok && j == 0) sc[i] = st * (dot - static_cast<float>(zt) * qs) * scale;
    }
    __syncthreads();

    float m = -INFINITY;
    for (int i = threadIdx.x; i < nt; i += kKvThreads) m = fmaxf(m, sc[i]);
    m = block_max(m, wred);
    float l = 0.0f;
    for (int i = threadIdx.x; i < nt; i += kKvThreads) {
        const float p = expf(sc[i] - m);
        sc[i] = p;
        l += p;
    }
    l = block_sum(l, wred);                      // its barriers also publish sc

    // acc = sum_t p_t s_t (u_t - z_t)
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
#pragma unroll 2
    for (int it = 0; it < niter; ++it) {
        const int i = it * per_step + wave * TPW + sub;
        const bool ok = i < nt;
        uint32_t w = 0;
        float wt = 0.0f;
        int zt = 0;
        if (ok) {
            const size_t sl = base + i;
            w = *reinterpret_cast<const uint32_t*>(vc + sl * rb + 4 * j);
            wt = sc[i] * h2f(vs[sl]);
            zt = vz[sl];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] += wt * static_cast<float>(static_cast<int>((w >> (4 * c)) & 15u) - zt);
    }
    for (int o = D; o < 64; o <<= 1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], o);
    }
    if (sub == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) red[wave][8 * j + c] = acc[c];
    }
    __syncthreads();
    const size_t row = static_cast<size_t>(h) * nsplit + s;
    for (int i = threadIdx.x; i < d; i += kKvThreads)
        part[row * d + i] = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
    if (threadIdx.x == 0) {
        ml[2 * row] = m;
        ml[2 * row + 1] = l;
    }
}

__global__ __launch_bounds__(128) void kv4_attn_combine_kernel(const float* __restrict__ part,
                                                              const float* __restrict__ ml, int nsplit, int d,
                                                              uint16_t* __restrict__ out) {
    const int h = blockIdx.x;
    const float* mh = ml + static_cast<size_t>(h) * nsplit * 2;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, mh[2 * s]);
    float L = 0.0f;
    for (int s = 0; s < nsplit; ++s) L += expf(mh[2 * s] - M) * mh[2 * s + 1];
    const float invL = 1.0f / L;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        float a = 0.0f;
        for (int s = 0; s < nsplit; ++s)
            a += expf(mh[2 * s] - M) * part[(static_cast<size_t>(h) * nsplit + s) * d + i];
        out[static_cast<size_t>(h) * d + i] = __half_as_ushort(__float2half_rn(a * invL));
    }
}

}  // namespace

int launch_kv4_quantize(const uint16_t* X, int ntok, int H, int d, int ldx, int pos, int tcap, uint8_t* codes,
                        uint16_t* step, uint8_t* zero, void* stream) {
    const int nvec = ntok * H;
    const int per_block = kKvThreads / 64;
    kv4_quant_kernel<<<(nvec + per_block - 1) / per_block, kKvThreads, 0, static_cast<hipStream_t>(stream)>>>(
        X, nvec, H, d, ldx, pos, tcap, codes, step, zero);
    return static_cast<int>(hipGetLastError());
}

int launch_kv4_attention(const uint16_t* q, const uint8_t* kc, const uint16_t* ks, const uint8_t* kz,
                         const uint8_t* vc, const uint16_t* vs, const uint8_t* vz, int Hq, int group, int d, int T,
                         int tcap, uint16_t* out, float* workspace, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int nsplit = kv4_splits(T);
    float* part = workspace;
    float* ml = workspace + static_cast<size_t>(Hq) * nsplit * d;
    const float scale = 1.0f / sqrtf(static_cast<float>(d));
    kv4_attn_chunk_kernel<<<Hq * nsplit, kKvThreads, 0, st>>>(q, kc, ks, kz, vc, vs, vz, group, d, T, tcap, scale,
                                                              nsplit, part, ml);
    const int e = static_cast<int>(hipGetLastError());
    if (e != 0) return e;
    kv4_attn_combine_kernel<<<Hq, 128, 0, st>>>(part, ml, nsplit, d, out);
    return static_cast<int>(hipGetLastError());
}

}  // namespace comet
