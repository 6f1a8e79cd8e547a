// mhc_device.h -- device-side helpers shared by the libmhc kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

constexpr int kHC = 4;    // residual streams
constexpr int kMix = 24;  // logits per token: pre(4) + post(4) + comb(16)
constexpr int kWave = 64; // CDNA wavefront

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Two fp32 -> packed bf16 pair, round to nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float v)
{
    __bf16 b = (__bf16)v;
    return __builtin_bit_cast(uint16_t, b);
}

// 16-byte streaming loads/stores (data touched once: non-temporal hint).
__device__ __forceinline__ u32x4 load_nt16(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void store_nt16(void *p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 1 / (1 + e^-z), using the hardware 2^x.
__device__ __forceinline__ float sigmoidf_fast(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Fixed-count Sinkhorn-Knopp on one 4x4 matrix held in registers (row-major P[4*i+j]):
// softmax over each row (row maximum subtracted) plus eps, then `iters` rounds of
// row normalisation followed by column normalisation.
__device__ __forceinline__ void sinkhorn4x4(float *P, int iters, float eps)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float mx = fmaxf(fmaxf(P[4 * i], P[4 * i + 1]), fmaxf(P[4 * i + 2], P[4 * i + 3]));
        float e0 = __expf(P[4 * i] - mx), e1 = __expf(P[4 * i + 1] - mx);
        float e2 = __expf(P[4 * i + 2] - mx), e3 = __expf(P[4 * i + 3] - mx);
        float r = fast_rcp((e0 + e1) + (e2 + e3));
        P[4 * i] = fmaf(e0, r, eps);
        P[4 * i + 1] = fmaf(e1, r, eps);
        P[4 * i + 2] = fmaf(e2, r, eps);
        P[4 * i + 3] = fmaf(e3, r, eps);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r = fast_rcp((P[4 * i] + P[4 * i + 1]) + (P[4 * i + 2] + P[4 * i + 3]));
            P[4 * i] *= r;
            P[4 * i + 1] *= r;
            P[4 * i + 2] *= r;
            P[4 * i + 3] *= r;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = fast_rcp((P[j] + P[4 + j]) + (P[8 + j] + P[12 + j]));
            P[j] *= r;
            P[4 + j] *= r;
            P[8 + j] *= r;
            P[12 + j] *= r;
        }
    }
}

// Wave-uniform value (forces an SGPR so coefficient loads become scalar loads).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

} // namespace mhc
