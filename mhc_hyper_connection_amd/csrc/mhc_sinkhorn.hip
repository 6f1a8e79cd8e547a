// mhc_sinkhorn.hip -- standalone fixed-count Sinkhorn-Knopp on 4x4 fp32 matrices.
//
// ("FlashInfer mHC 模块深度解析", section 5.2, Sinkhorn reference; rwkv-ops
// mhu_jax.py, sinkhorn_knopp.)
//
// One lane owns one matrix: 16 fp32 values in VGPRs, four 16-byte loads and
// stores, and the whole iteration with no cross-lane traffic.  The work is ALU
// bound (about 40 normalisation passes per matrix against 128 bytes moved), so
// the lane-per-matrix layout keeps every lane busy with independent work.
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

constexpr int kSkBlock = 256;

template <bool kVec4>
__global__ __launch_bounds__(kSkBlock) void sinkhorn_kernel(const float *logits, float *out, int64_t n, int iters,
                                                            float eps)
{
    const int64_t b = (int64_t)blockIdx.x * kSkBlock + threadIdx.x;
    if (b >= n) {
        return;
    }
    float P[16];
    const float *src = logits + b * 16;
    if (kVec4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src) + q);
            P[4 * q] = v[0];
            P[4 * q + 1] = v[1];
            P[4 * q + 2] = v[2];
            P[4 * q + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            P[e] = src[e];
        }
    }
    sinkhorn4x4(P, iters, eps);
    float *dst = out + b * 16;
    if (kVec4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = {P[4 * q], P[4 * q + 1], P[4 * q + 2], P[4 * q + 3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(dst) + q);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            dst[e] = P[e];
        }
    }
}

} // namespace

hipError_t launch_sinkhorn(const float *logits, float *out, int64_t n, int iters, float eps, hipStream_t stream,
                           bool vec4)
{
    return for_token_chunks(n, sinkhorn_items_per_matrix(), [&](int64_t c0, int64_t nc) {
        const int64_t blocks = (nc + kSkBlock - 1) / kSkBlock;
        const size_t o = (size_t)c0 * 16;
        if (vec4) {
            sinkhorn_kernel<true><<<dim3((unsigned)blocks), dim3(kSkBlock), 0, stream>>>(logits + o, out + o, nc, iters,
                                                                                         eps);
        } else {
            sinkhorn_kernel<false><<<dim3((unsigned)blocks), dim3(kSkBlock), 0, stream>>>(logits + o, out + o, nc,
                                                                                          iters, eps);
        }
        return hipGetLastError();
    });
}

int64_t sinkhorn_items_per_matrix() { return 1; }

} // namespace mhc
