// mhc_backward.hip -- reverse mode of the Sinkhorn projection and of the post-map.
//
// (rwkv-ops mhu_jax.py: sinkhorn_knopp and mhc_post_op with their custom VJPs,
// SinkhornBwd and MhcPostOpBwd; the forward formulas are those of the FlashInfer
// mHC article, sections 2.1 and 5.2.)
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

// ---------------------------------------------------------------- Sinkhorn backward
//
// 16 lanes per matrix (lane e holds entry (e / 4, e % 4)), 4 matrices per 64-thread
// workgroup.  The forward is replayed keeping the matrix after each full iteration in
// LDS ([iters + 1][64] floats, one per lane); the row-normalised matrix of an
// iteration is recomputed from the one before it with the same operations, so it is
// bit-identical to the replay's.  The reverse pass then runs, per iteration from the
// last:
//   column step Q = A / c:  dA = (dQ - sum_col(dQ * Q)) / c
//   row step    A = P / r:  dP = (dA - sum_row(dA * A)) / r
// and finally through + eps and the row softmax S: dL = S * (dS - sum_row(dS * S)).
// Divisions by a row or column sum multiply by its hardware reciprocal (1 ulp).
constexpr int kSBBlock = 64;

__device__ __forceinline__ float row_sum4(float v)
{
    v = v + dpp_quad_xor1(v);
    return v + dpp_quad_xor2(v);
}
__device__ __forceinline__ float col_sum4(float v)
{
    v = v + dpp_row_ror4(v);
    return v + dpp_row_ror8(v);
}

__global__ __launch_bounds__(kSBBlock) void sinkhorn_bwd_kernel(const float *__restrict__ grad,
                                                                const float *__restrict__ logits, int64_t n,
                                                                int iters, float eps, float *__restrict__ d_logits)
{
    extern __shared__ float hist[]; // [iters + 1][kSBBlock]
    const int tid = threadIdx.x;
    const int64_t gl = (int64_t)blockIdx.x * kSBBlock + tid;
    const bool live = (gl >> 4) < n; // uniform within each 16-lane row
    float L = 0.0f, G = 0.0f;
    if (live) {
        L = logits[gl];
        G = grad[gl];
    }
    // forward replay
    float mx = fmaxf(L, dpp_quad_xor1(L));
    mx = fmaxf(mx, dpp_quad_xor2(mx));
    const float ex = __expf(L - mx);
    const float S = ex * fast_rcp(row_sum4(ex));
    float P = S + eps;
    hist[tid] = P;
    for (int k = 1; k <= iters; ++k) {
        const float A = P * fast_rcp(row_sum4(P));
        P = A * fast_rcp(col_sum4(A));
        hist[k * kSBBlock + tid] = P;
    }
    // reverse pass (each lane reads back only what it wrote itself); P holds the
    // matrix after iteration k at the top of each step
    for (int k = iters; k >= 1; --k) {
        const float Q = P;
        P = hist[(k - 1) * kSBBlock + tid];
        const float rinv = fast_rcp(row_sum4(P));
        const float A = P * rinv;
        const float dA = (G - col_sum4(G * Q)) * fast_rcp(col_sum4(A));
        G = (dA - row_sum4(dA * A)) * rinv;
    }
    if (live) {
        d_logits[gl] = S * (G - row_sum4(G * S));
    }
}

// ---------------------------------------------------------------- post-map backward
//
// One workgroup per token.  With dO = d_out:
//   d_x[h] = sum_n dO[n][h] post[n],  d_res[o][h] = sum_n comb[o][n] dO[n][h]   (per element, bf16)
//   d_post[n] = sum_h dO[n][h] x[h],  d_comb[o][n] = sum_h res[o][h] dO[n][h]   (20 sums over h, fp32)
// Each thread handles its 8-element chunks (kCPT per stream on the 16-byte path,
// scalar elements otherwise); the 20 sums are reduced over the wavefront and then
// over the 4 wavefronts in a fixed order.
constexpr int kPBSums = kHC + kHC * kHC;

struct PostBwdArgs {
    const uint16_t *d_out, *x, *res;
    const float *post, *comb;
    int T, H;
    uint16_t *d_x, *d_res;
    float *d_post, *d_comb;
};

// One element h: d_x and the 4 d_res values (into column `slot` of vr) and the 20
// running sums.
__device__ __forceinline__ void post_bwd_element(const float (&gv)[kHC], const float (&rv)[kHC], float xs,
                                                 const float (&pw)[kHC], const float (&cw)[kHC][kHC],
                                                 float (&acc)[kPBSums], float &vx, float (&vr)[kHC][2], int slot)
{
    vx = gv[0] * pw[0];
#pragma unroll
    for (int n = 1; n < kHC; ++n) {
        vx = fmaf(gv[n], pw[n], vx);
    }
#pragma unroll
    for (int o = 0; o < kHC; ++o) {
        float v = cw[o][0] * gv[0];
#pragma unroll
        for (int n = 1; n < kHC; ++n) {
            v = fmaf(cw[o][n], gv[n], v);
        }
        vr[o][slot] = v;
    }
#pragma unroll
    for (int n = 0; n < kHC; ++n) {
        acc[n] = fmaf(gv[n], xs, acc[n]);
#pragma unroll
        for (int o = 0; o < kHC; ++o) {
            acc[kHC + o * kHC + n] = fmaf(rv[o], gv[n], acc[kHC + o * kHC + n]);
        }
    }
}

template <int kBlock, int kCPT>
__global__ __launch_bounds__(kBlock) void post_bwd_kernel(PostBwdArgs a)
{
    constexpr int kWaves = kBlock / kWave;
    __shared__ float part[kWaves][kPBSums];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int H = a.H;
    const uint16_t *go = a.d_out + (size_t)t * kHC * H;
    const uint16_t *xr = a.x + (size_t)t * H;
    const uint16_t *rr = a.res + (size_t)t * kHC * H;
    float pw[kHC], cw[kHC][kHC];
#pragma unroll
    for (int n = 0; n < kHC; ++n) {
        pw[n] = a.post[(size_t)t * kHC + n];
#pragma unroll
        for (int o = 0; o < kHC; ++o) {
            cw[o][n] = a.comb[((size_t)t * kHC + o) * kHC + n];
        }
    }
    float acc[kPBSums];
#pragma unroll
    for (int k = 0; k < kPBSums; ++k) {
        acc[k] = 0.0f;
    }
    if constexpr (kCPT > 0) {
        const int nch = H >> 3;
#pragma unroll
        for (int k = 0; k < kCPT; ++k) {
            const int j = tid + k * kBlock;
            if (j < nch) {
                const size_t col = (size_t)j * 8;
                u32x4 g[kHC], r[kHC];
#pragma unroll
                for (int i = 0; i < kHC; ++i) {
                    g[i] = load_nt16(go + (size_t)i * H + col);
                    r[i] = load_nt16(rr + (size_t)i * H + col);
                }
                const u32x4 xv = load_nt16(xr + col);
                u32x4 dx, dr[kHC];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float vx[2], vr[kHC][2];
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        float gv[kHC], rv[kHC];
#pragma unroll
                        for (int i = 0; i < kHC; ++i) {
                            // copy the element to a scalar before unpacking it
                            const uint32_t gw = g[i][q], rw = r[i][q];
                            gv[i] = half ? bf16_hi(gw) : bf16_lo(gw);
                            rv[i] = half ? bf16_hi(rw) : bf16_lo(rw);
                        }
                        const uint32_t xw = xv[q];
                        const float xs = half ? bf16_hi(xw) : bf16_lo(xw);
                        post_bwd_element(gv, rv, xs, pw, cw, acc, vx[half], vr, half);
                    }
                    dx[q] = pack_bf16x2(vx[0], vx[1]);
#pragma unroll
                    for (int o = 0; o < kHC; ++o) {
                        dr[o][q] = pack_bf16x2(vr[o][0], vr[o][1]);
                    }
                }
                store_nt16(a.d_x + (size_t)t * H + col, dx);
#pragma unroll
                for (int o = 0; o < kHC; ++o) {
                    store_nt16(a.d_res + ((size_t)t * kHC + o) * H + col, dr[o]);
                }
            }
        }
    } else {
        for (int h = tid; h < H; h += kBlock) {
            float gv[kHC], rv[kHC];
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                gv[i] = bf16_to_f32(go[(size_t)i * H + h]);
                rv[i] = bf16_to_f32(rr[(size_t)i * H + h]);
            }
            const float xs = bf16_to_f32(xr[h]);
            float vx, vr[kHC][2];
            post_bwd_element(gv, rv, xs, pw, cw, acc, vx, vr, 0);
            a.d_x[(size_t)t * H + h] = f32_to_bf16(vx);
#pragma unroll
            for (int o = 0; o < kHC; ++o) {
                a.d_res[((size_t)t * kHC + o) * H + h] = f32_to_bf16(vr[o][0]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kPBSums; ++k) {
        const float v = wave_sum(acc[k]);
        if (lane == 0) {
            part[w][k] = v;
        }
    }
    __syncthreads();
    if (tid < kPBSums) {
        float v = part[0][tid];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) {
            v += part[i][tid];
        }
        if (tid < kHC) {
            a.d_post[(size_t)t * kHC + tid] = v;
        } else {
            a.d_comb[(size_t)t * kHC * kHC + (tid - kHC)] = v;
        }
    }
}

} // namespace

size_t sinkhorn_bwd_lds_bytes(int iters) { return (size_t)(iters + 1) * kSBBlock * sizeof(float); }

hipError_t launch_sinkhorn_bwd(const float *grad, const float *logits, int64_t n, int iters, float eps,
                               float *d_logits, hipStream_t stream)
{
    const int64_t threads = n * 16;
    const int64_t blocks = (threads + kSBBlock - 1) / kSBBlock;
    sinkhorn_bwd_kernel<<<dim3((unsigned)blocks), dim3(kSBBlock), sinkhorn_bwd_lds_bytes(iters), stream>>>(
        grad, logits, n, iters, eps, d_logits);
    return hipGetLastError();
}

hipError_t launch_post_bwd(const uint16_t *d_out, const uint16_t *x, const uint16_t *res, const float *post,
                           const float *comb, int64_t T, int64_t H, uint16_t *d_x, uint16_t *d_res, float *d_post,
                           float *d_comb, hipStream_t stream, bool vec8)
{
    PostBwdArgs a;
    a.d_out = d_out;
    a.x = x;
    a.res = res;
    a.post = post;
    a.comb = comb;
    a.T = (int)T;
    a.H = (int)H;
    a.d_x = d_x;
    a.d_res = d_res;
    a.d_post = d_post;
    a.d_comb = d_comb;
    // 256 threads, kCPT 8-element chunks per thread and stream on the 16-byte path
    // (128- and 64-thread groups with exact chunk counts measured no faster at H=7168).
    const dim3 grid((unsigned)T), block(256);
    const int64_t per = (H / 8 + 255) / 256;
    if (vec8 && per <= 1) {
        post_bwd_kernel<256, 1><<<grid, block, 0, stream>>>(a);
    } else if (vec8 && per <= 2) {
        post_bwd_kernel<256, 2><<<grid, block, 0, stream>>>(a);
    } else if (vec8 && per <= 4) {
        post_bwd_kernel<256, 4><<<grid, block, 0, stream>>>(a);
    } else if (vec8 && per <= 8) {
        post_bwd_kernel<256, 8><<<grid, block, 0, stream>>>(a);
    } else {
        post_bwd_kernel<256, 0><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

} // namespace mhc
