// mhc_pre_dots.hip -- the mHC pre-map from an external projection.
//
// ("FlashInfer mHC 模块深度解析", sections 3.1-3.4, mhc_pre_big_fuse: the 24 dots
// come from outside, possibly as split-K partial sums; section 4,
// mhc_pre_big_fuse_with_prenorm: the sum of squares is computed here from the
// streams when the caller does not supply it.)
//
// With one split, a supplied sum of squares and 16-byte rows, the per-token mixes need
// no reduction and the pre-map's collapse kernel runs instead (one wavefront per token
// and 512-wide h tile, launch_collapse_dots).  Otherwise: one 256-thread workgroup per
// token.  On the 16-byte path each thread holds its
// 8-element chunks of all 4 streams in VGPRs, so the streams are read from HBM
// once: the sum of squares (when needed), the mixes and the collapse all use the
// same registers.  The whole workgroup sums the dot partials (staged through LDS,
// 64 splits at a time, in a fixed order), wavefront 0 computes rstd and the pre weights, and after the collapse the post weights and the 4x4
// Sinkhorn of comb, one matrix entry per lane of a 16-lane row.
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

constexpr int kDBlock = 256;
constexpr int kDWaves = kDBlock / kWave;

struct DotsArgs {
    const float *dot_mix; // [S][T][24], advanced to the launch's first token
    const float *sqrsum;  // [S][T], or null: computed from res (advanced likewise)
    int S;
    const uint16_t *res;
    const float *hc_scale;
    const float *hc_base;
    int T, H; // T: tokens of the whole call, the split arrays' split stride
    float k, rms_eps, pre_eps, sk_eps, post_mult;
    int iters;
    uint16_t *y;
    float *post, *comb, *pre_out;
};

// kCPT > 0: 16-byte path, kCPT chunks of 8 elements per thread and stream in VGPRs.
// kCPT == 0: any H and alignment, two scalar passes over the token's streams.
template <int kCPT>
__global__ __launch_bounds__(kDBlock) void pre_dots_kernel(DotsArgs a)
{
    __shared__ float wsum[kDWaves];
    __shared__ float dsum[kSplitFields]; // the summed dots, then the supplied sum of squares
    __shared__ float stage[kSplitStage * kSplitFields];
    __shared__ float wpart[4 * kSplitFields];
    __shared__ float prew[kHC];
    __shared__ float rstd_s;

    const int t = xcd_contiguous((int)blockIdx.x, (int)gridDim.x); // one token per workgroup
    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int H = a.H;
    const uint16_t *row = a.res + (size_t)t * kHC * H;
    const bool need_sq = a.sqrsum == nullptr;

    float sq = 0.0f;
    u32x4 r[kHC][kCPT > 0 ? kCPT : 1];
    if constexpr (kCPT > 0) {
        const int nch = H >> 3;
#pragma unroll
        for (int k = 0; k < kCPT; ++k) {
            const int j = tid + k * kDBlock;
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                r[i][k] = j < nch ? load16(row + (size_t)i * H + (size_t)j * 8) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        // the split partials, loaded while the streams are in flight
        sum_split_partials(a.dot_mix, a.sqrsum, a.S, a.T, t, stage, wpart, dsum);
        if (need_sq) {
#pragma unroll
            for (int k = 0; k < kCPT; ++k) {
#pragma unroll
                for (int i = 0; i < kHC; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // Copy to a scalar first: hipcc (clang 22) miscompiles __builtin_bit_cast
                        // applied directly to an ext_vector element (it reads element 0 for every q).
                        const uint32_t wq = r[i][k][q];
                        const bf16x2 pr = __builtin_bit_cast(bf16x2, wq);
                        sq = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, sq, false);
                    }
                }
            }
        }
    } else {
        sum_split_partials(a.dot_mix, a.sqrsum, a.S, a.T, t, stage, wpart, dsum);
        if (need_sq) {
            for (int h = tid; h < H; h += kDBlock) {
#pragma unroll
                for (int i = 0; i < kHC; ++i) {
                    const float v = bf16_to_f32(row[(size_t)i * H + h]);
                    sq = fmaf(v, v, sq);
                }
            }
        }
    }
    if (need_sq) {
        sq = wave_sum(sq);
        if (lane == 0) {
            wsum[w] = sq;
        }
    }
    __syncthreads();

    // rstd and the pre weights (wavefront 0)
    if (w == 0) {
        float S = 0.0f;
        if (need_sq) {
            S = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        } else {
            S = dsum[kMix];
        }
        const float rstd = 1.0f / sqrtf(S / a.k + a.rms_eps);
        if (lane < kHC) {
            prew[lane] = sigmoidf_fast(fmaf(dsum[lane] * rstd, a.hc_scale[0], a.hc_base[lane])) + a.pre_eps;
        }
        if (lane == 0) {
            rstd_s = rstd;
        }
    }
    __syncthreads();
    const float p0 = prew[0], p1 = prew[1], p2 = prew[2], p3 = prew[3];

    // collapse
    uint16_t *yrow = a.y + (size_t)t * H;
    if constexpr (kCPT > 0) {
        const int nch = H >> 3;
#pragma unroll
        for (int k = 0; k < kCPT; ++k) {
            const int j = tid + k * kDBlock;
            if (j < nch) {
                u32x4 yw;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float lo = bf16_lo(r[0][k][q]) * p0;
                    float hi = bf16_hi(r[0][k][q]) * p0;
                    lo = fmaf(bf16_lo(r[1][k][q]), p1, lo);
                    hi = fmaf(bf16_hi(r[1][k][q]), p1, hi);
                    lo = fmaf(bf16_lo(r[2][k][q]), p2, lo);
                    hi = fmaf(bf16_hi(r[2][k][q]), p2, hi);
                    lo = fmaf(bf16_lo(r[3][k][q]), p3, lo);
                    hi = fmaf(bf16_hi(r[3][k][q]), p3, hi);
                    yw[q] = pack_bf16x2(lo, hi);
                }
                store_nt16(yrow + (size_t)j * 8, yw);
            }
        }
    } else {
        for (int h = tid; h < H; h += kDBlock) {
            float v = bf16_to_f32(row[h]) * p0;
            v = fmaf(bf16_to_f32(row[(size_t)H + h]), p1, v);
            v = fmaf(bf16_to_f32(row[(size_t)2 * H + h]), p2, v);
            v = fmaf(bf16_to_f32(row[(size_t)3 * H + h]), p3, v);
            yrow[h] = f32_to_bf16(v);
        }
    }

    // post, comb and the optional pre output (wavefront 0)
    if (w == 0) {
        const float rstd = rstd_s;
        const int e = lane & 15;
        const float L = fmaf(dsum[2 * kHC + e] * rstd, a.hc_scale[2], a.hc_base[2 * kHC + e]);
        const float P = sinkhorn_row16(L, a.iters, a.sk_eps);
        if (lane < kHC * kHC) {
            a.comb[(size_t)t * kHC * kHC + lane] = P;
        }
        if (lane < kHC) {
            a.post[(size_t)t * kHC + lane] =
                sigmoidf_fast(fmaf(dsum[kHC + lane] * rstd, a.hc_scale[1], a.hc_base[kHC + lane])) * a.post_mult;
            if (a.pre_out) {
                a.pre_out[(size_t)t * kHC + lane] = prew[lane];
            }
        }
    }
}

} // namespace

hipError_t launch_pre_dots(const float *dot_mix, const float *sqrsum, int num_splits, const uint16_t *res,
                           const float *hc_scale, const float *hc_base, int64_t T, int64_t H, float k,
                           float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int iters,
                           uint16_t *y, float *post, float *comb, float *pre, hipStream_t stream, bool vec8)
{
    if (vec8 && num_splits == 1 && sqrsum != nullptr) {
        // nothing to reduce per token: the collapse kernel's one-wave-per-tile layout
        return launch_collapse_dots(dot_mix, sqrsum, res, hc_scale, hc_base, T, H, k, rms_eps, pre_eps,
                                    sinkhorn_eps, post_mult, iters, y, post, comb, pre, stream);
    }
    const int64_t per = (H / 8 + kDBlock - 1) / kDBlock; // 16-byte chunks per thread and stream
    return for_token_chunks(T, pre_dots_items_per_token(), [&](int64_t c0, int64_t Tc) {
        DotsArgs a{};
        a.dot_mix = dot_mix + (size_t)c0 * kMix; // split s of token c0 + t at ((s * T) + t) * 24
        a.sqrsum = sqrsum ? sqrsum + c0 : nullptr;
        a.S = num_splits;
        a.res = res + (size_t)c0 * kHC * H;
        a.hc_scale = hc_scale;
        a.hc_base = hc_base;
        a.T = (int)T;
        a.H = (int)H;
        a.k = k;
        a.rms_eps = rms_eps;
        a.pre_eps = pre_eps;
        a.sk_eps = sinkhorn_eps;
        a.post_mult = post_mult;
        a.iters = iters;
        a.y = y + (size_t)c0 * H;
        a.post = post + (size_t)c0 * kHC;
        a.comb = comb + (size_t)c0 * kHC * kHC;
        a.pre_out = pre ? pre + (size_t)c0 * kHC : nullptr;
        const dim3 grid((unsigned)Tc), block(kDBlock);
        if (vec8 && per <= 1) {
            pre_dots_kernel<1><<<grid, block, 0, stream>>>(a);
        } else if (vec8 && per <= 2) {
            pre_dots_kernel<2><<<grid, block, 0, stream>>>(a);
        } else if (vec8 && per <= 4) {
            pre_dots_kernel<4><<<grid, block, 0, stream>>>(a);
        } else if (vec8 && per <= 8) {
            pre_dots_kernel<8><<<grid, block, 0, stream>>>(a);
        } else {
            pre_dots_kernel<0><<<grid, block, 0, stream>>>(a);
        }
        return hipGetLastError();
    });
}

int64_t pre_dots_items_per_token() { return kDBlock; }

} // namespace mhc
