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

// Reverse mode of one matrix held by a 16-lane row (lane e: entry (e / 4, e % 4)):
// returns dL for logit L and output gradient G.  `hist` points at this lane's
// column of an [iters + 1][kSBBlock] LDS history; every lane of the wave runs it.
__device__ __forceinline__ float sinkhorn_row16_backward(float L, float G, int iters, float eps, float *hist)
{
    float mx = fmaxf(L, dpp_quad_xor1(L));
    mx = fmaxf(mx, dpp_quad_xor2(mx));
    const float ex = __expf(L - mx);
    const float S = ex * fast_rcp(row_sum4(ex));
    float P = S + eps;
    hist[0] = P;
    for (int k = 1; k <= iters; ++k) {
        const float A = P * fast_rcp(row_sum4(P));
        P = A * fast_rcp(col_sum4(A));
        hist[k * kSBBlock] = P;
    }
    // each lane reads back only what it wrote itself; P holds the matrix after
    // iteration k at the top of each step
    for (int k = iters; k >= 1; --k) {
        const float Q = P;
        P = hist[(k - 1) * kSBBlock];
        const float rinv = fast_rcp(row_sum4(P));
        const float A = P * rinv;
        const float dA = (G - col_sum4(G * Q)) * fast_rcp(col_sum4(A));
        G = (dA - row_sum4(dA * A)) * rinv;
    }
    return S * (G - row_sum4(G * S));
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
    const float dL = sinkhorn_row16_backward(L, G, iters, eps, hist + tid);
    if (live) {
        d_logits[gl] = dL;
    }
}

// ---------------------------------------------------------------- pre-map backward (external dots)
//
// One 256-thread workgroup per token, the reverse of pre_dots_kernel:
//   d_pre_i = sum_h dy[h] res_i[h]         (block reduction, with S = sum res^2 when not supplied)
//   wavefront 0: dots, S, rstd, m, z as in the forward; dz for pre (sigmoid'), post
//   (post_mult sigmoid') and comb (Sinkhorn reverse mode on lanes 0..15); dm = dz s_g,
//   d_dot = dm rstd, d_rstd = sum_r dm d_r, dS = -d_rstd rstd^3 / (2k)
//   d_res_i[h] = pre_i dy[h] + 2 dS res_i[h]   (the second term only when S was computed here)
// The token's dz_r (24) and sum over each group of dz_r m_r (3) go to a workspace row
// that pre_bwd_partial_kernel and pre_bwd_final_kernel sum over the tokens.
constexpr int kDBBlock = 256;
constexpr int kDBWaves = kDBBlock / kWave;
constexpr int kWsRow = 28; // floats per token in the workspace: 24 dz, 3 group sums, 1 pad

struct DotsBwdArgs {
    const uint16_t *dy;
    const float *d_post, *d_comb;
    const float *dot_mix; // [S][T][24]
    const float *sqrsum;  // [S][T] or null
    int S;
    const uint16_t *res;
    const float *hc_scale, *hc_base;
    int T, H;
    float k, rms_eps, pre_eps, sk_eps, post_mult;
    int iters;
    uint16_t *d_res;
    float *d_dot, *d_sqrsum;
    float *ws; // [T][kWsRow]
};

template <int kCPT>
__global__ __launch_bounds__(kDBBlock) void pre_dots_bwd_kernel(DotsBwdArgs a)
{
    extern __shared__ float hist[]; // [iters + 1][64], wavefront 0's Sinkhorn history
    __shared__ float part[kDBWaves][kHC + 1];
    __shared__ float dsum[kMix];
    __shared__ float bc[kHC + 1]; // pre weights, then the coefficient of res in d_res

    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int H = a.H;
    const uint16_t *row = a.res + (size_t)t * kHC * H;
    const uint16_t *grow = a.dy + (size_t)t * H;
    const bool need_sq = a.sqrsum == nullptr;

    float dv = 0.0f;
    if (w == 0 && lane < kMix) {
        for (int s = 0; s < a.S; ++s) {
            dv += a.dot_mix[((size_t)s * a.T + t) * kMix + lane];
        }
    }

    float dp[kHC] = {0.0f, 0.0f, 0.0f, 0.0f};
    float sq = 0.0f;
    u32x4 r[kHC][kCPT > 0 ? kCPT : 1], g[kCPT > 0 ? kCPT : 1];
    if constexpr (kCPT > 0) {
        const int nch = H >> 3;
#pragma unroll
        for (int k = 0; k < kCPT; ++k) {
            const int j = tid + k * kDBBlock;
            const bool in = j < nch;
            g[k] = in ? load16(grow + (size_t)j * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                r[i][k] = in ? load16(row + (size_t)i * H + (size_t)j * 8) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int k = 0; k < kCPT; ++k) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // copy each element to a scalar before reinterpreting it
                const uint32_t gq = g[k][q];
                const bf16x2 gp = __builtin_bit_cast(bf16x2, gq);
#pragma unroll
                for (int i = 0; i < kHC; ++i) {
                    const uint32_t rq = r[i][k][q];
                    const bf16x2 rp = __builtin_bit_cast(bf16x2, rq);
                    dp[i] = __builtin_amdgcn_fdot2_f32_bf16(gp, rp, dp[i], false);
                    if (need_sq) {
                        sq = __builtin_amdgcn_fdot2_f32_bf16(rp, rp, sq, false);
                    }
                }
            }
        }
    } else {
        for (int h = tid; h < H; h += kDBBlock) {
            const float gv = bf16_to_f32(grow[h]);
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                const float v = bf16_to_f32(row[(size_t)i * H + h]);
                dp[i] = fmaf(gv, v, dp[i]);
                sq = fmaf(v, v, sq);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        dp[i] = wave_sum(dp[i]);
    }
    sq = wave_sum(sq);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
            part[w][i] = dp[i];
        }
        part[w][kHC] = sq;
    }
    if (w == 0 && lane < kMix) {
        dsum[lane] = dv;
    }
    __syncthreads();

    if (w == 0) {
        float S = 0.0f;
        if (need_sq) {
            S = (part[0][kHC] + part[1][kHC]) + (part[2][kHC] + part[3][kHC]);
        } else {
            for (int s = 0; s < a.S; ++s) {
                S += a.sqrsum[(size_t)s * a.T + t];
            }
        }
        const float rstd = 1.0f / sqrtf(S / a.k + a.rms_eps);
        // comb: Sinkhorn reverse mode, entry e = lane & 15 on every 16-lane row (each row
        // computes the same matrix); lane 8 + e then takes entry e from lane e
        const int e = lane & 15;
        const float Lc = fmaf(dsum[2 * kHC + e] * rstd, a.hc_scale[2], a.hc_base[2 * kHC + e]);
        const float Gc = a.d_comb[(size_t)t * kHC * kHC + e];
        const float dLc = sinkhorn_row16_backward(Lc, Gc, a.iters, a.sk_eps, hist + lane);
        const float dLmine = __shfl(dLc, (lane - 2 * kHC) & 15);
        // lanes 0..23: one mix each
        const int grp = lane < kHC ? 0 : (lane < 2 * kHC ? 1 : 2);
        float dz = 0.0f, m = 0.0f, dm = 0.0f, d = 0.0f;
        if (lane < kMix) {
            d = dsum[lane];
            m = d * rstd;
            if (lane < 2 * kHC) {
                const float sg = sigmoidf_fast(fmaf(m, a.hc_scale[grp], a.hc_base[lane]));
                if (lane < kHC) {
                    const float dpre = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
                    dz = dpre * sg * (1.0f - sg);
                    bc[lane] = sg + a.pre_eps;
                } else {
                    dz = a.d_post[(size_t)t * kHC + lane - kHC] * a.post_mult * sg * (1.0f - sg);
                }
            } else {
                dz = dLmine;
            }
            dm = dz * a.hc_scale[grp];
            a.d_dot[(size_t)t * kMix + lane] = dm * rstd;
        }
        const float d_rstd = wave_sum(dm * d);
        const float dS = -d_rstd * rstd * rstd * rstd / (2.0f * a.k);
        float *wrow = a.ws + (size_t)t * kWsRow;
        const float zm = dz * m;
        // per-group sums of dz * m over lanes 0..3, 4..7 and 8..23 (fixed order)
        const float g0 = wave_sum(lane < kHC ? zm : 0.0f);
        const float g1 = wave_sum(lane >= kHC && lane < 2 * kHC ? zm : 0.0f);
        const float g2 = wave_sum(lane >= 2 * kHC && lane < kMix ? zm : 0.0f);
        if (lane < kMix) {
            wrow[lane] = dz;
        }
        if (lane == 0) {
            wrow[kMix] = g0;
            wrow[kMix + 1] = g1;
            wrow[kMix + 2] = g2;
            wrow[kMix + 3] = 0.0f;
            if (need_sq) {
                bc[kHC] = 2.0f * dS;
            } else {
                bc[kHC] = 0.0f;
                a.d_sqrsum[t] = dS;
            }
        }
    }
    __syncthreads();
    const float p0 = bc[0], p1 = bc[1], p2 = bc[2], p3 = bc[3], cr = bc[kHC];
    const float pw[kHC] = {p0, p1, p2, p3};

    uint16_t *drow = a.d_res + (size_t)t * kHC * H;
    if constexpr (kCPT > 0) {
        const int nch = H >> 3;
#pragma unroll
        for (int k = 0; k < kCPT; ++k) {
            const int j = tid + k * kDBBlock;
            if (j < nch) {
#pragma unroll
                for (int i = 0; i < kHC; ++i) {
                    u32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t gq = g[k][q], rq = r[i][k][q];
                        const float lo = fmaf(bf16_lo(rq), cr, bf16_lo(gq) * pw[i]);
                        const float hi = fmaf(bf16_hi(rq), cr, bf16_hi(gq) * pw[i]);
                        o[q] = pack_bf16x2(lo, hi);
                    }
                    store_nt16(drow + (size_t)i * H + (size_t)j * 8, o);
                }
            }
        }
    } else {
        for (int h = tid; h < H; h += kDBBlock) {
            const float gv = bf16_to_f32(grow[h]);
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                const float v = bf16_to_f32(row[(size_t)i * H + h]);
                drow[(size_t)i * H + h] = f32_to_bf16(fmaf(v, cr, gv * pw[i]));
            }
        }
    }
}

// d_hc_base[c] (c < 24) and d_hc_scale[c - 24] (c = 24..26) are the sums over the
// tokens of workspace column c, in two fixed-order passes.  Pass 1: one workgroup per
// 256 tokens; thread j reads token j's row, each wavefront reduces every column
// (butterfly), and the 4 wavefront sums are added in order into the block's partial
// row.  Pass 2: one thread per column adds the block partials in block order.
constexpr int kRedTok = 256;

__global__ __launch_bounds__(kRedTok) void pre_bwd_partial_kernel(const float *__restrict__ ws, int64_t T,
                                                                  float *__restrict__ part_out)
{
    __shared__ float wsum[kRedTok / kWave][kWsRow];
    const int tid = threadIdx.x;
    const int64_t t = (int64_t)blockIdx.x * kRedTok + tid;
    float v[kWsRow];
    if (t < T) {
        const f32x4 *row = reinterpret_cast<const f32x4 *>(ws + (size_t)t * kWsRow);
#pragma unroll
        for (int q = 0; q < kWsRow / 4; ++q) {
            const f32x4 x = row[q];
            v[4 * q] = x[0];
            v[4 * q + 1] = x[1];
            v[4 * q + 2] = x[2];
            v[4 * q + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int c = 0; c < kWsRow; ++c) {
            v[c] = 0.0f;
        }
    }
#pragma unroll
    for (int c = 0; c < kWsRow; ++c) {
        v[c] = wave_sum(v[c]);
    }
    if ((tid & (kWave - 1)) == 0) {
#pragma unroll
        for (int c = 0; c < kWsRow; ++c) {
            wsum[tid >> 6][c] = v[c];
        }
    }
    __syncthreads();
    if (tid < kWsRow) {
        part_out[(size_t)blockIdx.x * kWsRow + tid] = (wsum[0][tid] + wsum[1][tid]) + (wsum[2][tid] + wsum[3][tid]);
    }
}

__global__ __launch_bounds__(64) void pre_bwd_final_kernel(const float *__restrict__ part, int64_t nblk,
                                                           float *__restrict__ d_hc_scale,
                                                           float *__restrict__ d_hc_base)
{
    const int c = threadIdx.x;
    if (c >= kMix + 3) {
        return;
    }
    // eight independent loads in flight per step; the additions keep block order
    float v = 0.0f;
    int64_t b = 0;
    for (; b + 8 <= nblk; b += 8) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            e[j] = part[(size_t)(b + j) * kWsRow + c];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v += e[j];
        }
    }
    for (; b < nblk; ++b) {
        v += part[(size_t)b * kWsRow + c];
    }
    if (c < kMix) {
        d_hc_base[c] = v;
    } else {
        d_hc_scale[c - kMix] = v;
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

// Workspace: the [T][28] token rows, then the [ceil(T / 256)][28] block partials.
static size_t pre_bwd_rows_bytes(int64_t T) { return ((size_t)T * kWsRow * sizeof(float) + 255) & ~(size_t)255; }
size_t pre_bwd_workspace_bytes(int64_t T)
{
    const int64_t nblk = (T + kRedTok - 1) / kRedTok;
    return pre_bwd_rows_bytes(T) + (((size_t)nblk * kWsRow * sizeof(float) + 255) & ~(size_t)255);
}

hipError_t launch_pre_dots_bwd(const uint16_t *dy, const float *d_post, const float *d_comb, const float *dot_mix,
                               const float *sqrsum, int num_splits, const uint16_t *res, const float *hc_scale,
                               const float *hc_base, int64_t T, int64_t H, float k, float rms_eps, float pre_eps,
                               float sinkhorn_eps, float post_mult, int iters, uint16_t *d_res, float *d_dot,
                               float *d_sqrsum, float *d_hc_scale, float *d_hc_base, void *workspace,
                               hipStream_t stream, bool vec8)
{
    float *ws = reinterpret_cast<float *>(workspace);
    if (T > 0) {
        DotsBwdArgs a;
        a.dy = dy;
        a.d_post = d_post;
        a.d_comb = d_comb;
        a.dot_mix = dot_mix;
        a.sqrsum = sqrsum;
        a.S = num_splits;
        a.res = res;
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
        a.d_res = d_res;
        a.d_dot = d_dot;
        a.d_sqrsum = d_sqrsum;
        a.ws = ws;
        const dim3 grid((unsigned)T), block(kDBBlock);
        const size_t lds = (size_t)(iters + 1) * kWave * sizeof(float);
        const int64_t per = (H / 8 + kDBBlock - 1) / kDBBlock;
        if (vec8 && per <= 1) {
            pre_dots_bwd_kernel<1><<<grid, block, lds, stream>>>(a);
        } else if (vec8 && per <= 2) {
            pre_dots_bwd_kernel<2><<<grid, block, lds, stream>>>(a);
        } else if (vec8 && per <= 4) {
            pre_dots_bwd_kernel<4><<<grid, block, lds, stream>>>(a);
        } else if (vec8 && per <= 8) {
            pre_dots_bwd_kernel<8><<<grid, block, lds, stream>>>(a);
        } else {
            pre_dots_bwd_kernel<0><<<grid, block, lds, stream>>>(a);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
    }
    const int64_t nblk = (T + kRedTok - 1) / kRedTok;
    float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + pre_bwd_rows_bytes(T));
    if (nblk > 0) {
        pre_bwd_partial_kernel<<<dim3((unsigned)nblk), dim3(kRedTok), 0, stream>>>(ws, T, part);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
    }
    pre_bwd_final_kernel<<<dim3(1), dim3(64), 0, stream>>>(part, nblk, d_hc_scale, d_hc_base);
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
