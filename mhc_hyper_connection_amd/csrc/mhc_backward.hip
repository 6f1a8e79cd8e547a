// mhc_backward.hip -- reverse mode of the mHC path: the Sinkhorn projection, the
// post-map, the pre-map from external dots, and the whole pre-map with its projection
// inside (the projection's fields recomputed together with <dy, res_i>, the per-token
// chain, then the projection's reverse products).
//
// (rwkv-ops mhu_jax.py: sinkhorn_knopp, mhc_pre_op and mhc_post_op with their custom
// VJPs, SinkhornBwd, MhcPreOpBwd and MhcPostOpBwd; the forward formulas are those of the
// FlashInfer mHC article, sections 2.1, 3.2 and 5.2.)
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_view_b(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

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
    const float *dot_mix; // [S][T][24], advanced to the launch's first token
    const float *sqrsum;  // [S][T] or null (advanced likewise)
    int S;
    const uint16_t *res;
    const float *hc_scale, *hc_base;
    int T, H; // T: tokens of the whole call, the split arrays' split stride
    float k, rms_eps, pre_eps, sk_eps, post_mult;
    int iters;
    uint16_t *d_res;
    float *d_dot, *d_sqrsum;
    float *ws; // [T][kWsRow]
    // pre_tok_bwd_kernel (the reverse of the whole pre-map): the per-token fields come
    // from the projection's recompute, and instead of d_res it writes pre and 2 dS
    // ([T][8]) and d_dot as bf16 hi and lo halves, both row-major [T][32] and
    // transposed [32][ldT] (rows 24..31 zero).
    const float *sums; // [T][32]
    float *tok;
    uint16_t *dd_hi, *dd_lo, *ddT_hi, *ddT_lo;
    int ldT;
};

// The projection's per-token fields: pre dots 0..3, the sum of squares at 4, then
// post and comb dots.
__device__ __forceinline__ int sums_field(int col) { return col < kHC ? col : col + 1; }

template <int kCPT>
__global__ __launch_bounds__(kDBBlock) void pre_dots_bwd_kernel(DotsBwdArgs a)
{
    extern __shared__ float hist[]; // [iters + 1][64], wavefront 0's Sinkhorn history
    __shared__ float part[kDBWaves][kHC + 1];
    __shared__ float dsum[kSplitFields]; // the summed dots, then the supplied sum of squares
    __shared__ float stage[kSplitStage * kSplitFields];
    __shared__ float wpart[4 * kSplitFields];
    __shared__ float bc[kHC + 1]; // pre weights, then the coefficient of res in d_res

    const int t = xcd_contiguous((int)blockIdx.x, (int)gridDim.x); // one token per workgroup
    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int H = a.H;
    const uint16_t *row = a.res + (size_t)t * kHC * H;
    const uint16_t *grow = a.dy + (size_t)t * H;
    // S computed here from the streams (the RMS term of d_res applies), or supplied
    const bool need_sq = a.sqrsum == nullptr;

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
        // the split partials, loaded while the streams are in flight
        sum_split_partials(a.dot_mix, a.sqrsum, a.S, a.T, t, stage, wpart, dsum);
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
        sum_split_partials(a.dot_mix, a.sqrsum, a.S, a.T, t, stage, wpart, dsum);
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
    __syncthreads();

    if (w == 0) {
        float S = 0.0f;
        if (need_sq) {
            S = (part[0][kHC] + part[1][kHC]) + (part[2][kHC] + part[3][kHC]);
        } else {
            S = dsum[kMix];
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

// The whole pre-map's per-token reverse, after the projection's recompute left each
// token's fields in `sums` ([T][32]: pre dots 0..3, S at 4, post dots 5..8, comb dots
// 9..24, <dy, res_i> at 25..28).  The chain is that of pre_dots_bwd_kernel's wavefront
// 0 with S taken from the streams (the RMS term of d_res applies).  Four tokens per
// wavefront, one per 16-lane row: lane e of a row takes comb entry e (its Sinkhorn
// reverse on the row), and lanes e < 4 also pre_e and post_e; sums over a token's mixes
// are DPP sums over its row.  It writes pre and 2 dS, the dot gradients as bf16 hi + lo
// halves (row-major and transposed) for the projection's reverse, and the token's row
// of the d_hc_scale / d_hc_base sums.  No stream is read here.
constexpr int kSumsDy = kMix + 1; // first <dy, res_i> field in the sums

// Sum over the 16 lanes of a DPP row (every lane gets it): quads, then across them.
__device__ __forceinline__ float row16_sum(float v) { return col_sum4(row_sum4(v)); }

__device__ __forceinline__ void put_dd(const DotsBwdArgs &a, int t, int col, float v)
{
    const uint16_t hi = f32_to_bf16(v);
    const uint16_t lo = f32_to_bf16(v - bf16_to_f32(hi));
    a.dd_hi[(size_t)t * 32 + col] = hi;
    a.dd_lo[(size_t)t * 32 + col] = lo;
    a.ddT_hi[(size_t)col * a.ldT + t] = hi;
    a.ddT_lo[(size_t)col * a.ldT + t] = lo;
}

__global__ __launch_bounds__(kWave) void pre_tok_bwd_kernel(DotsBwdArgs a)
{
    extern __shared__ float hist[]; // [iters + 1][64]: the Sinkhorn history
    const int lane = threadIdx.x;
    const int e = lane & 15;
    const int t_row = blockIdx.x * 4 + (lane >> 4);
    const bool live = t_row < a.T; // uniform within each row
    const int t = live ? t_row : a.T - 1;
    const float *sm = a.sums + (size_t)t * 32;
    const float rstd = 1.0f / sqrtf(sm[kHC] / a.k + a.rms_eps);
    const float s0 = a.hc_scale[0], s1 = a.hc_scale[1], s2 = a.hc_scale[2];
    // comb entry e (mix 8 + e)
    const float dc = sm[sums_field(2 * kHC + e)];
    const float mc = dc * rstd;
    const float Lc = fmaf(mc, s2, a.hc_base[2 * kHC + e]);
    const float Gc = a.d_comb[(size_t)t * kHC * kHC + e];
    const float dzc = sinkhorn_row16_backward(Lc, Gc, a.iters, a.sk_eps, hist + lane);
    const float dmc = dzc * s2;
    // pre_e and post_e on lanes e < 4
    float dzp = 0.0f, mp = 0.0f, dmp = 0.0f, dp = 0.0f, pw = 0.0f;
    float dzq = 0.0f, mq = 0.0f, dmq = 0.0f, dq = 0.0f;
    const int eq = e & (kHC - 1);
    {
        dp = sm[sums_field(eq)];
        mp = dp * rstd;
        const float sg = sigmoidf_fast(fmaf(mp, s0, a.hc_base[eq]));
        dzp = sm[kSumsDy + eq] * sg * (1.0f - sg);
        pw = sg + a.pre_eps;
        dq = sm[sums_field(kHC + eq)];
        mq = dq * rstd;
        const float sq = sigmoidf_fast(fmaf(mq, s1, a.hc_base[kHC + eq]));
        dzq = a.d_post[(size_t)t * kHC + eq] * a.post_mult * sq * (1.0f - sq);
        if (e >= kHC) {
            dzp = 0.0f;
            dzq = 0.0f;
        }
        dmp = dzp * s0;
        dmq = dzq * s1;
    }
    // d_rstd = sum over the 24 mixes of dm * dot; the group sums of dz * m
    const float d_rstd = row16_sum(dmc * dc + (dmp * dp + dmq * dq));
    const float g0 = row16_sum(dzp * mp);
    const float g1 = row16_sum(dzq * mq);
    const float g2 = row16_sum(dzc * mc);
    const float dS = -d_rstd * rstd * rstd * rstd / (2.0f * a.k);
    if (!live) {
        return;
    }
    put_dd(a, t, 2 * kHC + e, dmc * rstd);
    float *wrow = a.ws + (size_t)t * kWsRow;
    wrow[2 * kHC + e] = dzc;
    if (e < kHC) {
        put_dd(a, t, e, dmp * rstd);
        put_dd(a, t, kHC + e, dmq * rstd);
        wrow[e] = dzp;
        wrow[kHC + e] = dzq;
        a.tok[(size_t)t * 8 + e] = pw;
    } else if (e < 2 * kHC) {
        a.tok[(size_t)t * 8 + e] = e == kHC ? 2.0f * dS : 0.0f;
    } else {
        put_dd(a, t, kMix + e - 2 * kHC, 0.0f); // d_dot rows 24..31 of the MFMA tiles: zero
    }
    if (e == 0) {
        wrow[kMix] = g0;
        wrow[kMix + 1] = g1;
        wrow[kMix + 2] = g2;
        wrow[kMix + 3] = 0.0f;
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

// ---------------------------------------------------------------- the projection's reverse
//
// dot[t][r] = sum_k W[r][k] res_flat[t][k] (k = i*H + h) gives
//   d_res_flat[t][k] += sum_r dd[t][r] W[r][k]      and      d_W[r][k] = sum_t dd[t][r] res_flat[t][k].
// One workgroup owns one stream i, a strip of 256 consecutive h and a range of tokens,
// walked in 32-token chunks.  Each chunk's streams, dy, dd, dd^T and token scalars come
// in with whole-row 16-byte loads (512 contiguous bytes per row) and go to LDS; the 4
// wavefronts then do the MFMA work on 64 columns each, reading their operands from LDS,
// and the d_res tile leaves through LDS as whole rows again.  The next chunk's loads
// are in flight (in registers) while the current chunk is worked on.
//   d_res: v_mfma_f32_16x16x32_bf16 with A = W^T (64 columns x 32 logit rows, rows
//     24..31 zero) and B = dd (logit rows x 16 tokens); W and dd each as bf16 hi + lo,
//     three products (hi hi, hi lo, lo hi).  The MFMA row order inside a 64-column block
//     is permuted so that result register q of tile j in lane (g, c) is h = 16g + 4j + q
//     of token c: each lane ends with 16 consecutive h of one token, which it combines
//     with pre_i dy + 2 dS res and writes back over dy in LDS.
//   d_W: A = dd^T (logit rows x 32 tokens, hi and lo), B = res (32 tokens x 16 columns),
//     read transposed from the LDS tile; the accumulators stay in VGPRs over the token
//     range and give one partial per (column block, token range), summed over the
//     ranges in order by a second kernel.
// The 16-byte pieces of an LDS tile row are XOR-swizzled by a function of the row, so
// that the 16-byte MFMA-operand reads (16 rows, one piece each) and the transposed
// 2-byte reads (rows 8g + r over g, 2 pieces) both fall on distinct banks.
constexpr int kPBCols = 64;                 // columns per wavefront
constexpr int kPBStrip = 4 * kPBCols;       // columns per workgroup
constexpr int kPBChunk = 32;                // tokens per step
constexpr int kPBRowB = kPBStrip * 2;       // bytes per LDS tile row
constexpr int kPBTile = kPBChunk * kPBRowB; // 16 KiB
constexpr int kPBSmallRow = 80;             // bytes per LDS dd / dd^T row (64 + 16: conflict-free 16-byte reads)
constexpr int kPBSmall = kPBChunk * kPBSmallRow;
constexpr int kPBOffRes = 0;                      // streams tile
constexpr int kPBOffDy = kPBOffRes + kPBTile;     // 2 dy tiles (d_res written over them)
constexpr int kPBOffDd = kPBOffDy + 2 * kPBTile;  // dd hi, dd lo: [token][32 rows]
constexpr int kPBOffDdT = kPBOffDd + 2 * kPBSmall; // dd^T hi, lo: [row][32 tokens]
constexpr int kPBOffTok = kPBOffDdT + 2 * kPBSmall; // [token][8] floats
constexpr int kPBSmem = kPBOffTok + kPBChunk * 8 * 4;
constexpr int kPBTargetBlocks = 1024; // about 2 rounds of 2 workgroups per CU

struct ProjBwdArgs {
    const uint16_t *dy, *res;
    const float *tok;              // [T][8]: pre[4], 2 dS
    const uint16_t *dd_hi, *dd_lo;   // [T][32]
    const uint16_t *ddT_hi, *ddT_lo; // [32][ldT]
    const u32x4 *wfrag;            // [blocks][4 tiles][2 terms][64 lanes]
    int T, H, ldT, nbh, nstrip, nblocks, tok_per_split;
    uint16_t *d_res;
    float *dw_part;                // [splits][24][4H]
};

// W^T fragments in the permuted MFMA row order: one thread per (block, tile, lane);
// term 0 = hi, term 1 = lo of the fp32 weight.  The same threads also zero the
// dd^T columns T .. ldT - 1, so that the main kernel reads whole 8-token pieces of
// dd^T with no tail test (the pad multiplies zero streams; it must only be finite).
__global__ __launch_bounds__(256) void proj_bwd_wfrag_kernel(const float *__restrict__ hc_fn, int H, int nbh,
                                                             u32x4 *__restrict__ wfrag, int T, int ldT,
                                                             uint16_t *__restrict__ ddT_hi,
                                                             uint16_t *__restrict__ ddT_lo)
{
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int pad = ldT - T; // 0 .. 31
    if (gid < 32 * pad) {
        const size_t at = (size_t)(gid / pad) * ldT + T + gid % pad;
        ddT_hi[at] = 0;
        ddT_lo[at] = 0;
    }
    const int nblk = kHC * nbh;
    if (gid >= nblk * 4 * kWave) {
        return;
    }
    const int l = gid & (kWave - 1);
    const int j = (gid >> 6) & 3;
    const int b = gid >> 8;
    const int i = b / nbh, h0 = (b - i * nbh) * kPBCols;
    const int m = l & 15, rg = l >> 4;
    const int h = h0 + 16 * (m >> 2) + 4 * j + (m & 3);
    u32x4 hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float v[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int r = 8 * rg + 2 * q + e;
            v[e] = (r < kMix && h < H) ? hc_fn[(size_t)r * kHC * H + (size_t)i * H + h] : 0.0f;
        }
        const uint16_t h0b = f32_to_bf16(v[0]), h1b = f32_to_bf16(v[1]);
        hi[q] = (uint32_t)h0b | ((uint32_t)h1b << 16);
        lo[q] = (uint32_t)f32_to_bf16(v[0] - bf16_to_f32(h0b)) |
                ((uint32_t)f32_to_bf16(v[1] - bf16_to_f32(h1b)) << 16);
    }
    wfrag[((size_t)(b * 4 + j) * 2 + 0) * kWave + l] = hi;
    wfrag[((size_t)(b * 4 + j) * 2 + 1) * kWave + l] = lo;
}

// Byte offset of 16-byte piece `ch` (0..31) of row t in an LDS tile.  Over any 16
// consecutive rows from a multiple of 16 the swizzle takes every value 0..15 once, and
// over rows 8g + r (g = 0..3, r fixed) its top three bits differ.
__device__ __forceinline__ int pb_at(int t, int ch)
{
    const int swz = (t & 15) ^ (2 * ((t >> 3) & 3));
    return t * kPBRowB + ((ch ^ swz) << 4);
}

__device__ __forceinline__ u32x4 lds16(const unsigned char *smem, int off)
{
    return *reinterpret_cast<const u32x4 *>(smem + off);
}

// One chunk's loads, held in registers until they go to LDS.  Thread tid takes piece
// tid & 31 of tile rows (tid >> 5) + 8k; piece tid & 127 of dd and of dd^T (hi for
// wavefronts 0 and 1, lo for 2 and 3); piece tid & 63 of the token scalars.
struct ProjBwdStage {
    u32x4 r[4], d[4];
    u32x4 dd, ddT, tk;
};

__device__ __forceinline__ void pb_issue(const ProjBwdArgs &a, int t0, int te, int i, int tid, int w, uint32_t colo,
                                         ProjBwdStage &P)
{
    const int H = a.H;
    const int ntok = min(kPBChunk, te - t0);
    const __amdgpu_buffer_rsrc_t vres =
        buf_view_b(a.res + (size_t)t0 * kHC * H, (uint32_t)((size_t)ntok * kHC * H * 2));
    const __amdgpu_buffer_rsrc_t vdy = buf_view_b(a.dy + (size_t)t0 * H, (uint32_t)((size_t)ntok * H * 2));
    const int row0 = tid >> 5;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int row = row0 + 8 * k;
        P.r[k] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, (int)((uint32_t)((row * kHC + i) * H) * 2u + colo), 0, 0));
        P.d[k] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(vdy, (int)((uint32_t)(row * H) * 2u + colo), 0, 0));
    }
    const int hl = w >> 1, pc = tid & 127;
    // past the range dd and the token scalars read as zero; dd^T columns up to ldT exist
    // (t0 is a multiple of 32 below T) and are zero past T
    const __amdgpu_buffer_rsrc_t vdd = buf_view_b((hl ? a.dd_lo : a.dd_hi) + (size_t)t0 * 32, (uint32_t)(ntok * 64));
    P.dd = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vdd, pc * 16, 0, 0));
    P.ddT = *reinterpret_cast<const u32x4 *>((hl ? a.ddT_lo : a.ddT_hi) + (size_t)(pc >> 2) * a.ldT + t0 +
                                              8 * (pc & 3));
    const __amdgpu_buffer_rsrc_t vtok = buf_view_b(a.tok + (size_t)t0 * 8, (uint32_t)(ntok * 32));
    P.tk = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vtok, (tid & 63) * 16, 0, 0));
}

__device__ __forceinline__ void pb_commit(unsigned char *smem, const ProjBwdStage &P, int slot, int tid, int w)
{
    const int row0 = tid >> 5, ch = tid & 31;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int at = pb_at(row0 + 8 * k, ch);
        *reinterpret_cast<u32x4 *>(smem + kPBOffRes + at) = P.r[k];
        *reinterpret_cast<u32x4 *>(smem + kPBOffDy + slot * kPBTile + at) = P.d[k];
    }
    const int hl = w >> 1, pc = tid & 127;
    const int so = hl * kPBSmall + (pc >> 2) * kPBSmallRow + (pc & 3) * 16;
    *reinterpret_cast<u32x4 *>(smem + kPBOffDd + so) = P.dd;
    *reinterpret_cast<u32x4 *>(smem + kPBOffDdT + so) = P.ddT;
    if (w == 0) {
        *reinterpret_cast<u32x4 *>(smem + kPBOffTok + tid * 16) = P.tk;
    }
}

__global__ __launch_bounds__(256, 2) void proj_bwd_kernel(ProjBwdArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char smem[kPBSmem];

    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int g = lane >> 4, c = lane & 15;
    // workgroup -> (stream i, unit u = strip + nstrip * range); blocks are dealt to the 8
    // XCDs in turn, so this sends the four streams of a unit to one XCD back to back,
    // where they share its dy and dd reads in L2
    const int L = blockIdx.x;
    const int n32 = a.nblocks & ~31;
    int u, i;
    if (L < n32) {
        u = (L >> 5) * 8 + (L & 7);
        i = (L >> 3) & 3;
    } else {
        u = (n32 >> 2) + ((L - n32) >> 2);
        i = (L - n32) & 3;
    }
    const int hb = u % a.nstrip, split = u / a.nstrip;
    const int H = a.H;
    const int hs = hb * kPBStrip;
    const int tb = split * a.tok_per_split;
    const int te = min(a.T, tb + a.tok_per_split);
    // this thread's 16-byte piece of every tile row it moves (past H: loads read zero,
    // stores are dropped)
    const int hp = hs + 8 * (tid & 31);
    const uint32_t colo = hp < H ? (uint32_t)hp * 2u : 0x80000000u;

    const int b = i * a.nbh + hb * 4 + w; // fragment block of this wavefront's 64 columns
    u32x4 wf[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) {
            wf[j][tm] = a.wfrag[((size_t)(b * 4 + j) * 2 + tm) * kWave + lane];
        }
    }
    f32x4 dw[2][4];
#pragma unroll
    for (int rtile = 0; rtile < 2; ++rtile) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            dw[rtile][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    ProjBwdStage P;
    int t0 = tb;
    if (t0 < te) {
        pb_issue(a, t0, te, i, tid, w, colo, P);
        pb_commit(smem, P, 0, tid, w);
        if (t0 + kPBChunk < te) {
            pb_issue(a, t0 + kPBChunk, te, i, tid, w, colo, P);
        }
    }
    const float *tokf = reinterpret_cast<const float *>(smem + kPBOffTok);
    for (int k = 0; t0 < te; ++k, t0 += kPBChunk) {
        const int dyo = kPBOffDy + (k & 1) * kPBTile;
        lds_barrier(); // the chunk is in LDS
        // ---- d_res for the 2 token tiles of the chunk, written over dy
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int row = mt * 16 + c;
            const float pre = tokf[row * 8 + i], cr = tokf[row * 8 + kHC];
            const u32x4 bh = lds16(smem, kPBOffDd + row * kPBSmallRow + g * 16);
            const u32x4 bl = lds16(smem, kPBOffDd + kPBSmall + row * kPBSmallRow + g * 16);
            f32x4 acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j][0]),
                                                                __builtin_bit_cast(bf16x8, bh), acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j][0]),
                                                                __builtin_bit_cast(bf16x8, bl), acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j][1]),
                                                                __builtin_bit_cast(bf16x8, bh), acc[j], 0, 0, 0);
            }
            // lane (g, c): acc[j][q] is h = 16g + 4j + q; piece hf holds tiles 2hf, 2hf + 1
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int at = pb_at(row, 8 * w + 2 * g + hf);
                const u32x4 rv = lds16(smem, kPBOffRes + at), gv = lds16(smem, dyo + at);
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // element pair (2q, 2q + 1) of the piece: tile 2hf + (q >> 1), registers 2(q & 1), +1
                    const int j = 2 * hf + (q >> 1), e = 2 * (q & 1);
                    const float lo = fmaf(bf16_lo(rv[q]), cr, fmaf(bf16_lo(gv[q]), pre, acc[j][e]));
                    const float hi = fmaf(bf16_hi(rv[q]), cr, fmaf(bf16_hi(gv[q]), pre, acc[j][e + 1]));
                    o[q] = pack_bf16x2(lo, hi);
                }
                *reinterpret_cast<u32x4 *>(smem + dyo + at) = o;
            }
        }
        // ---- d_W: B = the chunk's streams read transposed (tokens 8g .. 8g + 7 of column 16 jj + c)
        u32x4 ah[2], al[2];
#pragma unroll
        for (int rtile = 0; rtile < 2; ++rtile) {
            ah[rtile] = lds16(smem, kPBOffDdT + (c + 16 * rtile) * kPBSmallRow + g * 16);
            al[rtile] = lds16(smem, kPBOffDdT + kPBSmall + (c + 16 * rtile) * kPBSmallRow + g * 16);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int ch = 8 * w + 2 * jj + (c >> 3);
            uint32_t bw[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r0 = 8 * g + 2 * q;
                const uint32_t e0 =
                    *reinterpret_cast<const uint16_t *>(smem + kPBOffRes + pb_at(r0, ch) + 2 * (c & 7));
                const uint32_t e1 =
                    *reinterpret_cast<const uint16_t *>(smem + kPBOffRes + pb_at(r0 + 1, ch) + 2 * (c & 7));
                bw[q] = e0 | (e1 << 16);
            }
            const bf16x8 B = __builtin_bit_cast(bf16x8, u32x4{bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
            for (int rtile = 0; rtile < 2; ++rtile) {
                dw[rtile][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah[rtile]), B,
                                                                       dw[rtile][jj], 0, 0, 0);
                dw[rtile][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al[rtile]), B,
                                                                       dw[rtile][jj], 0, 0, 0);
            }
        }
        lds_barrier(); // d_res of the chunk is in LDS; every wavefront is done with the chunk's operands
        // ---- d_res rows out (t0 is uniform; saying so keeps the descriptor in SGPRs)
        const int tu = uniform(t0);
        const int ntok = min(kPBChunk, te - tu);
        const __amdgpu_buffer_rsrc_t vout =
            buf_view_b(a.d_res + (size_t)tu * kHC * H, (uint32_t)((size_t)ntok * kHC * H * 2));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int row = (tid >> 5) + 8 * kk;
            __builtin_amdgcn_raw_buffer_store_b128(lds16(smem, dyo + pb_at(row, tid & 31)), vout,
                                                   (int)((uint32_t)((row * kHC + i) * H) * 2u + colo), 0, 0);
        }
        // ---- the next chunk to LDS (streams, dd, dd^T, scalars: single copies, free since
        // the barrier; dy: the other slot, free since the previous chunk's rows went out),
        // and the one after it in flight
        if (t0 + kPBChunk < te) {
            pb_commit(smem, P, (k + 1) & 1, tid, w);
            if (t0 + 2 * kPBChunk < te) {
                pb_issue(a, t0 + 2 * kPBChunk, te, i, tid, w, colo, P);
            }
        }
    }
    // ---- d_W partial of this (stream, 64 columns, token range): dw[rtile][jj][q] is
    // logit row 16 rtile + 4g + q, column hs + 64w + 16 jj + c
#pragma unroll
    for (int rtile = 0; rtile < 2; ++rtile) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int h = hs + kPBCols * w + 16 * jj + c;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = 16 * rtile + 4 * g + q;
                if (r < kMix && h < H) {
                    a.dw_part[((size_t)split * kMix + r) * kHC * H + (size_t)i * H + h] = dw[rtile][jj][q];
                }
            }
        }
    }
}

// d_W[r][k] = sum over the token ranges of the partials, in range order.
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float *__restrict__ part, int splits, int64_t n,
                                                        float *__restrict__ d_w)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) {
        return;
    }
    float v = 0.0f;
    for (int s = 0; s < splits; ++s) {
        v += part[(size_t)s * n + e];
    }
    d_w[e] = v;
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
    return for_token_chunks(n, sinkhorn_bwd_items_per_matrix(), [&](int64_t c0, int64_t nc) {
        const int64_t blocks = (nc * 16 + kSBBlock - 1) / kSBBlock;
        const size_t o = (size_t)c0 * 16;
        sinkhorn_bwd_kernel<<<dim3((unsigned)blocks), dim3(kSBBlock), sinkhorn_bwd_lds_bytes(iters), stream>>>(
            grad + o, logits + o, nc, iters, eps, d_logits + o);
        return hipGetLastError();
    });
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
    const int64_t per = (H / 8 + kDBBlock - 1) / kDBBlock;
    const size_t lds = (size_t)(iters + 1) * kWave * sizeof(float);
    const hipError_t ec = for_token_chunks(T, pre_dots_bwd_items_per_token(), [&](int64_t c0, int64_t Tc) {
        DotsBwdArgs a{};
        a.dy = dy + (size_t)c0 * H;
        a.d_post = d_post + (size_t)c0 * kHC;
        a.d_comb = d_comb + (size_t)c0 * kHC * kHC;
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
        a.d_res = d_res + (size_t)c0 * kHC * H;
        a.d_dot = d_dot + (size_t)c0 * kMix;
        a.d_sqrsum = d_sqrsum ? d_sqrsum + c0 : nullptr;
        a.ws = ws + (size_t)c0 * kWsRow;
        const dim3 grid((unsigned)Tc), block(kDBBlock);
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
        return hipGetLastError();
    });
    if (ec != hipSuccess) {
        return ec;
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

// Workspace of the whole pre-map's reverse, all parts 256-byte aligned.
struct PreBwdLayout {
    PreGeom g;
    int nbh, nstrip, splits, tok_per_split, ldT;
    size_t off_wfrag, off_tok, off_ddh, off_ddl, off_ddTh, off_ddTl, off_rows, off_dw, total;
};

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

static PreBwdLayout pre_bwd_layout(int64_t T, int64_t H)
{
    PreBwdLayout L{};
    L.g = pre_geometry(T, H, true);
    L.nstrip = (int)((H + kPBStrip - 1) / kPBStrip);
    L.nbh = 4 * L.nstrip; // 64-column fragment blocks per stream, whole strips
    const int nb = kHC * L.nbh;
    const int64_t steps = (T + kPBChunk - 1) / kPBChunk; // 32-token steps
    int64_t splits = kPBTargetBlocks / (kHC * L.nstrip);
    splits = splits > steps ? steps : splits;
    splits = splits < 1 ? 1 : splits;
    const int64_t per_steps = (steps + splits - 1) / splits;
    L.tok_per_split = (int)(per_steps * kPBChunk);
    L.splits = (int)((T + L.tok_per_split - 1) / L.tok_per_split);
    if (L.splits < 1) {
        L.splits = 1;
    }
    L.ldT = (int)((T + 31) & ~(int64_t)31);
    size_t off = up256(L.g.total_bytes);
    L.off_wfrag = off;
    off += up256((size_t)nb * 4 * 2 * kWave * sizeof(u32x4));
    L.off_tok = off;
    off += up256((size_t)T * 8 * sizeof(float));
    L.off_ddh = off;
    off += up256((size_t)T * 32 * 2);
    L.off_ddl = off;
    off += up256((size_t)T * 32 * 2);
    L.off_ddTh = off;
    off += up256((size_t)32 * L.ldT * 2);
    L.off_ddTl = off;
    off += up256((size_t)32 * L.ldT * 2);
    L.off_rows = off;
    off += up256(pre_bwd_workspace_bytes(T));
    L.off_dw = off;
    off += up256((size_t)L.splits * kMix * kHC * H * sizeof(float));
    L.total = off;
    return L;
}

size_t pre_fused_bwd_workspace_bytes(int64_t T, int64_t H) { return pre_bwd_layout(T, H).total; }

hipError_t launch_pre_fused_bwd(const uint16_t *dy, const float *d_post, const float *d_comb, const uint16_t *res,
                                const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
                                int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                                int iters, uint16_t *d_res, float *d_hc_fn, float *d_hc_scale, float *d_hc_base,
                                void *workspace, hipStream_t stream)
{
    if (T == 0) { // gradients summed over no tokens: zeros
        pre_bwd_final_kernel<<<dim3(1), dim3(64), 0, stream>>>(nullptr, 0, d_hc_scale, d_hc_base);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) {
            return e0;
        }
        const int64_t n0 = (int64_t)kMix * kHC * H;
        dw_reduce_kernel<<<dim3((unsigned)((n0 + 255) / 256)), dim3(256), 0, stream>>>(nullptr, 0, n0, d_hc_fn);
        return hipGetLastError();
    }
    const PreBwdLayout L = pre_bwd_layout(T, H);
    char *ws = reinterpret_cast<char *>(workspace);
    float *tok = reinterpret_cast<float *>(ws + L.off_tok);
    uint16_t *ddh = reinterpret_cast<uint16_t *>(ws + L.off_ddh);
    uint16_t *ddl = reinterpret_cast<uint16_t *>(ws + L.off_ddl);
    uint16_t *ddTh = reinterpret_cast<uint16_t *>(ws + L.off_ddTh);
    uint16_t *ddTl = reinterpret_cast<uint16_t *>(ws + L.off_ddTl);
    float *rows = reinterpret_cast<float *>(ws + L.off_rows);
    hipError_t e = launch_pre_split(hc_fn, L.g, workspace, stream);
    if (e != hipSuccess) {
        return e;
    }
    // forward fields and <dy, res_i>, then the per-token reverse, chunk by chunk
    for (int64_t c0 = 0; c0 < T; c0 += L.g.chunk) {
        const int Tc = (int)(T - c0 < L.g.chunk ? T - c0 : L.g.chunk);
        e = launch_pre_sums(res, dy, L.g, c0, Tc, workspace, stream, true);
        if (e != hipSuccess) {
            return e;
        }
        DotsBwdArgs a{};
        a.d_post = d_post + (size_t)c0 * kHC;
        a.d_comb = d_comb + (size_t)c0 * kHC * kHC;
        a.hc_scale = hc_scale;
        a.hc_base = hc_base;
        a.T = Tc;
        a.H = (int)H;
        a.k = (float)(kHC * H);
        a.rms_eps = rms_eps;
        a.pre_eps = pre_eps;
        a.sk_eps = sinkhorn_eps;
        a.post_mult = post_mult;
        a.iters = iters;
        a.ws = rows + (size_t)c0 * kWsRow;
        a.sums = reinterpret_cast<const float *>(ws + L.g.off_prew);
        a.tok = tok + (size_t)c0 * 8;
        a.dd_hi = ddh + (size_t)c0 * 32;
        a.dd_lo = ddl + (size_t)c0 * 32;
        a.ddT_hi = ddTh + c0;
        a.ddT_lo = ddTl + c0;
        a.ldT = L.ldT;
        const size_t lds = (size_t)(iters + 1) * kWave * sizeof(float);
        pre_tok_bwd_kernel<<<dim3((unsigned)((Tc + 3) / 4)), dim3(kWave), lds, stream>>>(a);
        e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
    }
    // token sums of d_hc_scale and d_hc_base
    const int64_t nblk = (T + kRedTok - 1) / kRedTok;
    float *part = reinterpret_cast<float *>(reinterpret_cast<char *>(rows) + pre_bwd_rows_bytes(T));
    pre_bwd_partial_kernel<<<dim3((unsigned)nblk), dim3(kRedTok), 0, stream>>>(rows, T, part);
    e = hipGetLastError();
    if (e != hipSuccess) {
        return e;
    }
    pre_bwd_final_kernel<<<dim3(1), dim3(64), 0, stream>>>(part, nblk, d_hc_scale, d_hc_base);
    e = hipGetLastError();
    if (e != hipSuccess) {
        return e;
    }
    // the projection's reverse
    const int nb = kHC * L.nbh;
    u32x4 *wfrag = reinterpret_cast<u32x4 *>(ws + L.off_wfrag);
    // nb >= 16, so the grid's 4096+ threads cover the 32 x 31 dd^T pad entries at most
    proj_bwd_wfrag_kernel<<<dim3((unsigned)((nb * 4 * kWave + 255) / 256)), dim3(256), 0, stream>>>(
        hc_fn, (int)H, L.nbh, wfrag, (int)T, L.ldT, ddTh, ddTl);
    e = hipGetLastError();
    if (e != hipSuccess) {
        return e;
    }
    ProjBwdArgs pa{};
    pa.dy = dy;
    pa.res = res;
    pa.tok = tok;
    pa.dd_hi = ddh;
    pa.dd_lo = ddl;
    pa.ddT_hi = ddTh;
    pa.ddT_lo = ddTl;
    pa.wfrag = wfrag;
    pa.T = (int)T;
    pa.H = (int)H;
    pa.ldT = L.ldT;
    pa.nbh = L.nbh;
    pa.nstrip = L.nstrip;
    pa.nblocks = kHC * L.nstrip * L.splits;
    pa.tok_per_split = L.tok_per_split;
    pa.d_res = d_res;
    pa.dw_part = reinterpret_cast<float *>(ws + L.off_dw);
    proj_bwd_kernel<<<dim3((unsigned)pa.nblocks), dim3(kHC * kWave), 0, stream>>>(pa);
    e = hipGetLastError();
    if (e != hipSuccess) {
        return e;
    }
    const int64_t n = (int64_t)kMix * kHC * H;
    dw_reduce_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(pa.dw_part, L.splits, n, d_hc_fn);
    return hipGetLastError();
}

hipError_t launch_post_bwd(const uint16_t *d_out, const uint16_t *x, const uint16_t *res, const float *post,
                           const float *comb, int64_t T, int64_t H, uint16_t *d_x, uint16_t *d_res, float *d_post,
                           float *d_comb, hipStream_t stream, bool vec8)
{
    // 256 threads, kCPT 8-element chunks per thread and stream on the 16-byte path
    // (128- and 64-thread groups with exact chunk counts measured no faster at H=7168).
    const int64_t per = (H / 8 + 255) / 256;
    return for_token_chunks(T, post_bwd_items_per_token(), [&](int64_t c0, int64_t Tc) {
        PostBwdArgs a{};
        const size_t s = (size_t)c0 * kHC * H;
        a.d_out = d_out + s;
        a.x = x + (size_t)c0 * H;
        a.res = res + s;
        a.post = post + (size_t)c0 * kHC;
        a.comb = comb + (size_t)c0 * kHC * kHC;
        a.T = (int)Tc;
        a.H = (int)H;
        a.d_x = d_x + (size_t)c0 * H;
        a.d_res = d_res + s;
        a.d_post = d_post + (size_t)c0 * kHC;
        a.d_comb = d_comb + (size_t)c0 * kHC * kHC;
        const dim3 grid((unsigned)Tc), block(256);
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
    });
}

int64_t pre_dots_bwd_items_per_token() { return kDBBlock; }
int64_t post_bwd_items_per_token() { return 256; }
int64_t sinkhorn_bwd_items_per_matrix() { return 16; }

} // namespace mhc
