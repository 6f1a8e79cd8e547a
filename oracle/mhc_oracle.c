/*
 * mhc_oracle.c -- plain, slow, fp64 CPU oracle for the mHC residual-mixing path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP library, and the product path never calls it.
 *
 * Every step is written from the pages' definitions, one scalar loop per
 * formula, with fp64 arithmetic throughout.  bf16 and fp32 inputs are widened
 * exactly; results are returned unrounded in fp64 (the tests round them, or
 * compare against the unrounded value).
 *
 * Sources (page title -> section):
 *  - "FlashInfer mHC 模块深度解析" (FlashInfer mHC article), section 1: HC = 4 and
 *    the 24-logit layout pre[0:4], post[4:8], comb[8:24] viewed as 4x4.
 *  - same article, section 2.1: the post-map formula
 *    out[n][h] = x[h]*post[n] + sum_o res[o][h]*comb[o][n].
 *  - same article, section 3.4: rstd = rsqrt(sqrsum/K + rms_eps), K = 4H
 *    (section 4: the denominator is fixed at 4*H when the sum is computed in-kernel).
 *  - same article, section 5.2 (test reference implementation): mixes = dot*rstd,
 *    per-group scale and base, pre = sigmoid + pre_eps, post = sigmoid * post_mult,
 *    comb = Sinkhorn of the comb logits, layer_input = sum_i pre_i * res_i;
 *    and the Sinkhorn schedule: softmax over the last axis, + eps, then
 *    `repeat` rounds of (row normalise, column normalise).
 *  - metrale glm5next_mhc.rs, `glm_hc_post` doc comment: the same post formula
 *    with comb[i][j] weighting old stream i into new stream j.
 *  - metrale glm5next_mhc.rs, `Glm5NextMhcSiteWeights`: hc_fn is
 *    [mix_hc, hc_mult*hidden] and hc_scale holds the pre, post, comb scales in
 *    that order.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - flatten order of [4, H] into the K = 4H projection axis: k = i*H + h;
 *  - the Sinkhorn eps is added once after the softmax; the row and column
 *    divisions carry no eps; the softmax subtracts the row maximum;
 *  - `num_iters` counts (row, column) pairs, with no early exit.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORC_HC 4
#define ORC_MIX 24

/* bf16 bit pattern -> double, exact (bf16 is the top half of an IEEE binary32). */
static double orc_bf16_to_f64(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 (ties to even), directly from fp64
 * (no intermediate binary32 rounding).  bf16 keeps 8 significant bits and the
 * binary32 exponent range. */
uint16_t orc_f64_to_bf16(double v)
{
    if (isnan(v)) {
        return (uint16_t)0x7FC0u;
    }
    double a = fabs(v);
    double r;
    if (a == 0.0 || isinf(v)) {
        r = v;
    } else {
        int e;
        frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1: leading bit has weight 2^(e-1) */
        int ulp_exp = e - 8; /* 8 significant bits */
        if (ulp_exp < -133) {
            ulp_exp = -133; /* binary32 subnormal spacing */
        }
        double q = ldexp(a, -ulp_exp);
        double qr = nearbyint(q); /* default rounding mode: nearest, ties to even */
        r = copysign(ldexp(qr, ulp_exp), v);
        if (fabs(r) >= ldexp(1.0, 128)) {
            r = copysign(INFINITY, v);
        }
    }
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void orc_round_bf16(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        out[i] = orc_f64_to_bf16(v[i]);
    }
}

/* Step A1 (FlashInfer mHC article, sections 3.4 and 5.2): per-token sum of
 * squares over the 4 streams and rstd = 1 / sqrt(S / (4H) + rms_eps). */
void orc_rms(const uint16_t *res, int64_t T, int64_t H, double rms_eps, double *sqsum, double *rstd)
{
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int64_t i = 0; i < ORC_HC; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                double v = orc_bf16_to_f64(res[(t * ORC_HC + i) * H + h]);
                s += v * v;
            }
        }
        if (sqsum) {
            sqsum[t] = s;
        }
        rstd[t] = 1.0 / sqrt(s / (double)(ORC_HC * H) + rms_eps);
    }
}

/* Step A2: dot[t][r] = sum_k hc_fn[r][k] * res_flat[t][k], with the streams
 * flattened as k = i*H + h.  hc_fn is [24, 4H] row-major. */
void orc_project(const uint16_t *res, const float *hc_fn, int64_t T, int64_t H, double *dot)
{
    const int64_t K = ORC_HC * H;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *row = res + t * K;
        for (int64_t r = 0; r < ORC_MIX; ++r) {
            const float *w = hc_fn + r * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                acc += (double)w[k] * orc_bf16_to_f64(row[k]);
            }
            dot[t * ORC_MIX + r] = acc;
        }
    }
}

static double orc_sigmoid(double z)
{
    return 1.0 / (1.0 + exp(-z));
}

/* Step A3 (FlashInfer mHC article, section 5.2): m = dot * rstd, then
 *   pre_i  = sigmoid(m_i * s0 + b_i) + pre_eps
 *   post_i = sigmoid(m_{4+i} * s1 + b_{4+i}) * post_mult
 *   L_ij   = m_{8+4i+j} * s2 + b_{8+4i+j}            (comb logits, 4x4 row-major)
 * with hc_scale = (s0, s1, s2) in the order pre, post, comb. */
void orc_mix_activation(const double *dot, const double *rstd, const float *hc_scale, const float *hc_base,
                        int64_t T, double pre_eps, double post_mult, double *pre, double *post, double *comb_logits)
{
    const double s_pre = hc_scale[0], s_post = hc_scale[1], s_comb = hc_scale[2];
    for (int64_t t = 0; t < T; ++t) {
        const double *d = dot + t * ORC_MIX;
        for (int i = 0; i < ORC_HC; ++i) {
            double m = d[i] * rstd[t];
            pre[t * ORC_HC + i] = orc_sigmoid(m * s_pre + (double)hc_base[i]) + pre_eps;
        }
        for (int i = 0; i < ORC_HC; ++i) {
            double m = d[ORC_HC + i] * rstd[t];
            post[t * ORC_HC + i] = orc_sigmoid(m * s_post + (double)hc_base[ORC_HC + i]) * post_mult;
        }
        for (int c = 0; c < ORC_HC * ORC_HC; ++c) {
            double m = d[2 * ORC_HC + c] * rstd[t];
            comb_logits[t * ORC_HC * ORC_HC + c] = m * s_comb + (double)hc_base[2 * ORC_HC + c];
        }
    }
}

/* Step A4 (FlashInfer mHC article, section 5.2, the Sinkhorn reference; rwkv-ops
 * sinkhorn_knopp docstring for the [.., N, N] -> doubly-stochastic contract):
 *   P = softmax(L, over each row) + eps
 *   repeat num_iters times: divide each row by its sum; divide each column by its sum.
 * `logits` and `out` are [n, 4, 4] row-major; they may be the same array. */
void orc_sinkhorn(const double *logits, int64_t n, int num_iters, double eps, double *out)
{
    for (int64_t b = 0; b < n; ++b) {
        double P[ORC_HC][ORC_HC];
        const double *L = logits + b * ORC_HC * ORC_HC;
        for (int i = 0; i < ORC_HC; ++i) {
            double mx = L[i * ORC_HC];
            for (int j = 1; j < ORC_HC; ++j) {
                if (L[i * ORC_HC + j] > mx) {
                    mx = L[i * ORC_HC + j];
                }
            }
            double s = 0.0;
            for (int j = 0; j < ORC_HC; ++j) {
                P[i][j] = exp(L[i * ORC_HC + j] - mx);
                s += P[i][j];
            }
            for (int j = 0; j < ORC_HC; ++j) {
                P[i][j] = P[i][j] / s + eps;
            }
        }
        for (int it = 0; it < num_iters; ++it) {
            for (int i = 0; i < ORC_HC; ++i) {
                double s = 0.0;
                for (int j = 0; j < ORC_HC; ++j) {
                    s += P[i][j];
                }
                for (int j = 0; j < ORC_HC; ++j) {
                    P[i][j] /= s;
                }
            }
            for (int j = 0; j < ORC_HC; ++j) {
                double s = 0.0;
                for (int i = 0; i < ORC_HC; ++i) {
                    s += P[i][j];
                }
                for (int i = 0; i < ORC_HC; ++i) {
                    P[i][j] /= s;
                }
            }
        }
        double *O = out + b * ORC_HC * ORC_HC;
        for (int i = 0; i < ORC_HC; ++i) {
            for (int j = 0; j < ORC_HC; ++j) {
                O[i * ORC_HC + j] = P[i][j];
            }
        }
    }
}

/* Step A5 (FlashInfer mHC article, sections 3.4 and 5.2; rwkv-ops
 * stream_aggregate): y[t][h] = sum_i pre[t][i] * res[t][i][h]. */
void orc_collapse(const uint16_t *res, const double *pre, int64_t T, int64_t H, double *y)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < ORC_HC; ++i) {
                acc += pre[t * ORC_HC + i] * orc_bf16_to_f64(res[(t * ORC_HC + i) * H + h]);
            }
            y[t * H + h] = acc;
        }
    }
}

/* Step A6 (FlashInfer mHC article, section 2.1; metrale glm_hc_post):
 *   out[t][n][h] = x[t][h] * post[t][n] + sum_o res[t][o][h] * comb[t][o][n]. */
void orc_post(const uint16_t *x, const uint16_t *res, const double *post, const double *comb, int64_t T, int64_t H,
              double *out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int n = 0; n < ORC_HC; ++n) {
            for (int64_t h = 0; h < H; ++h) {
                double acc = orc_bf16_to_f64(x[t * H + h]) * post[t * ORC_HC + n];
                for (int o = 0; o < ORC_HC; ++o) {
                    acc += orc_bf16_to_f64(res[(t * ORC_HC + o) * H + h]) * comb[(t * ORC_HC + o) * ORC_HC + n];
                }
                out[(t * ORC_HC + n) * H + h] = acc;
            }
        }
    }
}

/* The whole pre-map, one token at a time: A1 -> A2 -> A3 -> A4 -> A5.
 * Outputs (fp64, unrounded): y [T,H], post [T,4], comb [T,4,4], pre [T,4];
 * `dot` [T,24] and `rstd` [T] are optional (may be NULL). */
void orc_pre(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
             int64_t H, double rms_eps, double pre_eps, double sinkhorn_eps, double post_mult, int num_iters,
             double *y, double *post, double *comb, double *pre, double *dot_out, double *rstd_out)
{
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *r = res + t * ORC_HC * H;
        double rstd, dot[ORC_MIX], logits[ORC_HC * ORC_HC];
        orc_rms(r, 1, H, rms_eps, NULL, &rstd);
        orc_project(r, hc_fn, 1, H, dot);
        orc_mix_activation(dot, &rstd, hc_scale, hc_base, 1, pre_eps, post_mult, pre + t * ORC_HC,
                           post + t * ORC_HC, logits);
        orc_sinkhorn(logits, 1, num_iters, sinkhorn_eps, comb + t * ORC_HC * ORC_HC);
        orc_collapse(r, pre + t * ORC_HC, 1, H, y + t * H);
        if (dot_out) {
            memcpy(dot_out + t * ORC_MIX, dot, sizeof dot);
        }
        if (rstd_out) {
            rstd_out[t] = rstd;
        }
    }
}

/* The pre-map from an external projection (FlashInfer mHC article, section 3.1
 * to 3.3, mhc_pre_big_fuse: the dots arrive as input, optionally as num_splits
 * partial sums over split K; section 4, mhc_pre_big_fuse_with_prenorm: the sum of
 * squares is computed from the residual streams when it is not supplied):
 *   d[r]  = sum over splits s of dot_mix[s][t][r]
 *   S     = sum over splits of sqrsum[s][t], or sum_{i,h} res[t][i][h]^2 when sqrsum is NULL
 *   rstd  = 1 / sqrt(S / k + rms_eps)
 * then A3 -> A4 -> A5 exactly as in orc_pre.  dot_mix is [S][T][24] and sqrsum
 * [S][T], fp32. */
void orc_pre_from_dots(const float *dot_mix, const float *sqrsum, int64_t num_splits, const uint16_t *res,
                       const float *hc_scale, const float *hc_base, int64_t T, int64_t H, double k, double rms_eps,
                       double pre_eps, double sinkhorn_eps, double post_mult, int num_iters, double *y, double *post,
                       double *comb, double *pre)
{
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *r = res + t * ORC_HC * H;
        double dot[ORC_MIX], logits[ORC_HC * ORC_HC], S = 0.0;
        for (int64_t c = 0; c < ORC_MIX; ++c) {
            double acc = 0.0;
            for (int64_t sp = 0; sp < num_splits; ++sp) {
                acc += (double)dot_mix[(sp * T + t) * ORC_MIX + c];
            }
            dot[c] = acc;
        }
        if (sqrsum) {
            for (int64_t sp = 0; sp < num_splits; ++sp) {
                S += (double)sqrsum[sp * T + t];
            }
        } else {
            double rstd_unused;
            orc_rms(r, 1, H, rms_eps, &S, &rstd_unused); /* S = the sum of squares */
        }
        const double rstd = 1.0 / sqrt(S / k + rms_eps);
        orc_mix_activation(dot, &rstd, hc_scale, hc_base, 1, pre_eps, post_mult, pre + t * ORC_HC,
                           post + t * ORC_HC, logits);
        orc_sinkhorn(logits, 1, num_iters, sinkhorn_eps, comb + t * ORC_HC * ORC_HC);
        orc_collapse(r, pre + t * ORC_HC, 1, H, y + t * H);
    }
}

/* Reverse mode through the Sinkhorn steps of orc_sinkhorn (rwkv-ops mhu_jax.py,
 * sinkhorn_knopp with its custom VJP SinkhornBwd: the gradient of the fixed-count
 * iteration, not of its limit).  The forward is replayed keeping every
 * intermediate matrix; then, from the last step back:
 *   column step Q = A / c (c_j = sum_i A_ij):  dA_ij = (dQ_ij - sum_i' dQ_i'j Q_i'j) / c_j
 *   row step    A = P / r (r_i = sum_j P_ij):  dP_ij = (dA_ij - sum_j' dA_ij' A_ij') / r_i
 *   + eps:                                     dS = dP0
 *   row softmax S = softmax(L):                dL_ij = S_ij (dS_ij - sum_j' dS_ij' S_ij')
 * grad, logits and d_logits are [n, 4, 4]. */
void orc_sinkhorn_backward(const double *grad, const double *logits, int64_t n, int num_iters, double eps,
                           double *d_logits)
{
    for (int64_t b = 0; b < n; ++b) {
        const double *L = logits + b * ORC_HC * ORC_HC;
        /* hist[0] = softmax + eps; hist[2k-1] = after the k-th row step; hist[2k] = after the k-th column step */
        double hist[2 * 1024 + 1][ORC_HC][ORC_HC];
        double S[ORC_HC][ORC_HC];
        if (num_iters > 1024) {
            return;
        }
        for (int i = 0; i < ORC_HC; ++i) {
            double mx = L[i * ORC_HC];
            for (int j = 1; j < ORC_HC; ++j) {
                mx = L[i * ORC_HC + j] > mx ? L[i * ORC_HC + j] : mx;
            }
            double s = 0.0;
            for (int j = 0; j < ORC_HC; ++j) {
                S[i][j] = exp(L[i * ORC_HC + j] - mx);
                s += S[i][j];
            }
            for (int j = 0; j < ORC_HC; ++j) {
                S[i][j] /= s;
                hist[0][i][j] = S[i][j] + eps;
            }
        }
        for (int k = 1; k <= num_iters; ++k) {
            for (int i = 0; i < ORC_HC; ++i) {
                double r = 0.0;
                for (int j = 0; j < ORC_HC; ++j) {
                    r += hist[2 * k - 2][i][j];
                }
                for (int j = 0; j < ORC_HC; ++j) {
                    hist[2 * k - 1][i][j] = hist[2 * k - 2][i][j] / r;
                }
            }
            for (int j = 0; j < ORC_HC; ++j) {
                double c = 0.0;
                for (int i = 0; i < ORC_HC; ++i) {
                    c += hist[2 * k - 1][i][j];
                }
                for (int i = 0; i < ORC_HC; ++i) {
                    hist[2 * k][i][j] = hist[2 * k - 1][i][j] / c;
                }
            }
        }
        double G[ORC_HC][ORC_HC];
        for (int i = 0; i < ORC_HC; ++i) {
            for (int j = 0; j < ORC_HC; ++j) {
                G[i][j] = grad[b * ORC_HC * ORC_HC + i * ORC_HC + j];
            }
        }
        for (int k = num_iters; k >= 1; --k) {
            const double(*A)[ORC_HC] = hist[2 * k - 1];
            const double(*Q)[ORC_HC] = hist[2 * k];
            const double(*P)[ORC_HC] = hist[2 * k - 2];
            double dA[ORC_HC][ORC_HC];
            for (int j = 0; j < ORC_HC; ++j) {
                double c = 0.0, gq = 0.0;
                for (int i = 0; i < ORC_HC; ++i) {
                    c += A[i][j];
                    gq += G[i][j] * Q[i][j];
                }
                for (int i = 0; i < ORC_HC; ++i) {
                    dA[i][j] = (G[i][j] - gq) / c;
                }
            }
            for (int i = 0; i < ORC_HC; ++i) {
                double r = 0.0, ga = 0.0;
                for (int j = 0; j < ORC_HC; ++j) {
                    r += P[i][j];
                    ga += dA[i][j] * A[i][j];
                }
                for (int j = 0; j < ORC_HC; ++j) {
                    G[i][j] = (dA[i][j] - ga) / r;
                }
            }
        }
        for (int i = 0; i < ORC_HC; ++i) {
            double gs = 0.0;
            for (int j = 0; j < ORC_HC; ++j) {
                gs += G[i][j] * S[i][j];
            }
            for (int j = 0; j < ORC_HC; ++j) {
                d_logits[b * ORC_HC * ORC_HC + i * ORC_HC + j] = S[i][j] * (G[i][j] - gs);
            }
        }
    }
}

/* Reverse mode of the post-map orc_post (rwkv-ops mhu_jax.py, mhc_post_op with its
 * custom VJP MhcPostOpBwd; the forward formula of the FlashInfer mHC article,
 * section 2.1).  With dO = d_out [T, 4, H]:
 *   d_x[t][h]       = sum_n dO[t][n][h] * post[t][n]
 *   d_res[t][o][h]  = sum_n comb[t][o][n] * dO[t][n][h]
 *   d_post[t][n]    = sum_h dO[t][n][h] * x[t][h]
 *   d_comb[t][o][n] = sum_h res[t][o][h] * dO[t][n][h]
 * d_out, x and res are bf16 bit patterns; post and comb fp64; every output fp64. */
void orc_post_backward(const uint16_t *d_out, const uint16_t *x, const uint16_t *res, const double *post,
                       const double *comb, int64_t T, int64_t H, double *d_x, double *d_res, double *d_post,
                       double *d_comb)
{
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *g = d_out + t * ORC_HC * H;
        const uint16_t *r = res + t * ORC_HC * H;
        const double *p = post + t * ORC_HC;
        const double *cm = comb + t * ORC_HC * ORC_HC;
        for (int64_t h = 0; h < H; ++h) {
            double a = 0.0;
            for (int n = 0; n < ORC_HC; ++n) {
                a += orc_bf16_to_f64(g[n * H + h]) * p[n];
            }
            d_x[t * H + h] = a;
            for (int o = 0; o < ORC_HC; ++o) {
                double v = 0.0;
                for (int n = 0; n < ORC_HC; ++n) {
                    v += cm[o * ORC_HC + n] * orc_bf16_to_f64(g[n * H + h]);
                }
                d_res[(t * ORC_HC + o) * H + h] = v;
            }
        }
        for (int n = 0; n < ORC_HC; ++n) {
            double v = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                v += orc_bf16_to_f64(g[n * H + h]) * orc_bf16_to_f64(x[t * H + h]);
            }
            d_post[t * ORC_HC + n] = v;
        }
        for (int o = 0; o < ORC_HC; ++o) {
            for (int n = 0; n < ORC_HC; ++n) {
                double v = 0.0;
                for (int64_t h = 0; h < H; ++h) {
                    v += orc_bf16_to_f64(r[o * H + h]) * orc_bf16_to_f64(g[n * H + h]);
                }
                d_comb[(t * ORC_HC + o) * ORC_HC + n] = v;
            }
        }
    }
}


/* Reverse mode of the pre-map from an external projection (orc_pre_from_dots with
 * one split: the dots d[t][24] and, when supplied, the sum of squares S[t]).  It is
 * the rwkv-ops mhc_pre_op custom VJP (MhcPreOpBwd: sigmoid weights, Sinkhorn and
 * the stream aggregate), extended by the FlashInfer mixes in front of it
 * (FlashInfer mHC article, section 5.2: m = d * rstd, per-group scale and base,
 * pre_eps, post_mult).  Given dy [T,H] (bf16 bits), d_post [T,4] and d_comb
 * [T,4,4], from the output back:
 *   y = sum_i pre_i res_i:            d_pre_i = sum_h dy[h] res_i[h];  d_res_i[h] = pre_i dy[h]
 *   pre_i = sigma(z_i) + pre_eps:     dz_i = d_pre_i sigma(z_i) (1 - sigma(z_i))
 *   post_i = sigma(z_{4+i}) post_mult: dz_{4+i} = d_post_i post_mult sigma (1 - sigma)
 *   comb = Sinkhorn(L), L = z_{8..23}: dz_{8..23} = the Sinkhorn reverse mode of d_comb
 *   z_r = m_r s_g + b_r:              d_b_r += dz_r;  d_s_g += dz_r m_r;  dm_r = dz_r s_g
 *   m_r = d_r rstd:                   dd_r = dm_r rstd;  d_rstd = sum_r dm_r d_r
 *   rstd = (S / k + rms_eps)^(-1/2):  dS = -d_rstd rstd^3 / (2 k)
 *   S = sum res^2 (sqrsum NULL):      d_res_i[h] += 2 res_i[h] dS;   else d_sqrsum[t] = dS
 * dot is [T,24] fp64, sqrsum [T] fp64 or NULL.  d_res [T,4,H], d_dot [T,24],
 * d_sqrsum [T] (ignored when sqrsum is NULL), d_hc_scale [3] and d_hc_base [24]
 * (summed over the tokens in token order) are fp64 outputs. */
void orc_pre_from_dots_backward(const uint16_t *dy, const double *d_post, const double *d_comb, const double *dot,
                                const double *sqrsum, const uint16_t *res, const float *hc_scale,
                                const float *hc_base, int64_t T, int64_t H, double k, double rms_eps,
                                double pre_eps, double sinkhorn_eps, double post_mult, int num_iters, double *d_res,
                                double *d_dot, double *d_sqrsum, double *d_hc_scale, double *d_hc_base)
{
    for (int g = 0; g < 3; ++g) {
        d_hc_scale[g] = 0.0;
    }
    for (int r = 0; r < ORC_MIX; ++r) {
        d_hc_base[r] = 0.0;
    }
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *rr = res + t * ORC_HC * H;
        const uint16_t *g = dy + t * H;
        const double *d = dot + t * ORC_MIX;
        /* forward values */
        double S;
        if (sqrsum) {
            S = sqrsum[t];
        } else {
            double rstd_unused;
            orc_rms(rr, 1, H, rms_eps, &S, &rstd_unused);
        }
        const double rstd = 1.0 / sqrt(S / k + rms_eps);
        double m[ORC_MIX], z[ORC_MIX];
        for (int r = 0; r < ORC_MIX; ++r) {
            const int grp = r < ORC_HC ? 0 : (r < 2 * ORC_HC ? 1 : 2);
            m[r] = d[r] * rstd;
            z[r] = m[r] * (double)hc_scale[grp] + (double)hc_base[r];
        }
        /* reverse */
        double dz[ORC_MIX];
        for (int i = 0; i < ORC_HC; ++i) {
            double dp = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                dp += orc_bf16_to_f64(g[h]) * orc_bf16_to_f64(rr[i * H + h]);
            }
            const double s = orc_sigmoid(z[i]);
            dz[i] = dp * s * (1.0 - s);
            const double sp = orc_sigmoid(z[ORC_HC + i]);
            dz[ORC_HC + i] = d_post[t * ORC_HC + i] * post_mult * sp * (1.0 - sp);
        }
        orc_sinkhorn_backward(d_comb + t * ORC_HC * ORC_HC, z + 2 * ORC_HC, 1, num_iters, sinkhorn_eps,
                              dz + 2 * ORC_HC);
        double d_rstd = 0.0;
        for (int r = 0; r < ORC_MIX; ++r) {
            const int grp = r < ORC_HC ? 0 : (r < 2 * ORC_HC ? 1 : 2);
            d_hc_base[r] += dz[r];
            d_hc_scale[grp] += dz[r] * m[r];
            const double dm = dz[r] * (double)hc_scale[grp];
            d_dot[t * ORC_MIX + r] = dm * rstd;
            d_rstd += dm * d[r];
        }
        const double dS = -d_rstd * rstd * rstd * rstd / (2.0 * k);
        if (sqrsum) {
            d_sqrsum[t] = dS;
        }
        /* pre weights for the collapse term */
        double pre[ORC_HC];
        for (int i = 0; i < ORC_HC; ++i) {
            pre[i] = orc_sigmoid(z[i]) + pre_eps;
        }
        for (int i = 0; i < ORC_HC; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                double v = pre[i] * orc_bf16_to_f64(g[h]);
                if (!sqrsum) {
                    v += 2.0 * orc_bf16_to_f64(rr[i * H + h]) * dS;
                }
                d_res[(t * ORC_HC + i) * H + h] = v;
            }
        }
    }
}

/* Reverse mode of the whole pre-map orc_pre (projection inside).  The dots and the
 * sum of squares are recomputed from res (steps A1, A2), orc_pre_from_dots_backward
 * runs with k = 4H and the sum of squares taken from res, and the projection
 * dot[t][r] = sum_k hc_fn[r][k] res_flat[t][k] is reversed:
 *   d_res_flat[t][k] += sum_r dd[t][r] hc_fn[r][k]
 *   d_hc_fn[r][k]     = sum_t dd[t][r] res_flat[t][k]      (token order)
 * d_res [T,4,H], d_hc_fn [24,4H], d_hc_scale [3], d_hc_base [24] are fp64 outputs.
 * `scratch` holds 2 * 24 * T doubles. */
void orc_pre_backward(const uint16_t *dy, const double *d_post, const double *d_comb, const uint16_t *res,
                      const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T, int64_t H,
                      double rms_eps, double pre_eps, double sinkhorn_eps, double post_mult, int num_iters,
                      double *d_res, double *d_hc_fn, double *d_hc_scale, double *d_hc_base, double *scratch)
{
    const int64_t K = ORC_HC * H;
    double *dot = scratch;
    double *dd = scratch + ORC_MIX * T;
    orc_project(res, hc_fn, T, H, dot);
    orc_pre_from_dots_backward(dy, d_post, d_comb, dot, NULL, res, hc_scale, hc_base, T, H, (double)K, rms_eps,
                               pre_eps, sinkhorn_eps, post_mult, num_iters, d_res, dd, NULL, d_hc_scale, d_hc_base);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t kk = 0; kk < K; ++kk) {
            double v = 0.0;
            for (int r = 0; r < ORC_MIX; ++r) {
                v += dd[t * ORC_MIX + r] * (double)hc_fn[r * K + kk];
            }
            d_res[t * K + kk] += v;
        }
    }
    for (int r = 0; r < ORC_MIX; ++r) {
        for (int64_t kk = 0; kk < K; ++kk) {
            double v = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                v += dd[t * ORC_MIX + r] * orc_bf16_to_f64(res[t * K + kk]);
            }
            d_hc_fn[r * K + kk] = v;
        }
    }
}

/* Model entry (metrale glm5next_mhc.rs, glm_hc_expand: each hidden row is broadcast into
 * its hc_mult streams): streams[t][i][h] = hidden[t][h] for every stream i.  bf16 in,
 * bf16 out, an exact copy. */
void orc_expand(const uint16_t *hidden, int64_t T, int64_t H, uint16_t *streams)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int i = 0; i < ORC_HC; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                streams[(t * ORC_HC + i) * H + h] = hidden[t * H + h];
            }
        }
    }
}

/* Model exit, unweighted (metrale glm5next_mhc.rs, hc_head_mean: the mean of the
 * hc_mult streams, no weights): y[t][h] = (1/4) sum_i res[t][i][h], fp64, unrounded. */
void orc_head_mean(const uint16_t *res, int64_t T, int64_t H, double *y)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < ORC_HC; ++i) {
                acc += orc_bf16_to_f64(res[(t * ORC_HC + i) * H + h]);
            }
            y[t * H + h] = acc / ORC_HC;
        }
    }
}

/* Model exit, weighted (metrale hyper_connection_dispatch.rs, hc_head_site: the head
 * takes its own hc_fn, hc_scale and hc_base with norm_eps and hc_eps and returns one
 * row).  Read as the pre-map's pre group alone (steps A1, A2 for 4 rows, A3 for pre,
 * A5): rstd = 1/sqrt(S/(4H) + norm_eps), m_i = rstd * sum_k hc_fn[i][k] res_flat[k],
 * pre_i = sigmoid(m_i * s + b_i) + hc_eps, y = sum_i pre_i res_i.  hc_fn is [4, 4H],
 * hc_scale [1], hc_base [4].  y [T,H] and pre [T,4] are fp64, unrounded. */
void orc_head(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
              int64_t H, double norm_eps, double hc_eps, double *y, double *pre)
{
    const int64_t K = ORC_HC * H;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *r = res + t * K;
        double rstd;
        orc_rms(r, 1, H, norm_eps, NULL, &rstd);
        for (int i = 0; i < ORC_HC; ++i) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                acc += (double)hc_fn[i * K + k] * orc_bf16_to_f64(r[k]);
            }
            pre[t * ORC_HC + i] = orc_sigmoid(acc * rstd * (double)hc_scale[0] + (double)hc_base[i]) + hc_eps;
        }
        orc_collapse(r, pre + t * ORC_HC, 1, H, y + t * H);
    }
}

/* ---------------------------------------------------------------------------------------
 * FP32 residual streams (metrale hyper_connection_dispatch.rs, module header: both mixer
 * families run over FP32 [T, hc_mult, H] streams; metrale glm5next_mhc.rs: glm_hc_expand
 * broadcasts each BF16 hidden row into its FP32 highway streams, glm_hc_pre collapses the
 * FP32 streams to one BF16 row and writes post and comb, glm_hc_post writes the new
 * streams with the same formula).  Every step is the one of the bf16-stream functions
 * above, with the streams read as fp32 (widened exactly to fp64).
 * ------------------------------------------------------------------------------------- */

/* Step A1 on fp32 streams: S = sum_{i,h} res^2, rstd = 1 / sqrt(S / (4H) + rms_eps). */
void orc_rms_f32s(const float *res, int64_t T, int64_t H, double rms_eps, double *sqsum, double *rstd)
{
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int64_t i = 0; i < ORC_HC; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                double v = (double)res[(t * ORC_HC + i) * H + h];
                s += v * v;
            }
        }
        if (sqsum) {
            sqsum[t] = s;
        }
        rstd[t] = 1.0 / sqrt(s / (double)(ORC_HC * H) + rms_eps);
    }
}

/* Step A2 on fp32 streams: dot[t][r] = sum_k hc_fn[r][k] * res_flat[t][k], k = i*H + h. */
void orc_project_f32s(const float *res, const float *hc_fn, int64_t T, int64_t H, double *dot)
{
    const int64_t K = ORC_HC * H;
    for (int64_t t = 0; t < T; ++t) {
        const float *row = res + t * K;
        for (int64_t r = 0; r < ORC_MIX; ++r) {
            const float *w = hc_fn + r * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                acc += (double)w[k] * (double)row[k];
            }
            dot[t * ORC_MIX + r] = acc;
        }
    }
}

/* Step A5 on fp32 streams: y[t][h] = sum_i pre[t][i] * res[t][i][h] (fp64, unrounded;
 * the layer input is a BF16 row, so callers round it once). */
void orc_collapse_f32s(const float *res, const double *pre, int64_t T, int64_t H, double *y)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < ORC_HC; ++i) {
                acc += pre[t * ORC_HC + i] * (double)res[(t * ORC_HC + i) * H + h];
            }
            y[t * H + h] = acc;
        }
    }
}

/* The whole pre-map on fp32 streams, one token at a time: A1 -> A2 -> A3 -> A4 -> A5.
 * y [T,H], post [T,4], comb [T,4,4], pre [T,4] are fp64, unrounded. */
void orc_pre_f32s(const float *res, const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
                  int64_t H, double rms_eps, double pre_eps, double sinkhorn_eps, double post_mult, int num_iters,
                  double *y, double *post, double *comb, double *pre)
{
    for (int64_t t = 0; t < T; ++t) {
        const float *r = res + t * ORC_HC * H;
        double rstd, dot[ORC_MIX], logits[ORC_HC * ORC_HC];
        orc_rms_f32s(r, 1, H, rms_eps, NULL, &rstd);
        orc_project_f32s(r, hc_fn, 1, H, dot);
        orc_mix_activation(dot, &rstd, hc_scale, hc_base, 1, pre_eps, post_mult, pre + t * ORC_HC,
                           post + t * ORC_HC, logits);
        orc_sinkhorn(logits, 1, num_iters, sinkhorn_eps, comb + t * ORC_HC * ORC_HC);
        orc_collapse_f32s(r, pre + t * ORC_HC, 1, H, y + t * H);
    }
}

/* Step A6 on fp32 streams: out[t][n][h] = x[t][h] * post[t][n] + sum_o res[t][o][h] *
 * comb[t][o][n], with x the BF16 sublayer output and res the fp32 streams; fp64,
 * unrounded (the new streams are fp32, so callers round them once). */
void orc_post_f32s(const uint16_t *x, const float *res, const double *post, const double *comb, int64_t T,
                   int64_t H, double *out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int n = 0; n < ORC_HC; ++n) {
            for (int64_t h = 0; h < H; ++h) {
                double acc = orc_bf16_to_f64(x[t * H + h]) * post[t * ORC_HC + n];
                for (int o = 0; o < ORC_HC; ++o) {
                    acc += (double)res[(t * ORC_HC + o) * H + h] * comb[(t * ORC_HC + o) * ORC_HC + n];
                }
                out[(t * ORC_HC + n) * H + h] = acc;
            }
        }
    }
}

/* Model entry on fp32 streams (glm_hc_expand): streams[t][i][h] = hidden[t][h], the BF16
 * value widened exactly to fp32. */
void orc_expand_f32s(const uint16_t *hidden, int64_t T, int64_t H, float *streams)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int i = 0; i < ORC_HC; ++i) {
            for (int64_t h = 0; h < H; ++h) {
                streams[(t * ORC_HC + i) * H + h] = (float)orc_bf16_to_f64(hidden[t * H + h]);
            }
        }
    }
}

/* Model exit, unweighted, on fp32 streams (hc_head_mean): y[t][h] = (1/4) sum_i res[t][i][h],
 * fp64, unrounded. */
void orc_head_mean_f32s(const float *res, int64_t T, int64_t H, double *y)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < ORC_HC; ++i) {
                acc += (double)res[(t * ORC_HC + i) * H + h];
            }
            y[t * H + h] = acc / ORC_HC;
        }
    }
}
