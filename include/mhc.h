/*
 * mhc.h -- C ABI of libmhc, the MI355X (gfx950) manifold-constrained
 * hyper-connection (mHC) residual-mixing library.
 *
 * HC (the number of residual streams) is fixed at 4, and every token carries
 * 24 mixing logits laid out as pre[0:4], post[4:8], comb[8:24] (a 4x4 matrix,
 * row-major) -- "FlashInfer mHC 模块深度解析" (FlashInfer mHC article),
 * section 1.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 tensors as float.
 *    Streams and activations are bf16, mixing coefficients fp32 (FlashInfer
 *    mHC article, sections 2.2 and 3.1).
 *  - Every tensor pointer is a DEVICE pointer to dense row-major memory:
 *        res   [T, 4, H]  bf16   residual streams
 *        x     [T, H]     bf16   sublayer output (post-map input)
 *        y     [T, H]     bf16   layer input (pre-map output)
 *        out   [T, 4, H]  bf16   new residual streams (post-map output)
 *        post  [T, 4]     fp32   (the same memory as [T, 4, 1])
 *        comb  [T, 4, 4]  fp32   comb[t][o][n] weights old stream o into new stream n
 *        pre   [T, 4]     fp32
 *        hc_fn [24, 4H]   fp32   projection; column k = i*H + h (stream i, element h)
 *        hc_scale [3]     fp32   logit scales of pre, post, comb, in that order
 *        hc_base  [24]    fp32   logit biases
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously on it; no call synchronises the host.
 *  - Ownership: the caller owns every buffer.  The library never allocates,
 *    frees or retains device memory, apart from the static scratch array of
 *    mhc_pre_fused_noalloc; outputs are written in place.
 *  - Large calls: token-parallel kernels are launched over token chunks, so that
 *    every launch covers fewer than 2^31 work-items and at most 2^24 tokens (a HIP
 *    grid dimension holds fewer than 2^32 work-items); mhc_launch_plan reports
 *    the split.
 *  - Errors: arguments are validated on the host before anything is enqueued.
 *    On any error nothing is launched and no output is touched.  T == 0 is a
 *    successful no-op.  MHC_ERROR_LAUNCH reports a failed enqueue
 *    (hipGetLastError after the launch).
 *  - Results are deterministic: no floating-point atomics; for fixed shapes
 *    repeated calls give bit-identical outputs.
 *  - Any H >= 1 is accepted.  Rows whose byte size is not a multiple of 16,
 *    or base pointers that are not 16-byte aligned, take a scalar path.
 */
#ifndef MHC_H_
#define MHC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_ABI_VERSION 1
#define MHC_HC 4
#define MHC_MIX 24

typedef enum mhc_status {
    MHC_SUCCESS = 0,
    MHC_ERROR_INVALID_VALUE = 1, /* null required pointer, bad size or parameter, forbidden overlap */
    MHC_ERROR_WORKSPACE = 2,     /* workspace missing or smaller than mhc_pre_fused_workspace_bytes() */
    MHC_ERROR_LAUNCH = 3         /* the HIP runtime rejected a kernel launch */
} mhc_status;

/* Returns MHC_ABI_VERSION. */
int mhc_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *mhc_status_string(mhc_status status);

/*
 * mhc_set_exchange_test_hooks -- test hooks of the one-read and small-batch pre-maps
 * (mhc_pre_fused, its variants and mhc_post_pre_fused on 16-byte rows at T >= 1024,
 * 1024 < H <= 8192, or at T <= 192, H <= 8192), for tests of their failure path only.
 * Those forms' workgroups exchange partial sums through memory, tagged with the call (and
 * the step); a reader that finds a record not yet written loads it again, up to max_retry
 * times (negative: the default, 2^14), and then gives the step NaN outputs rather than
 * wait for ever or use a stale record.  A nonzero tag_skew makes every record look
 * missing, so every step takes that path and every output of the call is NaN.  The
 * setting is process-wide and read when a call is enqueued; normal use leaves
 * (-1, 0).  Host only, no GPU work.
 */
void mhc_set_exchange_test_hooks(int32_t max_retry, uint32_t tag_skew);

/*
 * mhc_launch_plan -- diagnostics, host only (no HIP call, nothing enqueued): how an entry
 * point splits a call into launches of its token-parallel kernel.  `entry` names the
 * entry point without the mhc_ prefix: "post", "expand", "head_mean", "pre_fused" (its
 * two-pass form; the collapse and the slice sums are its widest grids), "collapse" (the
 * collapse of pre_from_dots with one split and a supplied sum of squares on 16-byte
 * rows), "pre_from_dots" (its other forms), "pre_from_dots_backward", "post_backward",
 * "sinkhorn", "sinkhorn_backward", "post_f32", "expand_f32", "head_mean_f32".  T is the
 * token count (the matrix count for the Sinkhorn entry points), H the hidden size (unused
 * for the Sinkhorn entry points), vec8 != 0 for 16-byte rows.  Writes the number of
 * launches, the tokens per launch (the last launch may hold fewer) and the work-items of
 * the widest launch (grid blocks times block size), which stays below 2^31.  Returns
 * MHC_ERROR_INVALID_VALUE for an unknown name, a null output pointer, T < 0 or H < 1.
 */
mhc_status mhc_launch_plan(const char *entry, int64_t T, int64_t H, int32_t vec8, int64_t *launches,
                           int64_t *tokens_per_launch, int64_t *max_items);

/*
 * mhc_sinkhorn -- fixed-iteration Sinkhorn-Knopp projection of 4x4 logit
 * matrices (FlashInfer mHC article, section 5.2, the Sinkhorn reference;
 * rwkv-ops mhu_jax.py, sinkhorn_knopp):
 *     P = softmax(L over each row, row maximum subtracted) + eps
 *     repeat num_iters times: divide every row by its sum, then every column by its sum
 *
 *   logits   [n_mats, 4, 4] fp32, device
 *   out      [n_mats, 4, 4] fp32, device; may equal `logits` exactly (in place),
 *            must not overlap it otherwise
 *   n_mats   >= 0
 *   num_iters >= 1 (the count of (row, column) rounds; no early exit)
 *   eps      finite and > 0
 */
mhc_status mhc_sinkhorn(const float *logits, float *out, int64_t n_mats, int32_t num_iters, float eps,
                        void *stream);

/*
 * Size in bytes of the device workspace mhc_pre_fused needs for (T, H): enough for
 * either form of the pre-map.  The caller owns this scratch and passes it with every call,
 * as the mix scratch of a site is caller-owned device memory next to its weights in the
 * metrale GLM-5 mHC page (Glm5NextMhcSiteWeights); its contents on entry are ignored.  The one-read form (16-byte rows, 1024 < H <= 8192,
 * T >= 1024, on a 256-CU gfx950) keeps a ring of exchange records: 16-byte chunks of
 * partial sums for a few 16-token steps of every workgroup, at most 4.6 MB and
 * independent of T.  The small-batch form (16-byte rows, 1 <= T <= 192, H <= 8192, on a
 * 256-CU gfx950) keeps 851,968 bytes of exchange records (16-byte chunks of one call's
 * partial sums) behind the first mhc_pre_split_bytes(H) bytes, which it leaves untouched.
 * The two-pass form keeps the projection weights split into bf16
 * terms in MFMA operand order (576 * H bytes, rounded up), the per-slice partial sums of
 * the projection (100 bytes per token per 128-wide slice of H) and the per-token totals
 * (128 bytes per token); tokens beyond 2^31 bytes of partial sums are processed in
 * chunks that reuse the same space.  Returns 0 for T <= 0, H <= 0 or H beyond the
 * pre-map limit.
 */
size_t mhc_pre_fused_workspace_bytes(int64_t T, int64_t H);

/*
 * mhc_pre_fused -- the mHC pre-map (FlashInfer mHC article, sections 3.4 and
 * 5.2; metrale hyper_connection_dispatch.rs, hc_pre_site argument list):
 *     S_t      = sum_{i,h} res[t][i][h]^2,     rstd_t = 1 / sqrt(S_t / (4H) + rms_eps)
 *     m_t[r]   = rstd_t * sum_k hc_fn[r][k] * res_flat[t][k]          (k = i*H + h)
 *     pre[t][i]  = sigmoid(m_t[i]   * hc_scale[0] + hc_base[i]) + pre_eps
 *     post[t][i] = sigmoid(m_t[4+i] * hc_scale[1] + hc_base[4+i]) * post_mult
 *     comb[t]    = Sinkhorn(L), L[i][j] = m_t[8+4i+j] * hc_scale[2] + hc_base[8+4i+j]
 *     y[t][h]    = bf16( sum_i pre[t][i] * res[t][i][h] )   (fp32 accumulation, nearest-even)
 *
 *   res, hc_fn, hc_scale, hc_base   inputs (layouts above), device
 *   T >= 0, 1 <= H <= 2097152 (the streams of a 64-token tile are addressed with
 *                     32-bit byte offsets)
 *   rms_eps, pre_eps, sinkhorn_eps  finite; rms_eps and sinkhorn_eps > 0, pre_eps >= 0 (the
 *                     FlashInfer article's parameter table of mhc_pre_big_fuse asks for a
 *                     positive pre_eps; 0 is accepted here, since no later step divides by
 *                     pre: it is then the plain sigmoid, in (0, 1))
 *   post_mult                       finite
 *   num_iters                       >= 1
 *   y [T,H], post [T,4], comb [T,4,4]   outputs, device; y must not overlap res
 *   pre [T,4]                       optional output (may be NULL)
 *   workspace                       device scratch of at least
 *                                   mhc_pre_fused_workspace_bytes(T, H) bytes, 256-byte aligned;
 *                                   may be NULL only when that size is 0.  Its contents on entry
 *                                   are ignored; calls sharing one workspace must be ordered on
 *                                   one stream.
 */
mhc_status mhc_pre_fused(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                         int64_t T, int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                         int32_t num_iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * mhc_pre_split_weights / mhc_pre_fused_presplit -- mhc_pre_fused with its weight split
 * done once ahead of the calls, for weights that stay fixed over many calls (a decode
 * loop; metrale glm5next_mhc.rs, Glm5NextMhcSiteWeights: a site's weights are uploaded
 * once by the loader and every call reuses them).
 *
 * mhc_pre_split_weights writes the split of hc_fn ([24, 4H] fp32: three bf16 terms per
 * weight, in the projection's MFMA operand order) into the first mhc_pre_split_bytes(H)
 * bytes of `workspace` (256-byte aligned, device; must not overlap hc_fn).  1 <= H <=
 * 2097152.
 *
 * mhc_pre_fused_presplit takes mhc_pre_fused's arguments, with a workspace that holds the
 * split of this hc_fn: mhc_pre_split_weights ran on it, ordered before this call (same
 * stream or synchronised), and neither hc_fn nor the workspace's first
 * mhc_pre_split_bytes(H) bytes changed since (mhc_pre_fused calls on the same workspace
 * rewrite them with the same values or leave them alone, so they keep it valid).  The
 * two-pass form then skips its weight-split launch; the one-read form (16-byte rows,
 * T >= 1024, 1024 < H <= 8192) splits in-kernel and the small-batch form (16-byte rows,
 * T <= 192, H <= 8192) reads hc_fn as it is, both ignoring the stored split.  Results equal
 * mhc_pre_fused's bit for bit; a stale split gives the two-pass form the results of the
 * weights it was made from.
 */
size_t mhc_pre_split_bytes(int64_t H);
mhc_status mhc_pre_split_weights(const float *hc_fn, int64_t H, void *workspace, size_t workspace_bytes,
                                 void *stream);
mhc_status mhc_pre_fused_presplit(const uint16_t *res, const float *hc_fn, const float *hc_scale,
                                  const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                                  float sinkhorn_eps, float post_mult, int32_t num_iters, uint16_t *y, float *post,
                                  float *comb, float *pre, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mhc_pre_fused_noalloc -- mhc_pre_fused for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument.  Its scratch is a file-scope device array of
 * MHC_PRE_FUSED_NOALLOC_MAX_BYTES inside the library, one per GPU, held until the
 * process ends; the first call on a device resolves its address there.  The call
 * allocates and frees nothing.  Arguments, outputs and limits are those of
 * mhc_pre_fused, and so are the results (bit for bit).  A call whose form needs more
 * workspace than MHC_PRE_FUSED_NOALLOC_MAX_BYTES is rejected with MHC_ERROR_WORKSPACE
 * before anything is enqueued.  The one-read form (16-byte aligned res and y, H a multiple
 * of 8, T >= 1024, 1024 < H <= 8192, on a 256-CU gfx950) needs at most 4.6 MB whatever T,
 * so it always fits; the two-pass form's partial sums take roughly 1 to 1.5 KB per token
 * and 1024 of H (mhc_pre_fused_workspace_bytes(T, H) bounds either form).  Every call on one
 * GPU shares the array: calls that may overlap in time on one GPU (different streams,
 * concurrent host threads) race and give undefined results; order them on one stream.
 */
#define MHC_PRE_FUSED_NOALLOC_MAX_BYTES ((size_t)16 << 20)
mhc_status mhc_pre_fused_noalloc(const uint16_t *res, const float *hc_fn, const float *hc_scale,
                                 const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                                 float sinkhorn_eps, float post_mult, int32_t num_iters, uint16_t *y, float *post,
                                 float *comb, float *pre, void *stream);

/*
 * mhc_pre_fused_bf16 -- mhc_pre_fused with bf16 weights (metrale glm5next_mhc.rs,
 * glm5next_hc_mix_bf16: widening bf16 to fp32 is exact, so the result is the fp32
 * pre-map's on the widened weights).  hc_fn is [24, 4H] bf16 bit patterns; every other
 * argument, output, limit and the workspace are as in mhc_pre_fused.
 */
mhc_status mhc_pre_fused_bf16(const uint16_t *res, const uint16_t *hc_fn, const float *hc_scale,
                              const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                              float sinkhorn_eps, float post_mult, int32_t num_iters, uint16_t *y, float *post,
                              float *comb, float *pre, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mhc_pre_from_dots -- the mHC pre-map from an external projection (FlashInfer mHC
 * article, sections 3.1-3.3, mhc_pre_big_fuse, where the 24 dots and the sum of
 * squares come from outside, optionally as split-K partial sums; section 4,
 * mhc_pre_big_fuse_with_prenorm, where the sum of squares is computed from the
 * streams):
 *     d[t][r]  = sum over s < num_splits of dot_mix[s][t][r]
 *     S_t      = sum over s of sqrsum[s][t], or sum_{i,h} res[t][i][h]^2 when sqrsum is NULL
 *   Both split sums take a fixed order (four interleaved running sums over s mod 4,
 *   then (0 + 1) + (2 + 3)), so the results do not depend on the launch.
 *     rstd_t   = 1 / sqrt(S_t / k + rms_eps)
 *     m_t[r]   = d[t][r] * rstd_t, then pre, post, comb and y exactly as in mhc_pre_fused
 *
 *   dot_mix     [num_splits, T, 24] fp32, device
 *   sqrsum      [num_splits, T] fp32, device, or NULL
 *   num_splits  1 <= num_splits <= 65536
 *   res, hc_scale, hc_base   as in mhc_pre_fused
 *   T >= 0, H >= 1
 *   k           the RMS denominator (4H for the pre-map proper), finite and > 0
 *   rms_eps, pre_eps, sinkhorn_eps, post_mult, num_iters   as in mhc_pre_fused
 *   y [T,H], post [T,4], comb [T,4,4], pre [T,4] (nullable)   outputs, device; no output
 *               may overlap an input or another output
 * No workspace.  The streams of a token are read once.  With num_splits = 1, sqrsum
 * given and 16-byte rows (H % 8 == 0, res and y 16-byte aligned), the mixes need no
 * reduction and each 512-wide piece of a token's streams is read by its own wavefront.
 * Otherwise one workgroup per token holds the streams in registers when rows are
 * 16-byte aligned and H is a multiple of 8 up to 16384; other shapes read them twice.
 */
mhc_status mhc_pre_from_dots(const float *dot_mix, const float *sqrsum, int32_t num_splits, const uint16_t *res,
                             const float *hc_scale, const float *hc_base, int64_t T, int64_t H, float k,
                             float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int32_t num_iters,
                             uint16_t *y, float *post, float *comb, float *pre, void *stream);

/*
 * mhc_post -- the mHC post-map (FlashInfer mHC article, section 2.1; metrale
 * glm5next_mhc.rs, glm_hc_post):
 *     out[t][n][h] = bf16( x[t][h] * post[t][n] + sum_o res[t][o][h] * comb[t][o][n] )
 *   (fp32 accumulation, round to nearest-even)
 *
 *   x [T,H], res [T,4,H], post [T,4], comb [T,4,4]   inputs, device
 *   T >= 0, H >= 1
 *   out [T,4,H]   output, device; may equal `res` exactly (in-place update: every
 *                 element reads all four old streams before it is written), must
 *                 not overlap res otherwise, nor x, post or comb.
 */
mhc_status mhc_post(const uint16_t *x, const uint16_t *res, const float *post, const float *comb, int64_t T,
                    int64_t H, uint16_t *out, void *stream);

/*
 * mhc_expand -- model entry (metrale glm5next_mhc.rs, glm_hc_expand): each hidden row is
 * copied into the 4 residual streams, streams[t][i][h] = hidden[t][h] (bf16, exact).
 *   hidden [T,H] bf16 input, streams [T,4,H] bf16 output, device; no overlap.  T >= 0, H >= 1.
 */
mhc_status mhc_expand(const uint16_t *hidden, int64_t T, int64_t H, uint16_t *streams, void *stream);

/*
 * mhc_head_mean -- model exit, unweighted (metrale glm5next_mhc.rs, hc_head_mean):
 *     y[t][h] = bf16( (res[t][0][h] + res[t][1][h] + res[t][2][h] + res[t][3][h]) / 4 )
 *   (fp32 sum in that order, one rounding)
 *   res [T,4,H] bf16 input, y [T,H] bf16 output, device; no overlap.  T >= 0, H >= 1.
 */
mhc_status mhc_head_mean(const uint16_t *res, int64_t T, int64_t H, uint16_t *y, void *stream);

/*
 * FP32 residual streams.  The metrale dispatch page (hyper_connection_dispatch.rs, module
 * header) runs both mixer families over FP32 [T, hc_mult, H] streams, and glm5next_mhc.rs
 * expands each BF16 hidden row into its FP32 highway streams (glm_hc_expand), collapses
 * them to one BF16 row (glm_hc_pre) and writes new FP32 streams (glm_hc_post).  These entry
 * points are the bf16-stream ones with `res`, `out` and `streams` as float [T, 4, H]; x,
 * hidden and y stay bf16 and the mixing coefficients fp32.  1 <= H <= 1048576 (the
 * projection addresses a 64-token tile of fp32 streams with 32-bit byte offsets).  Rows
 * take a vector path when H % 4 == 0, the fp32 arrays are 16-byte aligned and the bf16
 * rows 8-byte aligned, and a scalar path otherwise; both give the same results.
 */

/*
 * mhc_pre_fused_f32 -- the pre-map over fp32 streams: steps and outputs of mhc_pre_fused,
 * with the sum of squares, the 24 dots and the collapse taken over the fp32 values
 * (fp32 arithmetic; y rounded once to bf16).  The workspace is mhc_pre_fused's: at least
 * mhc_pre_fused_workspace_bytes(T, H) bytes, 256-byte aligned, contents on entry ignored.
 */
mhc_status mhc_pre_fused_f32(const float *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                             int64_t T, int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                             int32_t num_iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * mhc_post_f32 -- the post-map over fp32 streams (metrale glm5next_mhc.rs, glm_hc_post):
 *     out[t][n][h] = x[t][h] * post[t][n] + sum_o res[t][o][h] * comb[t][o][n]
 *   fp32 arithmetic in that order (one rounding per fused multiply-add), out fp32.
 *   x [T,H] bf16; res, out [T,4,H] fp32; post [T,4], comb [T,4,4] fp32.  `out` may equal
 *   `res` exactly (in place); no other overlap.
 */
mhc_status mhc_post_f32(const uint16_t *x, const float *res, const float *post, const float *comb, int64_t T,
                        int64_t H, float *out, void *stream);

/*
 * mhc_expand_f32 -- model entry onto fp32 streams (glm_hc_expand): streams[t][i][h] =
 * hidden[t][h] widened exactly.  hidden [T,H] bf16, streams [T,4,H] fp32; no overlap.
 */
mhc_status mhc_expand_f32(const uint16_t *hidden, int64_t T, int64_t H, float *streams, void *stream);

/*
 * mhc_head_mean_f32 -- the unweighted head over fp32 streams (hc_head_mean):
 *     y[t][h] = bf16( (res[t][0][h] + res[t][1][h] + res[t][2][h] + res[t][3][h]) / 4 )
 *   (fp32 sum in that order, one rounding).  res [T,4,H] fp32, y [T,H] bf16; no overlap.
 */
mhc_status mhc_head_mean_f32(const float *res, int64_t T, int64_t H, uint16_t *y, void *stream);

/*
 * mhc_head -- model exit, weighted (metrale hyper_connection_dispatch.rs, hc_head_site:
 * the head's own hc_fn, hc_scale and hc_base, norm_eps and hc_eps, one output row), taken
 * as the pre-map's pre group alone:
 *     rstd_t  = 1 / sqrt(S_t / (4H) + norm_eps),   S_t = sum_{i,h} res[t][i][h]^2
 *     m_t[i]  = rstd_t * sum_k hc_fn[i][k] * res_flat[t][k]            (i < 4, k = i'*H + h)
 *     pre[t][i] = sigmoid(m_t[i] * hc_scale[0] + hc_base[i]) + hc_eps
 *     y[t][h] = bf16( sum_i pre[t][i] * res[t][i][h] )
 *   res [T,4,H] bf16, hc_fn [4, 4H] fp32, hc_scale [1] fp32, hc_base [4] fp32   inputs, device
 *   T >= 0, 1 <= H <= 2097152; norm_eps finite and > 0, hc_eps finite and >= 0
 *   y [T,H] bf16 output; pre [T,4] fp32 optional output (may be NULL)
 *   workspace   as for mhc_pre_fused: at least mhc_pre_fused_workspace_bytes(T, H) bytes,
 *               256-byte aligned
 * No output may overlap an input, the workspace or another output.
 */
mhc_status mhc_head(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
                    int64_t H, float norm_eps, float hc_eps, uint16_t *y, float *pre, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * Reverse mode (backward pass).  Each entry point returns the gradients of the
 * matching forward map for a given output gradient, as the custom VJPs of
 * rwkv-ops mhu_jax.py do (sinkhorn_knopp / SinkhornBwd, mhc_post_op /
 * MhcPostOpBwd).  The forward is recomputed from the saved inputs where needed;
 * no state is kept between a forward and a backward call.
 */

#define MHC_SINKHORN_BWD_MAX_ITERS 255

/*
 * mhc_post_project -- the post-map fused with the next sublayer's projection
 * (FlashInfer mHC article, sections 3.1-3.3: the pre-map that takes its 24 dots and the
 * sum of squares from outside, dot_mix and sqrsum; here the post-map that writes the
 * streams also produces them).  One call computes
 *     out[t][n][h] = bf16( x[t][h] post[t][n] + sum_o res[t][o][h] comb[t][o][n] )
 * exactly as mhc_post does (the same bits), and, over the bf16 `out` it writes, the
 * next pre-map's projection and sum of squares:
 *     dot_mix[t][r] = sum_{i,h} hc_fn_next[r][i*H + h] out[t][i][h]
 *     sqrsum[t]     = sum_{i,h} out[t][i][h]^2
 * (the weights as three exact bf16 terms on MFMA, fp32 partial sums per 128-wide slice
 * of h, added over the slices in a fixed order).  Passing them to mhc_pre_from_dots
 * with num_splits = 1 and res = out runs the next pre-map without reading the streams
 * for its projection.
 *
 *   x [T,H], res [T,4,H] bf16; post [T,4], comb [T,4,4] fp32   as in mhc_post
 *   hc_fn_next [24,4H] fp32   the next pre-map's weights
 *   T >= 0; 8 <= H <= 2097152 with H % 8 == 0; x, res and out 16-byte aligned
 *   out [T,4,H] bf16   output; may equal `res` exactly
 *   dot_mix [T][24], sqrsum [T] fp32   outputs
 *   workspace   at least mhc_post_project_workspace_bytes(T, H) bytes (the next weights
 *               split for the MFMA and the per-slice partial sums), 256-byte aligned;
 *               contents on entry ignored
 * No output may overlap an input, the workspace or another output, except as stated.
 * T == 0 is a no-op.
 */
size_t mhc_post_project_workspace_bytes(int64_t T, int64_t H); /* 0 for T == 0 or an unsupported H */
mhc_status mhc_post_project(const uint16_t *x, const uint16_t *res, const float *post, const float *comb,
                            const float *hc_fn_next, int64_t T, int64_t H, uint16_t *out, float *dot_mix,
                            float *sqrsum, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mhc_post_pre_fused -- the post-map of one sublayer and the whole pre-map of the next in
 * one call (FlashInfer mHC article: section 1 for the two stages around each layer,
 * section 2.1 for the post-map, sections 3.4 and 5.2 for the pre-map; metrale dispatch
 * page: hc_post_site and hc_pre_site).  It computes
 *     out[t][n][h] = bf16( x[t][h] post[t][n] + sum_o res[t][o][h] comb[t][o][n] )
 * bit for bit as mhc_post does, and then, over the bf16 `out`, everything mhc_pre_fused
 * computes with the next weights (hc_fn, hc_scale, hc_base):
 *     y, post_next, comb_next and optionally pre_next.
 * With 16-byte rows (H % 8 == 0; x, res, out and y 16-byte aligned) on a 256-CU gfx950,
 * and either T >= 1024 and 1024 < H <= 8192 or 1 <= T <= 192 and H <= 8192, this is one
 * pass: the new streams are written to `out` and kept on chip for the pre-map, so the
 * streams are read once and written once (x, res in; out, y out).  Otherwise it runs
 * mhc_post then mhc_pre_fused on `out`.
 *
 *   x [T,H] bf16; res [T,4,H] bf16; post [T,4], comb [T,4,4] fp32   the post-map's inputs
 *   hc_fn [24,4H], hc_scale [3], hc_base [24] fp32                     the next pre-map's weights
 *   T, H, rms_eps, pre_eps, sinkhorn_eps, post_mult, num_iters         as for mhc_pre_fused
 *   out [T,4,H] bf16       output; may equal `res` exactly (in place)
 *   y [T,H] bf16, post_next [T,4], comb_next [T,4,4] fp32, pre_next [T,4] fp32 or NULL
 *   workspace   at least mhc_pre_fused_workspace_bytes(T, H) bytes, 256-byte aligned
 * No output may overlap an input, the workspace or another output, except out == res;
 * in particular post_next and comb_next must not overlap post and comb.  Errors as for
 * mhc_pre_fused and mhc_post; T == 0 is a no-op.
 */
mhc_status mhc_post_pre_fused(const uint16_t *x, const uint16_t *res, const float *post, const float *comb,
                              const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T, int64_t H,
                              float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int32_t num_iters,
                              uint16_t *out, uint16_t *y, float *post_next, float *comb_next, float *pre_next,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * mhc_sinkhorn_backward -- gradient of mhc_sinkhorn with respect to its logits,
 * through the fixed count of iterations (not the limit of the iteration):
 *     d_logits = J(logits)^T grad,   J the Jacobian of the map computed by mhc_sinkhorn
 * The forward is replayed per matrix, keeping the matrix after every iteration on
 * chip; then, from the last iteration back, the column step Q = A / colsum(A) and
 * the row step A = P / rowsum(P) are reversed, then + eps and the row softmax.
 *
 *   grad      [n_mats, 4, 4] fp32, device: gradient with respect to mhc_sinkhorn's out
 *   logits    [n_mats, 4, 4] fp32, device: the forward's input
 *   n_mats    0 <= n_mats <= 2^32
 *   num_iters 1 <= num_iters <= MHC_SINKHORN_BWD_MAX_ITERS (the forward's count;
 *             the history of one matrix takes 64 * (num_iters + 1) bytes of LDS)
 *   eps       the forward's eps, finite and > 0
 *   d_logits  [n_mats, 4, 4] fp32, device output; may equal `grad` or `logits` exactly,
 *             must not overlap either otherwise
 */
mhc_status mhc_sinkhorn_backward(const float *grad, const float *logits, int64_t n_mats, int32_t num_iters,
                                 float eps, float *d_logits, void *stream);

/*
 * mhc_post_backward -- gradients of mhc_post (FlashInfer mHC article, section 2.1,
 * for the forward formula).  With dO = d_out:
 *     d_x[t][h]       = bf16( sum_n dO[t][n][h] * post[t][n] )
 *     d_res[t][o][h]  = bf16( sum_n comb[t][o][n] * dO[t][n][h] )
 *     d_post[t][n]    = sum_h dO[t][n][h] * x[t][h]                 (fp32)
 *     d_comb[t][o][n] = sum_h res[t][o][h] * dO[t][n][h]            (fp32)
 *   (fp32 accumulation; the sums over h are reduced in a fixed order, so repeated
 *   calls are bit-identical)
 *
 *   d_out [T,4,H] bf16   gradient with respect to mhc_post's out, device
 *   x [T,H], res [T,4,H], post [T,4], comb [T,4,4]   the forward's inputs, device
 *   T >= 0, H >= 1
 *   d_x [T,H] bf16, d_res [T,4,H] bf16, d_post [T,4] fp32, d_comb [T,4,4] fp32
 *             outputs, device.  d_res may equal d_out exactly (each element of d_out
 *             is read before the d_res element at the same place is written); no
 *             other overlap between an output and an input or another output is allowed.
 */
mhc_status mhc_post_backward(const uint16_t *d_out, const uint16_t *x, const uint16_t *res, const float *post,
                             const float *comb, int64_t T, int64_t H, uint16_t *d_x, uint16_t *d_res,
                             float *d_post, float *d_comb, void *stream);

/*
 * Size in bytes of the device workspace mhc_pre_from_dots_backward needs for T tokens:
 * one row of 28 fp32 per token (24 logit gradients and 3 per-group scale terms) and
 * one such row per 256 tokens for the partial sums over the tokens, each part rounded
 * up to 256 bytes.  Returns 0 for T <= 0.
 */
size_t mhc_pre_backward_workspace_bytes(int64_t T);

/*
 * mhc_pre_from_dots_backward -- gradients of mhc_pre_from_dots: the rwkv-ops
 * mhc_pre_op custom VJP (MhcPreOpBwd: sigmoid weights, Sinkhorn, stream aggregate),
 * extended by the FlashInfer mixes in front of it (FlashInfer mHC article,
 * section 5.2: m = d * rstd, per-group scale and base, pre_eps, post_mult).  The
 * forward's mixes are recomputed from the same inputs.  With z_r = m_r * s_g + b_r:
 *     d_pre_i   = sum_h dy[t][h] res[t][i][h];   dz_i = d_pre_i sigma'(z_i)            (i < 4)
 *     dz_{4+i}  = d_post[t][i] post_mult sigma'(z_{4+i})
 *     dz_{8..}  = Sinkhorn reverse mode of d_comb[t] at the comb logits (as mhc_sinkhorn_backward)
 *     d_dot[t][r] = dz_r s_g rstd_t                          (the same for every split)
 *     dS_t      = -(sum_r dz_r s_g d_r) rstd_t^3 / (2k)
 *     d_res[t][i][h] = bf16( pre_i dy[t][h] + 2 dS_t res[t][i][h] )   (second term only when
 *                      sqrsum is NULL, i.e. when the forward computed S from res)
 *     d_sqrsum[s][t] = dS_t for every split s                 (only when sqrsum is given)
 *     d_hc_base[r] = sum_t dz_r,  d_hc_scale[g] = sum_t sum_{r in group g} dz_r m_r
 *   (token sums in a fixed order; repeated calls are bit-identical)
 *
 *   dy [T,H] bf16, d_post [T,4] fp32, d_comb [T,4,4] fp32   gradients of y, post, comb
 *   dot_mix, sqrsum, num_splits, res, hc_scale, hc_base, T, H, k, rms_eps, pre_eps,
 *   sinkhorn_eps, post_mult, num_iters   the forward's inputs, as in mhc_pre_from_dots;
 *               here 1 <= num_iters <= MHC_SINKHORN_BWD_MAX_ITERS
 *   d_res [T,4,H] bf16   output; may equal `res` exactly (every element is read before
 *               it is written), no other overlap
 *   d_dot [T,24] fp32    output: gradient of each split's partial dots
 *   d_sqrsum [T] fp32    output, required when sqrsum is given (gradient of each split's
 *               partial), ignored (may be NULL) otherwise
 *   d_hc_scale [3], d_hc_base [24] fp32   outputs, overwritten (not accumulated).  For
 *               T == 0 they are set to zero (one small launch) and nothing else runs.
 *   workspace   device scratch of at least mhc_pre_backward_workspace_bytes(T) bytes,
 *               256-byte aligned (may be NULL when T == 0); contents on entry ignored
 * No output may overlap an input, the workspace or another output, except as stated.
 */
mhc_status mhc_pre_from_dots_backward(const uint16_t *dy, const float *d_post, const float *d_comb,
                                      const float *dot_mix, const float *sqrsum, int32_t num_splits,
                                      const uint16_t *res, const float *hc_scale, const float *hc_base, int64_t T,
                                      int64_t H, float k, float rms_eps, float pre_eps, float sinkhorn_eps,
                                      float post_mult, int32_t num_iters, uint16_t *d_res, float *d_dot,
                                      float *d_sqrsum, float *d_hc_scale, float *d_hc_base, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * Size in bytes of the device workspace mhc_pre_fused_backward needs for (T, H): the
 * forward's projection workspace, the weights split for the reverse products, per-token
 * values (pre, dS, the logit gradients as bf16 halves, row-major and transposed), the
 * token-sum rows and per-token-range partial sums of d_hc_fn.  Returns 0 for T <= 0,
 * H <= 0, H % 8 != 0 or H beyond the pre-map limit.
 */
size_t mhc_pre_fused_backward_workspace_bytes(int64_t T, int64_t H);

/*
 * mhc_pre_fused_backward -- gradients of mhc_pre_fused (the whole pre-map, projection
 * inside).  The forward's dots and sum of squares are recomputed from res and hc_fn;
 * then the reverse of mhc_pre_from_dots_backward's chain with the sum of squares taken
 * from the streams (k = 4H), and the projection's reverse:
 *     d_res[t][i][h] = bf16( pre_i dy[t][h] + 2 dS_t res[t][i][h] + sum_r dd[t][r] hc_fn[r][i*H+h] )
 *     d_hc_fn[r][k]  = sum_t dd[t][r] res_flat[t][k]            (dd = d_dot of the dots)
 *     d_hc_scale, d_hc_base as in mhc_pre_from_dots_backward
 *   (the weight products use bf16 hi + lo halves of both factors, three products,
 *   fp32 accumulation; every sum over tokens runs in a fixed order)
 *
 *   dy [T,H] bf16, d_post [T,4] fp32, d_comb [T,4,4] fp32   gradients of y, post, comb
 *   res, hc_fn, hc_scale, hc_base, rms_eps, pre_eps, sinkhorn_eps, post_mult   as in
 *               mhc_pre_fused; 1 <= num_iters <= MHC_SINKHORN_BWD_MAX_ITERS
 *   T >= 0; 8 <= H <= 2097152 with H % 8 == 0; dy, res and d_res 16-byte aligned
 *   d_res [T,4,H] bf16   output; may equal `res` exactly
 *   d_hc_fn [24,4H] fp32, d_hc_scale [3], d_hc_base [24]   outputs, overwritten.  For
 *               T == 0 they are set to zero and nothing else runs.
 *   workspace   at least mhc_pre_fused_backward_workspace_bytes(T, H) bytes, 256-byte
 *               aligned (may be NULL when T == 0)
 * No output may overlap an input, the workspace or another output, except as stated.
 */
mhc_status mhc_pre_fused_backward(const uint16_t *dy, const float *d_post, const float *d_comb, const uint16_t *res,
                                  const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
                                  int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                                  int32_t num_iters, uint16_t *d_res, float *d_hc_fn, float *d_hc_scale,
                                  float *d_hc_base, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H_ */
