// mhc_internal.h -- host-side launchers shared between the libmhc translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mhc {

// Token-parallel launches are split into token chunks so that every launch covers fewer
// than kLaunchItems work-items (a grid dimension holds fewer than 2^32; below 2^31 every
// int index a kernel forms from its block and thread ids is exact) and at most
// kLaunchTokens tokens (per-token offsets such as t * 24 stay far below 2^31).  Each
// chunk is launched on pointers advanced to its first token.
constexpr int64_t kLaunchItems = (int64_t)1 << 31;
constexpr int64_t kLaunchTokens = (int64_t)1 << 24;

// Tokens per launch of a grid with `items_per_token` work-items per token (a grid rounded
// up to whole blocks adds fewer than one block).
inline int64_t launch_tokens(int64_t items_per_token)
{
    const int64_t n = (kLaunchItems - 1024) / (items_per_token > 0 ? items_per_token : 1);
    return n < 1 ? 1 : (n < kLaunchTokens ? n : kLaunchTokens);
}

// Calls f(c0, Tc) for the chunks [c0, c0 + Tc) of [0, T), stopping at the first error.
template <typename F> hipError_t for_token_chunks(int64_t T, int64_t items_per_token, F &&f)
{
    const int64_t per = launch_tokens(items_per_token);
    for (int64_t c0 = 0; c0 < T; c0 += per) {
        const hipError_t e = f(c0, T - c0 < per ? T - c0 : per);
        if (e != hipSuccess) {
            return e;
        }
    }
    return hipSuccess;
}

// Work-items per token (per matrix for the Sinkhorn kernels) of each token-parallel
// kernel, as its launcher sizes the grid and its token chunks.
int64_t post_items_per_token(int64_t H, bool vec8);
int64_t stream_copy_items_per_token(int64_t H, bool vec8); // expand and head_mean
int64_t collapse_items_per_token(int64_t H, bool vec8);    // the pre-map's collapse
int64_t pre_dots_items_per_token();
int64_t pre_dots_bwd_items_per_token();
int64_t post_bwd_items_per_token();
int64_t sinkhorn_items_per_matrix();
int64_t sinkhorn_bwd_items_per_matrix();

// Post-map.  `vec8`: H % 8 == 0 and x/res/out 16-byte aligned.
hipError_t launch_post(const uint16_t *x, const uint16_t *res, const float *post, const float *comb, int64_t T,
                       int64_t H, uint16_t *out, hipStream_t stream, bool vec8);

// Standalone Sinkhorn.  `vec4`: logits and out 16-byte aligned.
hipError_t launch_sinkhorn(const float *logits, float *out, int64_t n, int iters, float eps, hipStream_t stream,
                           bool vec4);

// Pre-map geometry.  Tokens are processed in chunks of `chunk` (a multiple of
// 64) so that every buffer view the kernels build stays below 2^31 bytes.
struct PreGeom {
    int64_t T, H;
    int64_t chunk;     // tokens per launch chunk
    int tiles;         // 64-token tiles in one chunk
    int nhb;           // ceil(H / 32)
    int slices;        // workgroups per 64-token tile in the projection
    int nrec;          // fields per record: 25, or 29 with the reverse's <dy, res_i>
    size_t off_frag;   // split weights in MFMA operand order
    size_t off_rec;    // partial records of one chunk
    size_t rec_bytes;
    size_t off_prew;   // per-token field sums of one chunk
    size_t total_bytes;
};
PreGeom pre_geometry(int64_t T, int64_t H, bool with_dy = false);

// The pre-map (and, with `head`, the weighted head: `fn_rows` = 4 weight rows, pre
// weights and y only).  `hc_fn` is fp32, or bf16 bit patterns when `fn_bf16`.
hipError_t launch_pre(const uint16_t *res, const void *hc_fn, bool fn_bf16, int fn_rows, const float *hc_scale,
                      const float *hc_base, const PreGeom &g, float rms_eps, float pre_eps, float sinkhorn_eps,
                      float post_mult, int iters, bool head, uint16_t *y, float *post, float *comb, float *pre,
                      void *workspace, hipStream_t stream, bool vec8, bool presplit = false);
// The weight split of the two-pass pre-map (bf16 x 3 MFMA fragments of hc_fn, fp32 or
// bf16 with `fn_rows` rows) into the fragment area at the start of a pre-map workspace,
// pre_split_bytes(H) bytes; launch_pre with `presplit` then skips it.
hipError_t launch_pre_split_any(const void *hc_fn, bool fn_bf16, int fn_rows, int64_t H, void *workspace,
                                hipStream_t stream);
size_t pre_split_bytes(int64_t H);

// The pre-map with one read of the streams: on each of the 8 XCDs a group of 32
// workgroups splits K, holds 16-token steps of the streams in LDS and exchanges partial
// sums through the XCD's L2 (mhc_pre_coop.hip).  Usable for 16-byte rows with
// 2 <= ceil(ceil(H / 32) / 32) <= 8 (1024 < H <= 8192) and T >= 1024, on a 256-CU gfx950.
// Its workspace is a ring of exchange records, pre_coop_workspace_bytes(H) bytes.
size_t pre_coop_workspace_bytes(int64_t H);
bool pre_coop_shape_ok(int64_t T, int64_t H); // the shape alone (no device or alignment check)
bool pre_coop_usable(int64_t T, int64_t H, bool vec8);
hipError_t launch_pre_coop(const uint16_t *res, const void *hc_fn, bool fn_bf16, int fn_rows, const float *hc_scale,
                           const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                           float sinkhorn_eps, float post_mult, int iters, bool head, uint16_t *y, float *post,
                           float *comb, float *pre, void *workspace, hipStream_t stream);
// The post-map and the next pre-map in one pass (pre_coop_kernel with the post-map in front):
// the new streams out = post-map(x, res, post_in, comb_in) are written and also held on chip
// for the next pre-map, which reads them from there.  Same shape conditions and workspace as
// launch_pre_coop; fp32 weights.
hipError_t launch_post_pre_coop(const uint16_t *x, const uint16_t *res, const float *post_in, const float *comb_in,
                                const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T, int64_t H,
                                float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int iters,
                                uint16_t *out, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                                hipStream_t stream);
// Test hooks of the one-read form's exchange (mhc_set_exchange_test_hooks): the reloads of a
// step's records before its outputs become NaN (negative: the default 2^14) and a value
// mixed into the tags readers expect (0 in normal use).
void set_exchange_test_hooks(int max_retry, uint32_t tag_skew);
// What those hooks hold now, and whether the current device runs the exchange kernels
// (256 CUs on gfx950: one workgroup per CU, 32 on each XCD).
int exchange_max_retry();
uint32_t exchange_tag_skew();
bool exchange_device_ok();

// The pre-map for small batches in one launch (mhc_pre_decode.hip): on each XCD a group of
// 32 workgroups splits K over the group's ceil(T / 8) tokens and exchanges partial sums
// through the XCD's L2.  Usable for 16-byte rows, 1 <= T <= 192 and H <= 8192 on a 256-CU
// gfx950; the weights are read as given (fp32 or bf16), never split.  Its exchange records
// sit at pre_split_bytes(H) in the workspace, behind the place of a weight split, which it
// leaves as it is; pre_decode_workspace_bytes(H) bytes in all.
bool pre_decode_shape_ok(int64_t T, int64_t H);
bool pre_decode_usable(int64_t T, int64_t H, bool vec8);
size_t pre_decode_workspace_bytes(int64_t H);
hipError_t launch_pre_decode(const uint16_t *res, const void *hc_fn, bool fn_bf16, int fn_rows,
                             const float *hc_scale, const float *hc_base, int64_t T, int64_t H, float rms_eps,
                             float pre_eps, float sinkhorn_eps, float post_mult, int iters, bool head, uint16_t *y,
                             float *post, float *comb, float *pre, void *workspace, hipStream_t stream);
// The post-map and the next pre-map in one launch of the small-batch form: the new streams
// out = post-map(x, res, post_in, comb_in) are formed in the workgroups' tiles, written,
// and the pre-map proceeds on them.  Same shape conditions and workspace as
// launch_pre_decode; fp32 weights; out may equal res.
hipError_t launch_post_pre_decode(const uint16_t *x, const uint16_t *res, const float *post_in,
                                  const float *comb_in, const float *hc_fn, const float *hc_scale,
                                  const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                                  float sinkhorn_eps, float post_mult, int iters, uint16_t *out, uint16_t *y,
                                  float *post, float *comb, float *pre, void *workspace, hipStream_t stream);
// Workspace of the pre-map entry points: enough for either form.
size_t pre_fused_workspace_bytes(int64_t T, int64_t H);
// Workspace of the form a call with these sizes and 16-byte rows (vec8) or not takes on the
// current device; at most pre_fused_workspace_bytes.
size_t pre_path_workspace_bytes(int64_t T, int64_t H, bool vec8);

// The pre-map's first stages on their own: the weight split (once), then for the token
// chunk [c0, c0 + Tc) the projection and the slice sums, which leave the per-token
// fields in the workspace at g.off_prew ([Tc][32] fp32: pre dots 0..3, the sum of
// squares at 4, post dots 5..8, comb dots 9..24; with `dy` (the reverse's recompute,
// g from pre_geometry(T, H, true), vec8 only) also <dy, res_i> at 25..28).
hipError_t launch_pre_split(const float *hc_fn, const PreGeom &g, void *workspace, hipStream_t stream);
hipError_t launch_pre_sums(const uint16_t *res, const uint16_t *dy, const PreGeom &g, int64_t c0, int Tc,
                           void *workspace, hipStream_t stream, bool vec8);

// The post-map fused with the next sublayer's projection (H % 8 == 0, 16-byte aligned
// rows): out as launch_post writes it, plus the next pre-map's 24 dots and sum of
// squares over out (dot_mix [T][24], sqrsum [T]).  The workspace is laid out as the
// pre-map's (pre_geometry(T, H)): the next weights split for the MFMA and one token
// chunk's partial records.
size_t post_project_workspace_bytes(int64_t T, int64_t H);
hipError_t launch_post_project(const uint16_t *x, const uint16_t *res, const float *post, const float *comb,
                               const float *hc_fn_next, int64_t T, int64_t H, uint16_t *out, float *dot_mix,
                               float *sqrsum, void *workspace, hipStream_t stream);

// FP32 residual streams [T][4][H] (x, hidden and y stay bf16).  `vec4`: H % 4 == 0, the
// fp32 arrays 16-byte and the bf16 rows 8-byte aligned.  The pre-map takes the two-pass
// form with the workspace layout of pre_geometry(T, H) (its weight-fragment area unused).
hipError_t launch_pre_f32s(const float *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                           const PreGeom &g, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                           int iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                           hipStream_t stream, bool vec4);
hipError_t launch_post_f32s(const uint16_t *x, const float *res, const float *post, const float *comb, int64_t T,
                            int64_t H, float *out, hipStream_t stream, bool vec4);
hipError_t launch_expand_f32s(const uint16_t *hidden, int64_t T, int64_t H, float *streams, hipStream_t stream,
                              bool vec4);
hipError_t launch_head_mean_f32s(const float *res, int64_t T, int64_t H, uint16_t *y, hipStream_t stream, bool vec4);
int64_t post_f32s_items_per_token(int64_t H, bool vec4);
int64_t stream_copy_f32s_items_per_token(int64_t H, bool vec4);

// Model entry (each hidden row copied into the 4 streams) and the unweighted head (the
// mean of the 4 streams).  `vec8`: H % 8 == 0 and both pointers 16-byte aligned.
hipError_t launch_expand(const uint16_t *hidden, int64_t T, int64_t H, uint16_t *streams, hipStream_t stream,
                         bool vec8);
hipError_t launch_head_mean(const uint16_t *res, int64_t T, int64_t H, uint16_t *y, hipStream_t stream, bool vec8);

// Pre-map from external dots (one workgroup per token).  `vec8`: H % 8 == 0 and res/y
// 16-byte aligned.  One split with a supplied sum of squares and vec8 goes to
// launch_collapse_dots instead.
hipError_t launch_pre_dots(const float *dot_mix, const float *sqrsum, int num_splits, const uint16_t *res,
                           const float *hc_scale, const float *hc_base, int64_t T, int64_t H, float k,
                           float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int iters,
                           uint16_t *y, float *post, float *comb, float *pre, hipStream_t stream, bool vec8);

// The pre-map's collapse kernel fed external dots: one split, dots [T][24] and the sum
// of squares [T] supplied, H % 8 == 0 and res/y 16-byte aligned.  One wavefront per
// (token, 512-wide h tile), the first tile's also writing post, comb and pre.
hipError_t launch_collapse_dots(const float *dots, const float *sq, const uint16_t *res, const float *hc_scale,
                                const float *hc_base, int64_t T, int64_t H, float k, float rms_eps, float pre_eps,
                                float sinkhorn_eps, float post_mult, int iters, uint16_t *y, float *post,
                                float *comb, float *pre, hipStream_t stream);

// Reverse mode of the standalone Sinkhorn (16 lanes per matrix, LDS history).
size_t sinkhorn_bwd_lds_bytes(int iters);
hipError_t launch_sinkhorn_bwd(const float *grad, const float *logits, int64_t n, int iters, float eps,
                               float *d_logits, hipStream_t stream);

// Reverse mode of the pre-map from external dots (one workgroup per token), then the
// fixed-order token sums of d_hc_scale and d_hc_base from a [T][28] fp32 workspace.
size_t pre_bwd_workspace_bytes(int64_t T);
hipError_t launch_pre_dots_bwd(const uint16_t *dy, const float *d_post, const float *d_comb, const float *dot_mix,
                               const float *sqrsum, int num_splits, const uint16_t *res, const float *hc_scale,
                               const float *hc_base, int64_t T, int64_t H, float k, float rms_eps, float pre_eps,
                               float sinkhorn_eps, float post_mult, int iters, uint16_t *d_res, float *d_dot,
                               float *d_sqrsum, float *d_hc_scale, float *d_hc_base, void *workspace,
                               hipStream_t stream, bool vec8);

// Reverse mode of the whole pre-map (projection inside): forward fields recomputed,
// the per-token reverse, token sums, then the projection's reverse (d_res with the
// weight term, d_hc_fn over token ranges).  Needs H % 8 == 0 and 16-byte aligned rows.
size_t pre_fused_bwd_workspace_bytes(int64_t T, int64_t H);
hipError_t launch_pre_fused_bwd(const uint16_t *dy, const float *d_post, const float *d_comb, const uint16_t *res,
                                const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
                                int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                                int iters, uint16_t *d_res, float *d_hc_fn, float *d_hc_scale, float *d_hc_base,
                                void *workspace, hipStream_t stream);

// Reverse mode of the post-map (one workgroup per token).  `vec8`: H % 8 == 0 and
// d_out/x/res/d_x/d_res 16-byte aligned.
hipError_t launch_post_bwd(const uint16_t *d_out, const uint16_t *x, const uint16_t *res, const float *post,
                           const float *comb, int64_t T, int64_t H, uint16_t *d_x, uint16_t *d_res, float *d_post,
                           float *d_comb, hipStream_t stream, bool vec8);

} // namespace mhc
