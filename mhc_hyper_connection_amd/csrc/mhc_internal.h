// mhc_internal.h -- host-side launchers shared between the libmhc translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mhc {

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
                      void *workspace, hipStream_t stream, bool vec8);

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
