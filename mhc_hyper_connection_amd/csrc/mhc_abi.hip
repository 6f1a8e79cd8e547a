// mhc_abi.hip -- the extern "C" entry points of libmhc: argument validation on
// the host, then kernel launches on the caller's stream.  No entry point
// allocates, frees or synchronises.
#include "mhc.h"
#include "mhc_internal.h"

#include <atomic>
#include <math.h>
#include <string.h>

namespace {

using mhc::PreGeom;

constexpr int64_t kMaxDim = (int64_t)1 << 30;
// The pre-map addresses a 64-token tile of the streams with 32-bit byte offsets.
constexpr int64_t kPreMaxH = (int64_t)1 << 21;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void *p) { return ((uintptr_t)p & 7u) == 0; }

// FP32 streams: the projection addresses a 64-token tile ([64][4][H] fp32) with 32-bit
// byte offsets.
constexpr int64_t kF32MaxH = (int64_t)1 << 20;

// Do [a, a + an) and [b, b + bn) share a byte?
bool overlaps(const void *a, size_t an, const void *b, size_t bn)
{
    if (!a || !b || an == 0 || bn == 0) {
        return false;
    }
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

bool finite(float v) { return isfinite(v) != 0; }

// Every size the kernels index stays below 2^31 wavefronts / elements per row.
bool sizes_ok(int64_t T, int64_t H)
{
    if (T < 0 || H < 1 || H > kMaxDim || T > kMaxDim) {
        return false;
    }
    const int64_t waves = T * ((H + 63) / 64);
    return waves < ((int64_t)1 << 31) / 4;
}

mhc_status launch_status(hipError_t e) { return e == hipSuccess ? MHC_SUCCESS : MHC_ERROR_LAUNCH; }

constexpr int kMixRows = 24;

// Shared validation and launch of the pre-map forms: the full pre-map (24 weight
// rows, fp32 or bf16) and the weighted head (4 rows, pre weights and y only).
// 16-byte rows: the pre-map's wide loads and its one-read form need them
bool pre_vec8(const uint16_t *res, const uint16_t *y, int64_t H) { return (H % 8 == 0) && aligned16(res) && aligned16(y); }

mhc_status pre_common(const uint16_t *res, const void *hc_fn, bool fn_bf16, int fn_rows, const float *hc_scale,
                      int n_scale, const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                      float sinkhorn_eps, float post_mult, int32_t num_iters, bool head, uint16_t *y, float *post,
                      float *comb, float *pre, void *workspace, size_t workspace_bytes, void *stream,
                      bool validate_only = false, bool presplit = false)
{
    if (!sizes_ok(T, H) || H > kPreMaxH || num_iters < 1 || !finite(rms_eps) || !(rms_eps > 0.0f) || !finite(pre_eps) ||
        pre_eps < 0.0f || !finite(sinkhorn_eps) || !(sinkhorn_eps > 0.0f) || !finite(post_mult)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!res || !hc_fn || !hc_scale || !hc_base || !y || (!head && (!post || !comb))) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const PreGeom g = mhc::pre_geometry(T, H);
    const bool vec8 = pre_vec8(res, y, H);
    // the need of the form this call takes (never above mhc_pre_fused_workspace_bytes)
    const size_t ws_need = mhc::pre_path_workspace_bytes(T, H, vec8);
    if (!validate_only && (!workspace || workspace_bytes < ws_need || ((uintptr_t)workspace & 255u) != 0)) {
        return MHC_ERROR_WORKSPACE;
    }
    const size_t res_b = (size_t)T * 4 * H * 2, y_b = (size_t)T * H * 2;
    const size_t post_b = head ? 0 : (size_t)T * 4 * 4, comb_b = head ? 0 : (size_t)T * 16 * 4;
    const size_t pre_b = pre ? (size_t)T * 4 * 4 : 0;
    const size_t fn_b = (size_t)fn_rows * 4 * H * (fn_bf16 ? 2 : 4);
    // Outputs must not overlap inputs, each other, or the workspace.
    const void *outs[5] = {y, post, comb, pre, workspace};
    const size_t outn[5] = {y_b, post_b, comb_b, pre_b, ws_need};
    const void *ins[4] = {res, hc_fn, hc_scale, hc_base};
    const size_t inn[4] = {res_b, fn_b, (size_t)n_scale * 4, (size_t)fn_rows * 4};
    for (int a = 0; a < 5; ++a) {
        for (int b = 0; b < 4; ++b) {
            if (overlaps(outs[a], outn[a], ins[b], inn[b])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
        for (int b = a + 1; b < 5; ++b) {
            if (overlaps(outs[a], outn[a], outs[b], outn[b])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    if (validate_only) {
        return MHC_SUCCESS;
    }
    return launch_status(mhc::launch_pre(res, hc_fn, fn_bf16, fn_rows, hc_scale, hc_base, g, rms_eps, pre_eps,
                                         sinkhorn_eps, post_mult, num_iters, head, y, post, comb, pre, workspace,
                                         (hipStream_t)stream, vec8, presplit));
}

// The no-allocation pre-map's scratch: a file-scope device array.  In host code the name
// stands for a host-side handle, not a device address: the address on each device comes
// from hipGetSymbolAddress with that device current, once, and only that pointer is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[MHC_PRE_FUSED_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The array's address on the current device (resolved on the first call there), or
// nullptr with the HIP error in `err`.
void *scratch_on_current_device(hipError_t &err)
{
    int dev = -1;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || p == nullptr) {
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

} // namespace

extern "C" {

int mhc_abi_version(void) { return MHC_ABI_VERSION; }

void mhc_set_exchange_test_hooks(int32_t max_retry, uint32_t tag_skew)
{
    mhc::set_exchange_test_hooks(max_retry, tag_skew);
}

const char *mhc_status_string(mhc_status status)
{
    switch (status) {
    case MHC_SUCCESS:
        return "success";
    case MHC_ERROR_INVALID_VALUE:
        return "invalid argument";
    case MHC_ERROR_WORKSPACE:
        return "workspace missing, misaligned or too small (or above the no-allocation scratch)";
    case MHC_ERROR_LAUNCH:
        return "kernel launch failed";
    }
    return "unknown status";
}

mhc_status mhc_launch_plan(const char *entry, int64_t T, int64_t H, int32_t vec8, int64_t *launches,
                           int64_t *tokens_per_launch, int64_t *max_items)
{
    if (!entry || !launches || !tokens_per_launch || !max_items || T < 0 || H < 1) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool v = vec8 != 0;
    int64_t per_tok = 0, block = 256, per_launch = 0;
    if (!strcmp(entry, "post")) {
        per_tok = mhc::post_items_per_token(H, v);
    } else if (!strcmp(entry, "expand") || !strcmp(entry, "head_mean")) {
        per_tok = mhc::stream_copy_items_per_token(H, v);
    } else if (!strcmp(entry, "pre_fused")) {
        const PreGeom g = mhc::pre_geometry(T > 0 ? T : 1, H);
        per_tok = mhc::collapse_items_per_token(H, v);
        per_tok = per_tok > (int64_t)g.nrec * 4 ? per_tok : (int64_t)g.nrec * 4; // slice sums: nrec * 256 per 64
        per_launch = g.chunk;
    } else if (!strcmp(entry, "post_f32")) {
        per_tok = mhc::post_f32s_items_per_token(H, v);
    } else if (!strcmp(entry, "expand_f32") || !strcmp(entry, "head_mean_f32")) {
        per_tok = mhc::stream_copy_f32s_items_per_token(H, v);
    } else if (!strcmp(entry, "collapse")) {
        per_tok = mhc::collapse_items_per_token(H, v);
    } else if (!strcmp(entry, "pre_from_dots")) {
        per_tok = mhc::pre_dots_items_per_token();
    } else if (!strcmp(entry, "pre_from_dots_backward")) {
        per_tok = mhc::pre_dots_bwd_items_per_token();
    } else if (!strcmp(entry, "post_backward")) {
        per_tok = mhc::post_bwd_items_per_token();
    } else if (!strcmp(entry, "sinkhorn")) {
        per_tok = mhc::sinkhorn_items_per_matrix();
    } else if (!strcmp(entry, "sinkhorn_backward")) {
        per_tok = mhc::sinkhorn_bwd_items_per_matrix();
        block = 64;
    } else {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (per_launch == 0) {
        per_launch = mhc::launch_tokens(per_tok);
    }
    const int64_t n = T < per_launch ? T : per_launch;
    *launches = (T + per_launch - 1) / per_launch;
    *tokens_per_launch = per_launch;
    *max_items = (n * per_tok + block - 1) / block * block;
    return MHC_SUCCESS;
}

mhc_status mhc_sinkhorn(const float *logits, float *out, int64_t n_mats, int32_t num_iters, float eps, void *stream)
{
    if (n_mats < 0 || n_mats > ((int64_t)1 << 40) || num_iters < 1 || !finite(eps) || !(eps > 0.0f)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (n_mats == 0) {
        return MHC_SUCCESS;
    }
    if (!logits || !out) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t bytes = (size_t)n_mats * 16 * sizeof(float);
    if ((const void *)out != (const void *)logits && overlaps(out, bytes, logits, bytes)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec4 = aligned16(logits) && aligned16(out);
    return launch_status(mhc::launch_sinkhorn(logits, out, n_mats, num_iters, eps, (hipStream_t)stream, vec4));
}

size_t mhc_pre_fused_workspace_bytes(int64_t T, int64_t H)
{
    if (T <= 0 || H <= 0 || H > kPreMaxH || !sizes_ok(T, H)) {
        return 0;
    }
    return mhc::pre_fused_workspace_bytes(T, H);
}

mhc_status mhc_pre_fused(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                         int64_t T, int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                         int32_t num_iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    return pre_common(res, hc_fn, false, kMixRows, hc_scale, 3, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps,
                      post_mult, num_iters, false, y, post, comb, pre, workspace, workspace_bytes, stream);
}

size_t mhc_pre_split_bytes(int64_t H)
{
    if (H <= 0 || H > kPreMaxH) {
        return 0;
    }
    return mhc::pre_split_bytes(H);
}

mhc_status mhc_pre_split_weights(const float *hc_fn, int64_t H, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    if (H <= 0 || H > kPreMaxH || !hc_fn) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t need = mhc::pre_split_bytes(H);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) {
        return MHC_ERROR_WORKSPACE;
    }
    if (overlaps(workspace, need, hc_fn, (size_t)kMixRows * 4 * H * 4)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    return launch_status(mhc::launch_pre_split_any(hc_fn, false, kMixRows, H, workspace, (hipStream_t)stream));
}

mhc_status mhc_pre_fused_presplit(const uint16_t *res, const float *hc_fn, const float *hc_scale,
                                  const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                                  float sinkhorn_eps, float post_mult, int32_t num_iters, uint16_t *y, float *post,
                                  float *comb, float *pre, void *workspace, size_t workspace_bytes, void *stream)
{
    return pre_common(res, hc_fn, false, kMixRows, hc_scale, 3, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps,
                      post_mult, num_iters, false, y, post, comb, pre, workspace, workspace_bytes, stream, false,
                      true);
}

mhc_status mhc_pre_fused_noalloc(const uint16_t *res, const float *hc_fn, const float *hc_scale,
                                 const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                                 float sinkhorn_eps, float post_mult, int32_t num_iters, uint16_t *y, float *post,
                                 float *comb, float *pre, void *stream)
{
    // every check of mhc_pre_fused except the workspace, before the device is touched
    const mhc_status v = pre_common(res, hc_fn, false, kMixRows, hc_scale, 3, hc_base, T, H, rms_eps, pre_eps,
                                    sinkhorn_eps, post_mult, num_iters, false, y, post, comb, pre, nullptr, 0,
                                    stream, true);
    if (v != MHC_SUCCESS || T == 0) {
        return v;
    }
    if (mhc::pre_path_workspace_bytes(T, H, pre_vec8(res, y, H)) > MHC_PRE_FUSED_NOALLOC_MAX_BYTES) {
        return MHC_ERROR_WORKSPACE;
    }
    hipError_t e = hipSuccess;
    void *ws = scratch_on_current_device(e);
    if (ws == nullptr) {
        return MHC_ERROR_LAUNCH;
    }
    return pre_common(res, hc_fn, false, kMixRows, hc_scale, 3, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps,
                      post_mult, num_iters, false, y, post, comb, pre, ws, MHC_PRE_FUSED_NOALLOC_MAX_BYTES, stream);
}

mhc_status mhc_pre_fused_bf16(const uint16_t *res, const uint16_t *hc_fn, const float *hc_scale,
                              const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                              float sinkhorn_eps, float post_mult, int32_t num_iters, uint16_t *y, float *post,
                              float *comb, float *pre, void *workspace, size_t workspace_bytes, void *stream)
{
    return pre_common(res, hc_fn, true, kMixRows, hc_scale, 3, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps,
                      post_mult, num_iters, false, y, post, comb, pre, workspace, workspace_bytes, stream);
}

mhc_status mhc_head(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
                    int64_t H, float norm_eps, float hc_eps, uint16_t *y, float *pre, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    return pre_common(res, hc_fn, false, 4, hc_scale, 1, hc_base, T, H, norm_eps, hc_eps, 1.0f, 1.0f, 1, true, y,
                      nullptr, nullptr, pre, workspace, workspace_bytes, stream);
}

mhc_status mhc_head_mean(const uint16_t *res, int64_t T, int64_t H, uint16_t *y, void *stream)
{
    if (!sizes_ok(T, H)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!res || !y || overlaps(y, (size_t)T * H * 2, res, (size_t)T * 4 * H * 2)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec8 = (H % 8 == 0) && aligned16(res) && aligned16(y);
    return launch_status(mhc::launch_head_mean(res, T, H, y, (hipStream_t)stream, vec8));
}

mhc_status mhc_expand(const uint16_t *hidden, int64_t T, int64_t H, uint16_t *streams, void *stream)
{
    if (!sizes_ok(T, H)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!hidden || !streams || overlaps(streams, (size_t)T * 4 * H * 2, hidden, (size_t)T * H * 2)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec8 = (H % 8 == 0) && aligned16(hidden) && aligned16(streams);
    return launch_status(mhc::launch_expand(hidden, T, H, streams, (hipStream_t)stream, vec8));
}

mhc_status mhc_pre_from_dots(const float *dot_mix, const float *sqrsum, int32_t num_splits, const uint16_t *res,
                             const float *hc_scale, const float *hc_base, int64_t T, int64_t H, float k,
                             float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int32_t num_iters,
                             uint16_t *y, float *post, float *comb, float *pre, void *stream)
{
    if (!sizes_ok(T, H) || num_splits < 1 || num_splits > 65536 || num_iters < 1 || !finite(k) || !(k > 0.0f) ||
        !finite(rms_eps) || !(rms_eps > 0.0f) || !finite(pre_eps) || pre_eps < 0.0f || !finite(sinkhorn_eps) ||
        !(sinkhorn_eps > 0.0f) || !finite(post_mult)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!dot_mix || !res || !hc_scale || !hc_base || !y || !post || !comb) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t res_b = (size_t)T * 4 * H * 2, y_b = (size_t)T * H * 2;
    const size_t post_b = (size_t)T * 4 * 4, comb_b = (size_t)T * 16 * 4, pre_b = pre ? (size_t)T * 4 * 4 : 0;
    const size_t dm_b = (size_t)num_splits * T * 24 * 4, sq_b = sqrsum ? (size_t)num_splits * T * 4 : 0;
    const void *outs[4] = {y, post, comb, pre};
    const size_t outn[4] = {y_b, post_b, comb_b, pre_b};
    const void *ins[5] = {res, dot_mix, sqrsum, hc_scale, hc_base};
    const size_t inn[5] = {res_b, dm_b, sq_b, 3 * 4, 24 * 4};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 5; ++i) {
            if (overlaps(outs[o], outn[o], ins[i], inn[i])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
        for (int o2 = o + 1; o2 < 4; ++o2) {
            if (overlaps(outs[o], outn[o], outs[o2], outn[o2])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    const bool vec8 = (H % 8 == 0) && aligned16(res) && aligned16(y);
    return launch_status(mhc::launch_pre_dots(dot_mix, sqrsum, num_splits, res, hc_scale, hc_base, T, H, k, rms_eps,
                                              pre_eps, sinkhorn_eps, post_mult, num_iters, y, post, comb, pre,
                                              (hipStream_t)stream, vec8));
}

mhc_status mhc_post(const uint16_t *x, const uint16_t *res, const float *post, const float *comb, int64_t T,
                    int64_t H, uint16_t *out, void *stream)
{
    if (!sizes_ok(T, H)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!x || !res || !post || !comb || !out) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t res_b = (size_t)T * 4 * H * 2, x_b = (size_t)T * H * 2;
    const size_t post_b = (size_t)T * 4 * 4, comb_b = (size_t)T * 16 * 4;
    if ((const void *)out != (const void *)res && overlaps(out, res_b, res, res_b)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (overlaps(out, res_b, x, x_b) || overlaps(out, res_b, post, post_b) || overlaps(out, res_b, comb, comb_b)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec8 = (H % 8 == 0) && aligned16(x) && aligned16(res) && aligned16(out);
    return launch_status(mhc::launch_post(x, res, post, comb, T, H, out, (hipStream_t)stream, vec8));
}

// ---------------------------------------------------------------- FP32 residual streams

mhc_status mhc_post_f32(const uint16_t *x, const float *res, const float *post, const float *comb, int64_t T,
                        int64_t H, float *out, void *stream)
{
    if (!sizes_ok(T, H) || H > kF32MaxH) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!x || !res || !post || !comb || !out) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t res_b = (size_t)T * 4 * H * 4, x_b = (size_t)T * H * 2;
    const size_t post_b = (size_t)T * 4 * 4, comb_b = (size_t)T * 16 * 4;
    if ((const void *)out != (const void *)res && overlaps(out, res_b, res, res_b)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (overlaps(out, res_b, x, x_b) || overlaps(out, res_b, post, post_b) || overlaps(out, res_b, comb, comb_b)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec4 = (H % 4 == 0) && aligned8(x) && aligned16(res) && aligned16(out);
    return launch_status(mhc::launch_post_f32s(x, res, post, comb, T, H, out, (hipStream_t)stream, vec4));
}

mhc_status mhc_expand_f32(const uint16_t *hidden, int64_t T, int64_t H, float *streams, void *stream)
{
    if (!sizes_ok(T, H) || H > kF32MaxH) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!hidden || !streams || overlaps(streams, (size_t)T * 4 * H * 4, hidden, (size_t)T * H * 2)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec4 = (H % 4 == 0) && aligned8(hidden) && aligned16(streams);
    return launch_status(mhc::launch_expand_f32s(hidden, T, H, streams, (hipStream_t)stream, vec4));
}

mhc_status mhc_head_mean_f32(const float *res, int64_t T, int64_t H, uint16_t *y, void *stream)
{
    if (!sizes_ok(T, H) || H > kF32MaxH) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!res || !y || overlaps(y, (size_t)T * H * 2, res, (size_t)T * 4 * H * 4)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec4 = (H % 4 == 0) && aligned16(res) && aligned8(y);
    return launch_status(mhc::launch_head_mean_f32s(res, T, H, y, (hipStream_t)stream, vec4));
}

mhc_status mhc_pre_fused_f32(const float *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                             int64_t T, int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                             int32_t num_iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    if (!sizes_ok(T, H) || H > kF32MaxH || num_iters < 1 || !finite(rms_eps) || !(rms_eps > 0.0f) ||
        !finite(pre_eps) || pre_eps < 0.0f || !finite(sinkhorn_eps) || !(sinkhorn_eps > 0.0f) || !finite(post_mult)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!res || !hc_fn || !hc_scale || !hc_base || !y || !post || !comb) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const PreGeom g = mhc::pre_geometry(T, H);
    if (!workspace || workspace_bytes < g.total_bytes || ((uintptr_t)workspace & 255u) != 0) {
        return MHC_ERROR_WORKSPACE;
    }
    const size_t res_b = (size_t)T * 4 * H * 4, y_b = (size_t)T * H * 2;
    const size_t post_b = (size_t)T * 4 * 4, comb_b = (size_t)T * 16 * 4, pre_b = pre ? (size_t)T * 4 * 4 : 0;
    const size_t fn_b = (size_t)kMixRows * 4 * H * 4;
    const void *outs[5] = {y, post, comb, pre, workspace};
    const size_t outn[5] = {y_b, post_b, comb_b, pre_b, g.total_bytes};
    const void *ins[4] = {res, hc_fn, hc_scale, hc_base};
    const size_t inn[4] = {res_b, fn_b, 3 * 4, (size_t)kMixRows * 4};
    for (int a = 0; a < 5; ++a) {
        for (int b = 0; b < 4; ++b) {
            if (overlaps(outs[a], outn[a], ins[b], inn[b])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
        for (int b = a + 1; b < 5; ++b) {
            if (overlaps(outs[a], outn[a], outs[b], outn[b])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    const bool vec4 = (H % 4 == 0) && aligned16(res) && aligned8(y);
    return launch_status(mhc::launch_pre_f32s(res, hc_fn, hc_scale, hc_base, g, rms_eps, pre_eps, sinkhorn_eps,
                                              post_mult, num_iters, y, post, comb, pre, workspace,
                                              (hipStream_t)stream, vec4));
}

size_t mhc_post_project_workspace_bytes(int64_t T, int64_t H)
{
    if (T <= 0 || H < 8 || H % 8 != 0 || H > kPreMaxH || !sizes_ok(T, H)) {
        return 0;
    }
    return mhc::post_project_workspace_bytes(T, H);
}

mhc_status mhc_post_project(const uint16_t *x, const uint16_t *res, const float *post, const float *comb,
                            const float *hc_fn_next, int64_t T, int64_t H, uint16_t *out, float *dot_mix,
                            float *sqrsum, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!sizes_ok(T, H) || H % 8 != 0 || H > kPreMaxH) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!x || !res || !post || !comb || !hc_fn_next || !out || !dot_mix || !sqrsum) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (!aligned16(x) || !aligned16(res) || !aligned16(out)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t need = mhc::post_project_workspace_bytes(T, H);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) {
        return MHC_ERROR_WORKSPACE;
    }
    const size_t res_b = (size_t)T * 4 * H * 2, x_b = (size_t)T * H * 2, fn_b = (size_t)24 * 4 * H * 4;
    const void *outs[4] = {out, dot_mix, sqrsum, workspace};
    const size_t outn[4] = {res_b, (size_t)T * 24 * 4, (size_t)T * 4, need};
    const void *ins[5] = {res, x, post, comb, hc_fn_next};
    const size_t inn[5] = {res_b, x_b, (size_t)T * 16, (size_t)T * 64, fn_b};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 5; ++i) {
            const bool in_place = o == 0 && i == 0 && (const void *)out == (const void *)res;
            if (!in_place && overlaps(outs[o], outn[o], ins[i], inn[i])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
        for (int o2 = o + 1; o2 < 4; ++o2) {
            if (overlaps(outs[o], outn[o], outs[o2], outn[o2])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    return launch_status(mhc::launch_post_project(x, res, post, comb, hc_fn_next, T, H, out, dot_mix, sqrsum,
                                                  workspace, (hipStream_t)stream));
}

mhc_status mhc_post_pre_fused(const uint16_t *x, const uint16_t *res, const float *post, const float *comb,
                              const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T, int64_t H,
                              float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int32_t num_iters,
                              uint16_t *out, uint16_t *y, float *post_next, float *comb_next, float *pre_next,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    // the next pre-map over `out`: its parameters, pointers and output overlaps (pre_common
    // with res = out, nothing launched)
    const mhc_status v = pre_common(out, hc_fn, false, kMixRows, hc_scale, 3, hc_base, T, H, rms_eps, pre_eps,
                                    sinkhorn_eps, post_mult, num_iters, false, y, post_next, comb_next, pre_next,
                                    workspace, workspace_bytes, stream, true);
    if (v != MHC_SUCCESS || T == 0) {
        return v;
    }
    if (!x || !res || !post || !comb) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const bool vec8_pre = pre_vec8(out, y, H);
    const size_t need = mhc::pre_path_workspace_bytes(T, H, vec8_pre);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) {
        return MHC_ERROR_WORKSPACE;
    }
    // the post-map's inputs against every output (out may equal res exactly)
    const size_t res_b = (size_t)T * 4 * H * 2, x_b = (size_t)T * H * 2, y_b = (size_t)T * H * 2;
    const size_t fn_b = (size_t)kMixRows * 4 * H * 4;
    const void *outs[6] = {out, y, post_next, comb_next, pre_next, workspace};
    const size_t outn[6] = {res_b, y_b, (size_t)T * 16, (size_t)T * 64, pre_next ? (size_t)T * 16 : 0, need};
    const void *ins[4] = {res, x, post, comb};
    const size_t inn[4] = {res_b, x_b, (size_t)T * 16, (size_t)T * 64};
    for (int o = 0; o < 6; ++o) {
        for (int i = 0; i < 4; ++i) {
            const bool in_place = o == 0 && i == 0 && (const void *)out == (const void *)res;
            if (!in_place && overlaps(outs[o], outn[o], ins[i], inn[i])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    if (overlaps(out, res_b, hc_fn, fn_b) || overlaps(out, res_b, hc_scale, 12) || overlaps(out, res_b, hc_base, 96)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    hipStream_t st = (hipStream_t)stream;
    const bool vec8_post = (H % 8 == 0) && aligned16(x) && aligned16(res) && aligned16(out);
    if (vec8_post && vec8_pre && mhc::pre_coop_usable(T, H, true)) {
        return launch_status(mhc::launch_post_pre_coop(x, res, post, comb, hc_fn, hc_scale, hc_base, T, H, rms_eps,
                                                       pre_eps, sinkhorn_eps, post_mult, num_iters, out, y, post_next,
                                                       comb_next, pre_next, workspace, st));
    }
    if (vec8_post && vec8_pre && mhc::pre_decode_usable(T, H, true)) {
        return launch_status(mhc::launch_post_pre_decode(x, res, post, comb, hc_fn, hc_scale, hc_base, T, H, rms_eps,
                                                         pre_eps, sinkhorn_eps, post_mult, num_iters, out, y,
                                                         post_next, comb_next, pre_next, workspace, st));
    }
    // other shapes: the post-map, then the pre-map over the streams it wrote
    hipError_t e = mhc::launch_post(x, res, post, comb, T, H, out, st, vec8_post);
    if (e != hipSuccess) {
        return MHC_ERROR_LAUNCH;
    }
    return launch_status(mhc::launch_pre(out, hc_fn, false, kMixRows, hc_scale, hc_base, mhc::pre_geometry(T, H),
                                         rms_eps, pre_eps, sinkhorn_eps, post_mult, num_iters, false, y, post_next,
                                         comb_next, pre_next, workspace, st, vec8_pre));
}

mhc_status mhc_sinkhorn_backward(const float *grad, const float *logits, int64_t n_mats, int32_t num_iters,
                                 float eps, float *d_logits, void *stream)
{
    if (n_mats < 0 || n_mats > ((int64_t)1 << 32) || num_iters < 1 || num_iters > MHC_SINKHORN_BWD_MAX_ITERS ||
        !finite(eps) || !(eps > 0.0f)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (n_mats == 0) {
        return MHC_SUCCESS;
    }
    if (!grad || !logits || !d_logits) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t bytes = (size_t)n_mats * 16 * sizeof(float);
    if (((const void *)d_logits != (const void *)grad && overlaps(d_logits, bytes, grad, bytes)) ||
        ((const void *)d_logits != (const void *)logits && overlaps(d_logits, bytes, logits, bytes))) {
        return MHC_ERROR_INVALID_VALUE;
    }
    return launch_status(
        mhc::launch_sinkhorn_bwd(grad, logits, n_mats, num_iters, eps, d_logits, (hipStream_t)stream));
}

mhc_status mhc_post_backward(const uint16_t *d_out, const uint16_t *x, const uint16_t *res, const float *post,
                             const float *comb, int64_t T, int64_t H, uint16_t *d_x, uint16_t *d_res,
                             float *d_post, float *d_comb, void *stream)
{
    if (!sizes_ok(T, H)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return MHC_SUCCESS;
    }
    if (!d_out || !x || !res || !post || !comb || !d_x || !d_res || !d_post || !d_comb) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t res_b = (size_t)T * 4 * H * 2, x_b = (size_t)T * H * 2;
    const size_t post_b = (size_t)T * 4 * 4, comb_b = (size_t)T * 16 * 4;
    const void *outs[4] = {d_x, d_res, d_post, d_comb};
    const size_t outn[4] = {x_b, res_b, post_b, comb_b};
    const void *ins[5] = {d_out, x, res, post, comb};
    const size_t inn[5] = {res_b, x_b, res_b, post_b, comb_b};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 5; ++i) {
            const bool in_place = o == 1 && i == 0 && (const void *)d_res == (const void *)d_out;
            if (!in_place && overlaps(outs[o], outn[o], ins[i], inn[i])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
        for (int o2 = o + 1; o2 < 4; ++o2) {
            if (overlaps(outs[o], outn[o], outs[o2], outn[o2])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    const bool vec8 = (H % 8 == 0) && aligned16(d_out) && aligned16(x) && aligned16(res) && aligned16(d_x) &&
                      aligned16(d_res);
    return launch_status(mhc::launch_post_bwd(d_out, x, res, post, comb, T, H, d_x, d_res, d_post, d_comb,
                                              (hipStream_t)stream, vec8));
}

size_t mhc_pre_backward_workspace_bytes(int64_t T)
{
    if (T <= 0 || T > kMaxDim) {
        return 0;
    }
    return mhc::pre_bwd_workspace_bytes(T);
}

mhc_status mhc_pre_from_dots_backward(const uint16_t *dy, const float *d_post, const float *d_comb,
                                      const float *dot_mix, const float *sqrsum, int32_t num_splits,
                                      const uint16_t *res, const float *hc_scale, const float *hc_base, int64_t T,
                                      int64_t H, float k, float rms_eps, float pre_eps, float sinkhorn_eps,
                                      float post_mult, int32_t num_iters, uint16_t *d_res, float *d_dot,
                                      float *d_sqrsum, float *d_hc_scale, float *d_hc_base, void *workspace,
                                      size_t workspace_bytes, void *stream)
{
    if (!sizes_ok(T, H) || num_splits < 1 || num_splits > 65536 || num_iters < 1 ||
        num_iters > MHC_SINKHORN_BWD_MAX_ITERS || !finite(k) || !(k > 0.0f) || !finite(rms_eps) ||
        !(rms_eps > 0.0f) || !finite(pre_eps) || pre_eps < 0.0f || !finite(sinkhorn_eps) || !(sinkhorn_eps > 0.0f) ||
        !finite(post_mult)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (!d_hc_scale || !d_hc_base || overlaps(d_hc_scale, 3 * 4, d_hc_base, 24 * 4)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return launch_status(mhc::launch_pre_dots_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, num_splits,
                                                      nullptr, nullptr, nullptr, 0, H, k, rms_eps, pre_eps,
                                                      sinkhorn_eps, post_mult, num_iters, nullptr, nullptr, nullptr,
                                                      d_hc_scale, d_hc_base, nullptr, (hipStream_t)stream, false));
    }
    if (!dy || !d_post || !d_comb || !dot_mix || !res || !hc_scale || !hc_base || !d_res || !d_dot ||
        (sqrsum && !d_sqrsum)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t need = mhc::pre_bwd_workspace_bytes(T);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) {
        return MHC_ERROR_WORKSPACE;
    }
    if (!sqrsum) {
        d_sqrsum = nullptr;
    }
    const size_t res_b = (size_t)T * 4 * H * 2, y_b = (size_t)T * H * 2;
    const size_t dm_b = (size_t)num_splits * T * 24 * 4, sq_b = sqrsum ? (size_t)num_splits * T * 4 : 0;
    const void *outs[6] = {d_res, d_dot, d_sqrsum, d_hc_scale, d_hc_base, workspace};
    const size_t outn[6] = {res_b, (size_t)T * 24 * 4, d_sqrsum ? (size_t)T * 4 : 0, 3 * 4, 24 * 4, need};
    const void *ins[8] = {dy, d_post, d_comb, dot_mix, sqrsum, res, hc_scale, hc_base};
    const size_t inn[8] = {y_b, (size_t)T * 16, (size_t)T * 64, dm_b, sq_b, res_b, 3 * 4, 24 * 4};
    for (int o = 0; o < 6; ++o) {
        for (int i = 0; i < 8; ++i) {
            const bool in_place = o == 0 && i == 5 && (const void *)d_res == (const void *)res;
            if (!in_place && overlaps(outs[o], outn[o], ins[i], inn[i])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
        for (int o2 = o + 1; o2 < 6; ++o2) {
            if (overlaps(outs[o], outn[o], outs[o2], outn[o2])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    const bool vec8 = (H % 8 == 0) && aligned16(dy) && aligned16(res) && aligned16(d_res);
    return launch_status(mhc::launch_pre_dots_bwd(dy, d_post, d_comb, dot_mix, sqrsum, num_splits, res, hc_scale,
                                                  hc_base, T, H, k, rms_eps, pre_eps, sinkhorn_eps, post_mult,
                                                  num_iters, d_res, d_dot, d_sqrsum, d_hc_scale, d_hc_base, workspace,
                                                  (hipStream_t)stream, vec8));
}

size_t mhc_pre_fused_backward_workspace_bytes(int64_t T, int64_t H)
{
    if (T <= 0 || H <= 0 || H > kPreMaxH || H % 8 != 0 || !sizes_ok(T, H)) {
        return 0;
    }
    return mhc::pre_fused_bwd_workspace_bytes(T, H);
}

mhc_status mhc_pre_fused_backward(const uint16_t *dy, const float *d_post, const float *d_comb, const uint16_t *res,
                                  const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T,
                                  int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                                  int32_t num_iters, uint16_t *d_res, float *d_hc_fn, float *d_hc_scale,
                                  float *d_hc_base, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!sizes_ok(T, H) || H > kPreMaxH || H % 8 != 0 || num_iters < 1 || num_iters > MHC_SINKHORN_BWD_MAX_ITERS ||
        !finite(rms_eps) || !(rms_eps > 0.0f) || !finite(pre_eps) || pre_eps < 0.0f || !finite(sinkhorn_eps) ||
        !(sinkhorn_eps > 0.0f) || !finite(post_mult)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t fn_b = (size_t)24 * 4 * H * 4;
    if (!d_hc_fn || !d_hc_scale || !d_hc_base || overlaps(d_hc_fn, fn_b, d_hc_scale, 3 * 4) ||
        overlaps(d_hc_fn, fn_b, d_hc_base, 24 * 4) || overlaps(d_hc_scale, 3 * 4, d_hc_base, 24 * 4)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (T == 0) {
        return launch_status(mhc::launch_pre_fused_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                       0, H, rms_eps, pre_eps, sinkhorn_eps, post_mult, num_iters,
                                                       nullptr, d_hc_fn, d_hc_scale, d_hc_base, nullptr,
                                                       (hipStream_t)stream));
    }
    if (!dy || !d_post || !d_comb || !res || !hc_fn || !hc_scale || !hc_base || !d_res) {
        return MHC_ERROR_INVALID_VALUE;
    }
    if (!aligned16(dy) || !aligned16(res) || !aligned16(d_res)) {
        return MHC_ERROR_INVALID_VALUE;
    }
    const size_t need = mhc::pre_fused_bwd_workspace_bytes(T, H);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0) {
        return MHC_ERROR_WORKSPACE;
    }
    const size_t res_b = (size_t)T * 4 * H * 2, y_b = (size_t)T * H * 2;
    const void *outs[5] = {d_res, d_hc_fn, d_hc_scale, d_hc_base, workspace};
    const size_t outn[5] = {res_b, fn_b, 3 * 4, 24 * 4, need};
    const void *ins[7] = {dy, d_post, d_comb, res, hc_fn, hc_scale, hc_base};
    const size_t inn[7] = {y_b, (size_t)T * 16, (size_t)T * 64, res_b, fn_b, 3 * 4, 24 * 4};
    for (int o = 0; o < 5; ++o) {
        for (int i = 0; i < 7; ++i) {
            const bool in_place = o == 0 && i == 3 && (const void *)d_res == (const void *)res;
            if (!in_place && overlaps(outs[o], outn[o], ins[i], inn[i])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
        for (int o2 = o + 1; o2 < 5; ++o2) {
            if (overlaps(outs[o], outn[o], outs[o2], outn[o2])) {
                return MHC_ERROR_INVALID_VALUE;
            }
        }
    }
    return launch_status(mhc::launch_pre_fused_bwd(dy, d_post, d_comb, res, hc_fn, hc_scale, hc_base, T, H, rms_eps,
                                                   pre_eps, sinkhorn_eps, post_mult, num_iters, d_res, d_hc_fn,
                                                   d_hc_scale, d_hc_base, workspace, (hipStream_t)stream));
}

} // extern "C"
