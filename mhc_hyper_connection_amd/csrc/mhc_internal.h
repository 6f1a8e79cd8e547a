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

// Pre-map geometry: split-K over `slices` contiguous ranges of 32-wide H blocks.
struct PreGeom {
    int64_t T, H;
    int tiles;        // token tiles of 64
    int nhb;          // ceil(H / 32)
    int slices;       // K splits
    int hb_per_slice; // H blocks per split
    size_t part_bytes;  // [slices][T][32] fp32 partial sums
    size_t prew_bytes;  // [T][4] fp32 pre weights
    size_t total_bytes; // workspace size
};
PreGeom pre_geometry(int64_t T, int64_t H);

hipError_t launch_pre(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                      const PreGeom &g, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                      int iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                      hipStream_t stream, bool vec8);

} // namespace mhc
