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

// Fused (read-once) pre-map: tiles of 64 tokens x slices of 128 h, persistent grid.
constexpr int64_t kFusedMaxH = 65536;
struct FusedGeom {
    bool valid;
    int tiles, nhb, S, nclass, nzero;
    size_t off_bfrag, off_part, off_prew, off_sync, bytes;
};
FusedGeom fused_geometry(int64_t T, int64_t H);
// Launches the prep and fused kernels.  Sets *fits = false (and launches nothing)
// when the device cannot keep enough workgroups resident for the tile barriers.
hipError_t launch_pre_fused(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                            const FusedGeom &f, int64_t T, int64_t H, float rms_eps, float pre_eps,
                            float sinkhorn_eps, float post_mult, int iters, uint16_t *y, float *post, float *comb,
                            float *pre, void *workspace, hipStream_t stream, bool vec8, bool *fits);

// Pre-map geometry.  The split-K fallback (three kernels, streams read twice)
// covers H beyond kFusedMaxH and devices that cannot host the fused grid.
struct PreGeom {
    int64_t T, H;
    int tiles;        // token tiles of 64
    int nhb;          // ceil(H / 32)
    int slices;       // K splits
    int hb_per_slice; // H blocks per split
    size_t part_bytes;  // [slices][T][32] fp32 partial sums
    size_t prew_bytes;  // [T][4] fp32 pre weights
    size_t split_bytes;  // split-K fallback workspace
    FusedGeom fused;
    size_t total_bytes; // workspace size: covers whichever path runs
};
PreGeom pre_geometry(int64_t T, int64_t H);

hipError_t launch_pre(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                      const PreGeom &g, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                      int iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                      hipStream_t stream, bool vec8);

} // namespace mhc
