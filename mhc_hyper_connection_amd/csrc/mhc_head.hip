// mhc_head.hip -- model entry and the unweighted head.
//
// (metrale glm5next_mhc.rs: glm_hc_expand broadcasts each hidden row into the
// hc_mult streams; hc_head_mean collapses the streams to their unweighted mean.)
//
// Both are pure streaming: one wavefront per (token, 512-wide H tile), each lane
// moving 8 consecutive h with 16-byte non-temporal accesses; a scalar path (one
// element per lane) covers H % 8 != 0 and unaligned rows.  The weighted head
// runs on the pre-map's kernels (launch_pre with `head`).
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

constexpr int kHBlock = 256;
constexpr int kHWaves = kHBlock / kWave;
constexpr int kHVecTile = kWave * 8;

template <bool kVec>
__global__ __launch_bounds__(kHBlock) void expand_kernel(const uint16_t *__restrict__ hidden, int T, int H,
                                                         int tiles_per_token, uint16_t *__restrict__ streams)
{
    const int wave = uniform(blockIdx.x * kHWaves + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    if constexpr (kVec) {
        const int h = tile * kHVecTile + lane * 8;
        if (h < H) {
            const u32x4 v = load_nt16(hidden + (size_t)t * H + h);
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                store_nt16(streams + ((size_t)t * kHC + i) * H + h, v);
            }
        }
    } else {
        const int h = tile * kWave + lane;
        if (h < H) {
            const uint16_t v = hidden[(size_t)t * H + h];
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                streams[((size_t)t * kHC + i) * H + h] = v;
            }
        }
    }
}

// y = bf16((r0 + r1 + r2 + r3) * 0.25), fp32 sum in a fixed order
template <bool kVec>
__global__ __launch_bounds__(kHBlock) void head_mean_kernel(const uint16_t *__restrict__ res, int T, int H,
                                                            int tiles_per_token, uint16_t *__restrict__ y)
{
    const int wave = uniform(blockIdx.x * kHWaves + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    if constexpr (kVec) {
        const int h = tile * kHVecTile + lane * 8;
        if (h < H) {
            u32x4 r[kHC];
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                r[i] = load_nt16(res + ((size_t)t * kHC + i) * H + h);
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = ((bf16_lo(r[0][q]) + bf16_lo(r[1][q])) + bf16_lo(r[2][q])) + bf16_lo(r[3][q]);
                const float hi = ((bf16_hi(r[0][q]) + bf16_hi(r[1][q])) + bf16_hi(r[2][q])) + bf16_hi(r[3][q]);
                o[q] = pack_bf16x2(lo * 0.25f, hi * 0.25f);
            }
            store_nt16(y + (size_t)t * H + h, o);
        }
    } else {
        const int h = tile * kWave + lane;
        if (h < H) {
            const size_t row = (size_t)t * kHC * H + h;
            const float v = ((bf16_to_f32(res[row]) + bf16_to_f32(res[row + (size_t)H])) +
                             bf16_to_f32(res[row + (size_t)2 * H])) +
                            bf16_to_f32(res[row + (size_t)3 * H]);
            y[(size_t)t * H + h] = f32_to_bf16(v * 0.25f);
        }
    }
}

dim3 stream_grid(int64_t T, int64_t H, bool vec8, int &tiles)
{
    const int tile = vec8 ? kHVecTile : kWave;
    tiles = (int)((H + tile - 1) / tile);
    const int64_t waves = T * tiles;
    return dim3((unsigned)((waves + kHWaves - 1) / kHWaves));
}

} // namespace

hipError_t launch_expand(const uint16_t *hidden, int64_t T, int64_t H, uint16_t *streams, hipStream_t stream,
                         bool vec8)
{
    int tiles;
    const dim3 grid = stream_grid(T, H, vec8, tiles);
    if (vec8) {
        expand_kernel<true><<<grid, dim3(kHBlock), 0, stream>>>(hidden, (int)T, (int)H, tiles, streams);
    } else {
        expand_kernel<false><<<grid, dim3(kHBlock), 0, stream>>>(hidden, (int)T, (int)H, tiles, streams);
    }
    return hipGetLastError();
}

hipError_t launch_head_mean(const uint16_t *res, int64_t T, int64_t H, uint16_t *y, hipStream_t stream, bool vec8)
{
    int tiles;
    const dim3 grid = stream_grid(T, H, vec8, tiles);
    if (vec8) {
        head_mean_kernel<true><<<grid, dim3(kHBlock), 0, stream>>>(res, (int)T, (int)H, tiles, y);
    } else {
        head_mean_kernel<false><<<grid, dim3(kHBlock), 0, stream>>>(res, (int)T, (int)H, tiles, y);
    }
    return hipGetLastError();
}

} // namespace mhc
