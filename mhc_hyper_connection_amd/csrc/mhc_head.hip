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

// FP32 streams: the model entry widens each bf16 h exactly into the 4 fp32 streams, and the
// unweighted head sums them in the same order as the bf16 form.  Vector path: a wave per
// (token, 256-wide tile), 4 h per lane (8-byte bf16, 16-byte fp32 accesses); scalar path:
// a lane per h.
constexpr int kHVecTileF = kWave * 4;

template <bool kVec>
__global__ __launch_bounds__(kHBlock) void expand_f32s_kernel(const uint16_t *__restrict__ hidden, int T, int H,
                                                              int tiles_per_token, float *__restrict__ streams)
{
    const int wave = uniform(blockIdx.x * kHWaves + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    if constexpr (kVec) {
        const int h = tile * kHVecTileF + lane * 4;
        if (h < H) {
            const uint2 w = *reinterpret_cast<const uint2 *>(hidden + (size_t)t * H + h);
            const u32x4 v = __builtin_bit_cast(u32x4, f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)});
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                store_nt16(streams + ((size_t)t * kHC + i) * H + h, v);
            }
        }
    } else {
        const int h = tile * kWave + lane;
        if (h < H) {
            const float v = bf16_to_f32(hidden[(size_t)t * H + h]);
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                streams[((size_t)t * kHC + i) * H + h] = v;
            }
        }
    }
}

template <bool kVec>
__global__ __launch_bounds__(kHBlock) void head_mean_f32s_kernel(const float *__restrict__ res, int T, int H,
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
        const int h = tile * kHVecTileF + lane * 4;
        if (h < H) {
            f32x4 r[kHC];
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                r[i] = __builtin_bit_cast(f32x4, load_nt16(res + ((size_t)t * kHC + i) * H + h));
            }
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = (((r[0][j] + r[1][j]) + r[2][j]) + r[3][j]) * 0.25f;
            }
            *reinterpret_cast<uint2 *>(y + (size_t)t * H + h) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    } else {
        const int h = tile * kWave + lane;
        if (h < H) {
            const size_t row = (size_t)t * kHC * H + h;
            const float v = ((res[row] + res[row + (size_t)H]) + res[row + (size_t)2 * H]) + res[row + (size_t)3 * H];
            y[(size_t)t * H + h] = f32_to_bf16(v * 0.25f);
        }
    }
}

} // namespace

int64_t stream_copy_f32s_items_per_token(int64_t H, bool vec4)
{
    const int tile = vec4 ? kHVecTileF : kWave;
    return (H + tile - 1) / tile * kWave;
}

hipError_t launch_expand_f32s(const uint16_t *hidden, int64_t T, int64_t H, float *streams, hipStream_t stream,
                              bool vec4)
{
    const int tile = vec4 ? kHVecTileF : kWave;
    const int tiles = (int)((H + tile - 1) / tile);
    return for_token_chunks(T, stream_copy_f32s_items_per_token(H, vec4), [&](int64_t c0, int64_t Tc) {
        const dim3 grid((unsigned)((Tc * tiles + kHWaves - 1) / kHWaves));
        const uint16_t *hc = hidden + (size_t)c0 * H;
        float *sc = streams + (size_t)c0 * kHC * H;
        if (vec4) {
            expand_f32s_kernel<true><<<grid, dim3(kHBlock), 0, stream>>>(hc, (int)Tc, (int)H, tiles, sc);
        } else {
            expand_f32s_kernel<false><<<grid, dim3(kHBlock), 0, stream>>>(hc, (int)Tc, (int)H, tiles, sc);
        }
        return hipGetLastError();
    });
}

hipError_t launch_head_mean_f32s(const float *res, int64_t T, int64_t H, uint16_t *y, hipStream_t stream, bool vec4)
{
    const int tile = vec4 ? kHVecTileF : kWave;
    const int tiles = (int)((H + tile - 1) / tile);
    return for_token_chunks(T, stream_copy_f32s_items_per_token(H, vec4), [&](int64_t c0, int64_t Tc) {
        const dim3 grid((unsigned)((Tc * tiles + kHWaves - 1) / kHWaves));
        const float *rc = res + (size_t)c0 * kHC * H;
        uint16_t *yc = y + (size_t)c0 * H;
        if (vec4) {
            head_mean_f32s_kernel<true><<<grid, dim3(kHBlock), 0, stream>>>(rc, (int)Tc, (int)H, tiles, yc);
        } else {
            head_mean_f32s_kernel<false><<<grid, dim3(kHBlock), 0, stream>>>(rc, (int)Tc, (int)H, tiles, yc);
        }
        return hipGetLastError();
    });
}

int64_t stream_copy_items_per_token(int64_t H, bool vec8)
{
    const int tile = vec8 ? kHVecTile : kWave;
    return (H + tile - 1) / tile * kWave;
}

hipError_t launch_expand(const uint16_t *hidden, int64_t T, int64_t H, uint16_t *streams, hipStream_t stream,
                         bool vec8)
{
    const int tile = vec8 ? kHVecTile : kWave;
    const int tiles = (int)((H + tile - 1) / tile);
    return for_token_chunks(T, stream_copy_items_per_token(H, vec8), [&](int64_t c0, int64_t Tc) {
        const dim3 grid((unsigned)((Tc * tiles + kHWaves - 1) / kHWaves));
        const uint16_t *hc = hidden + (size_t)c0 * H;
        uint16_t *sc = streams + (size_t)c0 * kHC * H;
        if (vec8) {
            expand_kernel<true><<<grid, dim3(kHBlock), 0, stream>>>(hc, (int)Tc, (int)H, tiles, sc);
        } else {
            expand_kernel<false><<<grid, dim3(kHBlock), 0, stream>>>(hc, (int)Tc, (int)H, tiles, sc);
        }
        return hipGetLastError();
    });
}

hipError_t launch_head_mean(const uint16_t *res, int64_t T, int64_t H, uint16_t *y, hipStream_t stream, bool vec8)
{
    const int tile = vec8 ? kHVecTile : kWave;
    const int tiles = (int)((H + tile - 1) / tile);
    return for_token_chunks(T, stream_copy_items_per_token(H, vec8), [&](int64_t c0, int64_t Tc) {
        const dim3 grid((unsigned)((Tc * tiles + kHWaves - 1) / kHWaves));
        const uint16_t *rc = res + (size_t)c0 * kHC * H;
        uint16_t *yc = y + (size_t)c0 * H;
        if (vec8) {
            head_mean_kernel<true><<<grid, dim3(kHBlock), 0, stream>>>(rc, (int)Tc, (int)H, tiles, yc);
        } else {
            head_mean_kernel<false><<<grid, dim3(kHBlock), 0, stream>>>(rc, (int)Tc, (int)H, tiles, yc);
        }
        return hipGetLastError();
    });
}

} // namespace mhc
