// mhc_post.hip -- the mHC post-map on gfx950.
//
//   out[t][n][h] = bf16( x[t][h] * post[t][n] + sum_o res[t][o][h] * comb[t][o][n] )
//
// ("FlashInfer mHC 模块深度解析", section 2.1; metrale glm5next_mhc.rs, glm_hc_post.)
//
// Layout of the work: one wavefront owns one (token, 512-element H tile).  Each
// lane moves 8 consecutive h of x and of the four old streams with 16-byte
// loads, and writes 8 h of the four new streams with 16-byte stores.  The
// token's 20 coefficients are wave-uniform and live in SGPRs (scalar loads), so
// no LDS and no cross-lane traffic is needed.  Every lane reads all four old
// streams of its elements before writing them, which makes out == res safe.
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

constexpr int kPostBlock = 256;
constexpr int kPostWavesPerBlock = kPostBlock / kWave;
constexpr int kVecTile = kWave * 8; // h elements per wave tile (vector path)

__device__ __forceinline__ void unpack8(const u32x4 &w, float *f)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf16_lo(w[q]);
        f[2 * q + 1] = bf16_hi(w[q]);
    }
}

__global__ __launch_bounds__(kPostBlock) void post_vec8_kernel(const uint16_t *__restrict__ x, const uint16_t *res,
                                                               const float *__restrict__ post,
                                                               const float *__restrict__ comb, int T, int H,
                                                               int tiles_per_token, uint16_t *out)
{
    const int wave = uniform(blockIdx.x * kPostWavesPerBlock + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    const int h = tile * kVecTile + lane * 8;
    if (h >= H) {
        return;
    }
    float p[kHC], c[kHC * kHC];
#pragma unroll
    for (int n = 0; n < kHC; ++n) {
        p[n] = post[(size_t)t * kHC + n];
    }
#pragma unroll
    for (int e = 0; e < kHC * kHC; ++e) {
        c[e] = comb[(size_t)t * kHC * kHC + e];
    }
    const size_t row = (size_t)t * kHC * H + h;
    const u32x4 xw = load_nt16(x + (size_t)t * H + h);
    u32x4 rw[kHC];
#pragma unroll
    for (int o = 0; o < kHC; ++o) {
        rw[o] = load_nt16(res + row + (size_t)o * H);
    }
    float xf[8], rf[kHC][8];
    unpack8(xw, xf);
#pragma unroll
    for (int o = 0; o < kHC; ++o) {
        unpack8(rw[o], rf[o]);
    }
#pragma unroll
    for (int n = 0; n < kHC; ++n) {
        u32x4 ow;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float v[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = 2 * q + e;
                float a = xf[j] * p[n];
                a = fmaf(rf[0][j], c[0 * kHC + n], a);
                a = fmaf(rf[1][j], c[1 * kHC + n], a);
                a = fmaf(rf[2][j], c[2 * kHC + n], a);
                a = fmaf(rf[3][j], c[3 * kHC + n], a);
                v[e] = a;
            }
            ow[q] = pack_bf16x2(v[0], v[1]);
        }
        store_nt16(out + row + (size_t)n * H, ow);
    }
}

// Scalar path: any H and any alignment.  One lane per h; wave tile of 64 h.
__global__ __launch_bounds__(kPostBlock) void post_scalar_kernel(const uint16_t *__restrict__ x, const uint16_t *res,
                                                                 const float *__restrict__ post,
                                                                 const float *__restrict__ comb, int T, int H,
                                                                 int tiles_per_token, uint16_t *out)
{
    const int wave = uniform(blockIdx.x * kPostWavesPerBlock + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    const int h = tile * kWave + lane;
    if (h >= H) {
        return;
    }
    const size_t row = (size_t)t * kHC * H + h;
    const float xf = bf16_to_f32(x[(size_t)t * H + h]);
    float rf[kHC];
#pragma unroll
    for (int o = 0; o < kHC; ++o) {
        rf[o] = bf16_to_f32(res[row + (size_t)o * H]);
    }
#pragma unroll
    for (int n = 0; n < kHC; ++n) {
        float a = xf * post[(size_t)t * kHC + n];
#pragma unroll
        for (int o = 0; o < kHC; ++o) {
            a = fmaf(rf[o], comb[(size_t)t * kHC * kHC + o * kHC + n], a);
        }
        out[row + (size_t)n * H] = f32_to_bf16(a);
    }
}

// FP32 streams (res and out fp32, x bf16): the same formula and FMA order.  Vector path:
// a wave per (token, 256-wide tile), 4 h per lane: an 8-byte x load and 16-byte stream
// loads and stores.  Scalar path: a lane per h, a wave tile of 64 h.
constexpr int kVecTileF = kWave * 4;

template <bool kVec>
__global__ __launch_bounds__(kPostBlock) void post_f32s_kernel(const uint16_t *__restrict__ x, const float *res,
                                                               const float *__restrict__ post,
                                                               const float *__restrict__ comb, int T, int H,
                                                               int tiles_per_token, float *out)
{
    const int wave = uniform(blockIdx.x * kPostWavesPerBlock + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    const int h = tile * (kVec ? kVecTileF : kWave) + lane * (kVec ? 4 : 1);
    if (h >= H) {
        return;
    }
    float p[kHC], c[kHC * kHC];
#pragma unroll
    for (int n = 0; n < kHC; ++n) {
        p[n] = post[(size_t)t * kHC + n];
    }
#pragma unroll
    for (int e = 0; e < kHC * kHC; ++e) {
        c[e] = comb[(size_t)t * kHC * kHC + e];
    }
    const size_t row = (size_t)t * kHC * H + h;
    constexpr int kE = kVec ? 4 : 1;
    float xf[kE], rf[kHC][kE];
    if constexpr (kVec) {
        const uint2 xw = *reinterpret_cast<const uint2 *>(x + (size_t)t * H + h);
        xf[0] = bf16_lo(xw.x);
        xf[1] = bf16_hi(xw.x);
        xf[2] = bf16_lo(xw.y);
        xf[3] = bf16_hi(xw.y);
#pragma unroll
        for (int o = 0; o < kHC; ++o) {
            const f32x4 v = __builtin_bit_cast(f32x4, load_nt16(res + row + (size_t)o * H));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                rf[o][j] = v[j];
            }
        }
    } else {
        xf[0] = bf16_to_f32(x[(size_t)t * H + h]);
#pragma unroll
        for (int o = 0; o < kHC; ++o) {
            rf[o][0] = res[row + (size_t)o * H];
        }
    }
#pragma unroll
    for (int n = 0; n < kHC; ++n) {
        float v[kE];
#pragma unroll
        for (int j = 0; j < kE; ++j) {
            float a = xf[j] * p[n];
            a = fmaf(rf[0][j], c[0 * kHC + n], a);
            a = fmaf(rf[1][j], c[1 * kHC + n], a);
            a = fmaf(rf[2][j], c[2 * kHC + n], a);
            a = fmaf(rf[3][j], c[3 * kHC + n], a);
            v[j] = a;
        }
        if constexpr (kVec) {
            store_nt16(out + row + (size_t)n * H, __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}));
        } else {
            out[row + (size_t)n * H] = v[0];
        }
    }
}

} // namespace

int64_t post_f32s_items_per_token(int64_t H, bool vec4)
{
    const int tile = vec4 ? kVecTileF : kWave;
    return (H + tile - 1) / tile * kWave;
}

hipError_t launch_post_f32s(const uint16_t *x, const float *res, const float *post, const float *comb, int64_t T,
                            int64_t H, float *out, hipStream_t stream, bool vec4)
{
    const int tile = vec4 ? kVecTileF : kWave;
    const int64_t tiles = (H + tile - 1) / tile;
    return for_token_chunks(T, post_f32s_items_per_token(H, vec4), [&](int64_t c0, int64_t Tc) {
        const int64_t blocks = (Tc * tiles + kPostWavesPerBlock - 1) / kPostWavesPerBlock;
        const size_t s = (size_t)c0 * kHC * H;
        if (vec4) {
            post_f32s_kernel<true><<<dim3((unsigned)blocks), dim3(kPostBlock), 0, stream>>>(
                x + (size_t)c0 * H, res + s, post + (size_t)c0 * kHC, comb + (size_t)c0 * kHC * kHC, (int)Tc,
                (int)H, (int)tiles, out + s);
        } else {
            post_f32s_kernel<false><<<dim3((unsigned)blocks), dim3(kPostBlock), 0, stream>>>(
                x + (size_t)c0 * H, res + s, post + (size_t)c0 * kHC, comb + (size_t)c0 * kHC * kHC, (int)Tc,
                (int)H, (int)tiles, out + s);
        }
        return hipGetLastError();
    });
}

int64_t post_items_per_token(int64_t H, bool vec8)
{
    const int tile = vec8 ? kVecTile : kWave;
    return (H + tile - 1) / tile * kWave;
}

hipError_t launch_post(const uint16_t *x, const uint16_t *res, const float *post, const float *comb, int64_t T,
                       int64_t H, uint16_t *out, hipStream_t stream, bool vec8)
{
    const int tile = vec8 ? kVecTile : kWave;
    const int64_t tiles = (H + tile - 1) / tile;
    return for_token_chunks(T, post_items_per_token(H, vec8), [&](int64_t c0, int64_t Tc) {
        const int64_t blocks = (Tc * tiles + kPostWavesPerBlock - 1) / kPostWavesPerBlock;
        const size_t s = (size_t)c0 * kHC * H;
        if (vec8) {
            post_vec8_kernel<<<dim3((unsigned)blocks), dim3(kPostBlock), 0, stream>>>(
                x + (size_t)c0 * H, res + s, post + (size_t)c0 * kHC, comb + (size_t)c0 * kHC * kHC, (int)Tc,
                (int)H, (int)tiles, out + s);
        } else {
            post_scalar_kernel<<<dim3((unsigned)blocks), dim3(kPostBlock), 0, stream>>>(
                x + (size_t)c0 * H, res + s, post + (size_t)c0 * kHC, comb + (size_t)c0 * kHC * kHC, (int)Tc,
                (int)H, (int)tiles, out + s);
        }
        return hipGetLastError();
    });
}

} // namespace mhc
