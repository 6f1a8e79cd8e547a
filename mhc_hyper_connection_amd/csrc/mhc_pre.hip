// mhc_pre.hip -- the mHC pre-map on gfx950.
//
// ("FlashInfer mHC 模块深度解析", sections 3.4 and 5.2; metrale
// hyper_connection_dispatch.rs, hc_pre_site; metrale glm5next_mhc.rs, the
// hc_mix / hc_finish split.)
//
// This file holds the split-K fallback used for H beyond the fused kernel's
// range (mhc_pre_fused.hip holds the read-once path).  Three kernels on one
// stream:
//
//  1. pre_proj_kernel -- the 24 x 4H projection and the sum of squares, on MFMA.
//     A workgroup owns 64 tokens x one contiguous range of H (all four streams),
//     i.e. a split-K slice.  The streams are bf16, so they feed
//     v_mfma_f32_16x16x32_bf16 unchanged.  hc_fn is fp32; each value is split
//     exactly into three bf16 terms hi + mid + lo (truncations: 8 + 8 + 8
//     significant bits), so three bf16 products accumulated in fp32 reproduce
//     the fp32 weight without rounding it.  The sum of squares rides along on
//     v_dot2_f32_bf16 from the same registers.  Each workgroup writes one
//     partial record [25] per token and slice (no atomics; fixed reduction order).
//  2. pre_mix_kernel -- one lane per token: sums the partials in slice order,
//     rstd, the sigmoid mixes and the 4x4 Sinkhorn in registers; writes post,
//     comb, pre.
//  3. pre_collapse_kernel -- y = sum_i pre_i * res_i, one wavefront per
//     (token, 512-element H tile), 16-byte loads, coefficients in SGPRs.
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

constexpr int kProjBlock = 256;
constexpr int kProjWaves = kProjBlock / kWave;
constexpr int kTileTokens = 64; // 4 MFMA row tiles of 16 tokens
constexpr int kMTiles = kTileTokens / 16;
constexpr int kHBlock = 32;     // h per MFMA step per stream: 4 lane groups x 8
constexpr int kPartStride = 32; // floats per (slice, token) partial: 24 dots, sum of squares, padding
constexpr int kSqSlot = kMix;   // index of the sum of squares inside a partial record
constexpr int kTargetBlocks = 2048;
// The read-once cooperative kernel is correct but its cross-workgroup exchange
// is still latency-bound; the split-K path is faster until that is fixed.
constexpr bool kUseFusedPre = false;

constexpr int kColBlock = 256;
constexpr int kColWaves = kColBlock / kWave;
constexpr int kColVecTile = kWave * 8;

// v == hi + mid + lo exactly for normal fp32 v: each term is a truncation of
// what remains to bf16 (8 significant bits), and a 24-bit significand has no
// bits left after three of them.
__device__ __forceinline__ void split3(const float *v, bf16x8 &hi, bf16x8 &mid, bf16x8 &lo)
{
    u32x4 ph, pm, pl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t h0 = __float_as_uint(v[2 * q]) & 0xFFFF0000u;
        uint32_t h1 = __float_as_uint(v[2 * q + 1]) & 0xFFFF0000u;
        float r0 = v[2 * q] - __uint_as_float(h0);
        float r1 = v[2 * q + 1] - __uint_as_float(h1);
        uint32_t m0 = __float_as_uint(r0) & 0xFFFF0000u;
        uint32_t m1 = __float_as_uint(r1) & 0xFFFF0000u;
        float l0 = r0 - __uint_as_float(m0);
        float l1 = r1 - __uint_as_float(m1);
        ph[q] = (h0 >> 16) | h1;
        pm[q] = (m0 >> 16) | m1;
        pl[q] = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u);
    }
    hi = __builtin_bit_cast(bf16x8, ph);
    mid = __builtin_bit_cast(bf16x8, pm);
    lo = __builtin_bit_cast(bf16x8, pl);
}

// Eight consecutive bf16 of a stream row starting at h (zeros past H or past T).
template <bool kVec>
__device__ __forceinline__ u32x4 load_a(const uint16_t *p, int h, int H, bool ok)
{
    u32x4 w = {0u, 0u, 0u, 0u};
    if (kVec) {
        if (ok && h < H) {
            w = load_nt16(p);
        }
    } else if (ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t lo = (h + 2 * q < H) ? (uint32_t)p[2 * q] : 0u;
            uint32_t hi = (h + 2 * q + 1 < H) ? (uint32_t)p[2 * q + 1] : 0u;
            w[q] = lo | (hi << 16);
        }
    }
    return w;
}

template <bool kVec>
__device__ __forceinline__ void load_b(const float *p, int h, int H, bool ok, float *v)
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[j] = 0.0f;
    }
    if (kVec) {
        if (ok && h < H) {
            const f32x4 v0 = *reinterpret_cast<const f32x4 *>(p);
            const f32x4 v1 = *reinterpret_cast<const f32x4 *>(p + 4);
            v[0] = v0[0], v[1] = v0[1], v[2] = v0[2], v[3] = v0[3];
            v[4] = v1[0], v[5] = v1[1], v[6] = v1[2], v[7] = v1[3];
        }
    } else if (ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[j] = (h + j < H) ? p[j] : 0.0f;
        }
    }
}

// MFMA operand layout (16x16x32 bf16): lane l holds row/column (l % 16) and the
// 8 k-values of lane group g = l / 16; the result lane l, register q holds
// row 4g + q, column l % 16.  Here a k-step is one stream i and 32 consecutive
// h (lane group g takes h = 32*hb + 8g .. +8), identically for A and B.
template <bool kVec>
__global__ __launch_bounds__(kProjBlock) void pre_proj_kernel(const uint16_t *__restrict__ res,
                                                              const float *__restrict__ hc_fn, int T, int H,
                                                              int nhb, int hb_per_slice, float *__restrict__ part)
{
    const int tile = blockIdx.x;
    const int slice = blockIdx.y;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;
    const int c = lane & 15;
    const int t0 = tile * kTileTokens;
    const int hb_begin = slice * hb_per_slice;
    const int hb_end = min(nhb, hb_begin + hb_per_slice);
    const size_t K = (size_t)kHC * H;

    f32x4 acc[kMTiles][2];
    float sq[kMTiles];
#pragma unroll
    for (int m = 0; m < kMTiles; ++m) {
        acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        sq[m] = 0.0f;
    }

    for (int hb = hb_begin + w; hb < hb_end; hb += kProjWaves) {
        const int h = hb * kHBlock + g * 8;
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
            bf16x8 a[kMTiles];
#pragma unroll
            for (int m = 0; m < kMTiles; ++m) {
                const int t = t0 + m * 16 + c;
                const u32x4 wa = load_a<kVec>(res + ((size_t)t * kHC + i) * H + h, h, H, t < T);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // Copy the element to a scalar first: hipcc (clang 22) miscompiles
                    // __builtin_bit_cast applied directly to an ext_vector element
                    // (it reads element 0 for every q).
                    const uint32_t wq = wa[q];
                    const bf16x2 pr = __builtin_bit_cast(bf16x2, wq);
                    sq[m] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, sq[m], false);
                }
                a[m] = __builtin_bit_cast(bf16x8, wa);
            }
            bf16x8 b[2][3];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int r = n * 16 + c;
                float v[8];
                load_b<kVec>(hc_fn + (size_t)r * K + (size_t)i * H + h, h, H, r < kMix, v);
                split3(v, b[n][0], b[n][1], b[n][2]);
            }
#pragma unroll
            for (int s = 0; s < 3; ++s) {
#pragma unroll
                for (int m = 0; m < kMTiles; ++m) {
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[n][s], acc[m][n], 0, 0, 0);
                    }
                }
            }
        }
    }

    // Reduce the four waves (and, for the sum of squares, the four lane groups)
    // through LDS in a fixed order.
    __shared__ float red[kProjWaves][kTileTokens][kMix];
    __shared__ float sqr[kProjWaves][4][kTileTokens];
#pragma unroll
    for (int m = 0; m < kMTiles; ++m) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int col = n * 16 + c;
            if (col < kMix) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    red[w][m * 16 + 4 * g + q][col] = acc[m][n][q];
                }
            }
        }
        sqr[w][g][m * 16 + c] = sq[m];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kTileTokens * (kMix + 1); e += kProjBlock) {
        const int tok = e / (kMix + 1);
        const int r = e - tok * (kMix + 1);
        float v;
        if (r < kMix) {
            v = ((red[0][tok][r] + red[1][tok][r]) + red[2][tok][r]) + red[3][tok][r];
        } else {
            v = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kProjWaves; ++ww) {
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    v += sqr[ww][gg][tok];
                }
            }
        }
        const int t = t0 + tok;
        if (t < T) {
            part[((size_t)slice * T + t) * kPartStride + r] = v;
        }
    }
}

__global__ __launch_bounds__(256) void pre_mix_kernel(const float *__restrict__ part, int T, int slices, float k_denom,
                                                      const float *__restrict__ hc_scale,
                                                      const float *__restrict__ hc_base, float rms_eps,
                                                      float pre_eps, float sk_eps, float post_mult, int iters,
                                                      float *__restrict__ post, float *__restrict__ comb,
                                                      float *__restrict__ pre_out, float *__restrict__ pre_ws)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) {
        return;
    }
    float d[kPartStride];
#pragma unroll
    for (int r = 0; r < kPartStride; ++r) {
        d[r] = 0.0f;
    }
    for (int s = 0; s < slices; ++s) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(part + ((size_t)s * T + t) * kPartStride);
#pragma unroll
        for (int q = 0; q < 7; ++q) { // records hold 25 used floats: 7 float4 cover them
            const f32x4 v = p[q];
            d[4 * q] += v[0];
            d[4 * q + 1] += v[1];
            d[4 * q + 2] += v[2];
            d[4 * q + 3] += v[3];
        }
    }
    const float rstd = 1.0f / sqrtf(d[kSqSlot] / k_denom + rms_eps);
    const float s_pre = hc_scale[0], s_post = hc_scale[1], s_comb = hc_scale[2];
    float pw[kHC];
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        pw[i] = sigmoidf_fast(fmaf(d[i] * rstd, s_pre, hc_base[i])) + pre_eps;
        post[t * kHC + i] = sigmoidf_fast(fmaf(d[kHC + i] * rstd, s_post, hc_base[kHC + i])) * post_mult;
    }
    float P[kHC * kHC];
#pragma unroll
    for (int e = 0; e < kHC * kHC; ++e) {
        P[e] = fmaf(d[2 * kHC + e] * rstd, s_comb, hc_base[2 * kHC + e]);
    }
    sinkhorn4x4(P, iters, sk_eps);
#pragma unroll
    for (int e = 0; e < kHC * kHC; ++e) {
        comb[t * kHC * kHC + e] = P[e];
    }
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        pre_ws[t * kHC + i] = pw[i];
        if (pre_out) {
            pre_out[t * kHC + i] = pw[i];
        }
    }
}

__global__ __launch_bounds__(kColBlock) void pre_collapse_vec8_kernel(const uint16_t *__restrict__ res,
                                                                      const float *__restrict__ pre_ws, int T, int H,
                                                                      int tiles_per_token, uint16_t *__restrict__ y)
{
    const int wave = uniform(blockIdx.x * kColWaves + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    const int h = tile * kColVecTile + lane * 8;
    if (h >= H) {
        return;
    }
    float p[kHC];
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        p[i] = pre_ws[t * kHC + i];
    }
    const size_t row = (size_t)t * kHC * H + h;
    u32x4 rw[kHC];
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        rw[i] = load_nt16(res + row + (size_t)i * H);
    }
    u32x4 yw;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float lo = bf16_lo(rw[0][q]) * p[0];
        float hi = bf16_hi(rw[0][q]) * p[0];
#pragma unroll
        for (int i = 1; i < kHC; ++i) {
            lo = fmaf(bf16_lo(rw[i][q]), p[i], lo);
            hi = fmaf(bf16_hi(rw[i][q]), p[i], hi);
        }
        yw[q] = pack_bf16x2(lo, hi);
    }
    store_nt16(y + (size_t)t * H + h, yw);
}

__global__ __launch_bounds__(kColBlock) void pre_collapse_scalar_kernel(const uint16_t *__restrict__ res,
                                                                        const float *__restrict__ pre_ws, int T,
                                                                        int H, int tiles_per_token,
                                                                        uint16_t *__restrict__ y)
{
    const int wave = uniform(blockIdx.x * kColWaves + (threadIdx.x >> 6));
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
    float a = bf16_to_f32(res[row]) * pre_ws[t * kHC];
#pragma unroll
    for (int i = 1; i < kHC; ++i) {
        a = fmaf(bf16_to_f32(res[row + (size_t)i * H]), pre_ws[t * kHC + i], a);
    }
    y[(size_t)t * H + h] = f32_to_bf16(a);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

} // namespace

PreGeom pre_geometry(int64_t T, int64_t H)
{
    PreGeom g{};
    g.T = T;
    g.H = H;
    if (T <= 0 || H <= 0) {
        return g;
    }
    g.tiles = (int)((T + kTileTokens - 1) / kTileTokens);
    g.nhb = (int)((H + kHBlock - 1) / kHBlock);
    int s = (kTargetBlocks + g.tiles - 1) / g.tiles;
    const int max_s = g.nhb / kProjWaves > 1 ? g.nhb / kProjWaves : 1; // >= one H block per wave
    s = s < 1 ? 1 : (s > max_s ? max_s : s);
    g.hb_per_slice = (g.nhb + s - 1) / s;
    g.slices = (g.nhb + g.hb_per_slice - 1) / g.hb_per_slice;
    g.part_bytes = (size_t)g.slices * (size_t)T * kPartStride * sizeof(float);
    g.prew_bytes = (size_t)T * kHC * sizeof(float);
    g.split_bytes = align256(g.part_bytes) + align256(g.prew_bytes);
    g.fused = kUseFusedPre ? fused_geometry(T, H) : FusedGeom{};
    g.total_bytes = g.fused.valid && g.fused.bytes > g.split_bytes ? g.fused.bytes : g.split_bytes;
    return g;
}

hipError_t launch_pre(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                      const PreGeom &g, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                      int iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                      hipStream_t stream, bool vec8)
{
    if (g.fused.valid) {
        bool fits = false;
        const hipError_t e = launch_pre_fused(res, hc_fn, hc_scale, hc_base, g.fused, g.T, g.H, rms_eps, pre_eps,
                                              sinkhorn_eps, post_mult, iters, y, post, comb, pre, workspace, stream,
                                              vec8, &fits);
        if (e != hipSuccess || fits) {
            return e;
        }
    }
    float *part = reinterpret_cast<float *>(workspace);
    float *pre_ws = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + align256(g.part_bytes));
    const int T = (int)g.T, H = (int)g.H;
    const dim3 pgrid((unsigned)g.tiles, (unsigned)g.slices);
    if (vec8) {
        pre_proj_kernel<true><<<pgrid, dim3(kProjBlock), 0, stream>>>(res, hc_fn, T, H, g.nhb, g.hb_per_slice, part);
    } else {
        pre_proj_kernel<false><<<pgrid, dim3(kProjBlock), 0, stream>>>(res, hc_fn, T, H, g.nhb, g.hb_per_slice,
                                                                        part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        return e;
    }
    pre_mix_kernel<<<dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream>>>(
        part, T, g.slices, (float)(kHC * g.H), hc_scale, hc_base, rms_eps, pre_eps, sinkhorn_eps, post_mult, iters,
        post, comb, pre, pre_ws);
    e = hipGetLastError();
    if (e != hipSuccess) {
        return e;
    }
    const int tile = vec8 ? kColVecTile : kWave;
    const int64_t tiles = (g.H + tile - 1) / tile;
    const int64_t blocks = (g.T * tiles + kColWaves - 1) / kColWaves;
    if (vec8) {
        pre_collapse_vec8_kernel<<<dim3((unsigned)blocks), dim3(kColBlock), 0, stream>>>(res, pre_ws, T, H,
                                                                                         (int)tiles, y);
    } else {
        pre_collapse_scalar_kernel<<<dim3((unsigned)blocks), dim3(kColBlock), 0, stream>>>(res, pre_ws, T, H,
                                                                                           (int)tiles, y);
    }
    return hipGetLastError();
}

} // namespace mhc
