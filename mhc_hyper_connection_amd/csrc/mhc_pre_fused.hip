// mhc_pre_fused.hip -- the mHC pre-map as one persistent, cooperative kernel (gfx950).
//
// ("FlashInfer mHC 模块深度解析", sections 3.4 and 5.2; metrale
// hyper_connection_dispatch.rs, hc_pre_site.)
//
// The pre-map needs the full 4H-long projection of a token before it can
// collapse that token's streams, and a token's streams (57 KB at H=7168) are
// too large to keep on one CU for the 64 tokens an MFMA tile amortises the
// weights over.  Reading the streams twice from HBM costs 8H bytes per token
// more than the method has to move, so the streams are read once:
//
//  * A work item is (tile of 64 tokens, slice of 128 h across all 4 streams).
//    Its workgroup (4 wavefronts, 32 h each) loads the slice into VGPRs
//    (64 KB), feeds it to v_mfma_f32_16x16x32_bf16 against the projection
//    weights, accumulates the sum of squares with v_dot2_f32_bf16, and writes
//    one 25-float partial record per token.
//  * Barrier 1 (per tile counter): when all slices of the tile have written
//    their records, each workgroup reduces a share of the tile's tokens (fixed
//    slice order, so the result does not depend on timing), computes rstd, the
//    sigmoid mixes and the 4x4 Sinkhorn, and publishes post, comb, pre.
//  * Barrier 2: every workgroup reads the tile's pre weights and collapses its
//    slice straight from the VGPRs it loaded: y = sum_i pre_i * res_i.
//
// The projection weights are fp32.  A small prep kernel splits every weight
// exactly into three bf16 terms hi + mid + lo (each a truncation of what
// remains, 8 + 8 + 8 significant bits) and stores them in MFMA operand order,
// so the main loop issues only 16-byte loads and MFMAs.  Three bf16 products
// accumulated in fp32 reproduce the fp32 weight without rounding it.
//
// Scheduling: the grid is persistent (sized to the resident capacity).
// Workgroups are split into `nclass` classes by blockIdx % nclass; class v owns
// the slices s with s % nclass == v and takes work items from its own ticket
// counter in tile order.  With round-robin dispatch a class lives on one XCD,
// so its share of the split weights stays in that XCD's L2.  Because each class
// claims items in tile order, the earliest unfinished tile always has every
// item claimed by a running workgroup, so the barriers cannot deadlock as long
// as each class has at least as many resident workgroups as it has slices per
// tile (checked on the host).  Every wait is bounded; a timeout sets a status
// word instead of hanging.
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

constexpr int kFWaves = 4;
constexpr int kFBlock = kFWaves * kWave;
constexpr int kFTok = 64;             // tokens per tile
constexpr int kFMT = kFTok / 16;      // MFMA row tiles per wave
constexpr int kFHB = 32;              // h per wave: 4 lane groups x 8
constexpr int kFSliceH = kFWaves * kFHB;
constexpr int kRec = kMix + 1;        // partial record: 24 dots + sum of squares
constexpr int kBFragPerHbStream = 3 * 64 + 3 * 32; // hi/mid/lo for column tile 0 (64 lanes) and 1 (32 lanes)
constexpr uint32_t kSpinLimit = 1u << 20;

// Cross-workgroup data (partial records, pre weights, counters) is exchanged only
// through relaxed agent-scope atomic loads and stores.  On gfx950 these are
// coherent accesses (sc1) that neither rely on nor disturb the non-coherent
// cache state, so no L2 writeback/invalidate (what a release/acquire fence adds
// for ordinary stores and loads) is needed.  Ordering is enforced by waiting for
// every outstanding memory operation of the wave before it reaches the
// workgroup barrier that precedes a counter increment, and, on the reading side,
// by issuing the data loads only after the counter load has returned.
__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this wave's memory operations have completed (stores acknowledged).
__device__ __forceinline__ void drain_memory()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Bounded wait until *p >= target.  Returns false (and records it) on timeout.
__device__ bool wait_count(uint32_t *p, uint32_t target, uint32_t *status)
{
    uint32_t n = 0;
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (++n > kSpinLimit) {
            __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

// v == hi + mid + lo exactly for normal fp32 v (three successive bf16 truncations).
__device__ __forceinline__ void split3x8(const float *v, u32x4 &ph, u32x4 &pm, u32x4 &pl)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t h0 = __float_as_uint(v[2 * q]) & 0xFFFF0000u;
        const uint32_t h1 = __float_as_uint(v[2 * q + 1]) & 0xFFFF0000u;
        const float r0 = v[2 * q] - __uint_as_float(h0);
        const float r1 = v[2 * q + 1] - __uint_as_float(h1);
        const uint32_t m0 = __float_as_uint(r0) & 0xFFFF0000u;
        const uint32_t m1 = __float_as_uint(r1) & 0xFFFF0000u;
        const float l0 = r0 - __uint_as_float(m0);
        const float l1 = r1 - __uint_as_float(m1);
        ph[q] = (h0 >> 16) | h1;
        pm[q] = (m0 >> 16) | m1;
        pl[q] = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u);
    }
}

// One thread per (h block, stream, operand slot): split 8 weights of one hc_fn
// row into hi/mid/lo MFMA B fragments.  Slot < 64: column tile 0, lane = slot
// (row = lane % 16).  Slot >= 64: column tile 1, rows 16..23 only (lane g*8+c
// stands for MFMA lane 16g + c).  Also clears the barrier counters and tickets.
__global__ __launch_bounds__(256) void pre_prep_kernel(const float *__restrict__ hc_fn, int H, int nhb,
                                                       u32x4 *__restrict__ bfrag, uint32_t *__restrict__ zero,
                                                       int nzero)
{
    const int gid = blockIdx.x * 256 + threadIdx.x;
    if (gid < nzero) {
        zero[gid] = 0u;
    }
    const int slots = kBFragPerHbStream / 3; // 96
    if (gid >= nhb * kHC * slots) {
        return;
    }
    const int slot = gid % slots;
    const int hbi = gid / slots; // hb * 4 + i
    const int i = hbi % kHC;
    const int hb = hbi / kHC;
    int n, g, c;
    if (slot < 64) {
        n = 0;
        g = slot >> 4;
        c = slot & 15;
    } else {
        n = 1;
        g = (slot - 64) >> 3;
        c = (slot - 64) & 7;
    }
    const int r = n * 16 + c;
    const int h = hb * kFHB + g * 8;
    float v[8];
    const float *src = hc_fn + (size_t)r * kHC * H + (size_t)i * H + h;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[j] = (h + j < H) ? src[j] : 0.0f;
    }
    u32x4 ph, pm, pl;
    split3x8(v, ph, pm, pl);
    u32x4 *dst = bfrag + (size_t)hbi * kBFragPerHbStream;
    if (n == 0) {
        dst[0 * 64 + slot] = ph;
        dst[1 * 64 + slot] = pm;
        dst[2 * 64 + slot] = pl;
    } else {
        const int k = slot - 64;
        dst[192 + 0 * 32 + k] = ph;
        dst[192 + 1 * 32 + k] = pm;
        dst[192 + 2 * 32 + k] = pl;
    }
}

template <bool kVec>
__device__ __forceinline__ u32x4 load_row8(const uint16_t *p, int h, int H, bool ok)
{
    u32x4 w = {0u, 0u, 0u, 0u};
    if (kVec) {
        if (ok && h < H) {
            w = load_nt16(p);
        }
    } else if (ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (h + 2 * q < H) ? (uint32_t)p[2 * q] : 0u;
            const uint32_t hi = (h + 2 * q + 1 < H) ? (uint32_t)p[2 * q + 1] : 0u;
            w[q] = lo | (hi << 16);
        }
    }
    return w;
}

template <bool kVec>
__device__ __forceinline__ void store_row8(uint16_t *p, int h, int H, u32x4 w)
{
    if (kVec) {
        store_nt16(p, w);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (h + 2 * q < H) {
                p[2 * q] = (uint16_t)(w[q] & 0xFFFFu);
            }
            if (h + 2 * q + 1 < H) {
                p[2 * q + 1] = (uint16_t)(w[q] >> 16);
            }
        }
    }
}

struct FusedArgs {
    const uint16_t *res;
    const u32x4 *bfrag;
    const float *hc_scale;
    const float *hc_base;
    int T, H, nhb, S, tiles, nclass;
    float k_denom, rms_eps, pre_eps, sk_eps, post_mult;
    int iters;
    uint16_t *y;
    float *post, *comb, *pre_out;
    float *part;     // [tiles][S][64][25]
    float *prew;     // [tiles][64][4]
    uint32_t *cnt;   // [tiles][2]
    uint32_t *sync;  // [0..7] class tickets, [8] status
};

template <bool kVec>
__global__ __launch_bounds__(kFBlock) void pre_fused_kernel(FusedArgs a)
{
    __shared__ float red[kFWaves][kFTok][kMix];
    __shared__ float sqp[kFWaves][4][kFTok];
    __shared__ float rsum[8][32];
    __shared__ float mixv[kFTok][kRec];
    __shared__ int s_item;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & (kWave - 1);
    const int g = lane >> 4;
    const int c = lane & 15;
    const int cls = blockIdx.x % a.nclass;
    const int S = a.S;
    const int nS = (S - cls + a.nclass - 1) / a.nclass; // slices of this class per tile
    const int items = a.tiles * nS;
    const int H = a.H;
    uint32_t *const status = a.sync + 8;

    if (tid == 0) {
        s_item = (int)__hip_atomic_fetch_add(&a.sync[cls], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    int q = s_item;

    while (q < items) {
        const int tile = q / nS;
        const int slice = cls + a.nclass * (q - tile * nS);
        const int t0 = tile * kFTok;
        const int hb = slice * kFWaves + w;
        const bool hb_ok = hb < a.nhb;
        const int h = hb * kFHB + g * 8;

        // ---------------- phase 1: load the slice, project it, sum its squares
        u32x4 d[kFMT][kHC];
#pragma unroll
        for (int m = 0; m < kFMT; ++m) {
            const int t = t0 + m * 16 + c;
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                d[m][i] = load_row8<kVec>(a.res + ((size_t)t * kHC + i) * H + h, h, H, hb_ok && t < a.T);
            }
        }
        f32x4 acc[kFMT][2];
#pragma unroll
        for (int m = 0; m < kFMT; ++m) {
            acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (hb_ok) {
            const u32x4 *bp = a.bfrag + (size_t)hb * kHC * kBFragPerHbStream;
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                u32x4 b0[3], b1[3];
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    b0[s] = bp[i * kBFragPerHbStream + s * 64 + lane];
                    b1[s] = (c < 8) ? bp[i * kBFragPerHbStream + 192 + s * 32 + g * 8 + c] : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    const bf16x8 B0 = __builtin_bit_cast(bf16x8, b0[s]);
                    const bf16x8 B1 = __builtin_bit_cast(bf16x8, b1[s]);
#pragma unroll
                    for (int m = 0; m < kFMT; ++m) {
                        const bf16x8 A = __builtin_bit_cast(bf16x8, d[m][i]);
                        acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B0, acc[m][0], 0, 0, 0);
                        acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B1, acc[m][1], 0, 0, 0);
                    }
                }
            }
        }
        float sq[kFMT];
#pragma unroll
        for (int m = 0; m < kFMT; ++m) {
            sq[m] = 0.0f;
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // copy to a scalar first: bit_cast of an ext_vector element miscompiles
                    const uint32_t wk = d[m][i][k];
                    const bf16x2 pr = __builtin_bit_cast(bf16x2, wk);
                    sq[m] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, sq[m], false);
                }
            }
        }

        // ---------------- workgroup reduction -> one partial record per token
#pragma unroll
        for (int m = 0; m < kFMT; ++m) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int col = n * 16 + c;
                if (col < kMix) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        red[w][m * 16 + 4 * g + k][col] = acc[m][n][k];
                    }
                }
            }
            sqp[w][g][m * 16 + c] = sq[m];
        }
        __syncthreads();
        float *rec = a.part + ((size_t)tile * S + slice) * (kFTok * kRec);
        for (int e = tid; e < kFTok * kRec; e += kFBlock) {
            const int tok = e / kRec;
            const int r = e - tok * kRec;
            float v;
            if (r < kMix) {
                v = ((red[0][tok][r] + red[1][tok][r]) + red[2][tok][r]) + red[3][tok][r];
            } else {
                v = 0.0f;
#pragma unroll
                for (int ww = 0; ww < kFWaves; ++ww) {
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        v += sqp[ww][gg][tok];
                    }
                }
            }
            st_agent(&rec[e], v);
        }

        // ---------------- barrier 1: every slice of the tile has its record out
        drain_memory();
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_fetch_add(&a.cnt[2 * tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_count(&a.cnt[2 * tile], (uint32_t)S, status);
            // All items of this tile are claimed, so the next ticket belongs to a later tile.
            s_item = (int)__hip_atomic_fetch_add(&a.sync[cls], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();

        // ---------------- reduce this workgroup's share of the tile's tokens
        // tokens slice, slice + S, slice + 2S, ... (< 64)
        const int ntok = slice < kFTok ? (kFTok - 1 - slice) / S + 1 : 0;
        for (int base = 0; base < ntok; base += 8) {
            const int P = min(8, ntok - base);
            const int G = P == 1 ? 8 : (P == 2 ? 4 : (P <= 4 ? 2 : 1)); // slice groups per token
            const int grp = tid >> 5;
            const int j = grp / G;
            const int k = grp - j * G;
            const int r = tid & 31;
            if (j < P && r < kRec) {
                const int tok = slice + (base + j) * S;
                const float *src = a.part + ((size_t)tile * S) * (kFTok * kRec) + tok * kRec + r;
                float v = 0.0f;
                for (int s = k; s < S; s += G) {
                    v += ld_agent(src + (size_t)s * (kFTok * kRec));
                }
                rsum[grp][r] = v;
            }
            __syncthreads();
            if (tid < P * kRec) {
                const int jj = tid / kRec;
                const int rr = tid - jj * kRec;
                float v = 0.0f;
                for (int kk = 0; kk < G; ++kk) {
                    v += rsum[jj * G + kk][rr];
                }
                mixv[base + jj][rr] = v;
            }
            __syncthreads();
        }
        if (tid < ntok) {
            const int tok = slice + tid * S;
            const int t = t0 + tok;
            if (t < a.T) {
                const float *d25 = mixv[tid];
                const float rstd = 1.0f / sqrtf(d25[kMix] / a.k_denom + a.rms_eps);
                const float s0 = a.hc_scale[0], s1 = a.hc_scale[1], s2 = a.hc_scale[2];
                float pw[kHC];
#pragma unroll
                for (int i = 0; i < kHC; ++i) {
                    pw[i] = sigmoidf_fast(fmaf(d25[i] * rstd, s0, a.hc_base[i])) + a.pre_eps;
                    a.post[(size_t)t * kHC + i] =
                        sigmoidf_fast(fmaf(d25[kHC + i] * rstd, s1, a.hc_base[kHC + i])) * a.post_mult;
                }
                float P16[kHC * kHC];
#pragma unroll
                for (int e = 0; e < kHC * kHC; ++e) {
                    P16[e] = fmaf(d25[2 * kHC + e] * rstd, s2, a.hc_base[2 * kHC + e]);
                }
                sinkhorn4x4(P16, a.iters, a.sk_eps);
#pragma unroll
                for (int e = 0; e < kHC * kHC; ++e) {
                    a.comb[(size_t)t * kHC * kHC + e] = P16[e];
                }
                float *pwd = a.prew + ((size_t)tile * kFTok + tok) * kHC;
#pragma unroll
                for (int i = 0; i < kHC; ++i) {
                    st_agent(&pwd[i], pw[i]);
                    if (a.pre_out) {
                        a.pre_out[(size_t)t * kHC + i] = pw[i];
                    }
                }
            }
        }

        // ---------------- barrier 2: the tile's pre weights are published
        drain_memory();
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_fetch_add(&a.cnt[2 * tile + 1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_count(&a.cnt[2 * tile + 1], (uint32_t)S, status);
        }
        __syncthreads();

        // ---------------- phase 2: collapse the slice held in registers
        if (hb_ok && h < H) {
#pragma unroll
            for (int m = 0; m < kFMT; ++m) {
                const int t = t0 + m * 16 + c;
                if (t < a.T) {
                    const float *pp = a.prew + ((size_t)tile * kFTok + m * 16 + c) * kHC;
                    const float pw[kHC] = {ld_agent(pp), ld_agent(pp + 1), ld_agent(pp + 2), ld_agent(pp + 3)};
                    u32x4 yw;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        float lo = bf16_lo(d[m][0][k]) * pw[0];
                        float hi = bf16_hi(d[m][0][k]) * pw[0];
#pragma unroll
                        for (int i = 1; i < kHC; ++i) {
                            lo = fmaf(bf16_lo(d[m][i][k]), pw[i], lo);
                            hi = fmaf(bf16_hi(d[m][i][k]), pw[i], hi);
                        }
                        yw[k] = pack_bf16x2(lo, hi);
                    }
                    store_row8<kVec>(a.y + (size_t)t * H + h, h, H, yw);
                }
            }
        }
        q = s_item; // claimed after barrier 1; published by the barrier-2 __syncthreads
        __syncthreads(); // s_item is rewritten after the next barrier 1 only
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int fused_capacity(hipError_t *err)
{
    static int cached[64] = {0};
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) {
        return 0;
    }
    if (dev >= 0 && dev < 64 && cached[dev] > 0) {
        return cached[dev];
    }
    int cus = 0, per_cu = 0;
    *err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (*err != hipSuccess) {
        return 0;
    }
    *err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pre_fused_kernel<true>, kFBlock, 0);
    if (*err != hipSuccess) {
        return 0;
    }
    int per_cu2 = 0;
    *err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu2, pre_fused_kernel<false>, kFBlock, 0);
    if (*err != hipSuccess) {
        return 0;
    }
    const int cap = cus * min(per_cu, per_cu2);
    if (dev >= 0 && dev < 64) {
        cached[dev] = cap;
    }
    return cap;
}

} // namespace

FusedGeom fused_geometry(int64_t T, int64_t H)
{
    FusedGeom f{};
    if (T <= 0 || H <= 0 || H > kFusedMaxH) {
        return f;
    }
    f.tiles = (int)((T + kFTok - 1) / kFTok);
    f.nhb = (int)((H + kFHB - 1) / kFHB);
    f.S = (int)((H + kFSliceH - 1) / kFSliceH);
    f.nclass = f.S < 8 ? f.S : 8;
    size_t off = 0;
    f.off_bfrag = off;
    off += align256((size_t)f.nhb * kHC * kBFragPerHbStream * sizeof(u32x4));
    f.off_part = off;
    off += align256((size_t)f.tiles * f.S * kFTok * kRec * sizeof(float));
    f.off_prew = off;
    off += align256((size_t)f.tiles * kFTok * kHC * sizeof(float));
    f.off_sync = off; // 16 words: tickets, status; then the per-tile counters
    f.nzero = 16 + 2 * f.tiles;
    off += align256((size_t)f.nzero * sizeof(uint32_t));
    f.bytes = off;
    f.valid = true;
    return f;
}

hipError_t launch_pre_fused(const uint16_t *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                            const FusedGeom &f, int64_t T, int64_t H, float rms_eps, float pre_eps,
                            float sinkhorn_eps, float post_mult, int iters, uint16_t *y, float *post, float *comb,
                            float *pre, void *workspace, hipStream_t stream, bool vec8, bool *fits)
{
    hipError_t err = hipSuccess;
    const int cap = fused_capacity(&err);
    if (err != hipSuccess) {
        return err;
    }
    const int per_class = cap / f.nclass;
    const int nS_max = (f.S + f.nclass - 1) / f.nclass;
    *fits = per_class >= nS_max;
    if (!*fits) {
        return hipSuccess;
    }
    char *ws = reinterpret_cast<char *>(workspace);
    FusedArgs a;
    a.res = res;
    a.bfrag = reinterpret_cast<const u32x4 *>(ws + f.off_bfrag);
    a.hc_scale = hc_scale;
    a.hc_base = hc_base;
    a.T = (int)T;
    a.H = (int)H;
    a.nhb = f.nhb;
    a.S = f.S;
    a.tiles = f.tiles;
    a.nclass = f.nclass;
    a.k_denom = (float)(kHC * H);
    a.rms_eps = rms_eps;
    a.pre_eps = pre_eps;
    a.sk_eps = sinkhorn_eps;
    a.post_mult = post_mult;
    a.iters = iters;
    a.y = y;
    a.post = post;
    a.comb = comb;
    a.pre_out = pre;
    a.part = reinterpret_cast<float *>(ws + f.off_part);
    a.prew = reinterpret_cast<float *>(ws + f.off_prew);
    a.sync = reinterpret_cast<uint32_t *>(ws + f.off_sync);
    a.cnt = a.sync + 16;

    const int prep_threads = max(f.nhb * kHC * (kBFragPerHbStream / 3), f.nzero);
    pre_prep_kernel<<<dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, stream>>>(
        hc_fn, (int)H, f.nhb, reinterpret_cast<u32x4 *>(ws + f.off_bfrag), a.sync, f.nzero);
    err = hipGetLastError();
    if (err != hipSuccess) {
        return err;
    }
    // Persistent grid: every class gets the same number of workgroups, no more than it has items.
    const int64_t items_per_class = (int64_t)f.tiles * nS_max;
    int64_t per = per_class;
    if (per > items_per_class) {
        per = items_per_class;
    }
    const unsigned grid = (unsigned)(per * f.nclass);
    if (vec8) {
        pre_fused_kernel<true><<<dim3(grid), dim3(kFBlock), 0, stream>>>(a);
    } else {
        pre_fused_kernel<false><<<dim3(grid), dim3(kFBlock), 0, stream>>>(a);
    }
    return hipGetLastError();
}

} // namespace mhc
