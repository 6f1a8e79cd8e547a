// mhc_pre_decode.hip -- the mHC pre-map for small batches (T <= 192) in one launch (gfx950).
//
// ("FlashInfer mHC 模块深度解析", section 3.4: per token the RMS statistic and the 24 x 4H
// projection, then the pre and post weights and the Sinkhorn of the comb logits, then the
// collapse of the four streams by the pre weights; section 5.2 for the arithmetic.)
//
// At a few tokens nothing here is bound by bandwidth: the weights (24 x 4H) outweigh the
// streams, and the time goes to latency, one chain of it per launch.  This form takes one.
//
//  * One group of 32 workgroups per XCD (workgroup b runs on XCD b mod 8 under the
//    hardware's round-robin dispatch; 256 workgroups, one per CU).  Group x takes the
//    tokens [x Tg, x Tg + nt), Tg = ceil(T / 8), and workgroup s of the group the slice
//    [s hs, (s + 1) hs) of every stream, hs = 8 ceil(H / 256).
//  * The workgroup loads its tokens' slice of the streams into LDS and its slice of the
//    weights, rows 0..23 of the four streams, straight into VGPRs as fp32 (bf16 weights
//    widened exactly): thread (g, c), g = tid / 128, holds rows 12 g .. 12 g + 11 of the
//    8 h of chunk c (stream c / (hs / 8)).  It forms those 12 partial dots, and for g = 0
//    the partial sum of squares, with fp32 FMAs, P tokens at a time.
//  * A wave's partial sums are added over its 64 lanes in a fixed order: a swap-and-add on
//    v_permlane32_swap, one on v_permlane16_swap (each halves the values a lane holds), then
//    a DPP sum within each 16-lane row; the two waves of each row half add in LDS.  That
//    gives the workgroup's record: 24 dots and the sum of squares of each token.
//  * Records go through the XCD's L2 as 16-byte chunks of three values and a tag that names
//    the call (its dispatch id) and the group: the pre dots and sums of squares of the
//    group's tokens, then each token's 20 post and comb dots.  Every workgroup sums the first
//    part over the 32 slices (device-scope loads that miss the CU's L1; 32 lanes, one per
//    slice, added by a fixed butterfly), forms rstd and the pre weights, and collapses its
//    slice of every token out of LDS: the streams are read once.  Workgroup s < nt also sums
//    the second part of its token s and finishes the post weights and the Sinkhorn, on its
//    fourth wave while the other three collapse.
//  * A chunk whose tag does not match has not landed yet; the records are loaded again, up to
//    2^14 times, and then the group's outputs become NaN (its writer was never made resident,
//    e.g. behind a long kernel on another stream) rather than values from a stale record.
#include "mhc_device.h"
#include "mhc_internal.h"

#include <atomic>

namespace mhc {

namespace {

constexpr int kDGroups = 8;                  // one per XCD
constexpr int kDSlices = 32;                 // workgroups per group
constexpr int kDThreads = 256;
constexpr int kDMaxTok = 192;                // tokens of a call
constexpr int kDMaxTg = kDMaxTok / kDGroups; // tokens of a group (24)
constexpr int kDMaxHs = 256;                 // slice width (H <= 8192)
constexpr int kDMaxChunks = kHC * kDMaxHs / 8; // 16-byte chunks of a slice (128)
constexpr int kDRows = 12;                   // weight rows of a thread (two row halves)
constexpr int kDF = kDRows + 1;              // partial values of a thread per token
constexpr int kDUrgMax = (5 * kDMaxTg + 2) / 3;           // chunks of pre dots and sums of squares (40)
constexpr int kDDef = (kMix - kHC + 2) / 3;               // chunks of a token's post and comb dots (7)
constexpr int kDGroupChunks = kDUrgMax + kDMaxTg * kDDef; // record chunks of one slice (208)
constexpr int kDTileMaxB = kDMaxTg * kDMaxChunks * 16;    // LDS tile of the streams, at most (48 KB)

struct DecArgs {
    const uint16_t *res;
    const void *hc_fn;
    const float *hc_scale, *hc_base;
    int T, H, fn_rows, Tg, hs;
    int tile_b; // bytes of the LDS tile: [Tg][4][hs / 8] 16-byte chunks rounded up to 256 of them
    float inv_k, rms_eps, pre_eps, sk_eps, post_mult; // inv_k = 1 / (4H)
    int iters, head;
    uint16_t *y;
    float *post, *comb, *pre;
    u32x4 *rec;
    uint32_t rec_bytes;
    int max_retry;
    uint32_t tag_skew;
    // the post-map in front (kPost): the sublayer output x [T][H], the previous mixes post_in
    // [T][4] and comb_in [T][4][4]; the new streams go to out [T][4][H] (which may be res) and
    // are the streams the pre-map reads
    const uint16_t *x;
    const float *post_in, *comb_in;
    uint16_t *out;
};

// Eight weights of one row from offset o (elements), fp32 or bf16, into fp32.
__device__ __forceinline__ void load_w8(const float *, __amdgpu_buffer_rsrc_t v, uint32_t o, bool ok, float (&d)[8])
{
    const uint32_t b = ok ? o * 4u : kOob;
    const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)b, 0, 0));
    const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)(b + 16u), 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        d[e] = __uint_as_float(lo[e]);
        d[4 + e] = __uint_as_float(hi[e]);
    }
}
__device__ __forceinline__ void load_w8(const uint16_t *, __amdgpu_buffer_rsrc_t v, uint32_t o, bool ok,
                                        float (&d)[8])
{
    const uint32_t b = ok ? o * 2u : kOob;
    const u32x4 q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)b, 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        d[2 * e] = bf16_lo(q[e]);
        d[2 * e + 1] = bf16_hi(q[e]);
    }
}

// Sums over the wave's 64 lanes of V values (V a multiple of 4), stored to out[0 .. V).
// permlane32_swap exchanges rows 2, 3 of its first operand with rows 0, 1 of its second,
// so adding the two results gives value k over lanes l, l + 32 in lanes 0..31 and value
// k + V/2 in lanes 32..63; permlane16_swap (odd rows of the first with even rows of the
// second) does the same one level down, after which row r holds value k + r V/4 summed over
// four lanes, and a DPP sum within the row finishes it.  The order is fixed.
template <int V> __device__ __forceinline__ void wave_sums(const float (&v)[V], float *out, int lane)
{
    constexpr int V2 = V / 2, V4 = V / 4;
    float u[V2];
#pragma unroll
    for (int k = 0; k < V2; ++k) {
        const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + V2]), false, false);
        u[k] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    }
    float z[V4];
#pragma unroll
    for (int k = 0; k < V4; ++k) {
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[k]), __float_as_uint(u[k + V4]), false, false);
        z[k] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    }
#pragma unroll
    for (int k = 0; k < V4; ++k) {
        z[k] += dpp_perm<0xB1>(z[k]);  // quad_perm [1,0,3,2]
        z[k] += dpp_perm<0x4E>(z[k]);  // quad_perm [2,3,0,1]
        z[k] += dpp_perm<0x141>(z[k]); // row_half_mirror
        z[k] += dpp_perm<0x140>(z[k]); // row_mirror
    }
    if ((lane & 15) == 0) {
        const int r = lane >> 4;
#pragma unroll
        for (int k = 0; k < V4; ++k) {
            out[k + r * V4] = z[k];
        }
    }
}

// P tokens per projection pass (1, 2 or 4); a group of more than 4 tokens takes several.
// kPost: the post-map in front, on the workgroup's tile (mhc_post_pre_fused).
// kBig: more than 8 tokens per group (up to 24).  The tile of the streams is then dynamic
// LDS (a.tile_b bytes, then 16 zero bytes) and the rounds of loads past the group's tokens
// are skipped by wave-uniform tests; with at most 8 tokens every round is issued (a straight
// run of loads, the loads past the tile reading zero) and the tile is static.
template <typename WT, int P, bool kPost, bool kBig>
__global__ __launch_bounds__(kDThreads) void pre_decode_kernel(DecArgs a)
{
    constexpr int V = (P * kDF + 3) / 4 * 4; // a pass's values per thread, padded to a multiple of 4
    constexpr int kTg = kBig ? kDMaxTg : 8;  // tokens of a group, at most
    constexpr int kTileB = kTg * kDMaxChunks * 16;
    constexpr int kPR = kTileB / 16 / kDThreads;                 // 16-byte pieces per thread (4 or 12)
    constexpr int kUrg = (5 * kTg + 2) / 3;                      // urgent chunks, at most
    constexpr int kRnd = (kUrg + kDDef + 7) / 8;                 // rounds of record loads (3 or 6)
    constexpr int kNP = kTg / 4 > 0 ? kTg / 4 : 1;               // projection passes, at most
    __shared__ __align__(16) unsigned char tile_st[kBig ? 16 : kTileB + 16];
    extern __shared__ __align__(16) unsigned char tile_dyn[];
    unsigned char *const tile = kBig ? tile_dyn : tile_st;      // [nt][4][nch] chunks, then 16 zero bytes
    __shared__ float part[kNP][4][V];                           // [pass][wave][value]
    __shared__ float usum[3 * kUrg];                            // pre dots [4][nt], then sums of squares [nt]
    __shared__ float dsum[3 * kDDef];                           // the designated token's post and comb dots
    __shared__ float dummy[kWave];
    __shared__ float coefs[kTg * (kHC + kHC * kHC)]; // kPost: post [nt][4] at 0, comb [nt][16] at 4 kTg
    __shared__ int badf;

    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int x = (int)blockIdx.x & (kDGroups - 1);
    const int s = (int)blockIdx.x >> 3;
    const int T = a.T, H = a.H, Tg = a.Tg, hs = a.hs;
    const int t0 = x * Tg;
    const int nt = uniform(min(Tg, T - t0));
    if (nt <= 0) {
        return; // the whole group: no tokens
    }
    const int nch = hs >> 3; // chunks per stream row of the slice
    const int h0 = s * hs;
    const uint32_t key = coop_key();
    const uint32_t tag = coop_tag(key, x);

    // ---- the tokens' slice of the streams: piece p = tid + 256 k is chunk p of the tile
    // [nt][4][nch] (stream row (t, i), h = h0 + 8 j); pieces past the tile or past H read 0
    // (rounds k with k 256 >= npieces are skipped: a wave-uniform test)
    const int npieces = nt * kHC * nch;
    const __amdgpu_buffer_rsrc_t vres =
        buf_view_uniform(a.res + (size_t)t0 * kHC * H, (uint32_t)((size_t)nt * kHC * H * sizeof(uint16_t)));
    u32x4 rp[kPR];
#pragma unroll
    for (int k = 0; k < kPR; ++k) {
        if (!kBig || k * kDThreads < npieces) {
            const int p = tid + k * kDThreads;
            const int row = p / nch, j = p - row * nch; // row = 4 t + i
            const int h = h0 + 8 * j;
            const uint32_t o = p < npieces && h < H ? ((uint32_t)row * (uint32_t)H + (uint32_t)h) * 2u : kOob;
            rp[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vres, (int)o, 0, 0));
        }
    }
    // kPost: the x pieces of items tid + 256 k = (t, j) of the tile (nt nch <= 768 items)
    constexpr int kXR = kPost ? kTg * (kDMaxChunks / kHC) / kDThreads : 1; // 1 or 3
    const int nitems = nt * nch;
    u32x4 xw[kXR];
    if constexpr (kPost) {
        const __amdgpu_buffer_rsrc_t vx =
            buf_view_uniform(a.x + (size_t)t0 * H, (uint32_t)((size_t)nt * H * sizeof(uint16_t)));
#pragma unroll
        for (int k = 0; k < kXR; ++k) {
            if (!kBig || k * kDThreads < nitems) {
                const int q = tid + k * kDThreads;
                const int t = q / nch, j = q - t * nch;
                const int h = h0 + 8 * j;
                const uint32_t o = q < nitems && h < H ? ((uint32_t)t * (uint32_t)H + (uint32_t)h) * 2u : kOob;
                xw[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vx, (int)o, 0, 0));
            }
        }
        for (int v = tid; v < (kHC + kHC * kHC) * nt; v += kDThreads) {
            if (v < kHC * nt) {
                coefs[v] = a.post_in[(size_t)t0 * kHC + v];
            } else {
                coefs[kHC * kTg + v - kHC * nt] = a.comb_in[(size_t)t0 * kHC * kHC + v - kHC * nt];
            }
        }
    }
    // ---- this thread's weights: rows 12 g + r of chunk c
    const int g = uniform(tid >> 7), c = tid & 127;
    const bool cval = c < kHC * nch;
    const int ci = cval ? c / nch : 0;
    const int hc = h0 + 8 * (c - ci * nch);
    const bool hok = cval && hc < H;
    float wv[kDRows][8];
    {
        const WT *wt = reinterpret_cast<const WT *>(a.hc_fn);
        const __amdgpu_buffer_rsrc_t vw =
            buf_view_uniform(a.hc_fn, (uint32_t)((size_t)a.fn_rows * kHC * H * sizeof(WT)));
#pragma unroll
        for (int r = 0; r < kDRows; ++r) {
            const int row = kDRows * g + r;
            load_w8(wt, vw, ((uint32_t)(row * kHC + ci)) * (uint32_t)H + (uint32_t)hc, hok, wv[r]);
        }
    }
#pragma unroll
    for (int k = 0; k < kPR; ++k) {
        if (!kBig || k * kDThreads < npieces) {
            *reinterpret_cast<u32x4 *>(tile + (tid + k * kDThreads) * 16) = rp[k];
        }
    }
    const int zpad = kBig ? a.tile_b : kTileB; // the 16 zero bytes
    if (tid == 0) {
        *reinterpret_cast<u32x4 *>(tile + zpad) = u32x4{0u, 0u, 0u, 0u};
        badf = 0;
    }
    __syncthreads();

    // ---- kPost: the post-map of item (t, j): the new streams out[n] = x post[n] + sum_o res[o]
    // comb[o][n] (mhc_post's products in its order), over the old ones in the tile and to `out`
    if constexpr (kPost) {
        const __amdgpu_buffer_rsrc_t vo =
            buf_view_uniform(a.out + (size_t)t0 * kHC * H, (uint32_t)((size_t)nt * kHC * H * sizeof(uint16_t)));
#pragma unroll
        for (int k = 0; k < kXR; ++k) {
        const int q = tid + k * kDThreads;
        const int t = q / nch, j = q - t * nch;
        const int h = h0 + 8 * j;
        if ((!kBig || k * kDThreads < nitems) && q < nitems && h < H) {
            u32x4 rw[kHC];
#pragma unroll
            for (int o = 0; o < kHC; ++o) {
                rw[o] = *reinterpret_cast<const u32x4 *>(tile + ((t * kHC + o) * nch + j) * 16);
            }
            const float *cp = coefs + t * kHC;
            const float *cc = coefs + kHC * kTg + t * kHC * kHC;
#pragma unroll
            for (int n = 0; n < kHC; ++n) {
                u32x4 nw;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float lo = bf16_lo(xw[k][q]) * cp[n];
                    float hi = bf16_hi(xw[k][q]) * cp[n];
#pragma unroll
                    for (int o = 0; o < kHC; ++o) {
                        lo = fmaf(bf16_lo(rw[o][q]), cc[o * kHC + n], lo);
                        hi = fmaf(bf16_hi(rw[o][q]), cc[o * kHC + n], hi);
                    }
                    nw[q] = pack_bf16x2(lo, hi);
                }
                *reinterpret_cast<u32x4 *>(tile + ((t * kHC + n) * nch + j) * 16) = nw;
                __builtin_amdgcn_raw_buffer_store_b128(nw, vo, (int)(((uint32_t)(t * kHC + n) * (uint32_t)H + (uint32_t)h) * 2u),
                                                       0, 2);
            }
        }
        }
        __syncthreads();
    }

    // ---- partial dots and sums of squares, P tokens a pass.  Rows outermost: the products
    // of row r start as soon as that row's weights have landed, beside the later rows' loads.
    const int npass = (nt + P - 1) / P;
    for (int pass = 0; pass < npass; ++pass) {
        float xf[P][8];
#pragma unroll
        for (int tl = 0; tl < P; ++tl) {
            const int t = pass * P + tl;
            const int xo = cval && t < nt ? (t * kHC * nch + c) * 16 : zpad;
            const u32x4 xr = *reinterpret_cast<const u32x4 *>(tile + xo);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xf[tl][2 * e] = bf16_lo(xr[e]);
                xf[tl][2 * e + 1] = bf16_hi(xr[e]);
            }
        }
        float v[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            v[k] = 0.0f;
        }
        if (g == 0) {
#pragma unroll
            for (int tl = 0; tl < P; ++tl) {
                float sq = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sq = fmaf(xf[tl][e], xf[tl][e], sq);
                }
                v[tl * kDF + kDRows] = sq;
            }
        }
#pragma unroll
        for (int r = 0; r < kDRows; ++r) {
#pragma unroll
            for (int tl = 0; tl < P; ++tl) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    acc = fmaf(wv[r][e], xf[tl][e], acc);
                }
                v[tl * kDF + r] = acc;
            }
        }
        wave_sums<V>(v, &part[pass][w][0], lane);
    }
    __syncthreads();

    // ---- this workgroup's record.  Value (t, f), f = 0..23 a dot and f = 24 the sum of
    // squares, is the sum of the two waves of its row half.  Chunk q < nu holds urgent values
    // 3q .. 3q + 2 (value u: field u / nt, or the sum of squares for u / nt = 4, of token
    // u mod nt); chunk nu + 7 t + d holds post and comb dots 3d .. 3d + 2 of token t.
    const int nu = (5 * nt + 2) / 3;
    const int nck = nu + kDDef * nt;
    auto rec_val = [&](int t, int f) -> float {
        const int pass = t / P, tl = t - pass * P;
        const int gg = (f < kDRows || f == kMix) ? 0 : 1;
        const int r = f == kMix ? kDRows : f - kDRows * gg;
        const float *pp = &part[pass][2 * gg][tl * kDF + r];
        return pp[0] + pp[V];
    };
    const __amdgpu_buffer_rsrc_t vrec = buf_view_uniform(a.rec, a.rec_bytes);
    auto chunk_off = [&](int q, int sli) -> uint32_t {
        return (((uint32_t)x * kDGroupChunks + (uint32_t)q) * kDSlices + (uint32_t)sli) * 16u;
    };
    for (int q = tid; q < nck; q += kDThreads) {
        float vals[3];
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            float val = 0.0f;
            if (q < nu) {
                const int u = 3 * q + e;
                if (u < 5 * nt) {
                    const int f = u / nt, t = u - f * nt;
                    val = rec_val(t, f < kHC ? f : kMix);
                }
            } else {
                const int dq = q - nu;
                const int t = dq / kDDef, d = dq - kDDef * t;
                const int fi = 3 * d + e;
                if (fi < kMix - kHC) {
                    val = rec_val(t, kHC + fi);
                }
            }
            vals[e] = val;
        }
        const u32x4 chunk = {__float_as_uint(vals[0]), __float_as_uint(vals[1]), __float_as_uint(vals[2]), tag};
        __builtin_amdgcn_raw_buffer_store_b128(chunk, vrec, (int)chunk_off(q, s), 0, 0);
    }
    // the record is in L2 before this workgroup reads it back with the others'
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- the group's records: list entry e < nu is urgent chunk e, entries nu .. nu + 6 the
    // post and comb chunks of token s (workgroup s < nt, when there are post and comb).
    // Half-wave hw takes entries hw + 8 k; lane sl of it loads slice sl.  Rounds k with 8 k >=
    // nlist are skipped (a wave-uniform test).
    const bool designated = !a.head && s < nt;
    const int nlist = nu + (designated ? kDDef : 0);
    const int hw = tid >> 5, sl = tid & 31;
    const uint32_t want = tag ^ a.tag_skew;
    auto load_list = [&](u32x4(&rr)[kRnd]) {
#pragma unroll
        for (int k = 0; k < kRnd; ++k) {
            if (!kBig || k * 8 < nlist) {
                const int e = k * 8 + hw;
                const int q = e < nu ? e : nu + kDDef * s + (e - nu);
                const uint32_t o = e < nlist ? chunk_off(q, sl) : kOob;
                rr[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrec, (int)o, 0, 16));
            }
        }
    };
    auto take_list = [&](const u32x4(&rr)[kRnd]) {
        int bad = 0;
#pragma unroll
        for (int k = 0; k < kRnd; ++k) {
            if (!kBig || k * 8 < nlist) {
                const int e = k * 8 + hw;
                if (e < nlist && rr[k][3] != want) {
                    bad = 1;
                }
                const float v0 = half_sum(__uint_as_float(rr[k][0]));
                const float v1 = half_sum(__uint_as_float(rr[k][1]));
                const float v2 = half_sum(__uint_as_float(rr[k][2]));
                float *dst = sl == kHalfSumLane && e < nlist ? (e < nu ? usum + 3 * e : dsum + 3 * (e - nu))
                                                             : dummy + (lane & 0x3C);
                dst[0] = v0;
                dst[1] = v1;
                dst[2] = v2;
            }
        }
        if (bad) {
            badf = 1;
        }
    };
    {
        u32x4 rr[kRnd];
        load_list(rr);
        take_list(rr);
    }
    __syncthreads();
    if (badf) {
        // a record had not landed: load them all again
        for (int tries = 0; tries < a.max_retry; ++tries) {
            __syncthreads();
            if (tid == 0) {
                badf = 0;
            }
            __syncthreads();
            u32x4 rr[kRnd];
            asm volatile("" ::: "memory");
            load_list(rr);
            take_list(rr);
            __syncthreads();
            if (!badf) {
                break;
            }
        }
        // still missing after the bounded reloads: the sums become NaN, so the outputs are NaN
        if (badf) {
            if (tid < 3 * kUrg) {
                usum[tid] = __builtin_nanf("");
            }
            if (tid >= 3 * kWave && tid < 3 * kWave + 3 * kDDef) {
                dsum[tid - 3 * kWave] = __builtin_nanf("");
            }
        }
        __syncthreads();
    }

    // ---- token s's post weights and Sinkhorn (wave 3 of workgroup s < nt, as soon as the sums
    // are in; the four 16-lane rows compute the same matrix, lane e holding entry (e / 4, e mod 4))
    if (designated && w == 3) {
        const int e = lane & 15;
        const float rstd = rstd_of(usum[kHC * nt + s], a.inv_k, a.rms_eps);
        const float Lg = fmaf(dsum[kHC + e] * rstd, a.hc_scale[2], a.hc_base[2 * kHC + e]);
        const float zp = fmaf(dsum[e & 3] * rstd, a.hc_scale[1], a.hc_base[kHC + (e & 3)]);
        const float Pv = sinkhorn_row16(Lg, a.iters, a.sk_eps);
        const float pv = sigmoidf_fast(zp) * a.post_mult;
        const size_t t = (size_t)(t0 + s);
        if (lane < kHC * kHC) {
            a.comb[t * kHC * kHC + lane] = Pv;
        }
        if (lane < kHC) {
            a.post[t * kHC + lane] = pv;
        }
        return;
    }
    // ---- the collapse of this slice of every token (the other waves): y = sum_i pre_i res_i in
    // the order of the streams, each item forming its token's rstd and pre weights from the
    // sums (workgroup 0 also stores them to `pre`)
    const int nthr = designated ? 3 * kWave : kDThreads;
    for (int it = tid; it < nt * nch; it += nthr) {
        const int t = it / nch, j = it - t * nch;
        const int h = h0 + 8 * j;
        const float rstd = rstd_of(usum[kHC * nt + t], a.inv_k, a.rms_eps);
        float p[kHC];
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
            p[i] = sigmoid_rcp(fmaf(usum[i * nt + t] * rstd, a.hc_scale[0], a.hc_base[i])) + a.pre_eps;
        }
        if (s == 0 && j == 0 && a.pre != nullptr) {
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                a.pre[(size_t)(t0 + t) * kHC + i] = p[i];
            }
        }
        if (h < H) {
            const unsigned char *b = tile + (t * kHC * nch + j) * 16;
            u32x4 rw[kHC];
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                rw[i] = *reinterpret_cast<const u32x4 *>(b + i * nch * 16);
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
            store_nt16(a.y + (size_t)(t0 + t) * H + h, yw);
        }
    }
}

template <typename WT, bool kPost>
hipError_t launch_decode_big(const DecArgs &a, hipStream_t stream)
{
    // the dynamic-LDS limit is a per-device attribute: raised once on each device to the
    // largest tile
    static std::atomic<bool> attr_set[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        return e != hipSuccess ? e : hipErrorInvalidDevice;
    }
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute((const void *)pre_decode_kernel<WT, 4, kPost, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kDTileMaxB + 16);
        if (e != hipSuccess) {
            return e;
        }
        attr_set[dev].store(true, std::memory_order_release);
    }
    pre_decode_kernel<WT, 4, kPost, true>
        <<<dim3(kDGroups * kDSlices), dim3(kDThreads), (size_t)a.tile_b + 16, stream>>>(a);
    return hipGetLastError();
}

template <typename WT, bool kPost>
hipError_t launch_decode_t(const DecArgs &a, hipStream_t stream)
{
    const dim3 grid(kDGroups * kDSlices), block(kDThreads);
    if (a.Tg <= 1) {
        pre_decode_kernel<WT, 1, kPost, false><<<grid, block, 0, stream>>>(a);
    } else if (a.Tg <= 2) {
        pre_decode_kernel<WT, 2, kPost, false><<<grid, block, 0, stream>>>(a);
    } else if (a.Tg <= 8) {
        pre_decode_kernel<WT, 4, kPost, false><<<grid, block, 0, stream>>>(a);
    } else {
        return launch_decode_big<WT, kPost>(a, stream);
    }
    return hipGetLastError();
}

DecArgs decode_args(const uint16_t *res, const void *hc_fn, int fn_rows, const float *hc_scale,
                    const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps,
                    float post_mult, int iters, bool head, uint16_t *y, float *post, float *comb, float *pre,
                    void *workspace)
{
    DecArgs a{};
    a.res = res;
    a.hc_fn = hc_fn;
    a.hc_scale = hc_scale;
    a.hc_base = hc_base;
    a.T = (int)T;
    a.H = (int)H;
    a.fn_rows = fn_rows;
    a.Tg = (int)((T + kDGroups - 1) / kDGroups);
    a.hs = (int)(8 * ((H + 8 * kDSlices - 1) / (8 * kDSlices)));
    a.tile_b = (a.Tg * kHC * (a.hs / 8) + kDThreads - 1) / kDThreads * kDThreads * 16;
    a.inv_k = 1.0f / (float)(kHC * H);
    a.rms_eps = rms_eps;
    a.pre_eps = pre_eps;
    a.sk_eps = sinkhorn_eps;
    a.post_mult = post_mult;
    a.iters = iters;
    a.head = head ? 1 : 0;
    a.y = y;
    a.post = post;
    a.comb = comb;
    a.pre = pre;
    a.rec = reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(workspace) + pre_split_bytes(H));
    a.rec_bytes = (uint32_t)((size_t)kDGroups * kDGroupChunks * kDSlices * sizeof(u32x4));
    a.max_retry = exchange_max_retry();
    a.tag_skew = exchange_tag_skew();
    return a;
}

} // namespace

bool pre_decode_shape_ok(int64_t T, int64_t H)
{
    return T >= 1 && T <= kDMaxTok && H >= 8 && H <= (int64_t)kDSlices * kDMaxHs && H % 8 == 0;
}

bool pre_decode_usable(int64_t T, int64_t H, bool vec8) { return vec8 && pre_decode_shape_ok(T, H) && exchange_device_ok(); }

size_t pre_decode_workspace_bytes(int64_t H)
{
    return pre_split_bytes(H) + (size_t)kDGroups * kDGroupChunks * kDSlices * sizeof(u32x4);
}

hipError_t launch_pre_decode(const uint16_t *res, const void *hc_fn, bool fn_bf16, int fn_rows,
                             const float *hc_scale, const float *hc_base, int64_t T, int64_t H, float rms_eps,
                             float pre_eps, float sinkhorn_eps, float post_mult, int iters, bool head, uint16_t *y,
                             float *post, float *comb, float *pre, void *workspace, hipStream_t stream)
{
    if (!pre_decode_shape_ok(T, H)) {
        return hipErrorInvalidValue;
    }
    const DecArgs a = decode_args(res, hc_fn, fn_rows, hc_scale, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps,
                                  post_mult, iters, head, y, post, comb, pre, workspace);
    return fn_bf16 ? launch_decode_t<uint16_t, false>(a, stream) : launch_decode_t<float, false>(a, stream);
}

hipError_t launch_post_pre_decode(const uint16_t *x, const uint16_t *res, const float *post_in,
                                  const float *comb_in, const float *hc_fn, const float *hc_scale,
                                  const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                                  float sinkhorn_eps, float post_mult, int iters, uint16_t *out, uint16_t *y,
                                  float *post, float *comb, float *pre, void *workspace, hipStream_t stream)
{
    if (!pre_decode_shape_ok(T, H)) {
        return hipErrorInvalidValue;
    }
    DecArgs a = decode_args(res, hc_fn, kMix, hc_scale, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps, post_mult,
                            iters, false, y, post, comb, pre, workspace);
    a.x = x;
    a.post_in = post_in;
    a.comb_in = comb_in;
    a.out = out;
    return launch_decode_t<float, true>(a, stream);
}

} // namespace mhc
