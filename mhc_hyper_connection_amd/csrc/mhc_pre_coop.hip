// mhc_pre_coop.hip -- the mHC pre-map with one read of the streams (gfx950).
//
// ("FlashInfer mHC 模块深度解析", section 3.4: per token, the RMS statistic and the
// projection, then the mixes and the Sinkhorn, then the collapse, from one read of the
// residual; section 5.2 for the arithmetic.)
//
// A token's pre weights need all 4H products of the projection before its collapse can
// start, and no workgroup can hold the 24 x 4H weights, so the reduction over K is
// split across workgroups and the token's streams are held on chip until it is done.
//
//  * One group of 32 workgroups per XCD (workgroup b runs on XCD b mod 8 under the
//    hardware's round-robin dispatch; the grid is 256 workgroups, one per CU).  Workgroup
//    s of a group owns a slice of W x 32 h across the four streams and keeps that slice of
//    the weights in VGPRs, split exactly into three bf16 terms for the MFMA.
//  * The group walks its tokens in 16-token steps (group x takes steps x, x + 8, ...).
//    A step's slice of the streams is loaded two steps ahead, written into a ring of L + 1
//    LDS slots, projected with v_mfma_f32_16x16x32_bf16 (the sum of squares rides on
//    v_dot2_f32_bf16) into per-wave partial sums, and in the next iteration reduced over
//    the workgroup's waves into one record: 24 partial dots and the partial sum of squares
//    of its 16 tokens (the partial sums are double-buffered by step parity, so that the
//    reduction runs beside the next step's products instead of between two barriers).
//  * Records go through the XCD's L2 as 16-byte chunks of three values and a tag that
//    names the call (its dispatch id) and the step.  L iterations after producing a step,
//    every workgroup sums the pre dots and the sums of squares of that step from all 32
//    slices (device-scope loads, issued one iteration earlier: they miss the CU's L1) in a
//    fixed order; the next iteration forms rstd and the pre weights and collapses its slice
//    of the step, from registers loaded out of the ring: the streams are read from HBM
//    once.  A chunk whose tag does not match has not landed yet and is loaded again, up to
//    2^14 times; a step whose records are still missing then (its writer was never made
//    resident, e.g. behind a long kernel on another stream) gets NaN outputs rather than
//    stale ones.
//  * An iteration has two barriers.  Between them run the slice sums, the products, the
//    collapse (its arithmetic between the products), the record of the previous step and
//    the next record loads; between B2 and the next B1 only the pre weights, the new step's
//    slot and the stream loads.
//  * Each token's post weights and Sinkhorn are finished by one workgroup: workgroup s
//    takes token s mod 16 of the steps whose parity is s / 16.
//
// Reduction orders are fixed (waves in order, slices by a butterfly over 32 lanes), so a
// result does not depend on timing.  Every iteration issues the same memory operations
// (empty buffer views stand for steps outside the range), which keeps the compiler's
// in-order wait counts exact, so the loads of the next two steps stay in flight.
#include "mhc_device.h"
#include "mhc_internal.h"

#include <atomic>
#include <string.h>

namespace mhc {

namespace {

constexpr int kQTok = 16;                                           // tokens per step
constexpr int kQGroups = 8;                                         // one group per XCD
constexpr int kQSlices = 32;                                        // workgroups per group
constexpr int kQUrgVals = 5 * kQTok;                                // pre dots 0..3 and the sum of squares
constexpr int kQUrgChunks = (kQUrgVals + 2) / 3;                    // 27
constexpr int kQDefFields = kMix - kHC;                             // post and comb dots
constexpr int kQDefChunks = (kQDefFields + 2) / 3;                  // 7
constexpr int kQChunks = kQUrgChunks + kQTok * kQDefChunks;         // chunks of one record (139)
// row stride of the waves' partial sums: 24 dots and the sum of squares, padded to 28 floats
// (conflict-free writes) except at 8 waves, where the two parity buffers must fit beside a
// ring of 4 slots
constexpr int red_stride(int W) { return W == 8 ? 25 : 28; }
constexpr int kQMaxRetry = 1 << 14;                                 // reloads of a step's records before giving up
std::atomic<int> g_max_retry{kQMaxRetry};
std::atomic<uint32_t> g_tag_skew{0};
constexpr int64_t kCoopMinTokens = 1024; // below this the pipeline's fill and drain dominate

struct CoopArgs {
    const uint16_t *res;
    const void *hc_fn;
    const float *hc_scale, *hc_base;
    int T, H, nhb, fn_rows;
    int wvec; // hc_fn 16-byte aligned: each lane's 8 weights of a row in 16-byte loads
    int L, R, RR; // collapse lag in iterations, LDS ring slots, record ring slots
    float inv_k, rms_eps, pre_eps, sk_eps, post_mult; // inv_k = 1 / (4H)
    int iters, head;
    uint16_t *y;
    float *post, *comb, *pre;
    u32x4 *rec;
    uint32_t rec_bytes;
    // the post-map in front (kPost): the sublayer output x [T][H], the previous mixes
    // post_in [T][4] and comb_in [T][4][4]; the new streams go to out [T][4][H] and are
    // the streams the pre-map reads
    const uint16_t *x;
    const float *post_in, *comb_in;
    uint16_t *out;
    // reloads of a step's records before its outputs become NaN, and a value mixed into the
    // tags the readers expect (0; nonzero only to make every record look missing, a test of
    // the NaN path set through mhc_set_exchange_test_hooks)
    int max_retry;
    uint32_t tag_skew;
};
constexpr int kCoefVals = kQTok * (kHC + kHC * kHC); // post and comb of one step: 320 floats

__device__ __forceinline__ float weight_elem(const float *w, uint32_t i, __amdgpu_buffer_rsrc_t v)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(v, (int)(i * 4u), 0, 0));
}
__device__ __forceinline__ float weight_elem(const uint16_t *w, uint32_t i, __amdgpu_buffer_rsrc_t v)
{
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(v, (int)(i * 2u), 0, 0));
}

// Weights i .. i + 7 (i a multiple of 8, the buffer 16-byte aligned) in 16-byte loads;
// an index past the view reads zeros.
__device__ __forceinline__ void load_w8(const float *, uint32_t i, __amdgpu_buffer_rsrc_t v, float (&o)[8])
{
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const u32x4 p = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)(i * 4u + 16u * hf), 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[4 * hf + e] = __uint_as_float(p[e]);
        }
    }
}
__device__ __forceinline__ void load_w8(const uint16_t *, uint32_t i, __amdgpu_buffer_rsrc_t v, float (&o)[8])
{
    const u32x4 p = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)(i * 2u), 0, 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[2 * e] = __uint_as_float(p[e] << 16);
        o[2 * e + 1] = __uint_as_float(p[e] & 0xFFFF0000u);
    }
}

// Sum over the four 16-lane rows of the wave, same bits in every lane: rows (0 + 1) and
// (2 + 3) by v_permlane16_swap, then the two halves by v_permlane32_swap.
__device__ __forceinline__ float rows_sum(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int W, typename WT, bool kPost>
__global__ __launch_bounds__(W * 64) void pre_coop_kernel(CoopArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int kTh = W * 64;
    constexpr int kQRedStride = red_stride(W);
    constexpr int kPieces = 4 * W;        // 16-byte pieces of one stream row of the slice
    constexpr int kRowB = 64 * W;         // bytes of one stream row of the slice
    constexpr int kTokB = 4 * kRowB + 16; // token pitch in a slot: (16W + 1) x 16 bytes
    constexpr int kSlotB = kQTok * kTokB;
    constexpr int kHW = 2 * W;            // half-waves
    constexpr int kUR = (kQUrgChunks + kHW - 1) / kHW;
    constexpr int kDR = (kQDefChunks + kHW - 1) / kHW;
    constexpr int kRS = (kQChunks + kTh - 1) / kTh;
    constexpr int kCf = (kCoefVals + kTh - 1) / kTh; // coefficient values per thread (kPost)

    const int R = a.R, RR = a.RR, L = a.L;
    // the wave that computes the pre weights and this workgroup's token: wave 3 sits alone on
    // its SIMD when W < 8 (waves go to SIMDs round robin)
    constexpr int kAux = W >= 4 ? 3 : W - 1;
    unsigned char *ring = smem;
    float *red = reinterpret_cast<float *>(smem + R * kSlotB); // [2][W][16][stride], by step parity
    float *sums = red + 2 * W * kQTok * kQRedStride;           // [81]: value f * 16 + token
    float *dsum = sums + 96;                                   // [21]: the designated token's post and comb dots
    float *prel = dsum + 32;                                   // [16][4]
    int *badf = reinterpret_cast<int *>(prel + 64);
    float *dummy = prel + 64 + 4; // [64]: writes of lanes with nothing to write (no divergent branches)
    float *coefb = dummy + 64;    // [2][320] (kPost): post [16][4] then comb [16][16] of a step, by parity

    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int g = lane >> 4, c = lane & 15;
    const int hw = tid >> 5, sl = tid & 31;
    const int x = (int)blockIdx.x & (kQGroups - 1);
    const int s = (int)blockIdx.x >> 3;
    const int T = a.T, H = a.H;
    const int steps_total = (T + kQTok - 1) / kQTok;
    const int nst = steps_total > x ? (steps_total - x + kQGroups - 1) / kQGroups : 0;
    if (nst == 0) {
        return; // the whole group
    }
    const uint32_t key = coop_key();
    const float s0 = a.hc_scale[0];
    const float s1 = a.head ? 0.0f : a.hc_scale[1];
    const float s2 = a.head ? 0.0f : a.hc_scale[2];

    // ---- this wave's slice of the weights: 32 h of the 4 streams, rows 0..23, as three
    // bf16 terms in the MFMA B layout (lane (g, c): k = hb*32 + 8g .. +8 of stream i).  Column
    // tile 0 holds rows 0..15 (lane c: row c), one operand per term.  Rows 16..23 take two
    // operands: lanes c < 8 hold the hi term of row 16 + c and lanes c >= 8 the mid term of
    // row 8 + c in the first, lanes c < 8 the lo term of row 16 + c in the second; both
    // products go into one accumulator, whose columns c and c + 8 are added afterwards.
    const int hb = s * W + w;
    u32x4 b0[kHC][3], b1[kHC][2];
    // hc_base per lane: the pre entry lane / 16; with e = lane mod 16 the comb entry e and the
    // post entry e mod 4 (the designated token's row of lanes)
    const float bpre = a.hc_base[lane >> 4]; // lane = 16 k + token computes pre weight k
    const float bcomb = a.head ? 0.0f : a.hc_base[2 * kHC + (lane & 15)];
    const float bpost = a.head ? 0.0f : a.hc_base[kHC + (lane & 3)];

    // ---- geometry of this thread's loads and of the record chunks
    const int piece = tid % kPieces;
    // 0..15: this thread's rows of a step (row = token * 4 + stream) are prow + 16k, or with
    // the post-map in front the 4 streams 4 prow + k of token prow
    const int prow = tid / kPieces;
    const int hq = s * (32 * W) + piece * 8;
    const uint32_t colq = hq < H ? (uint32_t)hq * 2u : kOob;
    const __amdgpu_buffer_rsrc_t vrec = buf_view_uniform(a.rec, a.rec_bytes);
    const uint32_t def0 = (uint32_t)kQGroups * RR * kQUrgChunks * kQSlices; // first deferred chunk
    const int td = s & 15;                                                  // the token this workgroup finishes
    auto urg_chunk = [&](int q, int k, int sli) -> uint32_t {
        return (((uint32_t)(x * RR + q) * kQUrgChunks + k) * kQSlices + sli) * 16u;
    };
    auto def_chunk = [&](int q, int tok, int k, int sli) -> uint32_t {
        return (def0 + (((uint32_t)(x * RR + q) * kQTok + tok) * kQDefChunks + k) * kQSlices + sli) * 16u;
    };
    auto wrap = [](int v, int n) { return v >= n ? v - n : v; }; // v in [0, 2n)
    auto designated = [&](int j) { return j >= 0 && j < nst && (s >> 4) == (j & 1); };

    auto load_step = [&](int j, u32x4(&d)[4]) {
        const int t0 = (j * kQGroups + x) * kQTok;
        const int ntok = (j >= 0 && j < nst) ? min(kQTok, T - t0) : 0;
        const __amdgpu_buffer_rsrc_t v = buf_view_uniform(a.res + (size_t)(ntok > 0 ? t0 : 0) * kHC * H,
                                                          (uint32_t)((size_t)ntok * kHC * H * sizeof(uint16_t)));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = kPost ? 4 * prow + k : prow + 16 * k;
            d[k] = __builtin_bit_cast(u32x4,
                                      __builtin_amdgcn_raw_buffer_load_b128(v, (int)((uint32_t)(row * H) * 2u + colq), 0, 0));
        }
    };
    // kPost: the x row of token prow (this thread's piece) of step j
    auto load_x = [&](int j) -> u32x4 {
        const int t0 = (j * kQGroups + x) * kQTok;
        const int ntok = (kPost && j >= 0 && j < nst) ? min(kQTok, T - t0) : 0;
        const __amdgpu_buffer_rsrc_t v = buf_view_uniform(a.x + (size_t)(ntok > 0 ? t0 : 0) * H,
                                                          (uint32_t)((size_t)ntok * H * sizeof(uint16_t)));
        return __builtin_bit_cast(u32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(v, (int)((uint32_t)(prow * H) * 2u + colq), 0, 0));
    };
    // kPost: the post and comb values of step j this thread stages: value tid + k kTh of the
    // step's 320 (post [16][4] at 0..63, from wave 0; comb [16][16] at 64..319)
    auto load_coef = [&](int j, float(&cf)[kCf]) {
        const int t0 = (j * kQGroups + x) * kQTok;
        const int ntok = (kPost && j >= 0 && j < nst) ? min(kQTok, T - t0) : 0;
        const __amdgpu_buffer_rsrc_t vp =
            buf_view_uniform(a.post_in + (size_t)(ntok > 0 ? t0 : 0) * kHC, (uint32_t)(ntok * kHC * 4));
        const __amdgpu_buffer_rsrc_t vc =
            buf_view_uniform(a.comb_in + (size_t)(ntok > 0 ? t0 : 0) * kHC * kHC, (uint32_t)(ntok * kHC * kHC * 4));
#pragma unroll
        for (int k = 0; k < kCf; ++k) {
            const int v = tid + k * kTh;
            const bool from_post = k == 0 && w == 0; // wave-uniform
            const uint32_t o = from_post ? (uint32_t)v * 4u : (v < kCoefVals ? (uint32_t)(v - 4 * kQTok) * 4u : kOob);
            cf[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(from_post ? vp : vc, (int)o, 0, 0));
        }
    };
    auto store_coef = [&](int j, const float(&cf)[kCf]) {
        float *cb = coefb + (j & 1) * kCoefVals;
#pragma unroll
        for (int k = 0; k < kCf; ++k) {
            const int v = tid + k * kTh;
            *(v < kCoefVals ? cb + v : dummy + lane) = cf[k];
        }
    };
    // the records of step j this thread reads: chunk k of slice sl for its half-wave's k
    auto load_recs = [&](int j, int q, u32x4(&ru)[kUR], u32x4(&rd)[kDR]) {
        const bool ok = j >= 0 && j < nst;
#pragma unroll
        for (int r = 0; r < kUR; ++r) {
            const int k = r * kHW + hw;
            const uint32_t o = ok && k < kQUrgChunks ? urg_chunk(q, k, sl) : kOob;
            ru[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrec, (int)o, 0, 16));
        }
        const bool dz = designated(j);
#pragma unroll
        for (int r = 0; r < kDR; ++r) {
            const int k = r * kHW + hw;
            const uint32_t o = dz && k < kQDefChunks ? def_chunk(q, td, k, sl) : kOob;
            rd[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrec, (int)o, 0, 16));
        }
    };
    // tags of the loaded records of step j (0 if they all match), and their slice sums into LDS
    auto take_recs = [&](int j, const u32x4(&ru)[kUR], const u32x4(&rd)[kDR], int *flag) {
        const bool ok = j >= 0 && j < nst;
        const uint32_t tag = coop_tag(key, j * kQGroups + x) ^ a.tag_skew;
        const bool dz = designated(j);
        int bad = 0;
#pragma unroll
        for (int r = 0; r < kUR; ++r) {
            const int k = r * kHW + hw;
            if (ok && k < kQUrgChunks && ru[r][3] != tag) {
                bad = 1;
            }
            float v0 = half_sum(__uint_as_float(ru[r][0]));
            float v1 = half_sum(__uint_as_float(ru[r][1]));
            float v2 = half_sum(__uint_as_float(ru[r][2]));
            float *dst = sl == kHalfSumLane && k < kQUrgChunks ? sums + 3 * k : dummy + (lane & 0x3C);
            dst[0] = v0;
            dst[1] = v1;
            dst[2] = v2;
        }
        if (2 * w >= kQDefChunks) { // no deferred chunk in this wave (wave-uniform)
            if (bad) {
                *flag = 1;
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < kDR; ++r) {
            const int k = r * kHW + hw;
            if (dz && k < kQDefChunks && rd[r][3] != tag) {
                bad = 1;
            }
            float v0 = half_sum(__uint_as_float(rd[r][0]));
            float v1 = half_sum(__uint_as_float(rd[r][1]));
            float v2 = half_sum(__uint_as_float(rd[r][2]));
            float *dst = sl == kHalfSumLane && k < kQDefChunks ? dsum + 3 * k : dummy + (lane & 0x3C);
            dst[0] = v0;
            dst[1] = v1;
            dst[2] = v2;
        }
        if (bad) {
            *flag = 1;
        }
    };

    // The record chunks this thread writes: chunk ch = tid + rs * kTh of kQChunks (27 urgent
    // chunks: value 3ch + e is field (3ch + e) / 16 of token (3ch + e) mod 16, field 4 being
    // the sum of squares in column 24; then 16 tokens x 7 chunks of the 20 post and comb
    // dots, columns 4..23).  rc_off: the value's offset in a wave's [16][28] partials;
    // rc_base + q * rc_qstride: the chunk's byte offset in record slot q.
    int rc_off[kRS][3];
    int rc_valid[kRS];
    uint32_t rc_base[kRS], rc_qstride[kRS];
#pragma unroll
    for (int rs = 0; rs < kRS; ++rs) {
        const int ch = tid + rs * kTh;
        rc_valid[rs] = 0;
        rc_base[rs] = kOob;
        rc_qstride[rs] = 0;
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            rc_off[rs][e] = 0;
        }
        if (ch < kQUrgChunks) {
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                const int val = 3 * ch + e;
                if (val < kQUrgVals) {
                    const int f = val >> 4, tok = val & 15;
                    rc_off[rs][e] = tok * kQRedStride + (f < kHC ? f : kMix);
                    rc_valid[rs] |= 1 << e;
                }
            }
            rc_base[rs] = urg_chunk(0, ch, s);
            rc_qstride[rs] = (uint32_t)kQUrgChunks * kQSlices * 16u;
        } else if (ch < kQChunks) {
            const int dch = ch - kQUrgChunks;
            const int tok = dch / kQDefChunks, k = dch - kQDefChunks * (dch / kQDefChunks);
#pragma unroll
            for (int e = 0; e < 3; ++e) {
                const int f = 3 * k + e;
                if (f < kQDefFields) {
                    rc_off[rs][e] = tok * kQRedStride + kHC + f;
                    rc_valid[rs] |= 1 << e;
                }
            }
            rc_base[rs] = def_chunk(0, tok, k, s);
            rc_qstride[rs] = (uint32_t)kQTok * kQDefChunks * kQSlices * 16u;
        }
    }

    // ---- one iteration i (ri = i mod R, qi = i mod RR, kept as counters).  X = i - L.
    // Phase A (after the previous iteration's B2): reload the records of step X - 1 if one had
    // not landed; the auxiliary wave forms the pre weights of step X - 1 (and the designated
    // token's raw comb and post values); step i goes into its slot; the streams of step i + 2
    // are loaded.  Phase B (between B1 and B2): the records of step X are summed over the
    // slices; step i is projected while step X - 1 is collapsed from registers; the partial
    // sums of step i - 1 (written before the last B2) are reduced over the waves into its
    // record; the records of step X + 1 are loaded; step X's slot goes into registers for the
    // next iteration's collapse (the slot is written again, as step i + 1, after B2).
    auto iteration = [&](int i, int ri, int qi, u32x4(&cur)[4], u32x4 &xcur, float(&cf)[kCf], u32x4(&ru)[kUR],
                         u32x4(&rd)[kDR], u32x4(&hold)[kHC]) {
        const int X = i - L;
        const int Xp = X - 1;                        // pre weights formed and collapsed this iteration
        const int rx = wrap(ri + 1, R);              // slot of step X: i - L = i + 1 (mod R = L + 1)
        const int qxp = wrap(qi + RR - L - 1, RR);   // record slot of step X - 1
        const int qx1 = wrap(qi + RR - L + 1, RR);   // record slot of step X + 1
        const int qim1 = wrap(qi + RR - 1, RR);      // record slot of step i - 1
        const bool xp_ok = Xp >= 0 && Xp < nst;
        const bool p_ok = i >= 0 && i < nst;
        const bool pm1_ok = i - 1 >= 0 && i - 1 < nst;

        // ---- phase A
        // A1: a record of step X - 1 had not landed when it was summed: load them again
        {
            int *bfp = badf + ((i - 1) & 1);
            if (*bfp) {
                for (int tries = 0; tries < a.max_retry; ++tries) {
                    __syncthreads();
                    if (tid == 0) {
                        *bfp = 0;
                    }
                    __syncthreads();
                    u32x4 qu[kUR], qd[kDR];
                    asm volatile("" ::: "memory");
                    load_recs(Xp, qxp, qu, qd);
                    take_recs(Xp, qu, qd, bfp);
                    __syncthreads();
                    if (!*bfp) {
                        break;
                    }
                }
                // still missing after the bounded reloads (a workgroup of the group was not
                // resident in time): the step's sums become NaN, so its outputs are NaN, never
                // values from a stale record
                if (*bfp) {
                    if (tid < 96) {
                        sums[tid] = __builtin_nanf("");
                    } else if (tid < 128) {
                        dsum[tid - 96] = __builtin_nanf("");
                    }
                }
                __syncthreads();
            }
        }
        // A2: pre weights of step X - 1 (the auxiliary wave: lane = 16 k + token, one sigmoid
        // each); the designated token's comb logits (lane e) and post pre-activations (lanes
        // 0..3), stored raw into comb and post (the Sinkhorn and the sigmoids run after the
        // loop); its pre weights to `pre` if asked for.  Every wave issues the stores (elsewhere
        // into empty views), so that every wave's memory operations stay the same.
        const bool dz = designated(Xp) && !a.head;
        const int tdz = (Xp * kQGroups + x) * kQTok + td;
        {
            if (w == kAux && xp_ok) {
                const int tok = lane & 15, k = lane >> 4;
                const float rstd = rstd_of(sums[4 * kQTok + tok], a.inv_k, a.rms_eps);
                prel[tok * kHC + k] = sigmoid_rcp(fmaf(sums[k * kQTok + tok] * rstd, s0, bpre)) + a.pre_eps;
            }
            float Lg = 0.0f, zp = 0.0f;
            if (w == kAux && dz) {
                const float rstd = rstd_of(sums[4 * kQTok + td], a.inv_k, a.rms_eps);
                const int e = lane & 15;
                Lg = fmaf(dsum[kHC + e] * rstd, s2, bcomb);
                zp = fmaf(dsum[e & 3] * rstd, s1, bpost);
            }
            const bool tin = dz && tdz < T && w == kAux;
            const __amdgpu_buffer_rsrc_t vc =
                buf_view_uniform(a.comb + (size_t)(tin ? tdz : 0) * kHC * kHC, tin ? kHC * kHC * 4 : 0);
            const __amdgpu_buffer_rsrc_t vp =
                buf_view_uniform(a.post + (size_t)(tin ? tdz : 0) * kHC, tin ? kHC * 4 : 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Lg), vc, lane < 16 ? lane * 4 : (int)kOob, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(zp), vp, lane < 4 ? lane * 4 : (int)kOob, 0, 0);
            const bool pin = designated(Xp) && tdz < T && a.pre != nullptr && w == kAux;
            const __amdgpu_buffer_rsrc_t vq =
                buf_view_uniform(pin ? (const void *)(a.pre + (size_t)tdz * kHC) : (const void *)a.y, pin ? kHC * 4 : 0);
            const float pv = w == kAux ? prel[td * kHC + (lane & 3)] : 0.0f;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pv), vq, lane < 4 ? lane * 4 : (int)kOob, 0, 0);
        }
        // A3: step i into its slot
        unsigned char *slot = ring + ri * kSlotB;
        if constexpr (kPost) {
            // the post-map of step i for this thread's (token prow, piece): the new streams
            // out[n] = x post[n] + sum_o res[o] comb[o][n] (the post-map's own order of the
            // products), into the slot and to `out`
            const float *cb = coefb + (i & 1) * kCoefVals;
            const f32x4 pq = *reinterpret_cast<const f32x4 *>(cb + prow * kHC);
            f32x4 cq[kHC];
#pragma unroll
            for (int o = 0; o < kHC; ++o) {
                cq[o] = *reinterpret_cast<const f32x4 *>(cb + kHC * kQTok + prow * kHC * kHC + o * kHC);
            }
            const int t0 = (i * kQGroups + x) * kQTok;
            const int ntok = p_ok ? min(kQTok, T - t0) : 0;
            const __amdgpu_buffer_rsrc_t vo = buf_view_uniform(a.out + (size_t)(ntok > 0 ? t0 : 0) * kHC * H,
                                                               (uint32_t)((size_t)ntok * kHC * H * sizeof(uint16_t)));
#pragma unroll
            for (int n = 0; n < kHC; ++n) {
                u32x4 nw;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float lo = bf16_lo(xcur[q]) * pq[n];
                    float hi = bf16_hi(xcur[q]) * pq[n];
#pragma unroll
                    for (int o = 0; o < kHC; ++o) {
                        lo = fmaf(bf16_lo(cur[o][q]), cq[o][n], lo);
                        hi = fmaf(bf16_hi(cur[o][q]), cq[o][n], hi);
                    }
                    nw[q] = pack_bf16x2(lo, hi);
                }
                *reinterpret_cast<u32x4 *>(slot + prow * kTokB + n * kRowB + piece * 16) = nw;
                __builtin_amdgcn_raw_buffer_store_b128(nw, vo, (int)((uint32_t)((4 * prow + n) * H) * 2u + colq), 0, 2);
            }
            // the coefficients of step i + 1 (loaded with step i's streams) for the next iteration
            if (i + 1 >= 1) {
                store_coef(i + 1, cf);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int row = prow + 16 * k;
                *reinterpret_cast<u32x4 *>(slot + (row >> 2) * kTokB + (row & 3) * kRowB + piece * 16) = cur[k];
            }
        }
        // A4: the loads of step i + 2
        if constexpr (kPost) {
            load_coef(i + 3, cf);
            xcur = load_x(i + 2);
        }
        load_step(i + 2, cur);
        lds_barrier(); // B1: slot i, the pre weights of step X - 1 and the coefficients are in LDS

        // ---- phase B
        if (tid == 0) {
            badf[(i - 1) & 1] = 0; // every thread read it before B1
        }
        float holdp[kHC];
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            holdp[k] = prel[prow * kHC + k];
        }
        // B1': the records of step X (loaded last iteration): check and sum over the slices
        int *bf = badf + (i & 1);
        take_recs(X, ru, rd, bf);
        // B2': projection of step i (this wave's 32 h, all 4 streams; streams 0, 1 and 2, 3 in
        // two chains per column tile; a step outside the range projects zeros and stores
        // nothing), with the collapse of step X - 1 (y = sum_i pre_i * res_i for this thread's
        // token and piece) between the products
        u32x4 yw;
        float *rw = red + (i & 1) * (W * kQTok * kQRedStride) + w * (kQTok * kQRedStride);
        {
            u32x4 A[kHC];
#pragma unroll
            for (int st = 0; st < kHC; ++st) {
                A[st] = *reinterpret_cast<const u32x4 *>(slot + c * kTokB + st * kRowB + (4 * w + g) * 16);
            }
            f32x4 acc0[2], acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                acc0[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            float sq = 0.0f;
#pragma unroll
            for (int st = 0; st < kHC; ++st) {
                const int u = st >> 1;
                const bf16x8 Ab = __builtin_bit_cast(bf16x8, A[st]);
#pragma unroll
                for (int t3 = 0; t3 < 3; ++t3) {
                    acc0[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ab, __builtin_bit_cast(bf16x8, b0[st][t3]), acc0[u], 0, 0, 0);
                }
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ab, __builtin_bit_cast(bf16x8, b1[st][0]), acc1, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ab, __builtin_bit_cast(bf16x8, b1[st][1]), acc1, 0, 0, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // a scalar copy first: hipcc (clang 22) miscompiles __builtin_bit_cast applied
                    // directly to an ext_vector element (it reads element 0 for every k)
                    const uint32_t wk = A[st][k];
                    const bf16x2 pr = __builtin_bit_cast(bf16x2, wk);
                    sq = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, sq, false);
                }
                // one quarter of the collapse (h pair q = st) while these products run
                {
                    const int q = st;
                    float lo = bf16_lo(hold[0][q]) * holdp[0];
                    float hi = bf16_hi(hold[0][q]) * holdp[0];
#pragma unroll
                    for (int o = 1; o < kHC; ++o) {
                        lo = fmaf(bf16_lo(hold[o][q]), holdp[o], lo);
                        hi = fmaf(bf16_hi(hold[o][q]), holdp[o], hi);
                    }
                    yw[q] = pack_bf16x2(lo, hi);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // the token's sum of squares over the 4 lane groups: (g0 + g1) + (g2 + g3)
            sq = rows_sum(sq);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float d0 = acc0[0][k] + acc0[1][k];
                // rows 16..23: hi + lo in column c (one chain), the mid partial from column c + 8
                const float d1 = acc1[k] + dpp_row_ror8(acc1[k]);
                rw[(4 * g + k) * kQRedStride + c] = d0;
                *(c < 8 ? rw + (4 * g + k) * kQRedStride + 16 + c : dummy + lane) = d1;
            }
            rw[c * kQRedStride + kMix] = sq; // the same bits from all 4 lane groups
        }
        {
            const bool xp_in = xp_ok;
            const int t0 = (Xp * kQGroups + x) * kQTok;
            const int ntok = xp_in ? min(kQTok, T - t0) : 0;
            const __amdgpu_buffer_rsrc_t vy =
                buf_view_uniform(a.y + (size_t)(ntok > 0 ? t0 : 0) * H, (uint32_t)((size_t)ntok * H * sizeof(uint16_t)));
            __builtin_amdgcn_raw_buffer_store_b128(yw, vy, (int)((uint32_t)(prow * H) * 2u + colq), 0, 2);
        }
        // B3': the record of step i - 1: this thread's chunk(s), three slice sums over the waves
        // each (waves holding no chunk skip it)
        if (w * kWave < kQChunks) {
            const float *rp = red + ((i - 1) & 1) * (W * kQTok * kQRedStride);
            const uint32_t tag = coop_tag(key, (i - 1) * kQGroups + x);
            const uint32_t q = (uint32_t)qim1;
#pragma unroll
            for (int rs = 0; rs < kRS; ++rs) {
                float v[3];
#pragma unroll
                for (int e = 0; e < 3; ++e) {
                    float acc = 0.0f;
#pragma unroll
                    for (int ww = 0; ww < W; ++ww) {
                        acc += rp[ww * (kQTok * kQRedStride) + rc_off[rs][e]];
                    }
                    v[e] = (rc_valid[rs] >> e) & 1 ? acc : 0.0f;
                }
                const uint32_t o = pm1_ok && rc_base[rs] != kOob ? rc_base[rs] + q * rc_qstride[rs] : kOob;
                const u32x4 chunk = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), tag};
                __builtin_amdgcn_raw_buffer_store_b128(chunk, vrec, (int)o, 0, 0);
            }
        }
        // B4': the records of step X + 1
        load_recs(X + 1, qx1, ru, rd);
        // B5': step X's slot into registers for the next iteration's collapse
        {
            const unsigned char *cs = ring + rx * kSlotB + prow * kTokB + piece * 16;
#pragma unroll
            for (int st = 0; st < kHC; ++st) {
                hold[st] = *reinterpret_cast<const u32x4 *>(cs + st * kRowB);
            }
        }
        lds_barrier(); // B2: partial sums of step i, the slice sums of step X, slot X read
    };

    // Every trip of the loop issues the same memory operations (empty views stand for steps
    // outside the range), so that the compiler's in-order wait counts stay exact.
    u32x4 bufA[4], bufB[4], hold[kHC];
    u32x4 xA = {0u, 0u, 0u, 0u}, xB = {0u, 0u, 0u, 0u};
    float cfA[kCf], cfB[kCf];
#pragma unroll
    for (int k = 0; k < kCf; ++k) {
        cfA[k] = 0.0f;
        cfB[k] = 0.0f;
    }
    u32x4 ru[kUR], rd[kDR];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bufA[k] = u32x4{0u, 0u, 0u, 0u};
        bufB[k] = u32x4{0u, 0u, 0u, 0u};
        hold[k] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < kUR; ++r) {
        ru[r] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < kDR; ++r) {
        rd[r] = u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 2) {
        badf[tid] = 0;
    }
    if (tid < kQTok * kHC) {
        prel[tid] = 0.0f;
    }
    if constexpr (kPost) {
        // the coefficients of step 0 (the loop stages those of step j + 1 in iteration j)
        float c0[kCf];
        load_coef(0, c0);
        store_coef(0, c0);
    }
    __syncthreads();
    // The loads of steps 0 and 1 (what iterations -2 and -1 would issue: every other memory
    // operation of those iterations is out of range) go out around the weights, so that their
    // latency and the weights' overlap; the loop starts at step 0.  Step 1 goes last: the
    // first projection waits for step 0 and the weights only.
    if constexpr (kPost) {
        load_coef(1, cfA);
        xA = load_x(0);
    }
    load_step(0, bufA);
    {
        const __amdgpu_buffer_rsrc_t vw =
            buf_view_uniform(a.hc_fn, (uint32_t)((size_t)a.fn_rows * kHC * H * sizeof(WT)));
        const int h = hb * 32 + 8 * g;
        const bool hok = hb < a.nhb && h < H;
        const WT *wt = reinterpret_cast<const WT *>(a.hc_fn);
        const int r1 = 16 + (c & 7);
        float v0[kHC][8], v1[kHC][8];
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
            const uint32_t i0 = hok ? (uint32_t)c * kHC * H + (uint32_t)i * H + h : kOob / 4;
            const uint32_t i1 = hok ? (uint32_t)r1 * kHC * H + (uint32_t)i * H + h : kOob / 4;
            if (a.wvec) {
                // 16-byte loads: the four lanes g of a row share one 128-byte line, where
                // element loads touch a line per lane and instruction
                load_w8(wt, i0, vw, v0[i]);
                load_w8(wt, i1, vw, v1[i]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v0[i][e] = weight_elem(wt, i0 + e, vw);
                    v1[i][e] = weight_elem(wt, i1 + e, vw);
                }
            }
        }
        if constexpr (kPost) {
            load_coef(2, cfB);
            xB = load_x(1);
        }
        load_step(1, bufB);
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
            split3x8(v0[i], b0[i][0], b0[i][1], b0[i][2]);
            u32x4 hi, mid, lo;
            split3x8(v1[i], hi, mid, lo);
            b1[i][0] = c < 8 ? hi : mid;
            b1[i][1] = c < 8 ? lo : u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int iend = nst + L + 1; // the last collapse (of step nst - 1) is in iteration nst + L
    int ri = 0, qi = 0;           // step 0
    for (int i = 0; i < iend; i += 2) {
        iteration(i, ri, qi, bufA, xA, cfA, ru, rd, hold);
        ri = wrap(ri + 1, R);
        qi = wrap(qi + 1, RR);
        iteration(i + 1, ri, qi, bufB, xB, cfB, ru, rd, hold);
        ri = wrap(ri + 1, R);
        qi = wrap(qi + 1, RR);
    }
    if (a.head) {
        return;
    }
    // Post weights and the Sinkhorn of this workgroup's tokens: token td of the steps j with
    // j mod 2 == s / 16, whose raw comb logits and post pre-activations the loop stored.
    // Row r of wave w takes the ((round * W + w) * 4 + r)-th of them and, in the same lanes,
    // the one 4W further on (two matrices per row: one round where 32 tokens would take two).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int e = lane & 15;
    const int nmine = (nst - (s >> 4) + 1) / 2;
    for (int base = 0; base < nmine; base += 8 * W) {
        float Lg[2], zp[2];
        float *pc[2], *pp[2];
        bool ok[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int m = base + 4 * W * u + 4 * w + (lane >> 4);
            const int j = 2 * m + (s >> 4);
            const int t = (j * kQGroups + x) * kQTok + td;
            ok[u] = m < nmine && t < T;
            pc[u] = a.comb + (size_t)(ok[u] ? t : 0) * kHC * kHC + e;
            pp[u] = a.post + (size_t)(ok[u] ? t : 0) * kHC + (e & 3);
            // device-scope loads: the auxiliary wave stored these, and they must not come from a stale L1 line
            Lg[u] = ok[u] ? __hip_atomic_load(pc[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
            zp[u] = ok[u] && e < kHC ? __hip_atomic_load(pp[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
        }
        float P[2];
        sinkhorn_row16x2(Lg[0], Lg[1], a.iters, a.sk_eps, P[0], P[1]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float pv = sigmoidf_fast(zp[u]) * a.post_mult;
            if (ok[u]) {
                *pc[u] = P[u];
                if (e < kHC) {
                    *pp[u] = pv;
                }
            }
        }
    }
}

int coop_waves(int64_t H) { return (int)((((H + 31) / 32) + kQSlices - 1) / kQSlices); }

struct CoopCfg {
    int W, L, R, RR;
    size_t lds;
};

CoopCfg coop_config(int64_t H)
{
    CoopCfg k{};
    k.W = coop_waves(H);
    const size_t slot = (size_t)kQTok * (256 * k.W + 16);
    // the waves' partials, sums, dsum, prel, flags, dummy, and the post-map's coefficients
    const size_t scratch = (size_t)2 * k.W * kQTok * red_stride(k.W) * 4 + (96 + 32 + 64 + 4 + 64 + 2 * kCoefVals) * 4;
    // a record of step j is stored in iteration j + 1 and loaded in iteration j + L - 1, so the
    // lag must be at least 3; a ring of L + 1 slots fits at every W (161,296 bytes at W = 8)
    k.L = 3;
    k.R = k.L + 1;
    k.RR = 2 * k.L + 2;
    k.lds = (size_t)k.R * slot + scratch;
    return k;
}

int g_coop_device_ok[64]; // per device: 0 unknown, 1 usable (256 CUs on gfx950), 2 not

bool coop_device_ok()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        return false;
    }
    if (g_coop_device_ok[dev] == 0) {
        int cus = 0;
        hipDeviceProp_t prop;
        const bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                        hipGetDeviceProperties(&prop, dev) == hipSuccess && cus == kQGroups * kQSlices &&
                        strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_coop_device_ok[dev] = ok ? 1 : 2;
    }
    return g_coop_device_ok[dev] == 1;
}

template <int W, typename WT, bool kPost>
hipError_t launch_coop_w(const CoopArgs &a, size_t lds, hipStream_t stream)
{
    // the dynamic-LDS limit is a per-device attribute: raised once on each device
    static std::atomic<bool> attr_set[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        return e != hipSuccess ? e : hipErrorInvalidDevice;
    }
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute((const void *)pre_coop_kernel<W, WT, kPost>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
        if (e != hipSuccess) {
            return e;
        }
        attr_set[dev].store(true, std::memory_order_release);
    }
    pre_coop_kernel<W, WT, kPost><<<dim3(kQGroups * kQSlices), dim3(W * 64), lds, stream>>>(a);
    return hipGetLastError();
}

template <typename WT, bool kPost>
hipError_t launch_coop_t(const CoopArgs &a, int W, size_t lds, hipStream_t stream)
{
    switch (W) {
    case 2:
        return launch_coop_w<2, WT, kPost>(a, lds, stream);
    case 3:
        return launch_coop_w<3, WT, kPost>(a, lds, stream);
    case 4:
        return launch_coop_w<4, WT, kPost>(a, lds, stream);
    case 5:
        return launch_coop_w<5, WT, kPost>(a, lds, stream);
    case 6:
        return launch_coop_w<6, WT, kPost>(a, lds, stream);
    case 7:
        return launch_coop_w<7, WT, kPost>(a, lds, stream);
    case 8:
        return launch_coop_w<8, WT, kPost>(a, lds, stream);
    default:
        return hipErrorInvalidValue;
    }
}

CoopArgs coop_args(const CoopCfg &k, const uint16_t *res, const void *hc_fn, int fn_rows, const float *hc_scale,
                   const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps, float sinkhorn_eps,
                   float post_mult, int iters, bool head, uint16_t *y, float *post, float *comb, float *pre,
                   void *workspace)
{
    CoopArgs a{};
    a.res = res;
    a.hc_fn = hc_fn;
    a.wvec = ((uintptr_t)hc_fn & 15u) == 0;
    a.hc_scale = hc_scale;
    a.hc_base = hc_base;
    a.T = (int)T;
    a.H = (int)H;
    a.nhb = (int)((H + 31) / 32);
    a.fn_rows = fn_rows;
    a.L = k.L;
    a.R = k.R;
    a.RR = k.RR;
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
    a.rec = reinterpret_cast<u32x4 *>(workspace);
    a.rec_bytes = (uint32_t)pre_coop_workspace_bytes(H);
    a.max_retry = g_max_retry.load(std::memory_order_relaxed);
    a.tag_skew = g_tag_skew.load(std::memory_order_relaxed);
    return a;
}

} // namespace

size_t pre_coop_workspace_bytes(int64_t H)
{
    const CoopCfg k = coop_config(H);
    return (size_t)kQGroups * k.RR * kQSlices * kQChunks * sizeof(u32x4);
}

bool pre_coop_shape_ok(int64_t T, int64_t H)
{
    if (T < kCoopMinTokens || H > (int64_t)kQSlices * 8 * 32) {
        return false;
    }
    const int W = coop_waves(H);
    return W >= 2 && W <= 8;
}

bool pre_coop_usable(int64_t T, int64_t H, bool vec8) { return vec8 && pre_coop_shape_ok(T, H) && coop_device_ok(); }

hipError_t launch_pre_coop(const uint16_t *res, const void *hc_fn, bool fn_bf16, int fn_rows, const float *hc_scale,
                           const float *hc_base, int64_t T, int64_t H, float rms_eps, float pre_eps,
                           float sinkhorn_eps, float post_mult, int iters, bool head, uint16_t *y, float *post,
                           float *comb, float *pre, void *workspace, hipStream_t stream)
{
    const CoopCfg k = coop_config(H);
    const CoopArgs a = coop_args(k, res, hc_fn, fn_rows, hc_scale, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps,
                                 post_mult, iters, head, y, post, comb, pre, workspace);
    return fn_bf16 ? launch_coop_t<uint16_t, false>(a, k.W, k.lds, stream)
                   : launch_coop_t<float, false>(a, k.W, k.lds, stream);
}

bool exchange_device_ok() { return coop_device_ok(); }
int exchange_max_retry() { return g_max_retry.load(std::memory_order_relaxed); }
uint32_t exchange_tag_skew() { return g_tag_skew.load(std::memory_order_relaxed); }

void set_exchange_test_hooks(int max_retry, uint32_t tag_skew)
{
    g_max_retry.store(max_retry < 0 ? kQMaxRetry : max_retry, std::memory_order_relaxed);
    g_tag_skew.store(tag_skew, std::memory_order_relaxed);
}

hipError_t launch_post_pre_coop(const uint16_t *x, const uint16_t *res, const float *post_in, const float *comb_in,
                                const float *hc_fn, const float *hc_scale, const float *hc_base, int64_t T, int64_t H,
                                float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult, int iters,
                                uint16_t *out, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                                hipStream_t stream)
{
    const CoopCfg k = coop_config(H);
    CoopArgs a = coop_args(k, res, hc_fn, kMix, hc_scale, hc_base, T, H, rms_eps, pre_eps, sinkhorn_eps, post_mult,
                           iters, false, y, post, comb, pre, workspace);
    a.x = x;
    a.post_in = post_in;
    a.comb_in = comb_in;
    a.out = out;
    return launch_coop_t<float, true>(a, k.W, k.lds, stream);
}

} // namespace mhc
