// mhc_pre.hip -- the mHC pre-map on gfx950: the two-pass form and the dispatch.
//
// ("FlashInfer mHC 模块深度解析", sections 3.4 and 5.2; metrale
// hyper_connection_dispatch.rs, hc_pre_site; metrale glm5next_mhc.rs, the
// hc_mix / hc_finish split.)
//
// launch_pre takes the one-read form (mhc_pre_coop.hip) when the shape and the
// device allow it: 16-byte rows, 1024 < H <= 8192, T >= 1024, a 256-CU gfx950.
// Everything else runs the two-pass form here, four kernels on one stream:
//
//  1. pre_prep_kernel -- splits every fp32 weight of hc_fn exactly into three
//     bf16 terms hi + mid + lo (successive truncations: 8 + 8 + 8 significant
//     bits) and stores them in the order of the MFMA B operand, so the
//     projection loop issues only 16-byte loads and MFMAs.  Three bf16
//     products accumulated in fp32 reproduce the fp32 weight without rounding
//     it.
//  2. pre_proj_stream_kernel -- the 24 x 4H projection and the sum of squares.  A
//     workgroup owns a 128-wide slice of H across all 4 streams and a range of
//     tokens, walked 32 tokens at a time through an LDS tile (whole-row loads,
//     the next step in flight): the bf16 streams feed v_mfma_f32_16x16x32_bf16
//     unchanged, the sum of squares rides on v_dot2_f32_bf16 from the same
//     registers, and each step writes one 25-float partial record per token.
//     (pre_proj_kernel, one 64-token tile per workgroup, serves H % 8 != 0.)
//  3. pre_mixsum_kernel -- sums every record field of every token over the
//     slices in a fixed order, so the result does not depend on timing.
//  4. pre_collapse_kernel -- one wavefront per (token, 512-wide H tile): rstd
//     and the pre weights from the token's sums (wave-uniform, in SGPRs), then
//     y = sum_i pre_i * res_i with 16-byte loads.  The wavefront of each
//     token's first tile also computes post and the 4x4 Sinkhorn of comb.
//
// The two-pass form reads the streams twice (passes 2 and 4).
#include "mhc_device.h"
#include "mhc_internal.h"

#include <algorithm>
#include <type_traits>

namespace mhc {

namespace {

constexpr int kPWaves = 4;
constexpr int kPBlock = kPWaves * kWave;
constexpr int kPTok = 64;        // tokens per tile
constexpr int kPMT = kPTok / 16; // MFMA row tiles per wave
constexpr int kPHB = 32;         // h per block: 4 lane groups x 8
constexpr int kPNHB = 1;         // blocks per wave
constexpr int kPSliceH = kPWaves * kPNHB * kPHB;
constexpr int kRec = kMix + 1;                    // partial record fields: 24 dots + sum of squares
constexpr int kFragPerHbStream = 3 * 64 + 3 * 32; // hi/mid/lo of column tile 0 (64 lanes) and 1 (32 lanes)

constexpr int kColBlock = 256;
constexpr int kColWaves = kColBlock / kWave;
constexpr int kColVecTile = kWave * 8;

// The record field of projection column `col`: the 4 pre logits, then the sum
// of squares, then post and comb.  Records are field-major ([25][64]) so one
// field of the 64 tokens is 256 contiguous bytes.
constexpr int kFSq = kHC;
__device__ __forceinline__ int field_of_col(int col) { return col < kHC ? col : col + 1; }

// One thread per (h block, stream, operand slot).  Slot < 64: column tile 0,
// MFMA lane = slot (weight row = slot % 16).  Slot >= 64: column tile 1, rows
// 16..23 only; entry g*8 + c stands for MFMA lane 16g + c (c < 8).
// Weight rows at or past `rows` are zero (the weighted head has 4 rows).  bf16
// weights widen exactly to fp32, so their mid and lo terms come out zero.
__device__ __forceinline__ float weight_at(const float *w, size_t i) { return w[i]; }
__device__ __forceinline__ float weight_at(const uint16_t *w, size_t i) { return bf16_to_f32(w[i]); }

template <typename W>
__global__ __launch_bounds__(256) void pre_prep_kernel(const W *__restrict__ hc_fn, int H, int nhb, int rows,
                                                       u32x4 *__restrict__ frag)
{
    const int gid = blockIdx.x * 256 + threadIdx.x;
    constexpr int slots = kFragPerHbStream / 3; // 96
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
    const int h = hb * kPHB + g * 8;
    float v[8];
    const size_t base = (size_t)r * kHC * H + (size_t)i * H + h;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[j] = (r < rows && h + j < H) ? weight_at(hc_fn, base + j) : 0.0f;
    }
    u32x4 ph, pm, pl;
    split3x8(v, ph, pm, pl);
    u32x4 *dst = frag + (size_t)hbi * kFragPerHbStream;
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

struct ProjArgs {
    const uint16_t *res;
    const u32x4 *frag;
    int T, H, nhb, S;
    float *rec; // [tiles][S][25][64]
};

// MFMA operand layout (16x16x32 bf16): lane l holds row/column l % 16 and the 8
// k-values of lane group g = l / 16; result register q of lane l is row 4g + q,
// column l % 16.  A k-step here is one stream i and 32 consecutive h (lane group
// g takes h = 32*hb + 8g .. +8), identically for A (tokens) and B (weights).
// This one-tile-per-workgroup form serves H % 8 != 0 (element loads); for H % 8 == 0
// pre_proj_stream_kernel below does the same work.
__global__ __launch_bounds__(kPBlock, 2) void pre_proj_kernel(ProjArgs a)
{
    __shared__ float red[kPWaves][kPTok][kMix];
    __shared__ float sqp[kPWaves][4][kPTok];

    const int tile = blockIdx.x;
    const int slice = blockIdx.y;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & (kWave - 1);
    const int g = lane >> 4;
    const int c = lane & 15;
    const int S = a.S;
    const int H = a.H;
    const int t0 = tile * kPTok;
    const int ntok = min(kPTok, a.T - t0);

    // ---------------- load the slice (elements past T or H read as zero)
    u32x4 d[kPNHB][kPMT][kHC];
#pragma unroll
    for (int b = 0; b < kPNHB; ++b) {
        const int hb = (slice * kPNHB + b) * kPWaves + w;
        const int h = hb * kPHB + g * 8;
#pragma unroll
        for (int m = 0; m < kPMT; ++m) {
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                const int row = (m * 16 + c) * kHC + i;
                {
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (m * 16 + c < ntok) {
                        const uint16_t *p = a.res + ((size_t)t0 * kHC + row) * H + h;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint32_t lo = (h + 2 * q < H) ? (uint32_t)p[2 * q] : 0u;
                            const uint32_t hi = (h + 2 * q + 1 < H) ? (uint32_t)p[2 * q + 1] : 0u;
                            v[q] = lo | (hi << 16);
                        }
                    }
                    d[b][m][i] = v;
                }
            }
        }
    }

    // ---------------- project: 24 weight rows (hi/mid/lo) x 64 tokens
    f32x4 acc[kPMT][2];
#pragma unroll
    for (int m = 0; m < kPMT; ++m) {
        acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int b = 0; b < kPNHB; ++b) {
        const int hb = (slice * kPNHB + b) * kPWaves + w;
        if (hb < a.nhb) { // wave-uniform
            // All weight fragments of the block are requested before the first MFMA,
            // so their L2 latency overlaps with the stream loads above.
            const u32x4 *fp = a.frag + (size_t)hb * kHC * kFragPerHbStream;
            u32x4 b0[kHC][3], b1[kHC][3];
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    b0[i][s] = fp[i * kFragPerHbStream + s * 64 + lane];
                    b1[i][s] = fp[i * kFragPerHbStream + 192 + s * 32 + ((g * 8 + c) & 31)];
                }
            }
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    const bf16x8 B0 = __builtin_bit_cast(bf16x8, b0[i][s]);
                    // lanes with c >= 8 stand for weight rows >= 24: zero
                    const bf16x8 B1 = __builtin_bit_cast(bf16x8, c < 8 ? b1[i][s] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
                    for (int m = 0; m < kPMT; ++m) {
                        const bf16x8 A = __builtin_bit_cast(bf16x8, d[b][m][i]);
                        acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B0, acc[m][0], 0, 0, 0);
                        acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B1, acc[m][1], 0, 0, 0);
                    }
                }
            }
        }
    }
    float sq[kPMT];
#pragma unroll
    for (int m = 0; m < kPMT; ++m) {
        sq[m] = 0.0f;
#pragma unroll
        for (int b = 0; b < kPNHB; ++b) {
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // Copy to a scalar first: hipcc (clang 22) miscompiles __builtin_bit_cast
                    // applied directly to an ext_vector element (it reads element 0 for every k).
                    const uint32_t wk = d[b][m][i][k];
                    const bf16x2 pr = __builtin_bit_cast(bf16x2, wk);
                    sq[m] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, sq[m], false);
                }
            }
        }
    }

    // ---------------- workgroup reduction -> this slice's partial record
#pragma unroll
    for (int m = 0; m < kPMT; ++m) {
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
    float *rec = a.rec + ((size_t)tile * S + slice) * (kRec * kPTok);
    const int tok = tid & (kPTok - 1);
    for (int col = tid >> 6; col < kMix; col += kPWaves) {
        float v = red[0][tok][col];
#pragma unroll
        for (int ww = 1; ww < kPWaves; ++ww) {
            v += red[ww][tok][col];
        }
        rec[field_of_col(col) * kPTok + tok] = v;
    }
    if (tid < kPTok) {
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                v += sqp[ww][gg][tid];
            }
        }
        rec[kFSq * kPTok + tid] = v;
    }
}

// Streaming form of the projection (H % 8 == 0).  A workgroup owns one 128-wide
// slice and a range of tokens: it loads the slice's weight fragments once, keeps them
// in VGPRs, and walks the range in 32-token steps.  A step's streams come in with
// whole 256-byte row pieces (row = token * 4 + stream) into an LDS tile, whose 16-byte
// pieces are XOR-swizzled by the token so that the MFMA operand reads (16 tokens of one
// stream, one piece each) fall on distinct banks.  The next step's loads are in flight
// in registers while the current step is multiplied and reduced, across LDS-only
// barriers.  The products, their order and the reduction order are those of
// pre_proj_kernel, so the records are bit-identical to its.
constexpr int kPSTok = 32;                       // tokens per step
constexpr int kPSMT = kPSTok / 16;               // MFMA row tiles per step
constexpr int kPSRowB = kPSliceH * 2;            // 256 bytes per tile row
constexpr int kPSRows = kPSTok * kHC;            // 128 rows per step
constexpr int kPSLoads = kPSRows / (kPBlock / 16); // row pieces per thread per step (8)
constexpr int kPSTargetBlocks = 512;             // one round of two workgroups per CU
// Row stride (floats) of the per-wave partial dots in LDS.  36 = 4 (mod 16): a write of
// lanes (g, c) at token 4g + k, column c lands on 64 distinct banks, and the reduction's
// reads of 32 tokens of one column meet at most two to a bank.
constexpr int kPSRedStride = 36;
// With <dy, res_i> each lane also leaves its 4 lane-group partials (columns 24 + 4i + g):
// 44 = 12 (mod 16) keeps those writes, the dot writes and the reads as conflict-free.
constexpr int kPSRedStrideDy = 44;
template <bool kDy> struct PSRed {
    static constexpr int stride = kDy ? kPSRedStrideDy : kPSRedStride;
};

struct ProjStreamArgs {
    const uint16_t *res;
    const uint16_t *dy; // the reverse's recompute: the layer input's gradient [T][H], else null
    const u32x4 *frag;
    int T, H, nhb, S, tok_per_range;
    float *rec; // [64-token tiles][S][nrec][64]
    uint32_t rec_bytes;
};
// Record fields: 24 dots + the sum of squares; with dy also <dy, res_i> at 25 .. 28.
constexpr int kRecDy = kRec + kHC;
constexpr int kFDy = kRec;

__device__ __forceinline__ int pstile_at(int row, int piece)
{
    return row * kPSRowB + ((piece ^ ((row >> 2) & 15)) << 4);
}

// Thread tid moves piece tid & 15 of rows (tid >> 4) + 16k of the step at t0.  A step
// past the range gets an empty view: its loads read zero and touch no memory, so every
// step issues the same loads and the wait counts stay exact across the loop.
__device__ __forceinline__ void pre_stream_load(const ProjStreamArgs &a, int t0, int te, int tid, uint32_t colq,
                                                u32x4 (&d)[kPSLoads])
{
    const int H = a.H;
    const int ntok = max(0, min(kPSTok, te - t0));
    const __amdgpu_buffer_rsrc_t v =
        buf_view_uniform(a.res + (size_t)t0 * kHC * H, (uint32_t)((size_t)ntok * kHC * H * sizeof(uint16_t)));
#pragma unroll
    for (int k = 0; k < kPSLoads; ++k) {
        const int row = (tid >> 4) + 16 * k;
        d[k] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)((uint32_t)(row * H) * 2u + colq), 0, 0));
    }
}

// dy of the step at t0 for this slice: 32 rows (tokens) of 16 pieces; thread tid moves
// piece tid & 15 of rows (tid >> 4) + 16k, k < 2 (empty view past the range).
constexpr int kPSDyLoads = kPSTok / (kPBlock / 16);
__device__ __forceinline__ void pre_stream_load_dy(const ProjStreamArgs &a, int t0, int te, int tid, uint32_t colq,
                                                   u32x4 (&d)[kPSDyLoads])
{
    const int H = a.H;
    const int ntok = max(0, min(kPSTok, te - t0));
    const __amdgpu_buffer_rsrc_t v =
        buf_view_uniform(a.dy + (size_t)t0 * H, (uint32_t)((size_t)ntok * H * sizeof(uint16_t)));
#pragma unroll
    for (int k = 0; k < kPSDyLoads; ++k) {
        const int row = (tid >> 4) + 16 * k;
        d[k] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)((uint32_t)(row * H) * 2u + colq), 0, 0));
    }
}

// Byte offset of piece p of dy row (token) r in its LDS tile: the same swizzle by token.
__device__ __forceinline__ int psdy_at(int row, int piece) { return row * kPSRowB + ((piece ^ (row & 15)) << 4); }

struct PreStreamCtx {
    int tid, w, lane, g, c, slice, S, te;
    uint32_t colq;
    __amdgpu_buffer_rsrc_t vrec; // the chunk's records (under 2 GiB)
};

// One 32-token step at t0 (its streams, and with kDy its dy, in the LDS tiles):
// products, sum of squares (and <dy, res_i>), and the workgroup reduction into the
// records.  After the second barrier the tiles take step t0 + 32 from the registers,
// which then load step t0 + 64.
template <bool kDy>
__device__ __forceinline__ void pre_stream_step(const ProjStreamArgs &a, const PreStreamCtx &x, int tu,
                                                unsigned char *tile, unsigned char *dyt,
                                                float (*red)[kPSTok][PSRed<kDy>::stride], float (*sqp)[kPSTok][4],
                                                const u32x4 (&b0)[kHC][3], const u32x4 (&b1)[kHC][3],
                                                u32x4 (&ld)[kPSLoads], u32x4 (&ldy)[kPSDyLoads])
{
    const int w = x.w, g = x.g, c = x.c, tid = x.tid;
    lds_barrier(); // the step's streams are in LDS
    f32x4 acc[kPSMT][2];
    float sq[kPSMT];
#pragma unroll
    for (int m = 0; m < kPSMT; ++m) {
        acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        sq[m] = 0.0f;
    }
    // this lane's 8 h of dy for its two tokens (the same h as its stream operands)
    u32x4 gy[kPSMT];
    float pd[kPSMT][kHC];
    if (kDy) {
#pragma unroll
        for (int m = 0; m < kPSMT; ++m) {
            gy[m] = *reinterpret_cast<const u32x4 *>(dyt + psdy_at(m * 16 + c, 4 * w + g));
        }
    }
    // stream by stream (the operands of one stream read from LDS when needed); each
    // token's sum of squares still runs stream-major, as in pre_proj_kernel
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        u32x4 dc[kPSMT];
#pragma unroll
        for (int m = 0; m < kPSMT; ++m) {
            dc[m] = *reinterpret_cast<const u32x4 *>(tile + pstile_at((m * 16 + c) * kHC + i, 4 * w + g));
        }
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const bf16x8 B0 = __builtin_bit_cast(bf16x8, b0[i][s]);
            const bf16x8 B1 = __builtin_bit_cast(bf16x8, b1[i][s]);
#pragma unroll
            for (int m = 0; m < kPSMT; ++m) {
                const bf16x8 A = __builtin_bit_cast(bf16x8, dc[m]);
                acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B0, acc[m][0], 0, 0, 0);
                acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B1, acc[m][1], 0, 0, 0);
            }
        }
#pragma unroll
        for (int m = 0; m < kPSMT; ++m) {
            if (kDy) {
                pd[m][i] = 0.0f;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // a scalar copy first (see pre_proj_kernel)
                const uint32_t wk = dc[m][k];
                const bf16x2 pr = __builtin_bit_cast(bf16x2, wk);
                sq[m] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, sq[m], false);
                if (kDy) {
                    const uint32_t yk = gy[m][k];
                    pd[m][i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, yk), pr, pd[m][i], false);
                }
            }
        }
    }
    // ---- workgroup reduction -> the slice's partial records of these 32 tokens
#pragma unroll
    for (int m = 0; m < kPSMT; ++m) {
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
        sqp[w][m * 16 + c][g] = sq[m];
        if (kDy) {
            // this lane's partial of token m*16 + c over its 8 h; the 4 lane groups are
            // summed with the 4 waves below
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
                red[w][m * 16 + c][kMix + 4 * i + g] = pd[m][i];
            }
        }
    }
    lds_barrier(); // the partial dots are in LDS; every wave is done with the tiles
    // step t0 + 32 to the tiles (zeros past the range), step t0 + 64 into the registers
#pragma unroll
    for (int k = 0; k < kPSLoads; ++k) {
        *reinterpret_cast<u32x4 *>(tile + pstile_at((tid >> 4) + 16 * k, tid & 15)) = ld[k];
    }
    if (kDy) {
#pragma unroll
        for (int k = 0; k < kPSDyLoads; ++k) {
            *reinterpret_cast<u32x4 *>(dyt + psdy_at((tid >> 4) + 16 * k, tid & 15)) = ldy[k];
        }
    }
    pre_stream_load(a, tu + 2 * kPSTok, x.te, tid, x.colq, ld);
    if (kDy) {
        pre_stream_load_dy(a, tu + 2 * kPSTok, x.te, tid, x.colq, ldy);
    }
    // records are per 64-token tile; t0 is a multiple of 32, so these are entries
    // (t0 & 63) .. + 31 of tile t0 >> 6.  Every thread issues the same stores (a lane
    // with nothing to store gets an offset past the view: the store is dropped).
    constexpr int nrec = kDy ? kRecDy : kRec;
    const uint32_t rec0 = (uint32_t)((((size_t)(tu >> 6) * x.S + x.slice) * (nrec * kPTok) + (tu & (kPTok - 1))) * 4);
    const int tok = tid & (kPSTok - 1);
#pragma unroll
    for (int j = 0; j < kMix / (kPBlock / kPSTok); ++j) {
        const int col = (tid >> 5) + j * (kPBlock / kPSTok);
        float v = red[0][tok][col];
#pragma unroll
        for (int ww = 1; ww < kPWaves; ++ww) {
            v += red[ww][tok][col];
        }
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), x.vrec,
                                              (int)(rec0 + (uint32_t)(field_of_col(col) * kPTok + tok) * 4u), 0, 0);
    }
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kPWaves; ++ww) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            v += sqp[ww][tok][gg];
        }
    }
    const uint32_t sqo = tid < kPSTok ? rec0 + (uint32_t)(kFSq * kPTok + tok) * 4u : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), x.vrec, (int)sqo, 0, 0);
    if (kDy) {
        // <dy, res_i> of the slice: threads 0..127 take stream tid >> 5 of token tok,
        // summing wave by wave, lane group by lane group
        const int i = (tid >> 5) & (kHC - 1);
        float u = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                u += red[ww][tok][kMix + 4 * i + gg];
            }
        }
        const uint32_t o = tid < kHC * kPSTok ? rec0 + (uint32_t)((kFDy + i) * kPTok + tok) * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(u), x.vrec, (int)o, 0, 0);
    }
}

template <bool kDy>
__global__ __launch_bounds__(kPBlock, 2) void pre_proj_stream_kernel(ProjStreamArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char tile[kPSRows * kPSRowB];
    __shared__ __attribute__((aligned(16))) unsigned char dyt[kDy ? kPSTok * kPSRowB : 16];
    __shared__ float red[kPWaves][kPSTok][PSRed<kDy>::stride];
    __shared__ float sqp[kPWaves][kPSTok][4];

    PreStreamCtx x;
    x.tid = threadIdx.x;
    x.w = uniform(x.tid >> 6);
    x.lane = x.tid & (kWave - 1);
    x.g = x.lane >> 4;
    x.c = x.lane & 15;
    x.slice = blockIdx.x;
    x.S = a.S;
    const int H = a.H;
    const int tb = blockIdx.y * a.tok_per_range;
    x.te = min(a.T, tb + a.tok_per_range);
    const int hb = x.slice * kPWaves + x.w;
    // this thread's 16-byte piece of each row it moves (past H: loads read zero)
    const int hq = x.slice * kPSliceH + 8 * (x.tid & 15);
    x.colq = hq < H ? (uint32_t)hq * 2u : 0x80000000u;
    x.vrec = buf_view_uniform(a.rec, a.rec_bytes);

    // the weight fragments of this wave's 32 h of the 4 streams; lanes with c >= 8
    // stand for weight rows >= 24 in column tile 1 and hold zero; past H all zero
    u32x4 b0[kHC][3], b1[kHC][3];
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 *fp = a.frag + (size_t)hb * kHC * kFragPerHbStream;
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            b0[i][s] = hb < a.nhb ? fp[i * kFragPerHbStream + s * 64 + x.lane] : z;
            b1[i][s] = hb < a.nhb && x.c < 8 ? fp[i * kFragPerHbStream + 192 + s * 32 + ((x.g * 8 + x.c) & 31)] : z;
        }
    }

    // step t0 in the tiles, step t0 + 32 in flight in registers
    u32x4 ld[kPSLoads], ldy[kPSDyLoads];
    if (tb >= x.te) {
        return;
    }
    pre_stream_load(a, uniform(tb), x.te, x.tid, x.colq, ld);
    if (kDy) {
        pre_stream_load_dy(a, uniform(tb), x.te, x.tid, x.colq, ldy);
    }
#pragma unroll
    for (int k = 0; k < kPSLoads; ++k) {
        *reinterpret_cast<u32x4 *>(tile + pstile_at((x.tid >> 4) + 16 * k, x.tid & 15)) = ld[k];
    }
    if (kDy) {
#pragma unroll
        for (int k = 0; k < kPSDyLoads; ++k) {
            *reinterpret_cast<u32x4 *>(dyt + psdy_at((x.tid >> 4) + 16 * k, x.tid & 15)) = ldy[k];
        }
    }
    pre_stream_load(a, uniform(tb + kPSTok), x.te, x.tid, x.colq, ld);
    if (kDy) {
        pre_stream_load_dy(a, uniform(tb + kPSTok), x.te, x.tid, x.colq, ldy);
    }
    for (int t0 = tb; t0 < x.te; t0 += kPSTok) {
        pre_stream_step<kDy>(a, x, uniform(t0), tile, dyt, red, sqp, b0, b1, ld, ldy);
    }
}

// ---------------------------------------------------------------- post-map fused with the next projection
//
// A post-map whose output feeds the next sublayer's pre-map, and that sublayer's
// projection and sum of squares on the way.  One 256-thread workgroup per (128-wide
// slice of H across the 4 streams, token range), walked in 32-token steps as in
// pre_proj_stream_kernel.  In a step each thread takes two (token, 16-byte piece)
// pairs: it loads x, the four old streams and the token's coefficients, computes the
// four new streams with the arithmetic of post_vec8_kernel (so they are the same bits),
// stores them and writes them to the LDS tile.  The waves then project the tile with the
// next weights and reduce the slice's 24 dots and sum of squares into the projection's
// partial records ([64-token tile][slice][25][64], as pre_proj_stream_kernel writes
// them), which pre_mixsum_kernel sums over the slices.  The next step's loads are in
// flight meanwhile.  out may equal res: each pair's old
// streams are read, by the thread that writes them, before they are written.
struct PostProjArgs {
    const uint16_t *x, *res;
    const float *post, *comb;
    const u32x4 *frag; // the next weights, split by pre_prep_kernel
    int T, H, nhb, S, tok_per_range;
    uint16_t *out;
    float *rec; // [64-token tiles][S][25][64]
    uint32_t rec_bytes;
};

constexpr int kPPPairs = kPSTok * (kPSliceH / 8) / kPBlock; // (token, piece) pairs per thread per step (2)
constexpr int kPPCoef = kHC + kHC * kHC;                     // post (4) and comb (16) of a token
constexpr int kPPCoefPieces = kPSTok * kPPCoef / 4;          // 16-byte pieces per step (160)

// What a thread loads for a step: x and the four old streams of its two pairs (token
// (tid >> 4) + 16k, piece tid & 15), and piece tid of the step's coefficient block
// ([32 tokens][20] fp32; threads past 160 load nothing).
struct PostStepIn {
    u32x4 x[kPPPairs], r[kPPPairs][kHC], cf;
};

// Past the range the views are empty and read zero.
__device__ __forceinline__ void post_proj_load(const PostProjArgs &a, int t0, int te, int tid, uint32_t colq,
                                               PostStepIn &in)
{
    const int H = a.H;
    const int ntok = max(0, min(kPSTok, te - t0));
    const __amdgpu_buffer_rsrc_t vx = buf_view_uniform(a.x + (size_t)t0 * H, (uint32_t)((size_t)ntok * H * 2));
    const __amdgpu_buffer_rsrc_t vr =
        buf_view_uniform(a.res + (size_t)t0 * kHC * H, (uint32_t)((size_t)ntok * kHC * H * 2));
#pragma unroll
    for (int k = 0; k < kPPPairs; ++k) {
        const int tl = (tid >> 4) + 16 * k;
        in.x[k] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(vx, (int)((uint32_t)(tl * H) * 2u + colq), 0, 0));
#pragma unroll
        for (int o = 0; o < kHC; ++o) {
            in.r[k][o] = __builtin_bit_cast(
                u32x4,
                __builtin_amdgcn_raw_buffer_load_b128(vr, (int)((uint32_t)((tl * kHC + o) * H) * 2u + colq), 0, 0));
        }
    }
    // coefficient piece tid: token tid / 5, word 4 (tid % 5) of its 20 (post, then comb)
    const int ct = tid / 5, cq = tid - 5 * (tid / 5);
    const __amdgpu_buffer_rsrc_t vp = buf_view_uniform(a.post + (size_t)t0 * kHC, (uint32_t)(ntok * kHC * 4));
    const __amdgpu_buffer_rsrc_t vc =
        buf_view_uniform(a.comb + (size_t)t0 * kHC * kHC, (uint32_t)(ntok * kHC * kHC * 4));
    const int off = tid < kPPCoefPieces ? (cq == 0 ? ct * 16 : ct * 64 + (cq - 1) * 16) : (int)0x80000000;
    const u32x4 pv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vp, cq == 0 ? off : (int)0x80000000, 0, 0));
    const u32x4 cv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vc, cq != 0 ? off : (int)0x80000000, 0, 0));
    in.cf = cq == 0 ? pv : cv;
}

// The pairs' new streams: stored to `out` and written to the LDS tile (row token*4 + n).
// coef: [32][20] fp32 in LDS.
__device__ __forceinline__ void post_proj_emit(const PostProjArgs &a, int t0, int te, int tid, uint32_t colq,
                                               const PostStepIn &in, const float *coef, unsigned char *tile)
{
    const int H = a.H;
    const int ntok = max(0, min(kPSTok, te - t0));
    const __amdgpu_buffer_rsrc_t vo =
        buf_view_uniform(a.out + (size_t)t0 * kHC * H, (uint32_t)((size_t)ntok * kHC * H * 2));
#pragma unroll
    for (int k = 0; k < kPPPairs; ++k) {
        const int tl = (tid >> 4) + 16 * k;
        const float *cf = coef + tl * kPPCoef; // post[n] at n, comb[o][n] at 4 + 4o + n
        float xf[8], rf[kHC][8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xf[2 * q] = bf16_lo(in.x[k][q]);
            xf[2 * q + 1] = bf16_hi(in.x[k][q]);
#pragma unroll
            for (int o = 0; o < kHC; ++o) {
                rf[o][2 * q] = bf16_lo(in.r[k][o][q]);
                rf[o][2 * q + 1] = bf16_hi(in.r[k][o][q]);
            }
        }
#pragma unroll
        for (int n = 0; n < kHC; ++n) {
            const float pn = cf[n];
            const float c0 = cf[kHC + n], c1 = cf[2 * kHC + n], c2 = cf[3 * kHC + n], c3 = cf[4 * kHC + n];
            u32x4 ow;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int j = 2 * q + e;
                    float acc = xf[j] * pn;
                    acc = fmaf(rf[0][j], c0, acc);
                    acc = fmaf(rf[1][j], c1, acc);
                    acc = fmaf(rf[2][j], c2, acc);
                    acc = fmaf(rf[3][j], c3, acc);
                    v[e] = acc;
                }
                ow[q] = pack_bf16x2(v[0], v[1]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(ow, vo, (int)((uint32_t)((tl * kHC + n) * H) * 2u + colq), 0, 0);
            *reinterpret_cast<u32x4 *>(tile + pstile_at(tl * kHC + n, tid & 15)) = ow;
        }
    }
}

__global__ __launch_bounds__(kPBlock, 2) void post_proj_stream_kernel(PostProjArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char tile[kPSRows * kPSRowB];
    __shared__ __attribute__((aligned(16))) float coef[kPSTok * kPPCoef];
    __shared__ float red[kPWaves][kPSTok][kPSRedStride];
    __shared__ float sqp[kPWaves][kPSTok][4];

    const int tid = threadIdx.x;
    const int w = uniform(tid >> 6);
    const int lane = tid & (kWave - 1);
    const int g = lane >> 4, c = lane & 15;
    const int slice = blockIdx.x;
    const int H = a.H;
    const int tb = blockIdx.y * a.tok_per_range;
    const int te = min(a.T, tb + a.tok_per_range);
    const int hb = slice * kPWaves + w;
    const int hq = slice * kPSliceH + 8 * (tid & 15);
    const uint32_t colq = hq < H ? (uint32_t)hq * 2u : 0x80000000u;

    u32x4 b0[kHC][3], b1[kHC][3];
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 *fp = a.frag + (size_t)hb * kHC * kFragPerHbStream;
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            b0[i][s] = hb < a.nhb ? fp[i * kFragPerHbStream + s * 64 + lane] : z;
            b1[i][s] = hb < a.nhb && c < 8 ? fp[i * kFragPerHbStream + 192 + s * 32 + ((g * 8 + c) & 31)] : z;
        }
    }
    if (tb >= te) {
        return;
    }
    const __amdgpu_buffer_rsrc_t vrec = buf_view_uniform(a.rec, a.rec_bytes);
    PostStepIn in;
    post_proj_load(a, uniform(tb), te, tid, colq, in);
    for (int t0 = tb; t0 < te; t0 += kPSTok) {
        const int tu = uniform(t0);
        // the step's coefficients to LDS (free since the last step's second barrier)
        if (tid < kPPCoefPieces) {
            *reinterpret_cast<u32x4 *>(coef + 4 * tid) = in.cf;
        }
        lds_barrier(); // coefficients in; the tile is free
        // the step's new streams out and into the tile, then the next step's loads
        post_proj_emit(a, tu, te, tid, colq, in, coef, tile);
        post_proj_load(a, tu + kPSTok, te, tid, colq, in);
        lds_barrier(); // the tile holds the step's new streams
        f32x4 acc[kPSMT][2];
        float sq[kPSMT];
#pragma unroll
        for (int m = 0; m < kPSMT; ++m) {
            acc[m][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            sq[m] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
            u32x4 dc[kPSMT];
#pragma unroll
            for (int m = 0; m < kPSMT; ++m) {
                dc[m] = *reinterpret_cast<const u32x4 *>(tile + pstile_at((m * 16 + c) * kHC + i, 4 * w + g));
            }
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                const bf16x8 B0 = __builtin_bit_cast(bf16x8, b0[i][s]);
                const bf16x8 B1 = __builtin_bit_cast(bf16x8, b1[i][s]);
#pragma unroll
                for (int m = 0; m < kPSMT; ++m) {
                    const bf16x8 A = __builtin_bit_cast(bf16x8, dc[m]);
                    acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B0, acc[m][0], 0, 0, 0);
                    acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B1, acc[m][1], 0, 0, 0);
                }
            }
#pragma unroll
            for (int m = 0; m < kPSMT; ++m) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t wk = dc[m][k];
                    const bf16x2 pr = __builtin_bit_cast(bf16x2, wk);
                    sq[m] = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, sq[m], false);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < kPSMT; ++m) {
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
            sqp[w][m * 16 + c][g] = sq[m];
        }
        lds_barrier(); // the partial dots are in LDS; every wave is done with the tile and the coefficients
        // the slice's records of these 32 tokens: entries (tu & 63) .. + 31 of tile tu >> 6
        // (tokens past the end land in the last tile's unused entries)
        const uint32_t rec0 =
            (uint32_t)((((size_t)(tu >> 6) * a.S + slice) * (kRec * kPTok) + (tu & (kPTok - 1))) * 4);
        const int tok = tid & (kPSTok - 1);
#pragma unroll
        for (int j = 0; j < kMix / (kPBlock / kPSTok); ++j) {
            const int col = (tid >> 5) + j * (kPBlock / kPSTok);
            float v = red[0][tok][col];
#pragma unroll
            for (int ww = 1; ww < kPWaves; ++ww) {
                v += red[ww][tok][col];
            }
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), vrec,
                                                  (int)(rec0 + (uint32_t)(field_of_col(col) * kPTok + tok) * 4u), 0, 0);
        }
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kPWaves; ++ww) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                v += sqp[ww][tok][gg];
            }
        }
        const uint32_t sqo = tid < kPSTok ? rec0 + (uint32_t)(kFSq * kPTok + tok) * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), vrec, (int)sqo, 0, 0);
    }
}

// Token ranges of the streaming projection for Tc tokens and S slices.
static void pre_stream_ranges(int Tc, int S, int &ranges, int &tok_per_range)
{
    const int steps = (Tc + kPSTok - 1) / kPSTok;
    int r = kPSTargetBlocks / S;
    r = r < 1 ? 1 : (r > steps ? steps : r);
    tok_per_range = ((steps + r - 1) / r) * kPSTok;
    ranges = (Tc + tok_per_range - 1) / tok_per_range;
}

// Per-token sums of the 25 record fields over the slices.  Block = (tile,
// field): thread (token, slice group k) adds slices k, k+4, ... (independent
// loads in flight), then the four group sums are added in a fixed order.
constexpr int kSumStride = 32; // floats per token in the sums array (25 used)
// Up to this many tokens per chunk the collapse sums the slices' records itself instead of
// a separate slice-sum launch (each of a token's waves redoes 5 sums over the slices).
constexpr int kFuseSumTokens = 64;
__global__ __launch_bounds__(256) void pre_mixsum_kernel(const float *__restrict__ rec, int T, int S, int nrec,
                                                         float *__restrict__ sums, float *__restrict__ dots,
                                                         float *__restrict__ sq)
{
    __shared__ float part[4][kPTok];
    const int tile = blockIdx.x / nrec;
    const int f = blockIdx.x - tile * nrec;
    const int tok = threadIdx.x & (kPTok - 1);
    const int k = threadIdx.x >> 6;
    const float *src = rec + (size_t)tile * S * (nrec * kPTok) + f * kPTok + tok;
    float v = 0.0f;
    int s = k;
    for (; s + 12 < S; s += 16) {
        const float e0 = src[(size_t)s * (nrec * kPTok)];
        const float e1 = src[(size_t)(s + 4) * (nrec * kPTok)];
        const float e2 = src[(size_t)(s + 8) * (nrec * kPTok)];
        const float e3 = src[(size_t)(s + 12) * (nrec * kPTok)];
        v += e0;
        v += e1;
        v += e2;
        v += e3;
    }
    for (; s < S; s += 4) {
        v += src[(size_t)s * (nrec * kPTok)];
    }
    part[k][tok] = v;
    __syncthreads();
    const int t = tile * kPTok + threadIdx.x;
    if (threadIdx.x < kPTok && t < T) {
        const float v = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
        if (dots == nullptr) {
            sums[(size_t)t * kSumStride + f] = v;
        } else if (f == kFSq) { // external form: dot_mix [T][24] and sqrsum [T]
            sq[t] = v;
        } else {
            dots[(size_t)t * kMix + (f < kFSq ? f : f - 1)] = v;
        }
    }
}

struct MixArgs {
    // Per token `stride` floats: the 4 pre dots at 0..3, the post and comb dots from
    // `off_post` on; the sum of squares at kFSq, or in `sq` [T] when that is given.
    // The projection's sums are [T][32] with off_post = 5; external dots [T][24] with
    // off_post = 4 and `sq`.
    const float *sums;
    int stride, off_post;
    const float *sq;
    const float *hc_scale;
    const float *hc_base;
    float k_denom, rms_eps, pre_eps, sk_eps, post_mult;
    int iters;
    int head; // the weighted head: pre weights and y only
    float *post, *comb, *pre_out;
    // Small batches: the projection's partial records ([tiles][S][nrec][64]) instead of
    // `sums`; each token's fields are summed over the S slices where they are used.
    const float *rec;
    int S, nrec;
};

// Fields f0 .. f0 + N - 1 of token t: from the sums, or (m.rec set) summed over the slices'
// records, lane l adding slices l, l + 64, ... in order (all N loads in flight together) and
// then a butterfly over the wave, so every lane holds the same totals.  Called by whole
// waves with a wave-uniform t.
template <int N> __device__ __forceinline__ void mix_fields(const MixArgs &m, int t, int f0, float (&out)[N])
{
    if (m.rec == nullptr) {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            out[k] = m.sums[(size_t)t * m.stride + f0 + k];
        }
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const size_t rs = (size_t)m.nrec * kPTok; // floats per slice record
    const float *p = m.rec + (size_t)(t / kPTok) * m.S * rs + (size_t)f0 * kPTok + (t % kPTok);
    float v[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        v[k] = 0.0f;
    }
    for (int s = lane; s < m.S; s += kWave) {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            v[k] += p[(size_t)s * rs + (size_t)k * kPTok];
        }
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
        out[k] = wave_sum_dpp(v[k]);
    }
}

// The fields of token t a wave needs: the pre dots and the sum of squares (d[0..4]), and
// with kAll (the wave that finishes post and comb) also the post and comb dots (d[5..24]);
// in the records' mode all in one batch of loads.
template <bool kAll> __device__ __forceinline__ void token_fields(const MixArgs &m, int t, float (&d)[kRec])
{
    if (m.rec != nullptr) {
        float v[kAll ? kRec : kHC + 1];
        mix_fields(m, t, 0, v);
#pragma unroll
        for (int k = 0; k < (kAll ? kRec : kHC + 1); ++k) {
            d[k] = v[k];
        }
        return;
    }
    float v[kHC + 1];
    mix_fields(m, t, 0, v); // field kFSq is the sum of squares only when m.sq is null
#pragma unroll
    for (int k = 0; k <= kHC; ++k) {
        d[k] = v[k];
    }
    if (kAll) {
        float w[kMix - kHC];
        mix_fields(m, t, m.off_post, w);
#pragma unroll
        for (int k = 0; k < kMix - kHC; ++k) {
            d[kHC + 1 + k] = w[k];
        }
    }
}

// pre weights of token t from its fields (wave-uniform).
__device__ __forceinline__ void token_pre(const MixArgs &m, int t, const float (&d)[kRec], float *p, float &rstd)
{
    // the supplied sum of squares through a buffer view: a plain ?: between m.sq[t] and
    // d[kFSq] becomes one load from a select of the two addresses, which puts d in scratch
    float S = d[kFSq];
    if (m.sq != nullptr) {
        S = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(buf_view_uniform(m.sq, (uint32_t)(t + 1) * 4u), t * 4, 0, 0));
    }
    rstd = 1.0f / sqrtf(S / m.k_denom + m.rms_eps);
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        p[i] = sigmoidf_fast(fmaf(d[i] * rstd, m.hc_scale[0], m.hc_base[i])) + m.pre_eps;
    }
}

// v where the lane's bit of `mask` is clear, a where it is set: one v_cndmask_b32.  Written
// as one instruction so that a chain of them over a register array stays in registers (the
// compiler turns a chain of ?: on lane-dependent conditions over an array into an indexed
// load from scratch memory).
__device__ __forceinline__ float lane_select(uint64_t mask, float a, float v)
{
    float r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(a), "s"(mask));
    return r;
}
constexpr uint64_t kLane16Mask = 0x0001000100010001ull; // lanes 0, 16, 32, 48
constexpr uint64_t kLane4Mask = 0x1111111111111111ull;  // lanes 0, 4, 8, ..., 60

// post, comb (Sinkhorn) and the optional pre output of token t; d from token_fields<true>.
// Called by a whole wave (all 64 lanes active: the Sinkhorn runs on DPP within 16-lane
// rows, lane e of each row holding entry (e / 4, e % 4); the four rows compute the same
// matrix).  Lanes 0..15 store comb, lanes 0..3 post and the pre output.
__device__ __forceinline__ void token_mix_outputs(const MixArgs &m, int t, const float (&d)[kRec], const float *p,
                                                  float rstd, int lane)
{
    const int e = lane & (kHC * kHC - 1);
    const int i = e & (kHC - 1);
    float pe = p[0];
#pragma unroll
    for (int k = 1; k < kHC; ++k) {
        pe = lane_select(kLane4Mask << k, p[k], pe);
    }
    if (m.head) {
        if (m.pre_out && lane < kHC) {
            m.pre_out[(size_t)t * kHC + lane] = pe;
        }
        return;
    }
    // this lane's comb logit (entry e) and post dot (entry e mod 4), from the wave-uniform fields
    float zc = d[2 * kHC + 1];
#pragma unroll
    for (int k = 1; k < kHC * kHC; ++k) {
        zc = lane_select(kLane16Mask << k, d[2 * kHC + 1 + k], zc);
    }
    float zp = d[kHC + 1];
#pragma unroll
    for (int k = 1; k < kHC; ++k) {
        zp = lane_select(kLane4Mask << k, d[kHC + 1 + k], zp);
    }
    const float post = sigmoidf_fast(fmaf(zp * rstd, m.hc_scale[1], m.hc_base[kHC + i])) * m.post_mult;
    const float P = sinkhorn_row16(fmaf(zc * rstd, m.hc_scale[2], m.hc_base[2 * kHC + e]), m.iters, m.sk_eps);
    if (lane < kHC * kHC) {
        m.comb[(size_t)t * kHC * kHC + lane] = P;
    }
    if (lane < kHC) {
        m.post[(size_t)t * kHC + lane] = post;
        if (m.pre_out) {
            m.pre_out[(size_t)t * kHC + lane] = pe;
        }
    }
}

// A collapse wave's token work: its fields (the first tile's wave all 25, for post and
// comb; the others the pre dots and the sum of squares), then the pre weights.  The two
// kinds of wave are compiled as separate paths (kFirst a template argument), so the field
// array never merges across a branch (such a merge put it in scratch memory).
template <bool kFirst>
__device__ __forceinline__ void token_start(const MixArgs &m, int t, float (&d)[kRec], float *p, float &rstd)
{
    token_fields<kFirst>(m, t, d);
    token_pre(m, t, d, p, rstd);
}

__global__ __launch_bounds__(kColBlock) void pre_collapse_vec8_kernel(const uint16_t *__restrict__ res, MixArgs mx,
                                                                      int T, int H, int tiles_per_token,
                                                                      uint16_t *__restrict__ y)
{
    const int wave = uniform(blockIdx.x * kColWaves + (threadIdx.x >> 6));
    const int lane = threadIdx.x & (kWave - 1);
    const int t = uniform(wave / tiles_per_token);
    const int tile = uniform(wave - t * tiles_per_token);
    if (t >= T) {
        return;
    }
    // the streams first: their loads are in flight while the token's fields are summed
    const int h = tile * kColVecTile + lane * 8;
    const bool hin = h < H;
    const size_t row = (size_t)t * kHC * H + (hin ? h : 0);
    u32x4 rw[kHC];
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        rw[i] = load_nt16(res + row + (size_t)i * H);
    }
    auto finish = [&](auto first) {
        constexpr bool kFirst = decltype(first)::value;
        float d[kRec], p[kHC], rstd;
        token_start<kFirst>(mx, t, d, p, rstd);
        if (hin) {
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
        if constexpr (kFirst) {
            token_mix_outputs(mx, t, d, p, rstd, lane);
        }
    };
    if (tile == 0) {
        finish(std::true_type{});
    } else {
        finish(std::false_type{});
    }
}

__global__ __launch_bounds__(kColBlock) void pre_collapse_scalar_kernel(const uint16_t *__restrict__ res,
                                                                        MixArgs mx, int T, int H,
                                                                        int tiles_per_token,
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
    const bool hin = h < H;
    const size_t row = (size_t)t * kHC * H + (hin ? h : 0);
    float r[kHC];
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        r[i] = bf16_to_f32(res[row + (size_t)i * H]);
    }
    auto finish = [&](auto first) {
        constexpr bool kFirst = decltype(first)::value;
        float d[kRec], p[kHC], rstd;
        token_start<kFirst>(mx, t, d, p, rstd);
        if (hin) {
            float a = r[0] * p[0];
#pragma unroll
            for (int i = 1; i < kHC; ++i) {
                a = fmaf(r[i], p[i], a);
            }
            y[(size_t)t * H + h] = f32_to_bf16(a);
        }
        if constexpr (kFirst) {
            token_mix_outputs(mx, t, d, p, rstd, lane);
        }
    };
    if (tile == 0) {
        finish(std::true_type{});
    } else {
        finish(std::false_type{});
    }
}

// ---------------------------------------------------------------- FP32 residual streams
// The pre-map over fp32 streams (the same steps; y is still a bf16 row).  The projection
// runs on the fp32 MFMA (16x16x4: one fp32 value per lane and step), so neither operand
// needs splitting: A holds 16 tokens, B 16 weight rows, and the 4 k of a step are one
// stream's h = h0 + 16u + 4g + e of lane group g.  A workgroup owns one 128-wide slice (a
// wave per 32-wide block, all 4 streams) and walks a range of 64-token tiles with the
// block's weights in VGPRs; the streams of the next two 16-token row tiles are in flight
// while one is multiplied.  Each tile leaves the same 25-field partial record as the bf16
// projection, which pre_mixsum_kernel sums and the fp32 collapse below finishes.
struct ProjF32Args {
    const float *res;   // the chunk's streams [T][4][H]
    const float *hc_fn; // [24][4H]
    int T, H, S, tiles_per_range, ntiles;
    float *rec; // [tiles][S][25][64]
};

template <bool kVec>
__global__ __launch_bounds__(kPBlock, 2) void pre_proj_f32s_kernel(ProjF32Args a)
{
    __shared__ float red[kPWaves][kPTok][kMix];
    __shared__ float sqp[kPWaves][4][kPTok];
    const int slice = blockIdx.x;
    const int tile0 = blockIdx.y * a.tiles_per_range;
    const int tile1 = min(a.ntiles, tile0 + a.tiles_per_range);
    if (tile0 >= tile1) {
        return; // the whole workgroup
    }
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & (kWave - 1);
    const int g = lane >> 4;
    const int c = lane & 15;
    const int H = a.H;
    const int S = a.S;
    const int h0 = (slice * kPWaves + w) * kPHB;
    const size_t K = (size_t)kHC * H;

    // B operands: weight row n * 16 + c (rows 24..31 zero) at stream i, h = h0 + 16u + 4g + e
    float wv[kHC][2][4][2];
    {
        const __amdgpu_buffer_rsrc_t vw = buf_view_uniform(a.hc_fn, (uint32_t)((size_t)kMix * K * sizeof(float)));
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int h = h0 + 16 * u + 4 * g;
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int r = n * 16 + c;
                    const uint32_t base = r < kMix ? (uint32_t)((size_t)r * K + (size_t)i * H) * 4u : 0x80000000u;
                    if constexpr (kVec) {
                        const uint32_t off = h < H ? base + (uint32_t)h * 4u : 0x80000000u;
                        const f32x4 q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vw, (int)off, 0, 0));
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            wv[i][u][e][n] = q[e];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t off = h + e < H ? base + (uint32_t)(h + e) * 4u : 0x80000000u;
                            wv[i][u][e][n] =
                                __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vw, (int)off, 0, 0));
                        }
                    }
                }
            }
        }
    }

    // row tile q of the range: 16 tokens (token c for this lane) of every stream at this
    // lane's h; tiles past the range or tokens past the chunk, and h past H, read zero
    const int nq = (tile1 - tile0) * kPMT;
    auto load = [&](int q, float (&d)[kHC][2][4]) {
        const int tok0 = tile0 * kPTok + q * 16;
        const int ntok = q < nq ? max(0, min(16, a.T - tok0)) : 0;
        const __amdgpu_buffer_rsrc_t v = buf_view_uniform(a.res + (size_t)(ntok > 0 ? tok0 : 0) * K,
                                                          (uint32_t)((size_t)ntok * K * sizeof(float)));
#pragma unroll
        for (int i = 0; i < kHC; ++i) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int h = h0 + 16 * u + 4 * g;
                const uint32_t base = ((uint32_t)(c * kHC + i) * (uint32_t)H) * 4u;
                if constexpr (kVec) {
                    const uint32_t off = h < H ? base + (uint32_t)h * 4u : 0x80000000u;
                    const f32x4 q4 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(v, (int)off, 0, 0));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        d[i][u][e] = q4[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t off = h + e < H ? base + (uint32_t)(h + e) * 4u : 0x80000000u;
                        d[i][u][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(v, (int)off, 0, 0));
                    }
                }
            }
        }
    };

    float buf[2][kHC][2][4];
    load(0, buf[0]);
    load(1, buf[1]);
    for (int q0 = 0; q0 < nq; q0 += kPMT) {
#pragma unroll
        for (int m = 0; m < kPMT; ++m) {
            float (&cur)[kHC][2][4] = buf[m & 1];
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            float sq = 0.0f;
#pragma unroll
            for (int i = 0; i < kHC; ++i) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = cur[i][u][e];
                        sq = fmaf(x, x, sq);
                        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, wv[i][u][e][0], acc[0], 0, 0, 0);
                        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, wv[i][u][e][1], acc[1], 0, 0, 0);
                    }
                }
            }
            load(q0 + m + 2, cur); // two row tiles ahead, into the registers just consumed
            // this row tile's partials (the order of pre_proj_kernel: waves summed after the barrier)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int col = n * 16 + c;
                if (col < kMix) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        red[w][m * 16 + 4 * g + k][col] = acc[n][k];
                    }
                }
            }
            sqp[w][g][m * 16 + c] = sq;
        }

        // workgroup reduction -> this slice's partial record of the tile; LDS-only barriers
        // keep the next loads in flight
        lds_barrier();
        const int tile = tile0 + q0 / kPMT;
        float *rec = a.rec + ((size_t)tile * S + slice) * (kRec * kPTok);
        const int tok = tid & (kPTok - 1);
        for (int col = tid >> 6; col < kMix; col += kPWaves) {
            float s = red[0][tok][col];
#pragma unroll
            for (int ww = 1; ww < kPWaves; ++ww) {
                s += red[ww][tok][col];
            }
            rec[field_of_col(col) * kPTok + tok] = s;
        }
        if (tid < kPTok) {
            float s = 0.0f;
#pragma unroll
            for (int ww = 0; ww < kPWaves; ++ww) {
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    s += sqp[ww][gg][tid];
                }
            }
            rec[kFSq * kPTok + tid] = s;
        }
        lds_barrier(); // the partials are read before the next tile writes them
    }
}

// y = sum_i pre_i * res_i over fp32 streams, and the token's post and comb (first tile).
// Vector path: a wave per (token, 256-wide tile), 4 h per lane, 16-byte loads and an
// 8-byte bf16 store; scalar path: a lane per h.
constexpr int kColVecTileF = kWave * 4;

template <bool kVec>
__global__ __launch_bounds__(kColBlock) void pre_collapse_f32s_kernel(const float *__restrict__ res, MixArgs mx, int T,
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
    // the streams first: their loads are in flight while the token's fields are summed
    const int h = tile * (kVec ? kColVecTileF : kWave) + lane * (kVec ? 4 : 1);
    const bool hin = h < H;
    const size_t row = (size_t)t * kHC * H + (hin ? h : 0);
    constexpr int kE = kVec ? 4 : 1;
    float r[kHC][kE];
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
        if constexpr (kVec) {
            const f32x4 v = __builtin_bit_cast(f32x4, load_nt16(res + row + (size_t)i * H));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                r[i][j] = v[j];
            }
        } else {
            r[i][0] = res[row + (size_t)i * H];
        }
    }
    auto finish = [&](auto first) {
        constexpr bool kFirst = decltype(first)::value;
        float d[kRec], p[kHC], rstd;
        token_start<kFirst>(mx, t, d, p, rstd);
        if (hin) {
            float o[kE];
#pragma unroll
            for (int j = 0; j < kE; ++j) {
                float s = r[0][j] * p[0];
#pragma unroll
                for (int i = 1; i < kHC; ++i) {
                    s = fmaf(r[i][j], p[i], s);
                }
                o[j] = s;
            }
            if constexpr (kVec) {
                *reinterpret_cast<uint2 *>(y + (size_t)t * H + h) =
                    uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            } else {
                y[(size_t)t * H + h] = f32_to_bf16(o[0]);
            }
        }
        if constexpr (kFirst) {
            token_mix_outputs(mx, t, d, p, rstd, lane);
        }
    };
    if (tile == 0) {
        finish(std::true_type{});
    } else {
        finish(std::false_type{});
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

} // namespace

PreGeom pre_geometry(int64_t T, int64_t H, bool with_dy)
{
    PreGeom g{};
    g.T = T;
    g.H = H;
    g.nrec = with_dy ? kRecDy : kRec;
    if (T <= 0 || H <= 0) {
        return g;
    }
    g.nhb = (int)((H + kPHB - 1) / kPHB);
    g.slices = (int)((H + kPSliceH - 1) / kPSliceH);
    const int64_t tiles_total = (T + kPTok - 1) / kPTok;
    const size_t rec_per_tile = (size_t)g.slices * g.nrec * kPTok * sizeof(float);
    int64_t max_tiles = (int64_t)(((size_t)1 << 31) / rec_per_tile);
    if (max_tiles < 1) {
        max_tiles = 1;
    }
    // and every launch of a chunk stays within the launch limits: the collapse (at most a
    // wave per 64 h of a token) and the slice sums (nrec blocks of 256 per tile) are its
    // widest grids
    const int64_t per_tok = std::max((H + kWave - 1) / kWave * kWave, (int64_t)g.nrec * 256 / kPTok);
    max_tiles = std::min(max_tiles, std::max<int64_t>(1, launch_tokens(per_tok) / kPTok));
    g.tiles = (int)(tiles_total < max_tiles ? tiles_total : max_tiles);
    g.chunk = (int64_t)g.tiles * kPTok;
    size_t off = 0;
    g.off_frag = off;
    off += align256((size_t)g.nhb * kHC * kFragPerHbStream * sizeof(u32x4));
    g.off_rec = off;
    g.rec_bytes = (size_t)g.tiles * rec_per_tile;
    off += align256(g.rec_bytes);
    g.off_prew = off;
    off += align256((size_t)g.chunk * kSumStride * sizeof(float));
    g.total_bytes = off;
    return g;
}

hipError_t launch_pre_split_any(const void *hc_fn, bool fn_bf16, int fn_rows, int64_t H, void *workspace,
                                hipStream_t stream)
{
    const PreGeom g = pre_geometry(1, H);
    u32x4 *frag = reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(workspace) + g.off_frag);
    const int prep_threads = g.nhb * kHC * (kFragPerHbStream / 3);
    const dim3 prep_grid((unsigned)((prep_threads + 255) / 256));
    if (fn_bf16) {
        pre_prep_kernel<uint16_t><<<prep_grid, dim3(256), 0, stream>>>(reinterpret_cast<const uint16_t *>(hc_fn),
                                                                       (int)H, g.nhb, fn_rows, frag);
    } else {
        pre_prep_kernel<float><<<prep_grid, dim3(256), 0, stream>>>(reinterpret_cast<const float *>(hc_fn), (int)H,
                                                                    g.nhb, fn_rows, frag);
    }
    return hipGetLastError();
}

size_t pre_split_bytes(int64_t H)
{
    const PreGeom g = pre_geometry(1, H);
    return g.off_rec; // the fragment area, from offset 0
}

hipError_t launch_pre_split(const float *hc_fn, const PreGeom &g, void *workspace, hipStream_t stream)
{
    u32x4 *frag = reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(workspace) + g.off_frag);
    const int prep_threads = g.nhb * kHC * (kFragPerHbStream / 3);
    pre_prep_kernel<float><<<dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, stream>>>(
        hc_fn, (int)g.H, g.nhb, kMix, frag);
    return hipGetLastError();
}

size_t post_project_workspace_bytes(int64_t T, int64_t H) { return pre_geometry(T, H).total_bytes; }

size_t pre_fused_workspace_bytes(int64_t T, int64_t H)
{
    const size_t two_pass = pre_geometry(T, H).total_bytes;
    const size_t coop = pre_coop_shape_ok(T, H) ? pre_coop_workspace_bytes(H) : 0;
    const size_t decode = pre_decode_shape_ok(T, H) ? pre_decode_workspace_bytes(H) : 0;
    return std::max(two_pass, std::max(coop, decode));
}

size_t pre_path_workspace_bytes(int64_t T, int64_t H, bool vec8)
{
    if (pre_decode_usable(T, H, vec8)) {
        return pre_decode_workspace_bytes(H);
    }
    return pre_coop_usable(T, H, vec8) ? pre_coop_workspace_bytes(H) : pre_geometry(T, H).total_bytes;
}

hipError_t launch_post_project(const uint16_t *x, const uint16_t *res, const float *post, const float *comb,
                               const float *hc_fn_next, int64_t T, int64_t H, uint16_t *out, float *dot_mix,
                               float *sqrsum, void *workspace, hipStream_t stream)
{
    const PreGeom g = pre_geometry(T, H);
    hipError_t e = launch_pre_split(hc_fn_next, g, workspace, stream);
    if (e != hipSuccess) {
        return e;
    }
    char *ws = reinterpret_cast<char *>(workspace);
    for (int64_t c0 = 0; c0 < T; c0 += g.chunk) {
        const int Tc = (int)(T - c0 < g.chunk ? T - c0 : g.chunk);
        const int tiles = (Tc + kPTok - 1) / kPTok;
        PostProjArgs a{};
        a.x = x + (size_t)c0 * H;
        a.res = res + (size_t)c0 * kHC * H;
        a.post = post + (size_t)c0 * kHC;
        a.comb = comb + (size_t)c0 * kHC * kHC;
        a.frag = reinterpret_cast<const u32x4 *>(ws + g.off_frag);
        a.T = Tc;
        a.H = (int)H;
        a.nhb = g.nhb;
        a.S = g.slices;
        a.out = out + (size_t)c0 * kHC * H;
        a.rec = reinterpret_cast<float *>(ws + g.off_rec);
        a.rec_bytes = (uint32_t)((size_t)tiles * g.slices * kRec * kPTok * sizeof(float));
        int ranges = 1;
        pre_stream_ranges(Tc, g.slices, ranges, a.tok_per_range);
        post_proj_stream_kernel<<<dim3((unsigned)g.slices, (unsigned)ranges), dim3(kPBlock), 0, stream>>>(a);
        e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
        pre_mixsum_kernel<<<dim3((unsigned)(tiles * kRec)), dim3(256), 0, stream>>>(
            a.rec, Tc, g.slices, kRec, nullptr, dot_mix + (size_t)c0 * kMix, sqrsum + c0);
        e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_collapse_dots(const float *dots, const float *sq, const uint16_t *res, const float *hc_scale,
                                const float *hc_base, int64_t T, int64_t H, float k, float rms_eps, float pre_eps,
                                float sinkhorn_eps, float post_mult, int iters, uint16_t *y, float *post,
                                float *comb, float *pre, hipStream_t stream)
{
    const int64_t htiles = (H + kColVecTile - 1) / kColVecTile;
    return for_token_chunks(T, collapse_items_per_token(H, true), [&](int64_t c0, int64_t Tc) {
        MixArgs mx{};
        mx.sums = dots + (size_t)c0 * kMix;
        mx.stride = kMix;
        mx.off_post = kHC;
        mx.sq = sq + c0;
        mx.hc_scale = hc_scale;
        mx.hc_base = hc_base;
        mx.k_denom = k;
        mx.rms_eps = rms_eps;
        mx.pre_eps = pre_eps;
        mx.sk_eps = sinkhorn_eps;
        mx.post_mult = post_mult;
        mx.iters = iters;
        mx.head = 0;
        mx.post = post + (size_t)c0 * kHC;
        mx.comb = comb + (size_t)c0 * kHC * kHC;
        mx.pre_out = pre ? pre + (size_t)c0 * kHC : nullptr;
        const int64_t blocks = (Tc * htiles + kColWaves - 1) / kColWaves;
        pre_collapse_vec8_kernel<<<dim3((unsigned)blocks), dim3(kColBlock), 0, stream>>>(
            res + (size_t)c0 * kHC * H, mx, (int)Tc, (int)H, (int)htiles, y + (size_t)c0 * H);
        return hipGetLastError();
    });
}

int64_t collapse_items_per_token(int64_t H, bool vec8)
{
    const int tile = vec8 ? kColVecTile : kWave;
    return (H + tile - 1) / tile * kWave;
}

hipError_t launch_pre_sums(const uint16_t *res, const uint16_t *dy, const PreGeom &g, int64_t c0, int Tc,
                           void *workspace, hipStream_t stream, bool vec8)
{
    if (dy != nullptr && (!vec8 || g.nrec != kRecDy)) {
        return hipErrorInvalidValue;
    }
    char *ws = reinterpret_cast<char *>(workspace);
    const int H = (int)g.H;
    const int tiles = (Tc + kPTok - 1) / kPTok;
    ProjArgs a{};
    a.res = res + (size_t)c0 * kHC * H;
    a.frag = reinterpret_cast<const u32x4 *>(ws + g.off_frag);
    a.T = Tc;
    a.H = H;
    a.nhb = g.nhb;
    a.S = g.slices;
    a.rec = reinterpret_cast<float *>(ws + g.off_rec);
    if (vec8) {
        ProjStreamArgs sa{};
        sa.res = a.res;
        sa.dy = dy != nullptr ? dy + (size_t)c0 * H : nullptr;
        sa.frag = a.frag;
        sa.T = a.T;
        sa.H = H;
        sa.nhb = g.nhb;
        sa.S = g.slices;
        sa.rec = a.rec;
        sa.rec_bytes = (uint32_t)g.rec_bytes;
        int ranges = 1;
        pre_stream_ranges(a.T, g.slices, ranges, sa.tok_per_range);
        const dim3 sgrid((unsigned)g.slices, (unsigned)ranges);
        if (dy != nullptr) {
            pre_proj_stream_kernel<true><<<sgrid, dim3(kPBlock), 0, stream>>>(sa);
        } else {
            pre_proj_stream_kernel<false><<<sgrid, dim3(kPBlock), 0, stream>>>(sa);
        }
    } else {
        pre_proj_kernel<<<dim3((unsigned)tiles, (unsigned)g.slices), dim3(kPBlock), 0, stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        return e;
    }
    pre_mixsum_kernel<<<dim3((unsigned)(tiles * g.nrec)), dim3(256), 0, stream>>>(
        a.rec, Tc, g.slices, g.nrec, reinterpret_cast<float *>(ws + g.off_prew), nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_pre(const uint16_t *res, const void *hc_fn, bool fn_bf16, int fn_rows, const float *hc_scale,
                      const float *hc_base, const PreGeom &g, float rms_eps, float pre_eps, float sinkhorn_eps,
                      float post_mult, int iters, bool head, uint16_t *y, float *post, float *comb, float *pre,
                      void *workspace, hipStream_t stream, bool vec8, bool presplit)
{
    if (pre_decode_usable(g.T, g.H, vec8)) { // small batches: one launch, weights as given
        return launch_pre_decode(res, hc_fn, fn_bf16, fn_rows, hc_scale, hc_base, g.T, g.H, rms_eps, pre_eps,
                                 sinkhorn_eps, post_mult, iters, head, y, post, comb, pre, workspace, stream);
    }
    if (pre_coop_usable(g.T, g.H, vec8)) {
        return launch_pre_coop(res, hc_fn, fn_bf16, fn_rows, hc_scale, hc_base, g.T, g.H, rms_eps, pre_eps,
                               sinkhorn_eps, post_mult, iters, head, y, post, comb, pre, workspace, stream);
    }
    char *ws = reinterpret_cast<char *>(workspace);
    u32x4 *frag = reinterpret_cast<u32x4 *>(ws + g.off_frag);
    const int H = (int)g.H;

    hipError_t e = hipSuccess;
    if (!presplit) { // else the caller split these weights into the workspace already
        e = launch_pre_split_any(hc_fn, fn_bf16, fn_rows, H, workspace, stream);
        if (e != hipSuccess) {
            return e;
        }
    }
    float *sums = reinterpret_cast<float *>(ws + g.off_prew);
    for (int64_t c0 = 0; c0 < g.T; c0 += g.chunk) {
        const int Tc = (int)(g.T - c0 < g.chunk ? g.T - c0 : g.chunk);
        const int tiles = (Tc + kPTok - 1) / kPTok;
        ProjArgs a{};
        a.res = res + (size_t)c0 * kHC * H;
        a.frag = frag;
        a.T = Tc;
        a.H = H;
        a.nhb = g.nhb;
        a.S = g.slices;
        a.rec = reinterpret_cast<float *>(ws + g.off_rec);
        if (vec8) {
            ProjStreamArgs sa{};
            sa.res = a.res;
            sa.frag = a.frag;
            sa.T = a.T;
            sa.H = H;
            sa.nhb = g.nhb;
            sa.S = g.slices;
            sa.rec = a.rec;
            sa.rec_bytes = (uint32_t)g.rec_bytes;
            int ranges = 1;
            pre_stream_ranges(a.T, g.slices, ranges, sa.tok_per_range);
            pre_proj_stream_kernel<false><<<dim3((unsigned)g.slices, (unsigned)ranges), dim3(kPBlock), 0, stream>>>(sa);
        } else {
            pre_proj_kernel<<<dim3((unsigned)tiles, (unsigned)g.slices), dim3(kPBlock), 0, stream>>>(a);
        }
        e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
        // small batches: the collapse sums the slices itself (one launch fewer)
        const bool fuse = Tc <= kFuseSumTokens;
        if (!fuse) {
            pre_mixsum_kernel<<<dim3((unsigned)(tiles * g.nrec)), dim3(256), 0, stream>>>(a.rec, Tc, g.slices, g.nrec,
                                                                                        sums, nullptr, nullptr);
            e = hipGetLastError();
            if (e != hipSuccess) {
                return e;
            }
        }
        MixArgs mx{};
        mx.rec = fuse ? a.rec : nullptr;
        mx.S = g.slices;
        mx.nrec = g.nrec;
        mx.sums = sums;
        mx.stride = kSumStride;
        mx.off_post = kFSq + 1;
        mx.sq = nullptr;
        mx.hc_scale = hc_scale;
        mx.hc_base = hc_base;
        mx.k_denom = (float)(kHC * g.H);
        mx.rms_eps = rms_eps;
        mx.pre_eps = pre_eps;
        mx.sk_eps = sinkhorn_eps;
        mx.post_mult = post_mult;
        mx.iters = iters;
        mx.head = head ? 1 : 0;
        mx.post = head ? nullptr : post + (size_t)c0 * kHC;
        mx.comb = head ? nullptr : comb + (size_t)c0 * kHC * kHC;
        mx.pre_out = pre ? pre + (size_t)c0 * kHC : nullptr;
        const int tile = vec8 ? kColVecTile : kWave;
        const int64_t htiles = (g.H + tile - 1) / tile;
        const int64_t blocks = ((int64_t)Tc * htiles + kColWaves - 1) / kColWaves;
        const uint16_t *rc = res + (size_t)c0 * kHC * H;
        uint16_t *yc = y + (size_t)c0 * H;
        if (vec8) {
            pre_collapse_vec8_kernel<<<dim3((unsigned)blocks), dim3(kColBlock), 0, stream>>>(rc, mx, Tc, H,
                                                                                             (int)htiles, yc);
        } else {
            pre_collapse_scalar_kernel<<<dim3((unsigned)blocks), dim3(kColBlock), 0, stream>>>(rc, mx, Tc, H,
                                                                                               (int)htiles, yc);
        }
        e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_pre_f32s(const float *res, const float *hc_fn, const float *hc_scale, const float *hc_base,
                           const PreGeom &g, float rms_eps, float pre_eps, float sinkhorn_eps, float post_mult,
                           int iters, uint16_t *y, float *post, float *comb, float *pre, void *workspace,
                           hipStream_t stream, bool vec4)
{
    char *ws = reinterpret_cast<char *>(workspace);
    float *sums = reinterpret_cast<float *>(ws + g.off_prew);
    const int H = (int)g.H;
    for (int64_t c0 = 0; c0 < g.T; c0 += g.chunk) {
        const int Tc = (int)(g.T - c0 < g.chunk ? g.T - c0 : g.chunk);
        const int tiles = (Tc + kPTok - 1) / kPTok;
        ProjF32Args a{};
        a.res = res + (size_t)c0 * kHC * H;
        a.hc_fn = hc_fn;
        a.T = Tc;
        a.H = H;
        a.S = g.slices;
        a.ntiles = tiles;
        a.rec = reinterpret_cast<float *>(ws + g.off_rec);
        // about two workgroups per CU over all slices, each walking a range of tiles
        int ranges = kPSTargetBlocks / g.slices;
        ranges = ranges < 1 ? 1 : (ranges > tiles ? tiles : ranges);
        a.tiles_per_range = (tiles + ranges - 1) / ranges;
        ranges = (tiles + a.tiles_per_range - 1) / a.tiles_per_range;
        if (vec4) {
            pre_proj_f32s_kernel<true><<<dim3((unsigned)g.slices, (unsigned)ranges), dim3(kPBlock), 0, stream>>>(a);
        } else {
            pre_proj_f32s_kernel<false><<<dim3((unsigned)g.slices, (unsigned)ranges), dim3(kPBlock), 0, stream>>>(a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
        const bool fuse = Tc <= kFuseSumTokens;
        if (!fuse) {
            pre_mixsum_kernel<<<dim3((unsigned)(tiles * kRec)), dim3(256), 0, stream>>>(a.rec, Tc, g.slices, kRec, sums,
                                                                                      nullptr, nullptr);
            e = hipGetLastError();
            if (e != hipSuccess) {
                return e;
            }
        }
        MixArgs mx{};
        mx.rec = fuse ? a.rec : nullptr;
        mx.S = g.slices;
        mx.nrec = kRec;
        mx.sums = sums;
        mx.stride = kSumStride;
        mx.off_post = kFSq + 1;
        mx.sq = nullptr;
        mx.hc_scale = hc_scale;
        mx.hc_base = hc_base;
        mx.k_denom = (float)(kHC * g.H);
        mx.rms_eps = rms_eps;
        mx.pre_eps = pre_eps;
        mx.sk_eps = sinkhorn_eps;
        mx.post_mult = post_mult;
        mx.iters = iters;
        mx.head = 0;
        mx.post = post + (size_t)c0 * kHC;
        mx.comb = comb + (size_t)c0 * kHC * kHC;
        mx.pre_out = pre ? pre + (size_t)c0 * kHC : nullptr;
        const int tile = vec4 ? kColVecTileF : kWave;
        const int64_t htiles = (g.H + tile - 1) / tile;
        const int64_t blocks = ((int64_t)Tc * htiles + kColWaves - 1) / kColWaves;
        const float *rc = res + (size_t)c0 * kHC * H;
        uint16_t *yc = y + (size_t)c0 * H;
        if (vec4) {
            pre_collapse_f32s_kernel<true><<<dim3((unsigned)blocks), dim3(kColBlock), 0, stream>>>(rc, mx, Tc, H,
                                                                                                 (int)htiles, yc);
        } else {
            pre_collapse_f32s_kernel<false><<<dim3((unsigned)blocks), dim3(kColBlock), 0, stream>>>(rc, mx, Tc, H,
                                                                                                  (int)htiles, yc);
        }
        e = hipGetLastError();
        if (e != hipSuccess) {
            return e;
        }
    }
    return hipSuccess;
}

} // namespace mhc
