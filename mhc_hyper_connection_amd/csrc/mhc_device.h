// mhc_device.h -- device-side helpers shared by the libmhc kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

constexpr int kHC = 4;    // residual streams
constexpr int kMix = 24;  // logits per token: pre(4) + post(4) + comb(16)
constexpr int kWave = 64; // CDNA wavefront

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Two fp32 -> packed bf16 pair, round to nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float v)
{
    __bf16 b = (__bf16)v;
    return __builtin_bit_cast(uint16_t, b);
}

// 16-byte streaming loads/stores (data touched once: non-temporal hint).
__device__ __forceinline__ u32x4 load_nt16(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void store_nt16(void *p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// 1 / (1 + e^-z), using the hardware 2^x.
__device__ __forceinline__ float sigmoidf_fast(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Fixed-count Sinkhorn-Knopp on one 4x4 matrix held in registers (row-major P[4*i+j]):
// softmax over each row (row maximum subtracted) plus eps, giving K, then `iters` rounds
// of row normalisation followed by column normalisation.  After any number of rounds
// the matrix is diag(r) K diag(c), so the rounds update only the scales:
//     r_i = 1 / sum_j K_ij c_j,   then   c_j = 1 / sum_i r_i K_ij
// (one multiply, three FMAs and a reciprocal per row or column: 40 instructions a
// round against 64 for rescaling all 16 entries twice), and P_ij = (r_i K_ij) c_j is
// formed once at the end.  Each column of the result sums to 1 up to rounding, as
// after a column normalisation of the entries themselves.
__device__ __forceinline__ void sinkhorn4x4(float *P, int iters, float eps)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float mx = fmaxf(fmaxf(P[4 * i], P[4 * i + 1]), fmaxf(P[4 * i + 2], P[4 * i + 3]));
        float e0 = __expf(P[4 * i] - mx), e1 = __expf(P[4 * i + 1] - mx);
        float e2 = __expf(P[4 * i + 2] - mx), e3 = __expf(P[4 * i + 3] - mx);
        float r = fast_rcp((e0 + e1) + (e2 + e3));
        P[4 * i] = fmaf(e0, r, eps);
        P[4 * i + 1] = fmaf(e1, r, eps);
        P[4 * i + 2] = fmaf(e2, r, eps);
        P[4 * i + 3] = fmaf(e3, r, eps);
    }
    float r[4] = {1.0f, 1.0f, 1.0f, 1.0f}, c[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float s = P[4 * i] * c[0];
            s = fmaf(P[4 * i + 1], c[1], s);
            s = fmaf(P[4 * i + 2], c[2], s);
            s = fmaf(P[4 * i + 3], c[3], s);
            r[i] = fast_rcp(s);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float s = r[0] * P[j];
            s = fmaf(r[1], P[4 + j], s);
            s = fmaf(r[2], P[8 + j], s);
            s = fmaf(r[3], P[12 + j], s);
            c[j] = fast_rcp(s);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            P[4 * i + j] = (r[i] * P[4 * i + j]) * c[j];
        }
    }
}

// Eight fp32 values split into three bf16 terms, packed in pairs: v == hi + mid + lo exactly
// for normal fp32 v (three successive bf16 truncations: 8 + 8 + 8 significant bits).
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

// Lane permutations within a 16-lane DPP row.  Every source lane exists for these
// patterns, so bound_ctrl (zero for a missing source) never applies; setting it and
// leaving `old` undefined lets the compiler fold the move into the consuming add.
template <int kCtrl>
__device__ __forceinline__ float dpp_perm(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor1(float v) { return dpp_perm<0xB1>(v); } // quad_perm [1,0,3,2]
__device__ __forceinline__ float dpp_quad_xor2(float v) { return dpp_perm<0x4E>(v); } // quad_perm [2,3,0,1]
__device__ __forceinline__ float dpp_row_ror4(float v) { return dpp_perm<0x124>(v); } // row_ror:4
__device__ __forceinline__ float dpp_row_ror8(float v) { return dpp_perm<0x128>(v); } // row_ror:8

// Fixed-count Sinkhorn of a 4x4 matrix spread over a 16-lane row (lane e holds entry
// (e / 4, e % 4)): row softmax (row maximum subtracted) plus eps, then `iters` rounds
// of row then column normalisation.  Row sums combine the lane's quad; column sums
// the lanes e, e +- 4, e +- 8 (rotations within the row).
__device__ __forceinline__ float sinkhorn_row16(float L, int iters, float eps)
{
    float mx = fmaxf(L, dpp_quad_xor1(L));
    mx = fmaxf(mx, dpp_quad_xor2(mx));
    const float e = __expf(L - mx);
    float s = e + dpp_quad_xor1(e);
    s = s + dpp_quad_xor2(s);
    float P = fmaf(e, fast_rcp(s), eps);
    for (int it = 0; it < iters; ++it) {
        float rs = P + dpp_quad_xor1(P);
        rs = rs + dpp_quad_xor2(rs);
        P *= fast_rcp(rs);
        float cs = P + dpp_row_ror4(P);
        cs = cs + dpp_row_ror8(cs);
        P *= fast_rcp(cs);
    }
    return P;
}

// Two matrices per 16-lane row (logits L0 and L1 in the same lane positions), the rounds of
// both in one loop so that their dependent chains interleave; each result has the bits
// sinkhorn_row16 gives for it.
__device__ __forceinline__ void sinkhorn_row16x2(float L0, float L1, int iters, float eps, float &P0, float &P1)
{
    float m0 = fmaxf(L0, dpp_quad_xor1(L0));
    float m1 = fmaxf(L1, dpp_quad_xor1(L1));
    m0 = fmaxf(m0, dpp_quad_xor2(m0));
    m1 = fmaxf(m1, dpp_quad_xor2(m1));
    const float e0 = __expf(L0 - m0);
    const float e1 = __expf(L1 - m1);
    float s0 = e0 + dpp_quad_xor1(e0);
    float s1 = e1 + dpp_quad_xor1(e1);
    s0 = s0 + dpp_quad_xor2(s0);
    s1 = s1 + dpp_quad_xor2(s1);
    P0 = fmaf(e0, fast_rcp(s0), eps);
    P1 = fmaf(e1, fast_rcp(s1), eps);
    for (int it = 0; it < iters; ++it) {
        float r0 = P0 + dpp_quad_xor1(P0);
        float r1 = P1 + dpp_quad_xor1(P1);
        r0 = r0 + dpp_quad_xor2(r0);
        r1 = r1 + dpp_quad_xor2(r1);
        P0 *= fast_rcp(r0);
        P1 *= fast_rcp(r1);
        float c0 = P0 + dpp_row_ror4(P0);
        float c1 = P1 + dpp_row_ror4(P1);
        c0 = c0 + dpp_row_ror8(c0);
        c1 = c1 + dpp_row_ror8(c1);
        P0 *= fast_rcp(c0);
        P1 *= fast_rcp(c1);
    }
}

// Sum over the 64 lanes of a wavefront (butterfly: every lane gets the total).
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        v += __shfl_xor(v, o);
    }
    return v;
}

// Sum over the 64 lanes of a wavefront on DPP moves and permlane swaps (no LDS round
// trip): within quads (lanes xor 1, 2), half rows and rows (mirrors), then the four rows
// ((0 + 1) and (2 + 3) by v_permlane16_swap, the halves by v_permlane32_swap).  Each add
// meets the same two partial sums in every lane, so every lane gets the same bits.
__device__ __forceinline__ float wave_sum_dpp(float v)
{
    v += dpp_quad_xor1(v);
    v += dpp_quad_xor2(v);
    v += dpp_perm<0x141>(v); // row_half_mirror
    v += dpp_perm<0x140>(v); // row_mirror
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Workgroup barrier over LDS only: waits for this wavefront's LDS accesses, not for
// its global loads, which stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-uniform value (forces an SGPR so coefficient loads become scalar loads).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A raw buffer view of `bytes` bytes at `base` (stride 0; offsets past the end read
// zero and drop stores).  Every piece goes through readfirstlane: the caller promises
// that base and bytes are the same in every lane, and the descriptor then stays in
// SGPRs even where the compiler would otherwise route it through VGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_view_uniform(const void *base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
    void *q = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, 0, (int)n, 0x00020000);
}

// Workgroups are dealt to the chip's 8 XCDs (each with its own L2) round robin.
// For a grid of n workgroups, one per item, this maps workgroup b to an item such that
// XCD b mod 8 walks a contiguous run of items: neighbouring items, whose small rows
// share cache lines, then meet in the same L2.  A bijection on [0, n).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous(int b, int n)
{
    const int q = n / kXcds, r = n - kXcds * q;
    const int x = b & (kXcds - 1), i = b / kXcds;
    return x * q + min(x, r) + i;
}

// A token's split partials summed by a whole 256-thread workgroup: dots [S][T][24] into
// out[0..23] and, when sqrsum is given, sums of squares [S][T] into out[24] (LDS).
// Splits are staged 64 at a time, every thread loading some of them, so the loads are
// in flight together instead of one after another.  Wave w adds the splits s = w mod 4
// in increasing order, and the four wave sums combine as (w0 + w1) + (w2 + w3): a fixed
// order, so the result is deterministic.  stage: 64 * 25 floats, wpart: 4 * 25 floats.
// Every thread of the workgroup must call it.  With one split there is nothing to
// reduce: threads 0..24 copy their field, and out is valid after the caller's next
// workgroup barrier; with several, out is valid when it returns.
constexpr int kSplitStage = 64;
constexpr int kSplitFields = kMix + 1;
__device__ __forceinline__ void sum_split_partials(const float *dot_mix, const float *sqrsum, int S, int T, int t,
                                                   float *stage, float *wpart, float *out)
{
    const int tid = threadIdx.x;
    if (S == 1) {
        if (tid < kMix) {
            out[tid] = dot_mix[(size_t)t * kMix + tid];
        } else if (tid == kMix && sqrsum != nullptr) {
            out[kMix] = sqrsum[t];
        }
        return;
    }
    const int w = tid >> 6;
    const int lane = tid & (kWave - 1);
    float acc = 0.0f;
    for (int s0 = 0; s0 < S; s0 += kSplitStage) {
        const int ns = min(kSplitStage, S - s0);
#pragma unroll
        for (int k = 0; k < (kSplitStage * kSplitFields + 255) / 256; ++k) {
            const int e = tid + 256 * k;
            const int s = e / kSplitFields, f = e - kSplitFields * s;
            float v = 0.0f;
            if (s < ns) {
                if (f < kMix) {
                    v = dot_mix[((size_t)(s0 + s) * T + t) * kMix + f];
                } else if (sqrsum != nullptr) {
                    v = sqrsum[(size_t)(s0 + s) * T + t];
                }
            }
            if (e < kSplitStage * kSplitFields) {
                stage[e] = v;
            }
        }
        __syncthreads();
        if (lane < kSplitFields) {
            for (int s = w; s < ns; s += 4) {
                acc += stage[s * kSplitFields + lane];
            }
        }
        __syncthreads();
    }
    if (lane < kSplitFields) {
        wpart[w * kSplitFields + lane] = acc;
    }
    __syncthreads();
    if (tid < kSplitFields) {
        out[tid] = (wpart[tid] + wpart[kSplitFields + tid]) + (wpart[2 * kSplitFields + tid] + wpart[3 * kSplitFields + tid]);
    }
    __syncthreads();
}

// ---- cross-workgroup exchange through an XCD's L2 (the one-read and small-batch pre-maps)

// A buffer offset that lies past every view: loads read zero, stores are dropped.
constexpr uint32_t kOob = 0x80000000u;

extern "C" __device__ uint64_t mhc_coop_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// Tags of exchange records: a key from the dispatch id (distinct for every launch), mixed
// with a record set's index.
__device__ __forceinline__ uint32_t coop_key()
{
    uint64_t z = mhc_coop_dispatch_id() + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(z >> 32));
}
// Distinct steps of one call get distinct tags (an odd multiplier is a bijection).
__device__ __forceinline__ uint32_t coop_tag(uint32_t key, int gs) { return key ^ ((uint32_t)gs * 0x85EBCA6Bu + 1u); }

// Sum of v over the 32 lanes of each half-wave, on DPP moves: within each quad (lanes
// xor 1, 2), the two quads of each 8-lane half row (mirror), the two halves of each
// 16-lane row (mirror), then row 0 into row 1 and row 2 into row 3 (row_bcast:15).  The
// total of lanes 0..31 lands in lanes 16..31 and that of lanes 32..63 in lanes 48..63;
// the order of the additions is fixed.
__device__ __forceinline__ float half_sum(float v)
{
    v += dpp_perm<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_perm<0x4E>(v);  // quad_perm [2,3,0,1]
    v += dpp_perm<0x141>(v); // row_half_mirror
    v += dpp_perm<0x140>(v); // row_mirror
    // rows 1 and 3 add the last lane of rows 0 and 2 (row_bcast:15; rows 0 and 2 are not
    // written); the s_nop covers the wait a DPP read needs after a VALU write of its source
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf" : "+v"(v));
    return v;
}
constexpr int kHalfSumLane = 16; // the lane of each half-wave (mod 32) that holds its sum

// rstd and sigmoid on the hardware reciprocal square root and reciprocal (1 ulp each, far
// inside the 1e-5 tolerance of the mixes), for the exchange kernels' per-token work.
__device__ __forceinline__ float rstd_of(float S, float inv_k, float eps) { return __builtin_amdgcn_rsqf(fmaf(S, inv_k, eps)); }
__device__ __forceinline__ float sigmoid_rcp(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

} // namespace mhc
