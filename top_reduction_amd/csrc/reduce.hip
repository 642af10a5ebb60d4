// reduce.hip -- per-row logsumexp, selected logprob and exact top-K of a
// logits matrix, on gfx950 (MTPLX PR #532, Change; openinfer issue #719,
// Suggested direction).
//
// Stage 1 (one coalesced read of every logit): a 1-D grid of rows x splits
// workgroups; each streams a contiguous, block-aligned slice of one row with
// 16-byte loads and produces
//   * an online (max, sum of exp(x - max)) partial in fp32, and
//   * the maximum of every 64-logit block it covers, stored as a monotone key
//     (16-bit for bf16 rows, 32-bit for fp32 rows).
// Stage 2 (one workgroup per row): combines the partials in a fixed order into
// the fp32 logsumexp, writes the selected logprob, keeps the min(K, nb) blocks
// with the largest maxima (equal maxima: lower block index first), gathers the
// entries of those blocks that are not below the K-th kept maximum, and ranks
// them by (value descending, id ascending) in LDS. The candidate set provably
// contains the exact top-K: a top-K entry outside the kept blocks, or below
// the K-th kept maximum, would have K kept block maxima ahead of it.
#include "lmh_internal.h"

namespace lmh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = 256;
constexpr int kHistBins = 256;     // key values resolved by one stage-2 histogram
constexpr int kSeg = 4096;          // logits per stage-1 work item (one wave)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maxima written as v_max_f32 / v_max3_f32. In IEEE mode the compiler quiets
// every fmaxf operand that is not the result of arithmetic first (here: all of
// them, being bit-cast loads), an extra instruction per logit. NaN operands:
// a quiet NaN loses to any number, a signalling one makes the result NaN.
__device__ inline float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ inline float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// max(v, v of the lane chosen by a full-row DPP pattern) as one instruction.
// The two wait states cover a DPP read of a VGPR written by the previous VALU
// instruction.
#define LMH_DPP_MAX(v, PATTERN)                                                                   \
    ([&]() {                                                                                      \
        float r_;                                                                                 \
        asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " PATTERN " row_mask:0xf bank_mask:0xf"         \
            : "=v"(r_)                                                                            \
            : "v"(v));                                                                            \
        return r_;                                                                                \
    }())
// Maximum over aligned lane groups of 8 or 16; every lane of a group ends with it.
template <int G>
__device__ inline float group_max(float v) {
    static_assert(G == 8 || G == 16 || G == 64, "group of 8, 16 or 64 lanes");
    v = LMH_DPP_MAX(v, "quad_perm:[1,0,3,2]");
    v = LMH_DPP_MAX(v, "quad_perm:[2,3,0,1]");
    v = LMH_DPP_MAX(v, "row_half_mirror");
    if (G >= 16) v = LMH_DPP_MAX(v, "row_mirror");
    if (G == 64) {
        const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
        const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
        v = fmaxf(fmaxf(a, b), fmaxf(c, d));   // wave-uniform
    }
    return v;
}

// Merge two (max, sum-exp) partials. A partial with max -inf has sum 0.
__device__ inline void lse_merge(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    const float Mr = (M == kNegInf) ? 0.f : M;
    s = s * ex2((m - Mr) * kLog2e) + s2 * ex2((m2 - Mr) * kLog2e);
    m = M;
}

template <bool BF16>
__device__ inline uint32_t elem_key(float x) {
    return BF16 ? (f32_key(x) & 0xFFFF0000u) : f32_key(x);
}

template <bool BF16>
__device__ inline float key_value(uint32_t k) {
    if (BF16) {
        const uint32_t k16 = k >> 16;
        const uint32_t b = (k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
        return __uint_as_float(b << 16);
    }
    return key_f32(k);
}

// ---------------------------------------------------------------------------
// Stage 1: a row is cut into fixed segments of kSeg logits (the last one
// partial); each segment is the work item of one wave, and items are numbered
// row-major so that consecutively dispatched waves stream consecutive memory.
// Lane l of a wave reads the item's 16-byte vectors l, l + 64, ...; all of an
// item's loads are in flight before its first vector is used, and the item's
// 64 logits per lane stay in registers for two passes:
//   1. the maximum of each lane's slice of every 64-logit block (the 8 bf16 or
//      16 fp32 lanes of a block then combine it with DPP), and of the lane;
//   2. with M the wave maximum, the sum of 2^(x*log2e + c) for c = -RN(M*log2e):
//      one fma, one exp2 and one add per logit. The rounding of c is the
//      exactly representable e = M*log2e + c (an fma), and the sum is scaled
//      by 2^-e once, so the partial is (M, sum of exp(x - M)) to fp32 rounding.
// The lane sums are added by a fixed DPP tree into lane 63. The block maxima
// are transposed across the wave (a register select, then ds_bpermute) so that
// lane b holds block b, and stored as keys with one coalesced store. Neither
// the segments nor the summation order depend on how many rows a call holds,
// so each row's results are bitwise independent of the batch around it.
// ---------------------------------------------------------------------------
// One (max, sum-exp) merge step with the partner chosen by a DPP control;
// lanes without a partner merge the identity (-inf, 0).
#define LMH_LSE_DPP_STEP(m, s, ctrl, rmask)                                                          \
    do {                                                                                             \
        const float m2_ = __int_as_float(                                                            \
            __builtin_amdgcn_update_dpp((int)0xFF800000, __float_as_int(m), ctrl, rmask, 0xF, false)); \
        const float s2_ = __int_as_float(                                                            \
            __builtin_amdgcn_update_dpp(0, __float_as_int(s), ctrl, rmask, 0xF, false));             \
        lse_merge(m, s, m2_, s2_);                                                                   \
    } while (0)

// Sum over the wave by row shifts, then row broadcasts; lane 63 ends with the
// total (a fixed order).
__device__ inline float wave_sum_to_63(float s) {
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x111, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x112, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x114, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x118, 0xF, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x142, 0xA, 0xF, false));
    s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x143, 0xC, 0xF, false));
    return s;
}

// v[r] for a lane-dependent r in [0, N), N a power of two, by a select tree.
template <int N>
__device__ inline float select_reg(const float (&v)[N], int r) {
    float t[N];
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = v[i];
#pragma unroll
    for (int w = N / 2, bit = 0; w >= 1; w /= 2, ++bit) {
        const bool hi = (r >> bit) & 1;
#pragma unroll
        for (int i = 0; i < w; ++i) t[i] = hi ? t[2 * i + 1] : t[2 * i];
    }
    return t[0];
}

template <bool BF16>
struct Stage1Item {
    static constexpr int EPV = BF16 ? 8 : 4;          // elements per 16-byte vector
    static constexpr int VPB = kBlock / EPV;          // lanes per 64-logit block
    static constexpr int VPL = kSeg / EPV / 64;       // vectors per lane (== VPB)
    static constexpr int GPV = 64 / VPB;              // blocks per wave-wide vector
    static_assert(VPL == VPB, "one block maximum per vector and lane group");
};

// Reduces one item held in buf (VPL vectors per lane; entries past V hold
// -inf) and writes its partial and block keys.
template <bool BF16, bool KEYS>
__device__ __forceinline__ void stage1_reduce(const u32x4 (&buf)[Stage1Item<BF16>::VPL], int lane,
                                              int64_t it, int64_t row, int32_t seg, int64_t V,
                                              int32_t kld, float2* __restrict__ part,
                                              void* __restrict__ keys) {
    using I = Stage1Item<BF16>;
    float x[I::VPL * I::EPV];
    float bm[I::VPL];
    float lm = kNegInf;
#pragma unroll
    for (int j = 0; j < I::VPL; ++j) {
        const uint32_t w[4] = {buf[j].x, buf[j].y, buf[j].z, buf[j].w};
        float* xv = x + j * I::EPV;
        float vm;
        if (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[2 * e] = bf16_lo(w[e]);
                xv[2 * e + 1] = bf16_hi(w[e]);
            }
            vm = vmax3(xv[6], xv[7], vmax(vmax3(xv[0], xv[1], xv[2]), vmax3(xv[3], xv[4], xv[5])));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[e] = __uint_as_float(w[e]);
            vm = vmax(vmax(xv[0], xv[1]), vmax(xv[2], xv[3]));
        }
        if (KEYS) bm[j] = group_max<I::VPB>(vm);
        lm = vmax(lm, vm);
    }

    const float M = group_max<64>(lm);
    const float Mr = (M == kNegInf) ? 0.f : M;
    const float c = -(Mr * kLog2e);
    const float e = fmaf(Mr, kLog2e, c);   // exact: Mr*log2e - RN(Mr*log2e)
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < I::VPL * I::EPV; i += 4) {
        s0 += ex2(fmaf(x[i], kLog2e, c));
        s1 += ex2(fmaf(x[i + 1], kLog2e, c));
        s2 += ex2(fmaf(x[i + 2], kLog2e, c));
        s3 += ex2(fmaf(x[i + 3], kLog2e, c));
    }
    const float s = wave_sum_to_63((s0 + s1) + (s2 + s3));
    if (lane == 63) part[it] = make_float2(M, s * ex2(-e));

    if (KEYS) {
        // lane g*VPB + r holds block r*GPV + g after the select; block b comes
        // from lane (b % GPV)*VPB + b / GPV
        const float mine = select_reg<I::VPL>(bm, lane % I::VPB);
        const int src = (lane % I::GPV) * I::VPB + lane / I::GPV;
        const float kbm = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(mine)));
        const int64_t blk = (int64_t)seg * (kSeg / kBlock) + lane;
        if (blk * kBlock < V) {
            const uint32_t kb = f32_key(kbm);
            if (BF16)
                reinterpret_cast<uint16_t*>(keys)[row * kld + blk] = (uint16_t)(kb >> 16);
            else
                reinterpret_cast<uint32_t*>(keys)[row * kld + blk] = kb;
        }
    }
}

template <bool BF16, bool KEYS>
__global__ __launch_bounds__(kThreads) void k_stage1(const uint8_t* __restrict__ logits, int64_t ld,
                                                     int64_t V, int32_t kld, int32_t P, int64_t nitems,
                                                     float2* __restrict__ part, void* __restrict__ keys) {
    using I = Stage1Item<BF16>;
    constexpr int EPV = I::EPV;
    constexpr int VPL = I::VPL;
    constexpr size_t ESZ = BF16 ? 2 : 4;

    const int lane = threadIdx.x & 63;
    // wave-uniform item arithmetic in scalar registers (item count < 2^32)
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t itu = blockIdx.x * (uint32_t)(kThreads / 64) + wave;
    if ((int64_t)itu >= nitems) return;
    const int64_t it = itu;
    const uint32_t rowu = itu / (uint32_t)P;
    const int64_t row = rowu;
    const int32_t seg = (int32_t)(itu - rowu * (uint32_t)P);
    const int64_t nvec_row = (V + EPV - 1) / EPV;
    const int64_t vb = (int64_t)seg * (kSeg / EPV);
    const bool full = vb + kSeg / EPV <= V / EPV;   // wave-uniform: no element past V
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp) + vb;
    const uint32_t ninf_word = BF16 ? 0xFF80FF80u : 0xFF800000u;

    u32x4 buf[VPL];
    if (full) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) buf[j] = vp[j * 64 + lane];
        // every load issued before any result is used (the scheduler would
        // otherwise hoist the first unpack between them and wait on it)
        __builtin_amdgcn_sched_barrier(0);
        stage1_reduce<BF16, KEYS>(buf, lane, it, row, seg, V, kld, part, keys);
    } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int64_t v = vb + j * 64 + lane;
            buf[j] = u32x4{ninf_word, ninf_word, ninf_word, ninf_word};
            if (v + 1 <= V / EPV) {
                buf[j] = vp[j * 64 + lane];
            } else if (v < nvec_row) {   // the one vector that straddles V
                uint32_t w[4] = {ninf_word, ninf_word, ninf_word, ninf_word};
                for (int e = 0; e < EPV; ++e) {
                    const int64_t i = v * EPV + e;
                    if (i < V) {
                        if (BF16) {
                            const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[i];
                            w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0x0000FFFFu) | (h << 16))
                                                : ((w[e >> 1] & 0xFFFF0000u) | h);
                        } else {
                            w[e] = reinterpret_cast<const uint32_t*>(rowp)[i];
                        }
                    }
                }
                buf[j] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
        stage1_reduce<BF16, KEYS>(buf, lane, it, row, seg, V, kld, part, keys);
    }
}

// ---------------------------------------------------------------------------
// Stage 2 helpers
// ---------------------------------------------------------------------------
struct SelectScratch {
    int32_t hist[256];
    uint64_t prefix;
    int32_t k;
};

// k-th largest (1-based, 1 <= k <= n) of n distinct 64-bit keys held in LDS.
// MSD radix select, 8 bits per pass. Every thread of the workgroup calls it.
// Only used when many candidates tie (e.g. constant rows): heavily repeated
// digits serialise its LDS atomics.
__device__ uint64_t radix_select(const uint64_t* keys, int n, int k, SelectScratch& sc) {
    const int tid = threadIdx.x;
    uint64_t prefix = 0, mask = 0;
    int kk = k;
    for (int shift = 56; shift >= 0; shift -= 8) {
        sc.hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            const uint64_t key = keys[i];
            if ((key & mask) == prefix) atomicAdd(&sc.hist[(key >> shift) & 255], 1);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns digits 255-4l .. 252-4l (descending)
            const int d0 = 255 - 4 * tid;
            const int c0 = sc.hist[d0], c1 = sc.hist[d0 - 1], c2 = sc.hist[d0 - 2], c3 = sc.hist[d0 - 3];
            const int sum = c0 + c1 + c2 + c3;
            int incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(incl, off);
                if (tid >= off) incl += t;
            }
            const int excl = incl - sum;
            if (excl < kk && kk <= incl) {
                int r = kk - excl, d;
                if (r <= c0) {
                    d = d0;
                } else if ((r -= c0) <= c1) {
                    d = d0 - 1;
                } else if ((r -= c1) <= c2) {
                    d = d0 - 2;
                } else {
                    r -= c2;
                    d = d0 - 3;
                }
                sc.prefix = prefix | ((uint64_t)d << shift);
                sc.k = r;
            }
        }
        __syncthreads();
        prefix = sc.prefix;
        kk = sc.k;
        mask |= (uint64_t)0xFF << shift;
    }
    return prefix;
}

// ---------------------------------------------------------------------------
// Wave and workgroup scans on DPP (row shifts, then row broadcasts of lanes
// 15 and 31): no LDS round trips inside a wave. `OP` 0 = add, 1 = max, 2 = min.
// ---------------------------------------------------------------------------
template <int OP>
__device__ inline uint32_t dpp_op(uint32_t a, uint32_t b) {
    return OP == 0 ? a + b : (OP == 1 ? max(a, b) : min(a, b));
}
#define LMH_DPP(v, ctrl, rmask, ident) \
    ((uint32_t)__builtin_amdgcn_update_dpp((int)(ident), (int)(v), ctrl, rmask, 0xF, false))

// Inclusive scan over the 64 lanes of a wave (lane i gets op over lanes 0..i).
template <int OP>
__device__ inline uint32_t wave_scan(uint32_t v) {
    constexpr uint32_t I = OP == 2 ? 0xFFFFFFFFu : 0u;
    v = dpp_op<OP>(v, LMH_DPP(v, 0x111, 0xF, I));   // row_shr:1
    v = dpp_op<OP>(v, LMH_DPP(v, 0x112, 0xF, I));   // row_shr:2
    v = dpp_op<OP>(v, LMH_DPP(v, 0x114, 0xF, I));   // row_shr:4
    v = dpp_op<OP>(v, LMH_DPP(v, 0x118, 0xF, I));   // row_shr:8
    v = dpp_op<OP>(v, LMH_DPP(v, 0x142, 0xA, I));   // row_bcast:15 -> rows 1, 3
    v = dpp_op<OP>(v, LMH_DPP(v, 0x143, 0xC, I));   // row_bcast:31 -> rows 2, 3
    return v;
}
template <int OP>
__device__ inline uint32_t wave_reduce(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan<OP>(v), 63);
}

// Workgroup-wide reduction of N values; every thread gets the results. `buf`
// alternates between two halves on consecutive calls, so one barrier each.
template <int OP, int N>
__device__ inline void block_reduce(uint32_t (&v)[N], uint32_t (*buf)[kThreads / 64][4], int& phase) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_reduce<OP>(v[i]);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) buf[phase][wave][i] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t t = buf[phase][0][i];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) t = dpp_op<OP>(t, buf[phase][w][i]);
        v[i] = t;
    }
    phase ^= 1;
}

// Workgroup-wide exclusive prefix sum in thread order; `total` gets the sum.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* wtot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_scan<0>(v);
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    uint32_t base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const uint32_t sw = wtot[w];
        base += (w < wave) ? sw : 0u;
        total += sw;
    }
    __syncthreads();
    return base + inc - v;
}

// ---------------------------------------------------------------------------
// Stage 2: one workgroup per row.
//  (1) lse from the row's partials (fixed merge order);
//  (2) the selected token's logprob;
//  (3) T = the K-th largest block-max key counted with multiplicity: a 5-way
//      search with exact counts over the key range [lo, max], where lo is the
//      smallest per-thread maximum (at least K keys reach it whenever K
//      threads hold blocks); the kept blocks are all keys above T plus the
//      lowest-indexed keys equal to T, K in all, placed by one prefix scan;
//  (4) one round of 16-byte loads gathers the kept blocks; entries with key
//      >= T become candidates, compacted by a prefix scan;
//  (5) each candidate's rank under (value desc, id asc) is counted in LDS and
//      the first K are written.
// Every thread holds the keys of KPT consecutive blocks in registers.
// ---------------------------------------------------------------------------
template <bool BF16, int KPT>
__global__ __launch_bounds__(kThreads) void k_stage2(const uint8_t* __restrict__ logits, int64_t ld,
                                                     int64_t V, int32_t nb, int32_t kld, int32_t splits,
                                                     const float2* __restrict__ part,
                                                     const void* __restrict__ keys,
                                                     const int32_t* __restrict__ sel, int32_t K,
                                                     float* __restrict__ lse_out,
                                                     float* __restrict__ sel_out,
                                                     int32_t* __restrict__ topk_ids,
                                                     float* __restrict__ topk_lp,
                                                     int32_t* __restrict__ err, int32_t cap) {
    extern __shared__ uint64_t smem[];   // [cap] candidates, [K] narrowed list
    uint64_t* cand = smem;
    uint64_t* list2 = smem + cap;
    __shared__ SelectScratch sc;
    __shared__ uint32_t sred[2][kThreads / 64][4];
    __shared__ uint32_t swtot[kThreads / 64];
    __shared__ float s_lse;
    __shared__ int32_t s_blk[kMaxCandidates / kBlock];
    __shared__ int32_t s_nlist, s_nblk;
    __shared__ uint32_t sh_hist[kHistBins];
    __shared__ uint32_t s_thr[3];
    constexpr size_t ESZ = BF16 ? 2 : 4;
    constexpr int EPV = BF16 ? 8 : 4;                 // elements per 16-byte vector
    constexpr int VPB = kBlock / EPV;                 // vectors per block
    constexpr int MAXV = kMaxCandidates / EPV / kThreads;   // vectors per thread, at most
    constexpr int MAXBLK = kMaxCandidates / kBlock;

    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;
    if (tid < MAXBLK) s_blk[tid] = -1;   // unfilled slots are skipped, never dereferenced

    // this thread's block keys, blocks [b0, b0 + KPT); 0 past nb (every real
    // key is above 0, so a 0 never counts and never ties)
    const int b0 = tid * KPT;
    uint32_t kr[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) kr[j] = 0u;
    if (K > 0 && K <= nb && b0 < nb) {
        if (BF16) {
            const uint16_t* kp = reinterpret_cast<const uint16_t*>(keys) + row * kld + b0;
            if (KPT == 4) {
                const uint2 q = *reinterpret_cast<const uint2*>(kp);
                const uint32_t wq[2] = {q.x, q.y};
#pragma unroll
                for (int j = 0; j < 4; ++j) kr[j] = (j & 1) ? (wq[j >> 1] & 0xFFFF0000u) : (wq[j >> 1] << 16);
            } else {
#pragma unroll
                for (int c = 0; c < KPT / 8; ++c) {
                    const u32x4 q = reinterpret_cast<const u32x4*>(kp)[c];
                    const uint32_t wq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        kr[c * 8 + j] = (j & 1) ? (wq[j >> 1] & 0xFFFF0000u) : (wq[j >> 1] << 16);
                }
            }
        } else {
            const uint32_t* kp = reinterpret_cast<const uint32_t*>(keys) + row * kld + b0;
#pragma unroll
            for (int c = 0; c < KPT / 4; ++c) {
                const u32x4 q = reinterpret_cast<const u32x4*>(kp)[c];
                kr[c * 4 + 0] = q.x;
                kr[c * 4 + 1] = q.y;
                kr[c * 4 + 2] = q.z;
                kr[c * 4 + 3] = q.w;
            }
        }
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (b0 + j >= nb) kr[j] = 0u;
    }

    // the selected token's id, issued now (thread 64: off the lse wave) and
    // used at the end, after the loads have long landed
    const bool sel_thread = sel != nullptr && sel_out != nullptr && tid == 64;
    int32_t sel_id = 0;
    if (sel_thread) sel_id = sel[row];

    // (1) logsumexp: wave 0 merges the row's partials in a fixed order (a
    // strided pass per lane, then a DPP tree into lane 63)
    if (tid < 64) {
        float m = kNegInf, s = 0.f;
        for (int i = tid; i < splits; i += 64) {
            const float2 p = part[row * splits + i];
            lse_merge(m, s, p.x, p.y);
        }
        LMH_LSE_DPP_STEP(m, s, 0x111, 0xF);
        LMH_LSE_DPP_STEP(m, s, 0x112, 0xF);
        LMH_LSE_DPP_STEP(m, s, 0x114, 0xF);
        LMH_LSE_DPP_STEP(m, s, 0x118, 0xF);
        LMH_LSE_DPP_STEP(m, s, 0x142, 0xA);
        LMH_LSE_DPP_STEP(m, s, 0x143, 0xC);
        if (tid == 63) {
            const float l = (m == kNegInf) ? kNegInf : m + logf(s);
            s_lse = l;
            lse_out[row] = l;
            s_nlist = 0;
            s_nblk = 0;
        }
    }
    __syncthreads();
    const float lse = s_lse;

    // (2) selected token: its logit load is issued here and consumed last
    const bool sel_ok = sel_thread && sel_id >= 0 && (int64_t)sel_id < V;
    float xsel = 0.f;
    if (sel_ok)
        xsel = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(rowp)[sel_id])
                    : reinterpret_cast<const float*>(rowp)[sel_id];
    auto write_selected = [&]() {
        if (sel_thread) {
            if (sel_ok) {
                sel_out[row] = xsel - lse;
            } else {
                sel_out[row] = __builtin_nanf("");
                if (err) atomicOr(err, LMH_DEVERR_INDEX);
            }
        }
    };
    if (K == 0) {
        write_selected();
        return;
    }

    if (K == 0) return;

    // (3) threshold and kept blocks
    int phase = 0;
    int nblk;
    uint32_t T = 0;                                     // key threshold (0: keep everything)
    if (K <= nb) {
        uint32_t tmax = 0u, tmin = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            tmax = max(tmax, kr[j]);
            if (b0 + j < nb) tmin = min(tmin, kr[j]);
        }
        // one max-reduction gives the maximum and (complemented) two minima:
        // of all keys, and of the per-thread maxima of threads holding blocks
        uint32_t mm[3] = {tmax, ~tmin, b0 < nb ? ~tmax : 0u};
        block_reduce<1, 3>(mm, sred, phase);
        const int nth = (nb + KPT - 1) / KPT;           // threads holding blocks
        const int sh = BF16 ? 16 : 0;
        // Largest t with count(key >= t) >= K; count(>= lo) >= K > count(>= hi).
        uint64_t lo = (uint64_t)((K <= nth ? ~mm[2] : ~mm[1]) >> sh);
        uint64_t hi = (uint64_t)(mm[0] >> sh) + 1;
        uint32_t c_hi = 0u;                              // count(key >= hi)
        // 5-way narrowing with exact counts until at most 256 key values remain
        while (hi - lo > kHistBins) {
            const uint64_t span = hi - lo;
            uint32_t t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t d = (span * (uint64_t)(i + 1)) / 5;
                t[i] = (uint32_t)(lo + (d < 1 ? 1 : d));
            }
            uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const uint32_t kv = kr[j] >> sh;
#pragma unroll
                for (int i = 0; i < 4; ++i) c[i] += (kv >= t[i]) ? 1u : 0u;
            }
            uint32_t pk[2] = {c[0] | (c[1] << 16), c[2] | (c[3] << 16)};
            block_reduce<0, 2>(pk, sred, phase);
            const uint32_t cc[4] = {pk[0] & 0xFFFFu, pk[0] >> 16, pk[1] & 0xFFFFu, pk[1] >> 16};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (cc[i] >= (uint32_t)K) {
                    if (t[i] > lo) lo = t[i];
                } else if (t[i] < hi) {
                    hi = t[i];
                    c_hi = cc[i];
                }
            }
        }
        // histogram of the keys in [lo, hi), then a suffix scan in wave 0:
        // T is the largest key value v with count(key >= v) >= K
        sh_hist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint64_t kv = kr[j] >> sh;
            if (kv >= lo && kv < hi) atomicAdd(&sh_hist[(int)(kv - lo)], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            const uint32_t h0 = sh_hist[4 * tid], h1 = sh_hist[4 * tid + 1];
            const uint32_t h2 = sh_hist[4 * tid + 2], h3 = sh_hist[4 * tid + 3];
            const uint32_t sum4 = h0 + h1 + h2 + h3;
            const uint32_t incl = wave_scan<0>(sum4);
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            // count(key >= bin 4l + 4) and the four suffix counts inside the lane
            const uint32_t above = c_hi + total - incl;
            const uint32_t s3 = above + h3, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
            const uint32_t k = (uint32_t)K;
            int b = -1;
            uint32_t gt = 0u, eqc = 0u;
            if (s3 >= k && above < k) { b = 4 * tid + 3; gt = above; eqc = h3; }
            else if (s2 >= k && s3 < k) { b = 4 * tid + 2; gt = s3; eqc = h2; }
            else if (s1 >= k && s2 < k) { b = 4 * tid + 1; gt = s2; eqc = h1; }
            else if (s0 >= k && s1 < k) { b = 4 * tid; gt = s1; eqc = h0; }
            if (b >= 0) {
                s_thr[0] = (uint32_t)((lo + (uint64_t)b) << sh);
                s_thr[1] = gt;
                s_thr[2] = eqc;
            }
        }
        __syncthreads();
        T = s_thr[0];
        const int need = K - (int)s_thr[1];             // blocks equal to T that are kept
        const bool all_ties = (uint32_t)need == s_thr[2];
        if (all_ties) {
            // every key >= T is kept: placement order does not matter
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if (kr[j] >= T) {
                    const int pos = atomicAdd(&s_nblk, 1);
                    if (pos < MAXBLK) s_blk[pos] = b0 + j;
                }
        } else {
            // the lowest-indexed keys equal to T are kept: one ordered scan
            uint32_t gt = 0u, eq = 0u;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                gt += (kr[j] > T) ? 1u : 0u;
                eq += (kr[j] == T) ? 1u : 0u;
            }
            uint32_t tot = 0u;
            const uint32_t ex = block_exclusive_scan(gt | (eq << 16), swtot, tot);
            const uint32_t gt_before = ex & 0xFFFFu, eq_before = ex >> 16;
            int pos = (int)gt_before + min(need, (int)eq_before);
            int ei = (int)eq_before;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                bool keep = kr[j] > T;
                if (kr[j] == T) {
                    keep = ei < need;
                    ++ei;
                }
                if (keep) {
                    if (pos < MAXBLK) s_blk[pos] = b0 + j;
                    ++pos;
                }
            }
        }
        nblk = min(K, MAXBLK);
    } else {
        for (int b = tid; b < nb; b += kThreads) s_blk[b] = b;
        nblk = nb;
    }
    __syncthreads();

    // (4) gather the kept blocks in one round of loads; keep entries >= T
    const int nvec = nblk * VPB;
    uint32_t w[MAXV][4];
    int64_t e0[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int j = tid + i * kThreads;
        e0[i] = -1;
        const int blk = j < nvec ? s_blk[j / VPB] : -1;
        if (blk >= 0 && blk < nb) {
            e0[i] = (int64_t)blk * kBlock + (int64_t)(j % VPB) * EPV;
            if (e0[i] + EPV <= V) {
                const u32x4 v4 = *reinterpret_cast<const u32x4*>(rowp + (size_t)e0[i] * ESZ);
                w[i][0] = v4.x; w[i][1] = v4.y; w[i][2] = v4.z; w[i][3] = v4.w;
            } else {
                const uint32_t ninf = BF16 ? 0xFF80FF80u : 0xFF800000u;
                w[i][0] = w[i][1] = w[i][2] = w[i][3] = ninf;
                for (int e = 0; e < EPV; ++e) {
                    const int64_t idx = e0[i] + e;
                    if (idx < V) {
                        if (BF16) {
                            const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[idx];
                            w[i][e >> 1] = (e & 1) ? ((w[i][e >> 1] & 0x0000FFFFu) | (h << 16))
                                                   : ((w[i][e >> 1] & 0xFFFF0000u) | h);
                        } else {
                            w[i][e] = reinterpret_cast<const uint32_t*>(rowp)[idx];
                        }
                    }
                }
            }
        }
    }
    // key >= T  <=>  x >= Tf for the values this row can hold (T == 0: all)
    const bool keep_all = T == 0u;
    const float Tf = keep_all ? kNegInf : key_value<BF16>(T);
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        if (e0[i] < 0) continue;
        const bool vfull = e0[i] + EPV <= V;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = BF16 ? ((e & 1) ? bf16_hi(w[i][e >> 1]) : bf16_lo(w[i][e >> 1]))
                                 : __uint_as_float(w[i][e]);
            cnt += ((vfull || e0[i] + e < V) && (keep_all || x >= Tf)) ? 1u : 0u;
        }
    }
    uint32_t ncand_u = 0;
    int cpos = (int)block_exclusive_scan(cnt, swtot, ncand_u);
    const int ncand = min((int)ncand_u, cap);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        if (e0[i] < 0) continue;
        const bool vfull = e0[i] + EPV <= V;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = BF16 ? ((e & 1) ? bf16_hi(w[i][e >> 1]) : bf16_lo(w[i][e >> 1]))
                                 : __uint_as_float(w[i][e]);
            const int64_t v = e0[i] + e;
            if ((vfull || v < V) && (keep_all || x >= Tf)) {
                if (cpos < cap)
                    cand[cpos] = ((uint64_t)elem_key<BF16>(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
                ++cpos;
            }
        }
    }
    __syncthreads();

    // (5) exact top-K by rank under the composite (value key, ~id) order
    const uint64_t* list = cand;
    int nlist = ncand;
    if (ncand > kThreads && ncand > K) {
        const uint64_t thr2 = radix_select(cand, ncand, K, sc);
        for (int i = tid; i < ncand; i += kThreads) {
            const uint64_t c = cand[i];
            if (c >= thr2) {
                const int q = atomicAdd(&s_nlist, 1);
                if (q < K) list2[q] = c;
            }
        }
        __syncthreads();
        list = list2;
        nlist = K;
    }
    // G lanes (a quad, a pair or one lane) count one candidate's predecessors
    // over interleaved slices of the list, then sum with DPP inside the quad
    const int G = nlist <= kThreads / 4 ? 4 : (nlist <= kThreads / 2 ? 2 : 1);
    const int q = tid & (G - 1);
    for (int i0 = 0; i0 < nlist * G; i0 += kThreads) {
        const int i = (i0 + tid) / G;
        const bool act = i0 + tid < nlist * G;
        const uint64_t c = act ? list[i] : 0ull;
        uint32_t rank = 0;
        if (act) {
            int j = q;
            for (; j + 7 * G < nlist; j += 8 * G) {
                uint64_t v8[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v8[u] = list[j + u * G];
#pragma unroll
                for (int u = 0; u < 8; ++u) rank += (v8[u] > c) ? 1u : 0u;
            }
            for (; j < nlist; j += G) rank += (list[j] > c) ? 1u : 0u;
        }
        if (G >= 2) rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0xB1, 0xF, 0xF, false);
        if (G == 4) rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0x4E, 0xF, 0xF, false);
        if (act && q == 0 && rank < (uint32_t)K) {
            topk_ids[row * K + rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
            topk_lp[row * K + rank] = key_value<BF16>((uint32_t)(c >> 32)) - lse;
        }
    }
    write_selected();
}

}  // namespace

ReducePlan plan_reduce(int64_t rows, int64_t vocab, int32_t k) {
    ReducePlan p{};
    p.rows = rows;
    p.vocab = vocab;
    p.k = k;
    p.nb = (int32_t)((vocab + kBlock - 1) / kBlock);
    p.kpt = 4;
    while (p.kpt * kThreads < p.nb && p.kpt < kMaxCandidates / kThreads) p.kpt *= 2;
    // stage 2 reads KPT keys per thread with 16-byte loads, so a key row spans
    // every thread's range; beyond the stage-2 limit only stage 1 touches keys
    p.kld = p.nb <= kMaxCandidates ? p.kpt * kThreads : (p.nb + 7) / 8 * 8;
    p.splits = (int32_t)((vocab + kSeg - 1) / kSeg);            // partials per row
    p.nitems = rows * (int64_t)p.splits;
    // one item per wave: short waves dispatched in address order keep the
    // active set on a compact stretch of memory, which streams fastest
    p.wgs = (p.nitems + kThreads / 64 - 1) / (kThreads / 64);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p.part_off = 0;
    p.keys_off = up((size_t)p.nitems * sizeof(float2));
    p.bytes = p.keys_off + up((size_t)rows * p.kld * sizeof(uint32_t));
    if (p.bytes == 0) p.bytes = 256;
    return p;
}

hipError_t launch_reduce_stage1(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    char* ws = static_cast<char*>(a.ws);
    float2* part = reinterpret_cast<float2*>(ws + p.part_off);
    void* keys = p.k > 0 ? ws + p.keys_off : nullptr;   // block maxima only feed the top-K
    const dim3 grid((unsigned)p.wgs);
    const uint8_t* lg = static_cast<const uint8_t*>(a.logits);
    const bool k = keys != nullptr;
    if (a.bf16 && k)
        hipLaunchKernelGGL((k_stage1<true, true>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.kld,
                           p.splits, p.nitems, part, keys);
    else if (a.bf16)
        hipLaunchKernelGGL((k_stage1<true, false>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.kld,
                           p.splits, p.nitems, part, keys);
    else if (k)
        hipLaunchKernelGGL((k_stage1<false, true>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.kld,
                           p.splits, p.nitems, part, keys);
    else
        hipLaunchKernelGGL((k_stage1<false, false>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.kld,
                           p.splits, p.nitems, part, keys);
    return hipGetLastError();
}

template <bool BF16, int KPT>
hipError_t launch_stage2_kpt(const ReducePlan& p, const ReduceArgs& a, hipStream_t s, const float2* part,
                             const void* keys, int32_t cap, size_t lds) {
    const void* fn = (const void*)k_stage2<BF16, KPT>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_stage2<BF16, KPT>), dim3((unsigned)p.rows), dim3(kThreads), lds, s,
                       static_cast<const uint8_t*>(a.logits), a.ld, p.vocab, p.nb, p.kld, p.splits, part,
                       keys, a.sel, p.k, a.lse, a.sel_lp, a.topk_ids, a.topk_lp, a.err, cap);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_stage2_dt(const ReducePlan& p, const ReduceArgs& a, hipStream_t s, const float2* part,
                            const void* keys, int32_t cap, size_t lds) {
    switch (p.kpt) {
        case 4: return launch_stage2_kpt<BF16, 4>(p, a, s, part, keys, cap, lds);
        case 8: return launch_stage2_kpt<BF16, 8>(p, a, s, part, keys, cap, lds);
        case 16: return launch_stage2_kpt<BF16, 16>(p, a, s, part, keys, cap, lds);
        default: return launch_stage2_kpt<BF16, 32>(p, a, s, part, keys, cap, lds);
    }
}

hipError_t launch_reduce_stage2(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    char* ws = static_cast<char*>(a.ws);
    const float2* part = reinterpret_cast<const float2*>(ws + p.part_off);
    const void* keys = ws + p.keys_off;
    int32_t cap = 0;
    size_t lds = 0;
    if (p.k > 0) {
        const int32_t nsel = p.k < p.nb ? p.k : p.nb;
        cap = nsel * kBlock;
        lds = ((size_t)cap + (size_t)p.k) * sizeof(uint64_t);
    }
    return a.bf16 ? launch_stage2_dt<true>(p, a, s, part, keys, cap, lds)
                  : launch_stage2_dt<false>(p, a, s, part, keys, cap, lds);
}

}  // namespace lmh
