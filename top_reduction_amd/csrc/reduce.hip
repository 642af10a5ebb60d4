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
constexpr int kUnroll = 4;        // 16-byte loads in flight per lane
constexpr int kTargetWgs = 2048;  // stage-1 workgroups to aim for (8 per CU)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over lane groups of 8 (quad swap, quad pair swap, half-row mirror) and,
// for 16, the row mirror. Every lane of a group ends with the group maximum.
__device__ inline float dpp_max8(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    return v;
}
__device__ inline float dpp_max16(float v) {
    v = dpp_max8(v);
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
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
// Stage 1
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_stage1(const uint8_t* __restrict__ logits, int64_t ld,
                                                     int64_t V, int32_t nb, int32_t bps,
                                                     int32_t splits, float2* __restrict__ part,
                                                     void* __restrict__ keys) {
    constexpr int EPV = BF16 ? 8 : 4;    // elements per 16-byte vector
    constexpr int VPB = kBlock / EPV;    // vectors (lanes) per 64-logit block
    constexpr size_t ESZ = BF16 ? 2 : 4;
    const int64_t wg = blockIdx.x;
    const int64_t row = wg / splits;
    const int32_t split = (int32_t)(wg - row * splits);
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    const int32_t b0 = split * bps;
    const int32_t b1 = min(nb, b0 + bps);
    const int64_t nvec_row = (V + EPV - 1) / EPV;
    const int64_t vb = (int64_t)b0 * VPB;
    const int64_t ve = min((int64_t)b1 * VPB, nvec_row);
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp);
    const int64_t ragged_vec = (V % EPV) ? nvec_row - 1 : -1;
    const uint32_t ninf_word = BF16 ? 0xFF80FF80u : 0xFF800000u;

    float m = kNegInf, s = 0.f;
    const int64_t n = ve - vb;
    for (int64_t base = 0; base < n; base += (int64_t)kThreads * kUnroll) {
        u32x4 buf[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t v = vb + base + u * kThreads + tid;
            buf[u] = u32x4{ninf_word, ninf_word, ninf_word, ninf_word};
            if (v < ve) {
                if (v != ragged_vec) {
                    buf[u] = vp[v];
                } else {
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
                    buf[u] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t v = vb + base + u * kThreads + tid;
            float x[EPV];
            const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
            if (BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = bf16_lo(w[e]);
                    x[2 * e + 1] = bf16_hi(w[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
            }
            float lm = x[0];
#pragma unroll
            for (int e = 1; e < EPV; ++e) lm = fmaxf(lm, x[e]);

            // block maximum over the VPB lanes of this 64-logit block
            const float bm = BF16 ? dpp_max8(lm) : dpp_max16(lm);
            if ((lane & (VPB - 1)) == 0 && v < ve) {
                const int64_t blk = v / VPB;
                if (BF16)
                    reinterpret_cast<uint16_t*>(keys)[row * nb + blk] = (uint16_t)(f32_key(bm) >> 16);
                else
                    reinterpret_cast<uint32_t*>(keys)[row * nb + blk] = f32_key(bm);
            }

            // online (max, sum-exp); a rescale by exp2(0) is exactly 1
            const float mn = fmaxf(m, lm);
            const float mr = (mn == kNegInf) ? 0.f : mn;
            float acc = s * ex2((m - mr) * kLog2e);
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc += ex2((x[e] - mr) * kLog2e);
            s = acc;
            m = mn;
        }
    }

    // workgroup combine in a fixed order: butterfly in each wave, then waves 0..3
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const float s2 = __shfl_xor(s, off);
        lse_merge(m, s, m2, s2);
    }
    __shared__ float2 wpart[kThreads / 64];
    if (lane == 0) wpart[tid >> 6] = make_float2(m, s);
    __syncthreads();
    if (tid == 0) {
        float M = wpart[0].x, S = wpart[0].y;
        for (int w = 1; w < kThreads / 64; ++w) lse_merge(M, S, wpart[w].x, wpart[w].y);
        part[row * splits + split] = make_float2(M, S);
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
// Stage 2
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_stage2(const uint8_t* __restrict__ logits, int64_t ld,
                                                     int64_t V, int32_t nb, int32_t splits,
                                                     const float2* __restrict__ part,
                                                     const void* __restrict__ keys,
                                                     const int32_t* __restrict__ sel, int32_t K,
                                                     float* __restrict__ lse_out,
                                                     float* __restrict__ sel_out,
                                                     int32_t* __restrict__ topk_ids,
                                                     float* __restrict__ topk_lp,
                                                     int32_t* __restrict__ err, int32_t region) {
    extern __shared__ uint64_t smem[];   // [region] keys/candidates, then [K] narrowed list
    __shared__ SelectScratch sc;
    __shared__ float s_lse;
    __shared__ int32_t s_blk[kMaxCandidates / kBlock];
    __shared__ int32_t s_nblk, s_ncand, s_nlist;
    constexpr size_t ESZ = BF16 ? 2 : 4;

    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;

    // (1) logsumexp: wave 0 merges the split partials in a fixed order
    if (tid < 64) {
        float m = kNegInf, s = 0.f;
        for (int i = tid; i < splits; i += 64) {
            const float2 p = part[row * splits + i];
            lse_merge(m, s, p.x, p.y);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float m2 = __shfl_xor(m, off);
            const float s2 = __shfl_xor(s, off);
            lse_merge(m, s, m2, s2);
        }
        if (tid == 0) {
            const float l = (m == kNegInf) ? kNegInf : m + logf(s);
            s_lse = l;
            lse_out[row] = l;
            s_nblk = 0;
            s_ncand = 0;
            s_nlist = 0;
        }
    }
    __syncthreads();
    const float lse = s_lse;

    // (2) selected token
    if (sel != nullptr && sel_out != nullptr && tid == 0) {
        const int32_t id = sel[row];
        float lp;
        if (id < 0 || (int64_t)id >= V) {
            lp = __builtin_nanf("");
            if (err) atomicOr(err, LMH_DEVERR_INDEX);
        } else {
            const float x = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(rowp)[id])
                                 : reinterpret_cast<const float*>(rowp)[id];
            lp = x - lse;
        }
        sel_out[row] = lp;
    }
    if (K == 0) return;

    // (3) block selection: composite key (block max key, ~block) makes ties
    // resolve to the lower block index
    uint64_t* comp = smem;
    for (int b = tid; b < nb; b += kThreads) {
        const uint32_t kb = BF16 ? ((uint32_t)reinterpret_cast<const uint16_t*>(keys)[row * nb + b] << 16)
                                 : reinterpret_cast<const uint32_t*>(keys)[row * nb + b];
        comp[b] = ((uint64_t)kb << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)b);
    }
    __syncthreads();
    uint64_t thr = 0;
    uint32_t tkey = 0;   // candidate threshold on the value key (0: everything)
    if (K <= nb) {
        thr = radix_select(comp, nb, K, sc);
        tkey = (uint32_t)(thr >> 32);
    }
    for (int b = tid; b < nb; b += kThreads) {
        if (comp[b] >= thr) s_blk[atomicAdd(&s_nblk, 1)] = b;
    }
    __syncthreads();
    const int nblk = s_nblk;

    // (4) candidates: entries of kept blocks whose key is >= tkey
    uint64_t* cand = smem;
    for (int j = wave; j < nblk; j += kThreads / 64) {
        const int64_t v = (int64_t)s_blk[j] * kBlock + lane;
        bool keep = false;
        uint64_t c = 0;
        if (v < V) {
            const float x = BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(rowp)[v])
                                 : reinterpret_cast<const float*>(rowp)[v];
            const uint32_t kx = elem_key<BF16>(x);
            keep = kx >= tkey;
            c = ((uint64_t)kx << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
        }
        const uint64_t ball = __ballot(keep);
        int basepos = 0;
        if (lane == 0) basepos = atomicAdd(&s_ncand, (int)__popcll(ball));
        basepos = __shfl(basepos, 0);
        if (keep) cand[basepos + (int)__popcll(ball & ((1ull << lane) - 1ull))] = c;
    }
    __syncthreads();
    const int ncand = s_ncand;

    // (5) narrow to exactly K when there are many candidates
    const uint64_t* list = cand;
    int nlist = ncand;
    if (ncand > kThreads && ncand > K) {
        const uint64_t thr2 = radix_select(cand, ncand, K, sc);
        uint64_t* list2 = smem + region;
        for (int i = tid; i < ncand; i += kThreads) {
            const uint64_t c = cand[i];
            if (c >= thr2) list2[atomicAdd(&s_nlist, 1)] = c;
        }
        __syncthreads();
        list = list2;
        nlist = K;
    }

    // (6) rank by (value desc, id asc) == composite descending; write top-K
    for (int i = tid; i < nlist; i += kThreads) {
        const uint64_t c = list[i];
        int rank = 0;
        for (int j = 0; j < nlist; ++j) rank += (list[j] > c) ? 1 : 0;
        if (rank < K) {
            const int32_t id = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
            topk_ids[row * K + rank] = id;
            topk_lp[row * K + rank] = key_value<BF16>((uint32_t)(c >> 32)) - lse;
        }
    }
}

}  // namespace

ReducePlan plan_reduce(int64_t rows, int64_t vocab, int32_t k) {
    ReducePlan p{};
    p.rows = rows;
    p.vocab = vocab;
    p.k = k;
    p.nb = (int32_t)((vocab + kBlock - 1) / kBlock);
    int64_t splits = rows > 0 ? (kTargetWgs + rows - 1) / rows : 1;
    const int64_t max_splits = (p.nb + 7) / 8;   // at least 8 blocks per split
    splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
    p.bps = (int32_t)((p.nb + splits - 1) / splits);
    p.splits = (int32_t)((p.nb + p.bps - 1) / p.bps);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p.part_off = 0;
    p.keys_off = up((size_t)rows * p.splits * sizeof(float2));
    p.bytes = p.keys_off + up((size_t)rows * p.nb * sizeof(uint32_t));
    if (p.bytes == 0) p.bytes = 256;
    return p;
}

hipError_t launch_reduce_stage1(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    char* ws = static_cast<char*>(a.ws);
    float2* part = reinterpret_cast<float2*>(ws + p.part_off);
    void* keys = ws + p.keys_off;
    const dim3 grid((unsigned)(p.rows * p.splits));
    const uint8_t* lg = static_cast<const uint8_t*>(a.logits);
    if (a.bf16)
        hipLaunchKernelGGL(k_stage1<true>, grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.nb, p.bps,
                           p.splits, part, keys);
    else
        hipLaunchKernelGGL(k_stage1<false>, grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.nb, p.bps,
                           p.splits, part, keys);
    return hipGetLastError();
}

hipError_t launch_reduce_stage2(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    char* ws = static_cast<char*>(a.ws);
    const float2* part = reinterpret_cast<const float2*>(ws + p.part_off);
    const void* keys = ws + p.keys_off;
    int32_t region = 0;
    size_t lds = 0;
    if (p.k > 0) {
        const int32_t nsel = p.k < p.nb ? p.k : p.nb;
        const int32_t cap = nsel * kBlock;
        region = p.nb > cap ? p.nb : cap;
        lds = ((size_t)region + (size_t)p.k) * sizeof(uint64_t);
    }
    const uint8_t* lg = static_cast<const uint8_t*>(a.logits);
    if (a.bf16) {
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute((const void*)k_stage2<true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_stage2<true>, dim3((unsigned)p.rows), dim3(kThreads), lds, s, lg, a.ld,
                           p.vocab, p.nb, p.splits, part, keys, a.sel, p.k, a.lse, a.sel_lp,
                           a.topk_ids, a.topk_lp, a.err, region);
    } else {
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute((const void*)k_stage2<false>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_stage2<false>, dim3((unsigned)p.rows), dim3(kThreads), lds, s, lg, a.ld,
                           p.vocab, p.nb, p.splits, part, keys, a.sel, p.k, a.lse, a.sel_lp,
                           a.topk_ids, a.topk_lp, a.err, region);
    }
    return hipGetLastError();
}

}  // namespace lmh
