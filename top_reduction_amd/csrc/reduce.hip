// reduce.hip -- per-row logsumexp, selected logprob and exact top-K of a
// logits matrix, on gfx950 (MTPLX PR #532, Change; openinfer issue #719,
// Suggested direction).
//
// Every logit is read once, with 16-byte loads, in 4096-logit items. An item
// yields a (max, sum of exp(x - max)) partial in fp32 and the maximum of each
// of its 64-logit blocks, as a monotone key (16-bit for bf16 rows, 32-bit for
// fp32 rows). The partials of a row are merged in one canonical order into
// the fp32 logsumexp; the min(K, nb) blocks with the largest maxima (equal
// maxima: lower block index first) are kept, the entries of those blocks
// that are not below the K-th kept maximum are gathered, and they are ranked
// by (value descending, id ascending) in LDS. The candidate set provably
// contains the exact top-K: a top-K entry outside the kept blocks, or below
// the K-th kept maximum, would have K kept block maxima ahead of it. With
// 16-bit logits, when few blocks reach the K-th largest maximum, all of them
// are kept (a superset; ties at that maximum need no ordering then), taken
// from blocks each thread prefetched while the threshold was searched.
//
// Two paths, with bitwise-identical results:
//   * k_rowreduce (rows fill the CUs evenly): one workgroup per row streams
//     the row, keeps the block keys in LDS and selects in the same launch;
//   * k_stage1 + k_stage2 (otherwise): a streaming launch over all rows
//     writes partials and keys to the workspace, then one workgroup per row
//     finishes it.
#include <type_traits>

#include "lmh_internal.h"

namespace lmh {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = 256;
constexpr int kHistBins = 256;     // key values resolved by one stage-2 histogram
constexpr int kSeg = 4096;          // logits per streaming work item (one wave)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Logits element types. Both 16-bit types stream 8 elements per 16-byte vector
// and keep 16-bit block keys (in the top half of a 32-bit key).
constexpr int kDtF32 = LMH_F32, kDtBf16 = LMH_BF16, kDtF16 = LMH_F16;
constexpr bool w16(int dt) { return dt != kDtF32; }

__device__ inline float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// The low and high 16-bit elements of a word as fp32 (exact).
template <int DT>
__device__ inline float lo16(uint32_t w) {
    return DT == kDtBf16 ? bf16_lo(w) : f16_bits_to_f32(w & 0xFFFFu);
}
template <int DT>
__device__ inline float hi16(uint32_t w) {
    return DT == kDtBf16 ? bf16_hi(w) : f16_bits_to_f32(w >> 16);
}
// One element of a 16-bit row.
template <int DT>
__device__ inline float elem16(const uint8_t* rowp, int64_t i) {
    const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[i];
    return DT == kDtBf16 ? bf16_to_f32((uint16_t)h) : f16_bits_to_f32(h);
}
// -inf in both halves of a word (16-bit types) or the word (fp32)
template <int DT>
constexpr uint32_t ninf_word() {
    return DT == kDtBf16 ? 0xFF80FF80u : (DT == kDtF16 ? 0xFC00FC00u : 0xFF800000u);
}

// Block keys: a monotone map of the block maximum, -0 folded into +0. fp32:
// the 32-bit key; bf16: its top 16 bits (exact for a bf16 value); f16: the
// 16-bit key of the f16 bits, in the top half.
template <int DT>
__device__ inline uint32_t block_key(float x) {
    if (DT == kDtF16) {
        uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)x);   // exact: x is an f16 value
        h = (x == 0.0f) ? 0u : h;
        return ((h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u)) << 16;
    }
    return DT == kDtBf16 ? (f32_key(x) & 0xFFFF0000u) : f32_key(x);
}
template <int DT>
__device__ inline float block_value(uint32_t k) {
    if (DT == kDtF32) return key_f32(k);
    const uint32_t k16 = k >> 16;
    const uint32_t b = (k16 & 0x8000u) ? (k16 & 0x7FFFu) : (~k16 & 0xFFFFu);
    return DT == kDtBf16 ? __uint_as_float(b << 16) : f16_bits_to_f32(b);
}
// Candidate keys (ranking among a row's candidates): the block key for bf16,
// the full 32-bit key otherwise.
template <int DT>
__device__ inline uint32_t elem_key(float x) {
    return DT == kDtBf16 ? (f32_key(x) & 0xFFFF0000u) : f32_key(x);
}
template <int DT>
__device__ inline float elem_value(uint32_t k) {
    return DT == kDtBf16 ? block_value<kDtBf16>(k) : key_f32(k);
}

// ---------------------------------------------------------------------------
// Stage 1: a row is cut into fixed segments of kSeg logits (the last one
// partial), the work items. Lane l of a wave reads an item's 16-byte vectors
// l, l + 64, ...; all of an item's loads are in flight before its first vector
// is used, and the item's 64 logits per lane stay in registers for two passes:
//   1. the maximum of each lane's slice of every 64-logit block (the 8 bf16 or
//      16 fp32 lanes of a block then combine it with DPP), and of the lane;
//   2. with M the wave maximum, the sum of 2^(x*log2e + c) for c = -RN(M*log2e):
//      one fma, one exp2 and one add per logit. The rounding of c is the
//      exactly representable e = M*log2e + c (an fma), and the sum is scaled
//      by 2^-e once, so the partial is (M, sum of exp(x - M)) to fp32 rounding.
// The lane sums are added by a fixed DPP tree. The block maxima are transposed
// across the wave (a register select, then ds_bpermute) so that lane b holds
// block b. The item partials of a row are merged in one canonical order:
// item i joins merge group i mod 16, each group merges its items in
// ascending order, and the 16 groups are merged as a pairwise tree (one lane
// per group, lower groups on the left). Both reduction
// paths (the split one and the one-workgroup-per-row one) use exactly this
// arithmetic, so each row's results are bitwise independent of the batch
// around it and of the path that served it.
// ---------------------------------------------------------------------------
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

template <int DT>
struct Stage1Item {
    static constexpr int EPV = w16(DT) ? 8 : 4;          // elements per 16-byte vector
    static constexpr int VPB = kBlock / EPV;          // lanes per 64-logit block
    static constexpr int VPL = kSeg / EPV / 64;       // vectors per lane (== VPB)
    static constexpr int GPV = 64 / VPB;              // blocks per wave-wide vector
    static_assert(VPL == VPB, "one block maximum per vector and lane group");
};

// Reduces one item held in buf (VPL vectors per lane; entries past V hold
// -inf) and writes its partial and block keys.
constexpr int kGroups = 16;   // merge groups of a row's item partials

// Reduces one item held in buf (VPL vectors per lane; entries past V hold
// -inf): M and S (the item's max and its sum of exp(x - M)) come back
// wave-uniform; with KEYS, kb is the monotone key of block seg*64 + lane.
template <int DT, bool KEYS>
__device__ __forceinline__ void stage1_item(const u32x4 (&buf)[Stage1Item<DT>::VPL], int lane, float& M,
                                            float& S, uint32_t& kb) {
    using I = Stage1Item<DT>;
    float x[I::VPL * I::EPV];
    float bm[I::VPL];
    float lm = kNegInf;
#pragma unroll
    for (int j = 0; j < I::VPL; ++j) {
        const uint32_t w[4] = {buf[j].x, buf[j].y, buf[j].z, buf[j].w};
        float* xv = x + j * I::EPV;
        float vm;
        if (w16(DT)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[2 * e] = lo16<DT>(w[e]);
                xv[2 * e + 1] = hi16<DT>(w[e]);
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

    M = group_max<64>(lm);
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
    const float s63 = wave_sum_to_63((s0 + s1) + (s2 + s3));
    S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s63), 63)) * ex2(-e);

    if (KEYS) {
        // lane g*VPB + r holds block r*GPV + g after the select; block b comes
        // from lane (b % GPV)*VPB + b / GPV
        const float mine = select_reg<I::VPL>(bm, lane % I::VPB);
        const int src = (lane % I::GPV) * I::VPB + lane / I::GPV;
        kb = block_key<DT>(__int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(mine))));
    }
}

// Loads full item `seg` of a row into buf: one 16-byte load per vector.
template <int DT>
__device__ __forceinline__ void stage1_load_full(const uint8_t* rowp, int32_t seg, int lane,
                                                 u32x4 (&buf)[Stage1Item<DT>::VPL]) {
    using I = Stage1Item<DT>;
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp) + (int64_t)seg * (kSeg / I::EPV);
#pragma unroll
    for (int j = 0; j < I::VPL; ++j) buf[j] = vp[j * 64 + lane];
}

// Loads item `seg` of a row into buf. Full items: one 16-byte load per vector,
// all issued before any is used. The partial last item fills entries past V
// with -inf (16-byte loads up to the last whole vector, then elementwise).
template <int DT>
__device__ __forceinline__ bool stage1_load(const uint8_t* rowp, int64_t V, int32_t seg, int lane,
                                            u32x4 (&buf)[Stage1Item<DT>::VPL]) {
    using I = Stage1Item<DT>;
    constexpr int EPV = I::EPV;
    const int64_t vb = (int64_t)seg * (kSeg / EPV);
    const bool full = vb + kSeg / EPV <= V / EPV;   // wave-uniform: no element past V
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp) + vb;
    if (full) {
#pragma unroll
        for (int j = 0; j < I::VPL; ++j) buf[j] = vp[j * 64 + lane];
        return true;
    }
    // all whole-vector loads issued unguarded (addresses clamped to the last
    // whole vector), then entries past V replaced by -inf; only the vector
    // that straddles V (when V is not a multiple of EPV) is read elementwise
    constexpr uint32_t ninf_w = ninf_word<DT>();
    const int64_t nwhole = V / EPV;                     // whole vectors in the row
    const u32x4* rv = reinterpret_cast<const u32x4*>(rowp);
    if (nwhole > 0) {
#pragma unroll
        for (int j = 0; j < I::VPL; ++j) {
            const int64_t v = vb + j * 64 + lane;
            buf[j] = rv[v < nwhole ? v : nwhole - 1];
        }
    }
#pragma unroll
    for (int j = 0; j < I::VPL; ++j) {
        const int64_t v = vb + j * 64 + lane;
        if (v >= nwhole) {
            uint32_t w[4] = {ninf_w, ninf_w, ninf_w, ninf_w};
            if (v == nwhole) {   // the vector that straddles V, if any
                for (int e = 0; e < EPV; ++e) {
                    const int64_t i = v * EPV + e;
                    if (i < V) {
                        if (w16(DT)) {
                            const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[i];
                            w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0x0000FFFFu) | (h << 16))
                                                : ((w[e >> 1] & 0xFFFF0000u) | h);
                        } else {
                            w[e] = reinterpret_cast<const uint32_t*>(rowp)[i];
                        }
                    }
                }
            }
            buf[j] = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
    return false;
}

// Split path, first kernel: one item per wave over all rows, items numbered
// row-major so that consecutively dispatched waves stream consecutive memory;
// writes each item's partial and its block keys to the workspace.
template <int DT, bool KEYS>
__global__ __launch_bounds__(kThreads) void k_stage1(const uint8_t* __restrict__ logits, int64_t ld,
                                                     int64_t V, int32_t kld, int32_t P, int64_t nitems,
                                                     float2* __restrict__ part, void* __restrict__ keys) {
    using I = Stage1Item<DT>;
    constexpr size_t ESZ = w16(DT) ? 2 : 4;
    const int lane = threadIdx.x & 63;
    // wave-uniform item arithmetic in scalar registers (item count < 2^32)
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t itu = blockIdx.x * (uint32_t)(kThreads / 64) + wave;
    if ((int64_t)itu >= nitems) return;
    const uint32_t rowu = itu / (uint32_t)P;
    const int64_t row = rowu;
    const int32_t seg = (int32_t)(itu - rowu * (uint32_t)P);
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;

    u32x4 buf[I::VPL];
    float M, S;
    uint32_t kb = 0;
    if (stage1_load<DT>(rowp, V, seg, lane, buf)) {
        // every load issued before any result is used (the scheduler would
        // otherwise hoist the first unpack between them and wait on it)
        __builtin_amdgcn_sched_barrier(0);
        stage1_item<DT, KEYS>(buf, lane, M, S, kb);
    } else {
        stage1_item<DT, KEYS>(buf, lane, M, S, kb);
    }
    if (lane == 0) part[itu] = make_float2(M, S);
    if (KEYS) {
        const int64_t blk = (int64_t)seg * (kSeg / kBlock) + lane;
        if (blk * kBlock < V) {
            if (w16(DT))
                reinterpret_cast<uint16_t*>(keys)[row * kld + blk] = (uint16_t)(kb >> 16);
            else
                reinterpret_cast<uint32_t*>(keys)[row * kld + blk] = kb;
        }
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
template <int NT>
__device__ uint64_t radix_select(const uint64_t* keys, int n, int k, SelectScratch& sc) {
    const int tid = threadIdx.x;
    uint64_t prefix = 0, mask = 0;
    int kk = k;
    for (int shift = 56; shift >= 0; shift -= 8) {
        if (tid < 256) sc.hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
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
template <int OP, int N, int NT>
__device__ inline void block_reduce(uint32_t (&v)[N], uint32_t (*buf)[NT / 64][4], int& phase) {
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
        for (int w = 1; w < NT / 64; ++w) t = dpp_op<OP>(t, buf[phase][w][i]);
        v[i] = t;
    }
    phase ^= 1;
}

// Workgroup-wide exclusive prefix sum in thread order; `total` gets the sum.
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* wtot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_scan<0>(v);
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    uint32_t base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t sw = wtot[w];
        base += (w < wave) ? sw : 0u;
        total += sw;
    }
    __syncthreads();
    return base + inc - v;
}

// ---------------------------------------------------------------------------
// Top-K of one row by NT threads (steps a6, a7):
//  * T = the K-th largest block-max key counted with multiplicity: a 5-way
//    search with exact counts over the key range [lo, max], where lo is the
//    smallest per-thread maximum (at least K keys reach it whenever K threads
//    hold blocks), finished by a 256-bin LDS histogram; the kept blocks are
//    all keys above T plus the lowest-indexed keys equal to T, K in all;
//  * the search runs on the keys' top 16 bits (all of a 16-bit key). For
//    fp32 logits, when the blocks with keys at or above the 16-bit bin of
//    the K-th key fit the candidate list whole (at most 2K blocks, 128 at
//    most) and that bin holds finite values, T is the bin's
//    lower edge and all of those blocks are kept (K or more); otherwise a
//    second search inside the bin on full keys gives the exact T. Every
//    bin-wide search step is a barrier round, so this skips the several
//    rounds that full 32-bit keys take to narrow;
//  * one round of 16-byte loads gathers the kept blocks; entries with key
//    >= T become candidates, compacted by a prefix scan;
//  * with PF (16-bit logits), each thread loads the block holding its own
//    largest key as soon as the keys are known, so those loads land while
//    T is searched (eight lanes load the eight 16-byte parts of a block, so
//    a wave instruction reads eight whole blocks); every block >= T is a
//    candidate block when at most capb blocks reach T, else the K kept
//    blocks above (one prefix count orders the blocks tied at T); the
//    candidate blocks are copied from those registers to an LDS staging
//    area (the other candidate blocks are loaded then, by all threads in
//    one round) and filtered there by all threads, instead of the
//    placement and gather above;
//  * each candidate's rank under (value desc, id asc) is counted in LDS and
//    the first K are written.
// Thread t holds the keys of blocks [t*KPT, t*KPT + KPT) in kr (0 past nb: a
// 0 never counts and never ties, every real key being above it).
// ---------------------------------------------------------------------------
template <int NT>
struct RowShared {
    SelectScratch sc;
    uint32_t sred[2][NT / 64][4];
    uint32_t swtot[NT / 64];
    int32_t blk[kMaxCandidates / kBlock];
    int32_t cslot[kMaxCandidates / kBlock];   // staging slot of each candidate block (PF path)
    int32_t nlist, nblk;
    uint32_t hist[kHistBins];
    uint32_t thr[3];
    int32_t ncand;
    float lse;
};

// (5) exact top-K of the ncand candidates by rank under the composite
// (value key, ~id) order; logprobs against the row's lse.
template <int DT, int NT>
__device__ __forceinline__ void rank_topk(int64_t row, int32_t K, uint64_t* cand, int ncand, uint64_t* list2,
                          RowShared<NT>& sh, int32_t* __restrict__ topk_ids, float* __restrict__ topk_lp,
                          const float* lse_p, const int32_t* lse_ready) {
    const int tid = threadIdx.x;
    const uint64_t* list = cand;
    int nlist = ncand;
    if (ncand > NT && ncand > K) {
        const uint64_t thr2 = radix_select<NT>(cand, ncand, K, sh.sc);
        for (int i = tid; i < ncand; i += NT) {
            const uint64_t c = cand[i];
            if (c >= thr2) {
                const int q = atomicAdd(&sh.nlist, 1);
                if (q < K) list2[q] = c;
            }
        }
        __syncthreads();
        list = list2;
        nlist = K;
    }
    // G lanes (a quad, a pair or one lane) count one candidate's predecessors
    // over interleaved slices of the list, then sum with DPP inside the quad
    // the row's lse: written before the first barrier above, or (lse_ready)
    // by another wave of the workgroup that raises the flag after it
    if (lse_ready != nullptr)
        while (__hip_atomic_load(lse_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
        }
    const float lse = lse_ready != nullptr ? __hip_atomic_load(lse_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                                           : *lse_p;
    const int G = nlist <= NT / 4 ? 4 : (nlist <= NT / 2 ? 2 : 1);
    const int q = tid & (G - 1);
    for (int i0 = 0; i0 < nlist * G; i0 += NT) {
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
            topk_lp[row * K + rank] = elem_value<DT>((uint32_t)(c >> 32)) - lse;
        }
    }
    // fewer candidates than K only when no entry compares (a row of NaN, the
    // head's mark for a row without a valid source): the places left are -1
    // and NaN, so every output of the row is written
    for (int r = nlist + tid; r < K; r += NT) {
        topk_ids[row * K + r] = -1;
        topk_lp[row * K + r] = __builtin_nanf("");
    }
}

// The 16-byte part of a row starting at entry e0 (a multiple of the entries
// per part); entries at or past V read as -inf and are not loaded.
template <int DT>
__device__ __forceinline__ u32x4 load_part(const uint8_t* __restrict__ rowp, int64_t V, int64_t e0) {
    constexpr int EPV = w16(DT) ? 8 : 4;
    if (e0 + EPV <= V) return *reinterpret_cast<const u32x4*>(rowp + (size_t)e0 * (w16(DT) ? 2 : 4));
    const uint32_t ninf = ninf_word<DT>();
    u32x4 v = u32x4{ninf, ninf, ninf, ninf};
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
        if (e0 + e >= V) continue;
        const int q = e / (w16(DT) ? 2 : 1);
        if (w16(DT)) {
            const uint32_t h = reinterpret_cast<const uint16_t*>(rowp)[e0 + e];
            v[q] = (e & 1) ? ((v[q] & 0x0000FFFFu) | (h << 16)) : ((v[q] & 0xFFFF0000u) | h);
        } else {
            v[q] = reinterpret_cast<const uint32_t*>(rowp)[e0 + e];
        }
    }
    return v;
}

// PRE: the caller already holds, per selection thread t, the maximum and
// minimum of its keys (tkey[0][t], tkey[1][t]; 0 and ~0 for a thread without
// blocks) and has zeroed sh.hist, which saves two workgroup barriers.
template <int DT, int KPT, int NT, bool PF = false, bool PRE = false>
__device__ __forceinline__ void row_topk(const uint8_t* __restrict__ rowp, int64_t row, int64_t V, int32_t nb, int32_t K,
                         const uint32_t (&kr)[KPT], const float* lse_p, uint64_t* cand, uint64_t* list2,
                         int32_t cap,
                         RowShared<NT>& sh, int32_t* __restrict__ topk_ids, float* __restrict__ topk_lp,
                         const int32_t* lse_ready = nullptr, int32_t capb = 0, u32x4* stage = nullptr,
                         const uint32_t (*tkey)[NT] = nullptr) {
    constexpr size_t ESZ = w16(DT) ? 2 : 4;
    constexpr int EPV = w16(DT) ? 8 : 4;                 // elements per 16-byte vector
    constexpr int VPB = kBlock / EPV;                 // vectors per block
    constexpr int MAXV = (kMaxCandidates / EPV + NT - 1) / NT;   // vectors per thread, at most
    constexpr int MAXBLK = kMaxCandidates / kBlock;
    const int tid = threadIdx.x;
    const int b0 = tid * KPT;

    // PF: the block of this thread's largest key (lowest index among equal
    // keys), loaded now and used after T is known
    int32_t pf_blk = -1, pf_j = -1;
    uint32_t pf_key = 0u;
    u32x4 pf[PF ? VPB : 1];
    if (PF && K <= nb) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (kr[j] > pf_key) {                        // slots past nb hold 0
                pf_key = kr[j];
                pf_j = j;
            }
        pf_blk = pf_j >= 0 ? b0 + pf_j : -1;
        if (pf_blk >= 0 && (int64_t)pf_blk * kBlock + kBlock > V)
            pf_blk = pf_j = -1;                          // the partial last block: loaded when needed
        // coalesced: load i of lane l brings the 16-byte part l % 8 of the
        // block of lane 8i + l / 8 (eight whole blocks per wave instruction)
        static_assert(!PF || VPB == 8, "the prefetch spreads a block over eight lanes");
        // (all lane exchanges first, then branch-free loads: a lane whose
        // owner has no block reads block 0, never used; a row shorter than
        // one block has no whole block and loads nothing)
        int blk[VPB];
#pragma unroll
        for (int i = 0; i < VPB; ++i) blk[i] = __shfl(pf_blk, i * 8 + ((tid & 63) >> 3));
        if (V >= kBlock) {
#pragma unroll
            for (int i = 0; i < VPB; ++i)
                pf[i] = *reinterpret_cast<const u32x4*>(
                    rowp + ((size_t)(blk[i] < 0 ? 0 : blk[i]) * kBlock + (size_t)(tid & 7) * EPV) * ESZ);
        }
    }

    // K = 1 with prefetched blocks (16-bit logits): the top entry is the
    // first entry equal to the row's largest block maximum T, and the block
    // holding it is the lowest-indexed block with key T -- the prefetched
    // block of the lowest selection thread whose largest key is T. So the
    // owner's wave reads the answer out of its prefetch registers, with no
    // threshold search, staging or rank. The partial last block is not
    // prefetched: when the winning thread holds it, the general path runs.
    if constexpr (PF) if (K == 1) {
        const int lane = tid & 63;
        uint32_t T1 = 0u;
        int tstar = NT;
        if constexpr (PRE) {
            // every wave reads the per-thread maxima itself (no barrier)
            uint32_t m = 0u;
#pragma unroll
            for (int i = 0; i < NT / 64; ++i) m = max(m, tkey[0][lane + 64 * i]);
            T1 = wave_reduce<1>(m);
#pragma unroll
            for (int i = 0; i < NT / 64; ++i) {
                const uint64_t b = __ballot(tkey[0][lane + 64 * i] == T1);
                if (tstar == NT && b != 0ull) tstar = 64 * i + __builtin_ctzll(b);
            }
        } else {
            uint32_t tmax = 0u;
#pragma unroll
            for (int j = 0; j < KPT; ++j) tmax = max(tmax, kr[j]);
            int fphase = 0;
            uint32_t mx[1] = {tmax};
            block_reduce<1, 1, NT>(mx, sh.sred, fphase);
            T1 = mx[0];
            uint32_t who[1] = {tmax == T1 ? (uint32_t)tid : (uint32_t)NT};
            block_reduce<2, 1, NT>(who, sh.sred, fphase);
            tstar = (int)who[0];
        }
        const bool partial_last = (int64_t)nb * kBlock > V;
        if (T1 != 0u && !(partial_last && tstar == (nb - 1) / KPT)) {
            if ((tstar >> 6) == (tid >> 6)) {            // the owner's wave
                const int o = tstar & 63;
                const int32_t bstar = __shfl(pf_blk, o);
                // lanes 8 (o % 8) .. +7 hold its eight 16-byte parts in pf[o / 8]
                u32x4 w = pf[0];
#pragma unroll
                for (int i = 1; i < VPB; ++i)
                    if ((o >> 3) == i) w = pf[i];
                const float Tf = block_value<DT>(T1);
                uint32_t m = 0u;
                if ((lane >> 3) == (o & 7)) {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const float x = (e & 1) ? hi16<DT>(w[e >> 1]) : lo16<DT>(w[e >> 1]);
                        if (x == Tf) m |= 1u << e;
                    }
                }
                const uint64_t bal = __ballot(m != 0u);
                if (lse_ready != nullptr)
                    while (__hip_atomic_load(lse_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
                    }
                const float lse = lse_ready != nullptr
                                      ? __hip_atomic_load(lse_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                                      : *lse_p;
                // no entry equals T only for a NaN T (a row of NaN): -1 and NaN
                const int lw = bal != 0ull ? __builtin_ctzll(bal) : o;
                if (lane == lw) {
                    topk_ids[row] = bal != 0ull ? bstar * kBlock + (lane & 7) * EPV + __builtin_ctz(m) : -1;
                    topk_lp[row] = bal != 0ull ? Tf - lse : __builtin_nanf("");
                }
            }
            return;
        }
        if constexpr (!PRE) __syncthreads();             // the general path's first reduction reuses sred
    }

    // (3) threshold and kept blocks
    int phase = 0;
    int nblk;
    uint32_t T = 0;                                     // key threshold (0: keep everything)
    bool coarse = false;                                // fp32: every block of T's 16-bit bin and above kept
    if (K <= nb) {
        // The search runs on the top 16 bits of every key first (the whole
        // key for 16-bit logits). For fp32 logits that gives the 16-bit bin
        // holding the K-th key; when the blocks of that bin and above are
        // few, all of them are kept (a superset of the K blocks, whose
        // entries the candidate filter and the rank below still order
        // exactly), else the search goes on inside the bin on full keys.
        constexpr int ksh = 16;
        // Largest t with count(key >= t) >= K; count(>= lo) >= K > count(>= hi).
        // one max-reduction gives the maximum and (complemented) two minima:
        // of all keys, and of the per-thread maxima of threads holding blocks
        uint32_t mm[3];
        if constexpr (PRE) {
            // every wave reduces the per-thread extremes itself (no barrier)
            const int lane = tid & 63;
            mm[0] = mm[1] = mm[2] = 0u;
#pragma unroll
            for (int i = 0; i < NT / 64; ++i) {
                const int t = lane + 64 * i;
                const uint32_t hi_t = tkey[0][t], lo_t = tkey[1][t];
                mm[0] = max(mm[0], hi_t);
                mm[1] = max(mm[1], ~lo_t);
                mm[2] = max(mm[2], t * KPT < nb ? ~hi_t : 0u);
            }
#pragma unroll
            for (int i = 0; i < 3; ++i) mm[i] = wave_reduce<1>(mm[i]);
        } else {
            uint32_t tmax = 0u, tmin = 0xFFFFFFFFu;
            const int nbt = nb - b0;                     // blocks of this thread
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                tmax = max(tmax, kr[j]);
                if (j < nbt) tmin = min(tmin, kr[j]);
            }
            mm[0] = tmax;
            mm[1] = ~tmin;
            mm[2] = b0 < nb ? ~tmax : 0u;
            block_reduce<1, 3, NT>(mm, sh.sred, phase);
        }
        const int nth = (nb + KPT - 1) / KPT;           // threads holding blocks
        // one search over key values [lo, hi) shifted right by `shift`:
        // sh.thr = {T << shift, count(key > T), count(key == T)} in shifted keys
        auto search = [&](uint64_t lo, uint64_t hi, uint32_t c_hi, int shift) {
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
                    const uint32_t kv = kr[j] >> shift;
#pragma unroll
                    for (int i = 0; i < 4; ++i) c[i] += (kv >= t[i]) ? 1u : 0u;
                }
                uint32_t pk[2] = {c[0] | (c[1] << 16), c[2] | (c[3] << 16)};
                block_reduce<0, 2, NT>(pk, sh.sred, phase);
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
            // histogram of the keys in [lo, hi) (cleared before the call),
            // then a suffix scan in wave 0: T is the largest key value v with
            // count(key >= v) >= K
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const uint64_t kv = kr[j] >> shift;
                if (kv >= lo && kv < hi) atomicAdd(&sh.hist[(int)(kv - lo)], 1u);
            }
            __syncthreads();
            if (tid < 64) {
                const uint32_t h0 = sh.hist[4 * tid], h1 = sh.hist[4 * tid + 1];
                const uint32_t h2 = sh.hist[4 * tid + 2], h3 = sh.hist[4 * tid + 3];
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
                    sh.thr[0] = (uint32_t)((lo + (uint64_t)b) << shift);
                    sh.thr[1] = gt;
                    sh.thr[2] = eqc;
                }
            }
            __syncthreads();
        };
        if constexpr (!PRE) {
            if (tid < kHistBins) sh.hist[tid] = 0u;
            __syncthreads();
        }
        search((uint64_t)((K <= nth ? ~mm[2] : ~mm[1]) >> ksh), (uint64_t)(mm[0] >> ksh) + 1, 0u, ksh);
        T = sh.thr[0];
        if constexpr (!w16(DT)) {
            // the bin's blocks and those above, when all their entries fit
            // the candidate list and the bin holds finite values only (its
            // lower edge decodes to a finite float)
            const uint32_t bin = T >> 16;
            const uint32_t nkeep = sh.thr[1] + sh.thr[2];
            if (nkeep <= (uint32_t)MAXBLK && nkeep * kBlock <= (uint32_t)cap && bin >= 0x0080u && bin < 0xFF80u) {
                coarse = true;
            } else {
                const uint32_t c_above = sh.thr[1];
                if (tid < kHistBins) sh.hist[tid] = 0u;   // wave 0's scan read it before the barrier
                __syncthreads();
                search((uint64_t)T, (uint64_t)T + 0x10000u, c_above, 0);
                T = sh.thr[0];
            }
        }
        if constexpr (PF) if (K <= capb && T != 0u) {   // T == 0 (all-NaN blocks) would keep empty slots
            // the candidate blocks are staged in LDS (sh.nblk counts the
            // slots), then filtered by all threads. They are the blocks with
            // key >= T while those fit in capb slots; otherwise the blocks
            // with key > T and the K - count(key > T) lowest-indexed blocks
            // with key == T: the first K blocks under (key desc, index asc),
            // whose maxima precede every entry of a dropped tied block
            static_assert(KPT <= 32, "one bit per block of a selection thread");
            uint32_t keep = 0u;                          // bit j: block b0 + j is a candidate
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if (kr[j] >= T) keep |= 1u << j;         // slots past nb hold 0 < T
            if (sh.thr[1] + sh.thr[2] > (uint32_t)capb) {
                uint32_t eqm = 0u;                       // bit j: block b0 + j has key == T
#pragma unroll
                for (int j = 0; j < KPT; ++j)
                    if (kr[j] == T) eqm |= 1u << j;
                uint32_t tot = 0u;
                const int need = K - (int)sh.thr[1];
                int ei = (int)block_exclusive_scan<NT>((uint32_t)__builtin_popcount(eqm), sh.swtot, tot);
                while (eqm != 0u) {                      // ascending block index
                    const int j = __builtin_ctz(eqm);
                    eqm &= eqm - 1u;
                    if (ei >= need) keep &= ~(1u << j);
                    ++ei;
                }
            }
            if (tid == 0) sh.ncand = 0;
            const uint32_t more = keep & ~(pf_blk >= 0 ? 1u << pf_j : 0u);   // kept, not prefetched
            // staging slot t holds thread t's prefetched block (every part
            // is written; only the slots of candidate blocks are read), slots
            // NT + c the blocks loaded now
#pragma unroll
            for (int i = 0; i < VPB; ++i) stage[((tid & ~63) + i * 8 + ((tid & 63) >> 3)) * VPB + (tid & 7)] = pf[i];
            if (pf_blk >= 0 && ((keep >> pf_j) & 1u)) {
                const int c = atomicAdd(&sh.nblk, 1);
                sh.blk[c] = pf_blk;
                sh.cslot[c] = tid;
            }
            for (uint32_t mb = more; mb != 0u; mb &= mb - 1u) {
                const int c = atomicAdd(&sh.nblk, 1);
                sh.blk[c] = b0 + __builtin_ctz(mb);
                sh.cslot[c] = NT + c;
            }
            __syncthreads();
            // the candidate blocks not prefetched, loaded by all threads in
            // one round (part i % VPB of candidate i / VPB: a thread's loads
            // are all issued before its first wait)
            {
                constexpr int MQ = (MAXBLK * VPB + NT - 1) / NT;
                const int nq = sh.nblk * VPB;
                u32x4 q[MQ];
                int qs[MQ];
#pragma unroll
                for (int i = 0; i < MQ; ++i) {
                    const int v = tid + i * NT;
                    const int c = v / VPB;
                    qs[i] = v < nq && sh.cslot[c] >= NT ? sh.cslot[c] * VPB + v % VPB : -1;
                    if (qs[i] >= 0)
                        q[i] = load_part<DT>(rowp, V, (int64_t)sh.blk[c] * kBlock + (int64_t)(v % VPB) * EPV);
                }
#pragma unroll
                for (int i = 0; i < MQ; ++i)
                    if (qs[i] >= 0) stage[qs[i]] = q[i];
            }
            __syncthreads();
            const bool keep_all = T == 0u;
            const float Tf = keep_all ? kNegInf : block_value<DT>(T);
            const int nvec = sh.nblk * VPB;
            for (int i = tid; i < nvec; i += NT) {
                const u32x4 w = stage[sh.cslot[i / VPB] * VPB + i % VPB];
                const int64_t e0 = (int64_t)sh.blk[i / VPB] * kBlock + (int64_t)(i % VPB) * EPV;
                uint32_t m = 0u;                         // bit e: entry e0 + e is a candidate
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const uint32_t wd = w[e / (w16(DT) ? 2 : 1)];
                    const float x = w16(DT) ? ((e & 1) ? hi16<DT>(wd) : lo16<DT>(wd)) : __uint_as_float(wd);
                    if (e0 + e < V && (keep_all || x >= Tf)) m |= 1u << e;
                }
                if (m != 0u) {
                    int pos = atomicAdd(&sh.ncand, __builtin_popcount(m));
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        if ((m >> e) & 1u) {
                            const uint32_t wd = w[e / (w16(DT) ? 2 : 1)];
                            const float x = w16(DT) ? ((e & 1) ? hi16<DT>(wd) : lo16<DT>(wd)) : __uint_as_float(wd);
                            cand[pos++] = ((uint64_t)elem_key<DT>(x) << 32) |
                                          (uint64_t)(0xFFFFFFFFu - (uint32_t)(e0 + e));
                        }
                    }
                }
            }
            __syncthreads();
            rank_topk<DT, NT>(row, K, cand, sh.ncand, list2, sh, topk_ids, topk_lp, lse_p, lse_ready);
            return;
        }
        const int need = K - (int)sh.thr[1];             // blocks equal to T that are kept
        const bool all_ties = coarse || (uint32_t)need == sh.thr[2];
        if (all_ties) {
            // every key >= T is kept: placement order does not matter
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if (kr[j] >= T) {
                    const int pos = atomicAdd(&sh.nblk, 1);
                    if (pos < MAXBLK) sh.blk[pos] = b0 + j;
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
            const uint32_t ex = block_exclusive_scan<NT>(gt | (eq << 16), sh.swtot, tot);
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
                    if (pos < MAXBLK) sh.blk[pos] = b0 + j;
                    ++pos;
                }
            }
        }
        nblk = coarse ? (int)(sh.thr[1] + sh.thr[2]) : min(K, MAXBLK);
    } else {
        for (int b = tid; b < nb; b += NT) sh.blk[b] = b;
        nblk = nb;
    }
    __syncthreads();

    // (4) gather the kept blocks in one round of loads; keep entries >= T
    const int nvec = nblk * VPB;
    uint32_t w[MAXV][4];
    int64_t e0[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int j = tid + i * NT;
        e0[i] = -1;
        const int blk = j < nvec ? sh.blk[j / VPB] : -1;
        if (blk >= 0 && blk < nb) {
            e0[i] = (int64_t)blk * kBlock + (int64_t)(j % VPB) * EPV;
            if (e0[i] + EPV <= V) {
                const u32x4 v4 = *reinterpret_cast<const u32x4*>(rowp + (size_t)e0[i] * ESZ);
                w[i][0] = v4.x; w[i][1] = v4.y; w[i][2] = v4.z; w[i][3] = v4.w;
            } else {
                const uint32_t ninf = ninf_word<DT>();
                w[i][0] = w[i][1] = w[i][2] = w[i][3] = ninf;
                for (int e = 0; e < EPV; ++e) {
                    const int64_t idx = e0[i] + e;
                    if (idx < V) {
                        if (w16(DT)) {
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
    const float Tf = keep_all ? kNegInf : block_value<DT>(T);
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        if (e0[i] < 0) continue;
        const bool vfull = e0[i] + EPV <= V;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = w16(DT) ? ((e & 1) ? hi16<DT>(w[i][e >> 1]) : lo16<DT>(w[i][e >> 1]))
                                 : __uint_as_float(w[i][e]);
            cnt += ((vfull || e0[i] + e < V) && (keep_all || x >= Tf)) ? 1u : 0u;
        }
    }
    uint32_t ncand_u = 0;
    int cpos = (int)block_exclusive_scan<NT>(cnt, sh.swtot, ncand_u);
    const int ncand = min((int)ncand_u, cap);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        if (e0[i] < 0) continue;
        const bool vfull = e0[i] + EPV <= V;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = w16(DT) ? ((e & 1) ? hi16<DT>(w[i][e >> 1]) : lo16<DT>(w[i][e >> 1]))
                                 : __uint_as_float(w[i][e]);
            const int64_t v = e0[i] + e;
            if ((vfull || v < V) && (keep_all || x >= Tf)) {
                if (cpos < cap)
                    cand[cpos] = ((uint64_t)elem_key<DT>(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
                ++cpos;
            }
        }
    }
    __syncthreads();

    rank_topk<DT, NT>(row, K, cand, ncand, list2, sh, topk_ids, topk_lp, lse_p, lse_ready);
}

// Canonical merge of a row's item partials: lane g < 16 holds the partial
// of group g (items i with i mod 16 == g, merged in ascending order); the 16
// groups are merged as a pairwise tree (2j with 2j+1, then the pairs, ...;
// the lower groups always the left operand), so every lane takes the same
// rounding steps. lse = m + log(s), -inf for a row whose entries are all
// -inf. Called by a whole wave (lanes 16-63 hold copies of no use); lanes
// 0-15 return the row's lse.
__device__ inline float lse_tree16(float m, float s) {
    const int lane = threadIdx.x & 63;
    // partner lane at each level: lane ^ 1, lane ^ 2 (quad permutes), then
    // the mirror lane in the half row and in the row; after each level the
    // lanes of a merged subgroup hold identical values, so any lane of the
    // partner subgroup serves
    auto level = [&](auto ctl, int d) {
        constexpr int C = decltype(ctl)::value;
        const float m2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), C, 0xF, 0xF, false));
        const float s2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), C, 0xF, 0xF, false));
        const bool left = (lane & d) == 0;
        float mL = left ? m : m2, sL = left ? s : s2;
        lse_merge(mL, sL, left ? m2 : m, left ? s2 : s);
        m = mL;
        s = sL;
    };
    level(std::integral_constant<int, 0xB1>{}, 1);
    level(std::integral_constant<int, 0x4E>{}, 2);
    level(std::integral_constant<int, 0x141>{}, 4);
    level(std::integral_constant<int, 0x140>{}, 8);
    // m = -inf: every entry is -inf (sum 0, lse -inf) or NaN (the sum is NaN
    // and so is the lse)
    return (m == kNegInf) ? (s == s ? kNegInf : s) : m + logf(s);
}

// The selected token's logit (a5), loaded long before its logprob is
// written; an id outside [0, V) gives NaN and the index error bit.
template <int DT>
__device__ inline float load_selected(const uint8_t* rowp, int64_t V, int32_t sel_id) {
    if (sel_id < 0 || (int64_t)sel_id >= V) return __builtin_nanf("");
    return w16(DT) ? elem16<DT>(rowp, sel_id)
                : reinterpret_cast<const float*>(rowp)[sel_id];
}
__device__ inline void write_selected(int64_t V, int32_t sel_id, float xsel, float lse, float* out,
                                      int32_t* err) {
    if (sel_id >= 0 && (int64_t)sel_id < V) {
        *out = xsel - lse;
    } else {
        *out = __builtin_nanf("");
        if (err) atomicOr(err, LMH_DEVERR_INDEX);
    }
}

// The (max, sum) of a wave's 64 lanes as a pairwise tree (partner lane ^ 1,
// ^ 2, the mirror lane in the half row and in the row, then lane ^ 16 and
// lane ^ 32; the lower half always the left operand); every lane ends with
// the wave's partial.
__device__ inline void lse_tree64(float& m, float& s) {
    const int lane = threadIdx.x & 63;
    auto merge_with = [&](float m2, float s2, int d) {
        const bool left = (lane & d) == 0;
        float mL = left ? m : m2, sL = left ? s : s2;
        lse_merge(mL, sL, left ? m2 : m, left ? s2 : s);
        m = mL;
        s = sL;
    };
    auto level = [&](auto ctl, int d) {
        constexpr int C = decltype(ctl)::value;
        merge_with(__int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), C, 0xF, 0xF, false)),
                   __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), C, 0xF, 0xF, false)), d);
    };
    level(std::integral_constant<int, 0xB1>{}, 1);
    level(std::integral_constant<int, 0x4E>{}, 2);
    level(std::integral_constant<int, 0x141>{}, 4);
    level(std::integral_constant<int, 0x140>{}, 8);
    merge_with(__int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x1F | (16 << 10))),
               __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(s), 0x1F | (16 << 10))), 16);
    const int x32 = ((lane ^ 32) << 2);
    merge_with(__int_as_float(__builtin_amdgcn_ds_bpermute(x32, __float_as_int(m))),
               __int_as_float(__builtin_amdgcn_ds_bpermute(x32, __float_as_int(s))), 32);
}

// ---------------------------------------------------------------------------
// Split path, second kernel: one workgroup of 256 threads per row reads the
// row's item partials and block keys from the workspace. BLOCKS: the
// partials are one per 64-logit block, written by the tiled head's epilogue
// (fp32 logits), and merge in their own fixed order: partial i goes to thread
// i mod 256, which merges its partials in ascending order; each wave's lanes
// then merge as a pairwise tree and the four waves in order.
// ---------------------------------------------------------------------------
template <int DT, int KPT, bool BLOCKS = false>
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
    // [cap] candidates, [K] narrowed list (even count), staged blocks (16-bit logits)
    extern __shared__ __attribute__((aligned(16))) uint64_t smem[];
    __shared__ RowShared<kThreads> sh;
    constexpr size_t ESZ = w16(DT) ? 2 : 4;
    constexpr int MAXBLK = kMaxCandidates / kBlock;

    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;
    if (tid < MAXBLK) sh.blk[tid] = -1;   // unfilled slots are skipped, never dereferenced
    if (tid == 0) {
        sh.nlist = 0;
        sh.nblk = 0;
    }

    // this thread's block keys, blocks [b0, b0 + KPT): the raw 32-bit words
    // now (two 16-bit keys per word for 16-bit logits), unpacked after the
    // partials' loads are issued
    const int b0 = tid * KPT;
    constexpr int KW = w16(DT) ? KPT / 2 : KPT;
    uint32_t kw[KW];
#pragma unroll
    for (int j = 0; j < KW; ++j) kw[j] = 0u;
    if (K > 0 && K <= nb && b0 < nb) {
        const uint32_t* kp = w16(DT)
            ? reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(keys) + row * kld + b0)
            : reinterpret_cast<const uint32_t*>(keys) + row * kld + b0;
        if constexpr (KW == 2) {
            const uint2 q = *reinterpret_cast<const uint2*>(kp);
            kw[0] = q.x;
            kw[1] = q.y;
        } else {
#pragma unroll
            for (int c = 0; c < KW / 4; ++c) {
                const u32x4 q = reinterpret_cast<const u32x4*>(kp)[c];
                kw[c * 4 + 0] = q.x;
                kw[c * 4 + 1] = q.y;
                kw[c * 4 + 2] = q.z;
                kw[c * 4 + 3] = q.w;
            }
        }
    }

    // the selected token's id, issued now (thread 64: off the lse wave)
    const bool sel_thread = sel != nullptr && sel_out != nullptr && tid == 64;
    int32_t sel_id = 0;
    if (sel_thread) sel_id = sel[row];

    if constexpr (BLOCKS) {
        __shared__ float2 swave[kThreads / 64];
        // rounds of KPT partials per thread, all loaded before the first
        // merge of the round (one round when the row has at most KPT * 256
        // blocks); the merge order is the loop's ascending i either way
        float m = kNegInf, sm = 0.f;
        for (int i0 = tid; i0 < splits; i0 += KPT * kThreads) {
            float2 pp[KPT];
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const int i = i0 + j * kThreads;
                pp[j] = i < splits ? part[row * splits + i] : make_float2(kNegInf, 0.f);
            }
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if (i0 + j * kThreads < splits) lse_merge(m, sm, pp[j].x, pp[j].y);
        }
        lse_tree64(m, sm);
        if ((tid & 63) == 0) swave[tid >> 6] = make_float2(m, sm);
        __syncthreads();
        if (tid == 0) {
            float mm = swave[0].x, ss = swave[0].y;
#pragma unroll
            for (int w = 1; w < kThreads / 64; ++w) lse_merge(mm, ss, swave[w].x, swave[w].y);
            // m = -inf: every entry -inf (lse -inf) or NaN (lse NaN)
            const float l = (mm == kNegInf) ? (ss == ss ? kNegInf : ss) : mm + logf(ss);
            sh.lse = l;
            lse_out[row] = l;
        }
    } else {
        // logsumexp: lanes 0..15 of wave 0 merge their groups' partials, then
        // the wave merges the groups
        if (tid < 64) {
            // a group's partials in rounds of four, each round's loads issued
            // before its first merge (merge order: ascending i)
            constexpr int kRound = 4;
            float m = kNegInf, sm = 0.f;
            if (tid < kGroups)
                for (int i0 = tid; i0 < splits; i0 += kRound * kGroups) {
                    float2 pp[kRound];
#pragma unroll
                    for (int j = 0; j < kRound; ++j) {
                        const int i = i0 + j * kGroups;
                        pp[j] = i < splits ? part[row * splits + i] : make_float2(kNegInf, 0.f);
                    }
#pragma unroll
                    for (int j = 0; j < kRound; ++j)
                        if (i0 + j * kGroups < splits) lse_merge(m, sm, pp[j].x, pp[j].y);
                }
            const float l = lse_tree16(m, sm);
            if (tid == 0) {
                sh.lse = l;
                lse_out[row] = l;
            }
        }
    }
    // the keys, 0 past nb
    uint32_t kr[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        kr[j] = !w16(DT) ? kw[j] : ((j & 1) ? (kw[j >> 1] & 0xFFFF0000u) : (kw[j >> 1] << 16));
        if (b0 + j >= nb) kr[j] = 0u;
    }
    __syncthreads();
    const float lse = sh.lse;
    // the selected logit: loaded now, written after the top-K
    const float xsel = sel_thread ? load_selected<DT>(rowp, V, sel_id) : 0.f;
    if (K > 0)
        row_topk<DT, KPT, kThreads, w16(DT)>(rowp, row, V, nb, K, kr, &sh.lse, smem, smem + cap, cap, sh,
                                              topk_ids, topk_lp, nullptr, cap / kBlock,
                                              reinterpret_cast<u32x4*>(smem + cap + ((K + 1) & ~1)));
    if (sel_thread) write_selected(V, sel_id, xsel, lse, sel_out + row, err);
}

// ---------------------------------------------------------------------------
// Single-launch path for a few rows (rows that leave most CUs idle; openinfer
// issue #719, Description: decode steps of a few rows): each row is spread
// over S = ceil(P / 4) workgroups of four waves, wave w of workgroup j
// streaming item 4j + w exactly as the split path's first kernel does (the
// same partials and block keys). Each workgroup then takes the exact top-K of
// its own slice: wave 0 finds the K-th largest of the slice's block keys by
// repeated wave maxima (counted with multiplicity, ties cut by ascending
// block index), the kept blocks' entries at or above it are gathered (the
// slice was just read: L2 hits), ranked, and the slice's K (id, value) pairs
// go to the scratch. A row's top-K lies in the union of its slices' top-K.
// The last workgroup of a row to arrive (one device-scope counter per row,
// incremented once per workgroup after a device-scope release of its writes)
// merges the row's item partials in the canonical order, ranks the union and
// writes the row's outputs, then puts the counter back to zero. No workgroup
// waits for another, so the results are bitwise those of the other paths.
// ---------------------------------------------------------------------------
constexpr int kSingleMaxK = LMH_SINGLE_MAX_K;
constexpr int kSingleMaxSlices = 16;   // P <= 64 items per row
constexpr int64_t kSingleMaxRows = LMH_SINGLE_MAX_ROWS;
static_assert(kSingleMaxK * kSingleMaxSlices <= 2 * kThreads, "the final union is read in two rounds");

template <int DT, bool KEYS>
__global__ __launch_bounds__(kThreads) void k_single(const uint8_t* __restrict__ logits, int64_t ld, int64_t V,
                                                     int32_t P, int32_t S, const int32_t* __restrict__ sel,
                                                     int32_t K, float* __restrict__ lse_out,
                                                     float* __restrict__ sel_out, int32_t* __restrict__ topk_ids,
                                                     float* __restrict__ topk_lp, int32_t* __restrict__ err,
                                                     float2* __restrict__ part, int32_t* __restrict__ loc_ids,
                                                     float* __restrict__ loc_vals,
                                                     uint32_t* __restrict__ counters) {
    using I = Stage1Item<DT>;
    constexpr size_t ESZ = w16(DT) ? 2 : 4;
    constexpr int EPV = I::EPV;
    constexpr int VPB = kBlock / EPV;
    __shared__ RowShared<kThreads> sh;
    __shared__ uint32_t skey[kThreads];                                 // the slice's block keys (0: none)
    __shared__ __attribute__((aligned(16))) uint64_t cand[kSingleMaxK * kBlock];
    __shared__ uint64_t list2[kSingleMaxK];
    __shared__ int32_t lids[kSingleMaxK];                              // the slice's top-K
    __shared__ float lvals[kSingleMaxK];
    __shared__ int32_t s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint32_t g = blockIdx.x;
    const uint32_t rowu = g / (uint32_t)S;
    const int64_t row = rowu;
    const int32_t j = (int32_t)(g - rowu * (uint32_t)S);
    const int32_t seg = 4 * j + wave;
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;
    if (tid == 0) {
        sh.nlist = 0;
        sh.ncand = 0;
        sh.nblk = 0;
        sh.lse = 0.f;
    }

    // (1) this wave's item, as in the split path's first kernel
    uint32_t kb = 0u;
    if (seg < P) {
        u32x4 buf[I::VPL];
        float M, Sm;
        if (stage1_load<DT>(rowp, V, seg, lane, buf)) {
            __builtin_amdgcn_sched_barrier(0);
            stage1_item<DT, KEYS>(buf, lane, M, Sm, kb);
        } else {
            stage1_item<DT, KEYS>(buf, lane, M, Sm, kb);
        }
        if (lane == 0)
            __hip_atomic_store(reinterpret_cast<uint64_t*>(part) + row * P + seg,
                               ((uint64_t)__float_as_uint(Sm) << 32) | __float_as_uint(M), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (((int64_t)seg * (kSeg / kBlock) + lane) * kBlock >= V) kb = 0u;   // a block past V has no key
    }

    if constexpr (KEYS) {
        skey[tid] = kb;                  // local block tid = block 4j*64 + tid of the row
        __syncthreads();
        // (2) wave 0: the slice's K-th largest key T and its kept blocks (all
        // keys above T, then the lowest-indexed keys equal to T up to K); a
        // slice with fewer than K blocks keeps all of them (T = 0)
        if (wave == 0) {
            uint32_t kk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) kk[i] = skey[i * 64 + lane];
            uint32_t T = 0u, gt = 0u;
            if (K <= 4) {
                // the distinct key values from the top, one per round
                uint32_t rem[4] = {kk[0], kk[1], kk[2], kk[3]};
                uint32_t before = 0u;
                for (int it = 0; it < K; ++it) {
                    const uint32_t m = wave_reduce<1>(max(max(rem[0], rem[1]), max(rem[2], rem[3])));
                    if (m == 0u) break;
                    uint32_t c = 0u;
#pragma unroll
                    for (int i = 0; i < 4; ++i) c += (uint32_t)__popcll(__ballot(rem[i] == m));
                    if (before + c >= (uint32_t)K) {
                        T = m;
                        gt = before;
                        break;
                    }
                    before += c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) rem[i] = rem[i] == m ? 0u : rem[i];
                }
            } else {
                // bitwise search from the top bit: T is the largest value
                // with at least K keys at or above it (16-bit keys occupy the
                // top half); keys 0 are empty slots
                uint32_t real = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) real += (uint32_t)__popcll(__ballot(kk[i] != 0u));
                if (real >= (uint32_t)K) {
                    uint32_t prefix = 0u, k_left = (uint32_t)K;
                    constexpr int lo_bit = w16(DT) ? 16 : 0;
                    for (int bit = 31; bit >= lo_bit; --bit) {
                        const uint32_t hi_mask = 0xFFFFFFFFu << bit;       // bits bit..31
                        const uint32_t want = prefix | (1u << bit);
                        uint32_t c = 0u;
#pragma unroll
                        for (int i = 0; i < 4; ++i) c += (uint32_t)__popcll(__ballot((kk[i] & hi_mask) == want));
                        if (c >= k_left)
                            prefix = want;
                        else
                            k_left -= c;
                    }
                    T = prefix;
                    gt = (uint32_t)K - k_left;                  // keys above T
                }
            }
            const uint32_t need = (uint32_t)K - gt;      // keys equal to T that are kept
            const uint64_t below = (1ull << lane) - 1ull;
            uint32_t eq_seen = 0u;
            int nk = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool eq = T != 0u && kk[i] == T;
                const uint64_t eqm = __ballot(eq);
                const bool keep = kk[i] != 0u &&
                                  (T == 0u || kk[i] > T || (eq && eq_seen + (uint32_t)__popcll(eqm & below) < need));
                const uint64_t km = __ballot(keep);
                if (keep) sh.blk[nk + __popcll(km & below)] = i * 64 + lane;
                nk += __popcll(km);
                eq_seen += (uint32_t)__popcll(eqm);
            }
            if (lane == 0) {
                sh.nblk = nk;
                sh.thr[0] = T;
            }
        }
        __syncthreads();

        // (3) the kept blocks' entries at or above T (all of them for T = 0),
        // then the slice's top-K as (id, value) pairs
        {
            const int nkb = sh.nblk;
            const uint32_t T = sh.thr[0];
            const bool keep_all = T == 0u;
            const float Tf = keep_all ? kNegInf : block_value<DT>(T);
            const int64_t blk0 = (int64_t)j * 4 * (kSeg / kBlock);
            for (int v = tid; v < nkb * VPB; v += kThreads) {
                const int64_t e0 = (blk0 + sh.blk[v / VPB]) * kBlock + (int64_t)(v % VPB) * EPV;
                const u32x4 w = load_part<DT>(rowp, V, e0);
                uint32_t m = 0u;
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const uint32_t wd = w[e / (w16(DT) ? 2 : 1)];
                    const float x = w16(DT) ? ((e & 1) ? hi16<DT>(wd) : lo16<DT>(wd)) : __uint_as_float(wd);
                    if (e0 + e < V && (keep_all || x >= Tf)) m |= 1u << e;
                }
                if (m != 0u) {
                    int pos = atomicAdd(&sh.ncand, __builtin_popcount(m));
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        if ((m >> e) & 1u) {
                            const uint32_t wd = w[e / (w16(DT) ? 2 : 1)];
                            const float x = w16(DT) ? ((e & 1) ? hi16<DT>(wd) : lo16<DT>(wd)) : __uint_as_float(wd);
                            cand[pos++] = ((uint64_t)elem_key<DT>(x) << 32) |
                                          (uint64_t)(0xFFFFFFFFu - (uint32_t)(e0 + e));
                        }
                    }
                }
            }
            __syncthreads();
            // sh.lse is 0 here: the values are written as they are, to LDS
            rank_topk<DT, kThreads>(0, K, cand, sh.ncand, list2, sh, lids, lvals, &sh.lse, nullptr);
            __syncthreads();
            if (tid < K) {
                const int64_t at = (int64_t)g * K + tid;
                __hip_atomic_store(reinterpret_cast<uint32_t*>(loc_ids) + at, (uint32_t)lids[tid],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(reinterpret_cast<uint32_t*>(loc_vals) + at, __float_as_uint(lvals[tid]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // (4) arrival. Everything another workgroup reads (the partials and the
    // top-K lists) was written with device-scope stores, which the caches
    // pass through to the device's point of coherence, and is read back with
    // device-scope loads, which do not hit a stale cached copy; so the
    // publication needs no cache write-back or invalidation (a device-scope
    // fence, measured at about 9 us per workgroup here), only that every
    // such store has completed before the workgroup's one increment of the
    // row's counter: each wave waits for its stores, then the barrier.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&counters[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (uint32_t)(S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    if (tid == 0) {
        sh.ncand = 0;
        sh.nlist = 0;
    }
    __syncthreads();

    // (5) the last workgroup of the row: lse from the item partials in the
    // canonical order (as stage 2), the union of the slices' top-K ranked
    const bool sel_thread = sel != nullptr && sel_out != nullptr && tid == 64;
    int32_t sel_id = 0;
    if (sel_thread) sel_id = sel[row];
    if (tid < 64) {
        constexpr int kRound = 4;
        float m = kNegInf, sm = 0.f;
        if (tid < kGroups)
            for (int i0 = tid; i0 < P; i0 += kRound * kGroups) {
                float2 pp[kRound];
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    const int i = i0 + u * kGroups;
                    const uint64_t b = i < P ? __hip_atomic_load(reinterpret_cast<const uint64_t*>(part) + row * P + i,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                             : ((uint64_t)__float_as_uint(0.f) << 32) | __float_as_uint(kNegInf);
                    pp[u] = make_float2(__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
                }
#pragma unroll
                for (int u = 0; u < kRound; ++u)
                    if (i0 + u * kGroups < P) lse_merge(m, sm, pp[u].x, pp[u].y);
            }
        const float l = lse_tree16(m, sm);
        if (tid == 0) {
            sh.lse = l;
            lse_out[row] = l;
        }
    }
    if constexpr (KEYS) {
        // (n <= 16 * 32 = 2 * kThreads: every thread's loads in one round)
        const int n = S * K;
        int32_t id[2];
        float val[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = tid + r * kThreads;
            const int64_t at = row * (int64_t)n + (i < n ? i : 0);
            id[r] = (int32_t)__hip_atomic_load(reinterpret_cast<const uint32_t*>(loc_ids) + at, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
            val[r] = __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(loc_vals) + at,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (i >= n) id[r] = -1;
        }
        // one LDS atomic per wave and round: lanes place their entries by
        // their rank among the wave's valid lanes
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const bool ok = id[r] >= 0;
            const uint64_t vm = __ballot(ok);
            int base = 0;
            if (lane == 0 && vm != 0ull) base = atomicAdd(&sh.ncand, __popcll(vm));
            base = __shfl(base, 0);
            if (ok)
                cand[base + __popcll(vm & ((1ull << lane) - 1ull))] =
                    ((uint64_t)elem_key<DT>(val[r]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id[r]);
        }
    }
    __syncthreads();
    const float lse = sh.lse;
    const float xsel = sel_thread ? load_selected<DT>(rowp, V, sel_id) : 0.f;
    if constexpr (KEYS)
        rank_topk<DT, kThreads>(row, K, cand, sh.ncand, list2, sh, topk_ids, topk_lp, &sh.lse, nullptr);
    if (sel_thread) write_selected(V, sel_id, xsel, lse, sel_out + row, err);
    if (tid == 0) counters[row] = 0u;                    // ready for the next call
}

// ---------------------------------------------------------------------------
// One-workgroup-per-row path (rows that fill the CUs evenly): 8 waves stream
// the row's items, handed out from an LDS counter (bf16 items double-
// buffered: the next item's loads are in flight while the current one is
// reduced), writing each item's partial and block keys to LDS; after one
// barrier wave 4 merges the partials in the canonical order while waves 0-3
// run the top-K selection on the LDS keys (waves 5-7 end there). One launch,
// and no workspace round trip between the stream and the selection. Eight
// waves keep two 8 KiB items per wave in flight, which holds the CU's share
// of HBM bandwidth; sixteen waves streamed no faster and took longer to
// dispatch (28.6 against 30.3 us on 256 rows of 248,320 bf16 logits).
// ---------------------------------------------------------------------------
constexpr int kRowWaves = 8;
static_assert(kRowWaves > kThreads / 64, "the lse wave follows the selection waves");
constexpr int kRowThreads = kRowWaves * 64;
constexpr int kRowMaxItems = 64;   // items per row on this path (V <= 64 * kSeg)
template <bool W16> struct KeyType { using type = uint32_t; };
template <> struct KeyType<true> { using type = uint16_t; };

template <int DT, int KPT, bool KEYS>
__global__ __launch_bounds__(kRowThreads) void k_rowreduce(const uint8_t* __restrict__ logits, int64_t ld,
                                                           int64_t V, int32_t nb, int32_t P,
                                                           const int32_t* __restrict__ sel, int32_t K,
                                                           float* __restrict__ lse_out,
                                                           float* __restrict__ sel_out,
                                                           int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_lp,
                                                           int32_t* __restrict__ err, int32_t cap) {
    using I = Stage1Item<DT>;
    using key_t = typename KeyType<w16(DT)>::type;
    // [KPT*256] keys, [cap] candidates, [K] narrowed list (even count), staged blocks
    extern __shared__ __attribute__((aligned(16))) uint64_t smem[];
    __shared__ RowShared<kThreads> sh;
    __shared__ float2 sitem[kRowMaxItems];
    __shared__ int32_t s_next, s_sel, s_lse_ready;
    __shared__ float s_xsel;
    // per selection thread t (blocks t*KPT .. t*KPT + KPT - 1): the maximum
    // and minimum of its keys, gathered while the items are reduced
    __shared__ uint32_t s_tkey[2][kThreads];
    constexpr size_t ESZ = w16(DT) ? 2 : 4;
    constexpr int MAXBLK = kMaxCandidates / kBlock;
    key_t* skeys = reinterpret_cast<key_t*>(smem);
    uint64_t* cand = smem + (KPT * kThreads * sizeof(key_t) + 7) / 8;

    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint8_t* rowp = logits + (size_t)row * (size_t)ld * ESZ;
    if (tid < MAXBLK) sh.blk[tid] = -1;
    if (tid == 0) {
        sh.nlist = 0;
        sh.nblk = 0;
        s_next = kRowWaves;
        s_lse_ready = 0;
    }
    if (KEYS) {
        for (int t = tid; t < kThreads; t += kRowThreads) {
            s_tkey[0][t] = 0u;
            s_tkey[1][t] = 0xFFFFFFFFu;
        }
        for (int i = tid; i < kHistBins; i += kRowThreads) sh.hist[i] = 0u;
    }
    __syncthreads();   // s_next before the first hand-out
    // key slots past nb read as 0
    if (KEYS)
        for (int b = nb + tid; b < KPT * kThreads; b += kRowThreads) skeys[b] = 0;

    // the selected id and logit, issued first by the last wave (its item
    // count is never above any other wave's, so its two dependent loads do
    // not hold up the workgroup)
    const bool sel_thread = sel != nullptr && sel_out != nullptr && tid == kRowThreads - 64;
    int32_t sel_id = 0;
    float xsel = 0.f;
    if (sel_thread) {
        sel_id = sel[row];
        s_sel = sel_id;
        xsel = load_selected<DT>(rowp, V, sel_id);
    }

    // Items are handed out dynamically (wave w starts with item w, then takes
    // the next index from an LDS counter), so the waves finish together;
    // each item's partial goes to LDS and the row's partials are merged in
    // the canonical order afterwards.
    auto reduce_item = [&](const u32x4 (&buf)[I::VPL], int32_t seg) {
        float M, S;
        uint32_t kb = 0;
        stage1_item<DT, KEYS>(buf, lane, M, S, kb);
        if (KEYS) {
            const int32_t blk = seg * (kSeg / kBlock) + lane;
            if (blk < nb) skeys[blk] = w16(DT) ? (key_t)(kb >> 16) : (key_t)kb;
            // the key as the selection holds it; extremes over the KPT lanes
            // of one selection thread (partners: lane ^ 1, ^ 2, then the
            // mirror lane in the half row and in the row)
            const uint32_t kv = w16(DT) ? (kb & 0xFFFF0000u) : kb;
            uint32_t hi = blk < nb ? kv : 0u, lo = blk < nb ? kv : 0xFFFFFFFFu;
            auto fold = [&](auto ctl) {
                constexpr int C = decltype(ctl)::value;
                hi = max(hi, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, C, 0xF, 0xF, false));
                lo = min(lo, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, C, 0xF, 0xF, false));
            };
            fold(std::integral_constant<int, 0xB1>{});
            fold(std::integral_constant<int, 0x4E>{});
            if (KPT >= 8) fold(std::integral_constant<int, 0x141>{});
            if (KPT >= 16) fold(std::integral_constant<int, 0x140>{});
            const int t = blk / KPT;
            if (lane % KPT == 0 && t < kThreads) {
                s_tkey[0][t] = hi;
                s_tkey[1][t] = lo;
            }
        }
        if (lane == 0) sitem[seg] = make_float2(M, S);
    };
    auto next_item = [&]() -> int32_t {
        int32_t v = 0;
        if (lane == 0) v = atomicAdd(&s_next, 1);
        return __builtin_amdgcn_readfirstlane(v);
    };
    // The partial last item (index Pf, when V is not a multiple of kSeg) goes
    // first to the last wave, so that its loads are not exposed at the end.
    const int32_t Pf = (int32_t)(V / kSeg);
    if (Pf < P && wave == kRowWaves - 1) {
        u32x4 buf[I::VPL];
        stage1_load<DT>(rowp, V, Pf, lane, buf);
        reduce_item(buf, Pf);
    }
    int32_t cur = wave < Pf ? wave : Pf;
    if (w16(DT)) {
        // double-buffered: the next item's loads are issued before the current
        // one is reduced (on the last pass the current item is loaded again,
        // an L2 hit, which keeps the loop free of load branches)
        u32x4 nxt[I::VPL];
        if (cur < Pf) stage1_load_full<DT>(rowp, cur, lane, nxt);
        while (cur < Pf) {
            u32x4 buf[I::VPL];
#pragma unroll
            for (int j = 0; j < I::VPL; ++j) buf[j] = nxt[j];
            const int32_t nx = next_item();
            stage1_load_full<DT>(rowp, nx < Pf ? nx : cur, lane, nxt);
            reduce_item(buf, cur);
            cur = nx;
        }
    } else {
        // fp32 items (twice the registers) one at a time
        while (cur < Pf) {
            u32x4 buf[I::VPL];
            stage1_load_full<DT>(rowp, cur, lane, buf);
            __builtin_amdgcn_sched_barrier(0);
            reduce_item(buf, cur);
            cur = next_item();
        }
    }
    if (sel_thread) s_xsel = xsel;
    __syncthreads();

    // lse: lanes 0..15 of wave 4 merge their groups, the wave the groups
    // (the split path's arithmetic), then lane 0 raises s_lse_ready; the
    // selection on waves 0..3 reads the lse only for its last step
    constexpr int kLseWave = kThreads / 64;
    if (wave == kLseWave) {
        float m = kNegInf, sm = 0.f;
        if (lane < kGroups)
            for (int32_t i = lane; i < P; i += kGroups) lse_merge(m, sm, sitem[i].x, sitem[i].y);
        const float l = lse_tree16(m, sm);
        if (lane == 0) {
            __hip_atomic_store(&sh.lse, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_store(&s_lse_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            lse_out[row] = l;
            if (sel != nullptr && sel_out != nullptr) write_selected(V, s_sel, s_xsel, l, sel_out + row, err);
        }
        return;
    }
    if (!KEYS) return;

    // the selection runs on waves 0..3 (the same 256-thread code as the split
    // path); the other waves end here (a barrier waits on surviving waves only)
    if (wave >= kThreads / 64) return;
    uint32_t kr[KPT];
    if (K <= nb) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            kr[j] = w16(DT) ? ((uint32_t)skeys[tid * KPT + j] << 16) : (uint32_t)skeys[tid * KPT + j];
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) kr[j] = 0u;
    }
    row_topk<DT, KPT, kThreads, w16(DT), true>(rowp, row, V, nb, K, kr, &sh.lse, cand, cand + cap, cap, sh,
                                                topk_ids, topk_lp, &s_lse_ready, cap / kBlock,
                                                reinterpret_cast<u32x4*>(cand + cap + ((K + 1) & ~1)), s_tkey);
}

// ---------------------------------------------------------------------------
// Full-vocabulary logprobs (K = -1; openinfer issue #719, Acceptance
// criteria): out[r][v] = fp32(x[r][v]) - lse[r], one rounding, the same
// value the top-K path writes for the ids it returns. One thread per 16-byte
// group of a row; entries past the vocabulary are not written.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_full_logprobs(const uint8_t* __restrict__ logits, int64_t ld,
                                                            int64_t V, uint32_t chunks,
                                                            const float* __restrict__ lse,
                                                            float* __restrict__ out) {
    constexpr int EPV = w16(DT) ? 8 : 4;
    constexpr size_t ESZ = w16(DT) ? 2 : 4;
    const uint32_t r = blockIdx.x / chunks;
    const int64_t e0 = ((int64_t)(blockIdx.x - r * chunks) * kThreads + threadIdx.x) * EPV;
    if (e0 >= V) return;
    const float l = lse[r];
    const u32x4 w = load_part<DT>(logits + (size_t)r * (size_t)ld * ESZ, V, e0);
    float* o = out + (int64_t)r * V + e0;
    float y[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
        const uint32_t wd = w[e / (w16(DT) ? 2 : 1)];
        const float x = w16(DT) ? ((e & 1) ? hi16<DT>(wd) : lo16<DT>(wd)) : __uint_as_float(wd);
        y[e] = x - l;
    }
    // whole groups on a 16-byte aligned output: 16-byte non-temporal stores
    // (scalar stores, each lane writing 4 of every 32 bytes, ran at a third
    // of the HBM rate)
    if (e0 + EPV <= V && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
#pragma unroll
        for (int q = 0; q < EPV / 4; ++q)
            __builtin_nontemporal_store(f32x4{y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]},
                                        reinterpret_cast<f32x4*>(o) + q);
    } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            if (e0 + e < V) o[e] = y[e];
    }
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

hipError_t launch_full_logprobs(const void* logits, int32_t dt, int64_t rows, int64_t vocab, int64_t ld,
                                const float* lse, float* out, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const int epv = w16(dt) ? 8 : 4;
    const int64_t groups = (vocab + epv - 1) / epv;
    const uint32_t chunks = (uint32_t)((groups + kThreads - 1) / kThreads);
    const dim3 grid((unsigned)(chunks * rows));
    const uint8_t* lg = static_cast<const uint8_t*>(logits);
    if (dt == kDtBf16)
        hipLaunchKernelGGL((k_full_logprobs<kDtBf16>), grid, dim3(kThreads), 0, s, lg, ld, vocab, chunks, lse, out);
    else if (dt == kDtF16)
        hipLaunchKernelGGL((k_full_logprobs<kDtF16>), grid, dim3(kThreads), 0, s, lg, ld, vocab, chunks, lse, out);
    else
        hipLaunchKernelGGL((k_full_logprobs<kDtF32>), grid, dim3(kThreads), 0, s, lg, ld, vocab, chunks, lse, out);
    return hipGetLastError();
}

hipError_t launch_reduce_stage1(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    char* ws = static_cast<char*>(a.ws);
    float2* part = reinterpret_cast<float2*>(ws + p.part_off);
    void* keys = p.k > 0 ? ws + p.keys_off : nullptr;   // block maxima only feed the top-K
    const dim3 grid((unsigned)p.wgs);
    const uint8_t* lg = static_cast<const uint8_t*>(a.logits);
    const bool k = keys != nullptr;
    auto go = [&](auto dt) {
        constexpr int DT = decltype(dt)::value;
        if (k)
            hipLaunchKernelGGL((k_stage1<DT, true>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.kld,
                               p.splits, p.nitems, part, keys);
        else
            hipLaunchKernelGGL((k_stage1<DT, false>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.kld,
                               p.splits, p.nitems, part, keys);
    };
    if (a.dt == kDtBf16)
        go(std::integral_constant<int, kDtBf16>{});
    else if (a.dt == kDtF16)
        go(std::integral_constant<int, kDtF16>{});
    else
        go(std::integral_constant<int, kDtF32>{});
    return hipGetLastError();
}

template <int DT, int KPT, bool BLOCKS>
hipError_t launch_stage2_kpt(const ReducePlan& p, const ReduceArgs& a, hipStream_t s, const float2* part,
                             const void* keys, int32_t cap, size_t lds) {
    const void* fn = (const void*)k_stage2<DT, KPT, BLOCKS>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_stage2<DT, KPT, BLOCKS>), dim3((unsigned)p.rows), dim3(kThreads), lds, s,
                       static_cast<const uint8_t*>(a.logits), a.ld, p.vocab, p.nb, p.kld, p.splits, part,
                       keys, a.sel, p.k, a.lse, a.sel_lp, a.topk_ids, a.topk_lp, a.err, cap);
    return hipGetLastError();
}

template <int DT, bool BLOCKS = false>
hipError_t launch_stage2_dt(const ReducePlan& p, const ReduceArgs& a, hipStream_t s, const float2* part,
                            const void* keys, int32_t cap, size_t lds) {
    switch (p.kpt) {
        case 4: return launch_stage2_kpt<DT, 4, BLOCKS>(p, a, s, part, keys, cap, lds);
        case 8: return launch_stage2_kpt<DT, 8, BLOCKS>(p, a, s, part, keys, cap, lds);
        case 16: return launch_stage2_kpt<DT, 16, BLOCKS>(p, a, s, part, keys, cap, lds);
        default: return launch_stage2_kpt<DT, 32, BLOCKS>(p, a, s, part, keys, cap, lds);
    }
}

// Candidate entries a row's selection can hold: up to 2K candidate blocks
// (at most 128), so that the prefetched-candidate path of 16-bit logits also
// takes blocks tied at T, and fp32 logits keep a whole 16-bit bin of blocks.
int32_t cand_cap(const ReducePlan& p) {
    if (p.k <= 0) return 0;
    return std::min(std::max(p.k, std::min(2 * p.k, kMaxCandidates / kBlock)), p.nb) * kBlock;
}

// candidates and LDS of the second kernel (fp32 logits: no staging)
void stage2_sizes(const ReducePlan& p, int32_t dt, int32_t& cap, size_t& lds) {
    cap = 0;
    lds = 0;
    if (p.k > 0) {
        cap = cand_cap(p);
        // (the staging path exists only when K <= nb)
        const size_t stage = w16(dt) && p.k <= p.nb ? ((size_t)kThreads * kBlock + (size_t)cap) * 2 : 0;
        lds = ((size_t)cap + (size_t)((p.k + 1) & ~1)) * sizeof(uint64_t) + stage;
    }
}

hipError_t launch_reduce_stage2_blocks(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    if (a.dt != kDtF32 || p.splits != p.nb) return hipErrorInvalidValue;
    char* ws = static_cast<char*>(a.ws);
    int32_t cap;
    size_t lds;
    stage2_sizes(p, a.dt, cap, lds);
    return launch_stage2_dt<kDtF32, true>(p, a, s, reinterpret_cast<const float2*>(ws + p.part_off),
                                          ws + p.keys_off, cap, lds);
}

hipError_t launch_reduce_stage2(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    char* ws = static_cast<char*>(a.ws);
    const float2* part = reinterpret_cast<const float2*>(ws + p.part_off);
    const void* keys = ws + p.keys_off;
    int32_t cap = 0;
    size_t lds = 0;
    stage2_sizes(p, a.dt, cap, lds);
    if (a.dt == kDtBf16) return launch_stage2_dt<kDtBf16>(p, a, s, part, keys, cap, lds);
    if (a.dt == kDtF16) return launch_stage2_dt<kDtF16>(p, a, s, part, keys, cap, lds);
    return launch_stage2_dt<kDtF32>(p, a, s, part, keys, cap, lds);
}

// Compute units of the current device (cached per device id).
int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

namespace {

template <int DT, int KPT, bool KEYS>
hipError_t launch_row_kpt(const ReducePlan& p, const ReduceArgs& a, hipStream_t s, int32_t cap, size_t lds) {
    const void* fn = (const void*)k_rowreduce<DT, KPT, KEYS>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_rowreduce<DT, KPT, KEYS>), dim3((unsigned)p.rows), dim3(kRowThreads), lds, s,
                       static_cast<const uint8_t*>(a.logits), a.ld, p.vocab, p.nb, p.splits, a.sel, p.k, a.lse,
                       a.sel_lp, a.topk_ids, a.topk_lp, a.err, cap);
    return hipGetLastError();
}

}  // namespace

bool reduce_row_path(const ReducePlan& p) {
    const int ncu = cu_count();
    if (ncu <= 0 || p.rows < ncu) return false;
    if (p.splits > kRowMaxItems) return false;   // vocab above 64 * 4096: the split path
    if (p.k > 0 && p.kpt > 16) return false;   // more than 4096 blocks: the split path
    // one workgroup per CU at a time: the rows must fill the CUs evenly
    const int64_t rounds = (p.rows + ncu - 1) / ncu;
    return p.rows * 4 >= rounds * ncu * 3;
}

bool single_ok(const ReducePlan& p) {
    return p.rows > 0 && p.rows <= kSingleMaxRows && p.k >= 0 && p.k <= kSingleMaxK &&
           p.splits <= 4 * kSingleMaxSlices && !reduce_row_path(p);
}

size_t single_bytes(const ReducePlan& p) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t S = (size_t)(p.splits + 3) / 4;
    return up((size_t)p.rows * p.splits * sizeof(float2)) + 2 * up((size_t)p.rows * S * p.k * 4);
}

hipError_t launch_reduce_single(const ReducePlan& p, const ReduceArgs& a, uint32_t* counters, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    if (!single_ok(p) || counters == nullptr) return hipErrorInvalidValue;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int32_t S = (p.splits + 3) / 4;
    char* ws = static_cast<char*>(a.ws);
    float2* part = reinterpret_cast<float2*>(ws);
    const size_t lb = up((size_t)p.rows * S * p.k * 4);
    int32_t* loc_ids = reinterpret_cast<int32_t*>(ws + up((size_t)p.rows * p.splits * sizeof(float2)));
    float* loc_vals = reinterpret_cast<float*>(reinterpret_cast<char*>(loc_ids) + lb);
    const dim3 grid((unsigned)(p.rows * S));
    auto go = [&](auto dt) {
        constexpr int DT = decltype(dt)::value;
        const uint8_t* lg = static_cast<const uint8_t*>(a.logits);
        if (p.k > 0)
            hipLaunchKernelGGL((k_single<DT, true>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.splits, S,
                               a.sel, p.k, a.lse, a.sel_lp, a.topk_ids, a.topk_lp, a.err, part, loc_ids,
                               loc_vals, counters);
        else
            hipLaunchKernelGGL((k_single<DT, false>), grid, dim3(kThreads), 0, s, lg, a.ld, p.vocab, p.splits, S,
                               a.sel, 0, a.lse, a.sel_lp, a.topk_ids, a.topk_lp, a.err, part, loc_ids,
                               loc_vals, counters);
    };
    if (a.dt == kDtBf16)
        go(std::integral_constant<int, kDtBf16>{});
    else if (a.dt == kDtF16)
        go(std::integral_constant<int, kDtF16>{});
    else
        go(std::integral_constant<int, kDtF32>{});
    return hipGetLastError();
}

hipError_t launch_reduce(const ReducePlan& p, const ReduceArgs& a, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    if (!reduce_row_path(p)) {
        const hipError_t e = launch_reduce_stage1(p, a, s);
        if (e != hipSuccess) return e;
        return launch_reduce_stage2(p, a, s);
    }
    int32_t cap = 0;
    size_t lds = 0;
    if (p.k > 0) {
        cap = cand_cap(p);
        const size_t kbytes = (size_t)p.kpt * kThreads * (w16(a.dt) ? 2 : 4);
        // staged blocks: one per selection thread, then the candidate blocks
        // (the staging path exists only when K <= nb)
        const size_t stage = w16(a.dt) && p.k <= p.nb ? ((size_t)kThreads * kBlock + (size_t)cap) * 2 : 0;
        lds = kbytes + ((size_t)cap + (size_t)((p.k + 1) & ~1)) * sizeof(uint64_t) + stage;
    }
    auto go = [&](auto dt) -> hipError_t {
        constexpr int DT = decltype(dt)::value;
        if (p.k == 0) return launch_row_kpt<DT, 4, false>(p, a, s, cap, lds);
        switch (p.kpt) {
            case 4: return launch_row_kpt<DT, 4, true>(p, a, s, cap, lds);
            case 8: return launch_row_kpt<DT, 8, true>(p, a, s, cap, lds);
            default: return launch_row_kpt<DT, 16, true>(p, a, s, cap, lds);
        }
    };
    if (a.dt == kDtBf16) return go(std::integral_constant<int, kDtBf16>{});
    if (a.dt == kDtF16) return go(std::integral_constant<int, kDtF16>{});
    return go(std::integral_constant<int, kDtF32>{});
}

}  // namespace lmh
