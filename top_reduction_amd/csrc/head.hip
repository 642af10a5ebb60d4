// head.hip -- gathered-row LM-head projection on gfx950 (vllm-metal release
// v0.4.0, Summary: project only the sampled rows; mlxcel PR #1969: the head
// acts per position, so a gathered row's logits equal the full projection's).
//
//   logits[r][v] = sum_k hidden[src(r)][k] * W[v][k]
//
// bf16 operands run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation. Both
// bf16 kernels feed every output element the same sequence of MFMAs: the
// hidden dimension in ascending 32-wide steps, lane l holding k = 8*(l/16) ..
// 8*(l/16)+7 of the step for row/column l%16, no split over k. A row's logits
// are therefore bitwise the same whichever kernel, tile position or set of
// companion rows produced them.
//
//   stream  (R <= 64): weight-streaming. Each workgroup owns a 128-row slab of
//           W and reads it once, straight from HBM into MFMA B fragments,
//           a full k-chunk ahead; the gathered hidden rows (small, L2
//           resident) are staged through LDS and shared by the 4 waves.
//   tiled   (any R): 256 x 256 output tiles, 8 waves of 128 x 64; both
//           operands pass through double-buffered LDS fed 3 k-steps ahead;
//           workgroups are mapped so that each XCD walks the row tiles of one
//           W slab together.
//   f32     fp32 operands: plain fp32 FMA in ascending k.
#include <type_traits>

#include "head_common.h"

namespace lmh {
namespace {


constexpr int kThreads = 256;
#ifndef LMH_STREAM_NT
#define LMH_STREAM_NT 1
#endif
#ifndef LMH_STREAM_KC
#define LMH_STREAM_KC 256
#endif
#ifndef LMH_STREAM_WAVES
#define LMH_STREAM_WAVES 4
#endif
#ifndef LMH_STREAMQ_NT
#define LMH_STREAMQ_NT 1
#endif
#ifndef LMH_STREAMQ_KC
#define LMH_STREAMQ_KC 256
#endif
constexpr int kStreamNT = LMH_STREAM_NT;   // 16-row W tiles per wave in the streaming head
constexpr int kStreamKC = LMH_STREAM_KC;   // hidden elements per streaming-head k-chunk
constexpr int kStreamThreads = 64 * LMH_STREAM_WAVES;    // threads per streaming-head workgroup
#ifndef LMH_STREAMQ_WAVES
#define LMH_STREAMQ_WAVES 8
#endif
constexpr int kStreamQNT = LMH_STREAMQ_NT; // the same for quantised weights
constexpr int kStreamQKC = LMH_STREAMQ_KC;
constexpr int kStreamQThreads = 64 * LMH_STREAMQ_WAVES;   // threads per quantised-stream workgroup

template <bool OUT_BF16>
__device__ inline void store_out(void* out, int64_t off, float v) {
    if (OUT_BF16)
        __builtin_nontemporal_store(f32_to_bf16_rne(v), reinterpret_cast<uint16_t*>(out) + off);
    else
        __builtin_nontemporal_store(v, reinterpret_cast<float*>(out) + off);
}

// Four consecutive bf16 logits (elements off .. off + 3, off a multiple of 4
// on an 8-byte aligned output) as one 8-byte store.
__device__ inline void store_bf16x4(void* out, int64_t off, const f32x4& v) {
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
    __builtin_nontemporal_store(((uint64_t)hi << 32) | lo,
                                reinterpret_cast<uint64_t*>(reinterpret_cast<uint16_t*>(out) + off));
}

// Drives step(PF, c, current, next) over chunks 0..n-1 with two weight
// register sets that alternate without copies (a copy of a prefetch
// destination would wait for the prefetch). Inside the loop every step
// prefetches, so the loop header is reached with the same loads in flight on
// every path and the wait counts stay exact; the last one or two steps, the
// last of which prefetches nothing, are peeled after it.
template <typename Step, typename W>
__device__ inline void chunk_loop(int n, Step& step, W& w0, W& w1) {
    using Y = std::integral_constant<bool, true>;
    using N = std::integral_constant<bool, false>;
    int c = 0;
    for (; c + 2 < n; c += 2) {
        step(Y{}, c, w0, w1);
        step(Y{}, c + 1, w1, w0);
    }
    if (c + 1 < n) {
        step(Y{}, c, w0, w1);
        step(N{}, c + 1, w1, w0);
    } else {
        step(N{}, c, w0, w1);
    }
}

// Logits of a streaming workgroup as whole row segments: each wave's MFMA
// results (lane: rows 4*(lane/16)+e of column lane%16 of each 16-row tile)
// go to an LDS staging tile of MT*16 rows x TPB/4*NT columns, then the
// workgroup stores 16-byte pieces of consecutive columns (4 fp32 or 8 bf16
// logits) -- vocabulary and row pitch multiples of that count, 16-byte
// aligned output. The caller's barrier must precede it (`so` reuses the
// hidden-row buffers).
template <bool OUT_BF16>
__device__ inline bool rows_vec_ok(const HeadParams& p) {
    constexpr int E = OUT_BF16 ? 8 : 4;
    return p.V % E == 0 && p.old % E == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
}
template <int MT, int NT, int TPB, bool OUT_BF16>
__device__ inline void store_rows_staged(const HeadParams& p, float* __restrict__ so,
                                         const f32x4 (&acc)[MT][NT], const int32_t* sIdx) {
    constexpr int ROWS = MT * 16;
    constexpr int CW = TPB / 4 * NT;            // the workgroup's columns
    constexpr int CWP = CW + 4;                 // staged row pitch (floats)
    constexpr int E = OUT_BF16 ? 8 : 4;         // logits per 16-byte piece
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = i * 16 + (lane >> 4) * 4 + e;
                const float val = (r < p.R && sIdx[r] < 0) ? kNaN : scale_logit(acc[i][j][e], p.scale_mode, p.scale);
                so[r * CWP + wave * 16 * NT + j * 16 + (lane & 15)] = val;
            }
    __syncthreads();
    const int64_t col0 = (int64_t)blockIdx.x * CW;
    constexpr int NCH = ROWS * (CW / E);        // 16-byte pieces
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += TPB) {
        const int c = c0 + tid;
        if (NCH % TPB == 0 || c < NCH) {
            const int r = c / (CW / E);
            const int cc = (c % (CW / E)) * E;
            const int64_t col = col0 + cc;
            if (r < p.R && col < p.V) {
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(&so[r * CWP + cc]);
                if constexpr (OUT_BF16) {
                    const f32x4 v1 = *reinterpret_cast<const f32x4*>(&so[r * CWP + cc + 4]);
                    const u32x4 wd{(uint32_t)f32_to_bf16_rne(v0[0]) | ((uint32_t)f32_to_bf16_rne(v0[1]) << 16),
                                   (uint32_t)f32_to_bf16_rne(v0[2]) | ((uint32_t)f32_to_bf16_rne(v0[3]) << 16),
                                   (uint32_t)f32_to_bf16_rne(v1[0]) | ((uint32_t)f32_to_bf16_rne(v1[1]) << 16),
                                   (uint32_t)f32_to_bf16_rne(v1[2]) | ((uint32_t)f32_to_bf16_rne(v1[3]) << 16)};
                    __builtin_nontemporal_store(
                        wd, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)r * p.old + col));
                } else {
                    __builtin_nontemporal_store(
                        v0, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + (int64_t)r * p.old + col));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel: MT row tiles of 16 (R <= 16*MT) against a slab of
// 64*NT W rows per workgroup (16*NT per wave), k in chunks of KC (256). Each
// wave loads its W fragments straight from HBM into MFMA B operands a whole
// chunk ahead; the gathered hidden rows come through double-buffered LDS,
// shared by the 4 waves. Small slabs keep the last, partly filled round of
// workgroups short. fp32 logits leave as whole row segments through LDS
// (store_rows_staged) where the vocabulary and the row pitch allow.
// ---------------------------------------------------------------------------
template <int MT, int NT, bool KFULL, bool OUT_BF16>
__global__ __launch_bounds__(kStreamThreads) void k_head_stream(HeadParams p) {
    constexpr int KC = kStreamKC;       // hidden elements per chunk
    constexpr int KS = KC / 32;         // MFMA k-steps per chunk
    constexpr int AP = KC + 8;          // LDS row pitch (elements): +16 B breaks bank aliasing
    constexpr int ROWS = MT * 16;
    constexpr int AVN = ROWS * KC / 8;                      // 16-B A vectors per chunk
    constexpr int TPB = kStreamThreads;
    constexpr int AV = (AVN + TPB - 1) / TPB;               // ... per thread
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][ROWS][AP];
    __shared__ int32_t sIdx[ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t nbase = (int64_t)blockIdx.x * (TPB / 4 * NT) + wave * (16 * NT);
    const int l16 = lane & 15;
    const int kq = (lane >> 4) * 8;

    if (tid < ROWS)
        sIdx[tid] = (tid < p.R) ? row_source(p.row0 + tid, p.cu, p.num_decode, p.num_tokens, p.ex) : -1;
    __syncthreads();

    const int nchunks = (int)((p.H + KC - 1) / KC);
    const int ksteps = (int)((p.H + 31) / 32);

    // Loads are branch-free (clamped address, then a select), so the compiler
    // can keep every prefetch in flight across the loop instead of draining
    // the memory counters at divergent joins.
    const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
    int64_t a_off[AV];    // element offset of this thread's A source rows
    int a_kv[AV];         // its 8-element column group within a chunk
#pragma unroll
    for (int j = 0; j < AV; ++j) {
        const int idx = j * TPB + tid;
        const bool in = (AVN % TPB == 0) || idx < AVN;
        const int row = in ? idx / (KC / 8) : 0;
        const int32_t t = sIdx[row];
        a_off[j] = (int64_t)(t >= 0 ? t : 0) * p.hld;
        a_kv[j] = in ? (idx % (KC / 8)) * 8 : 0;
    }
    int64_t w_off[NT];    // element offset of this lane's W rows
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int64_t n = nbase + j * 16 + l16;
        w_off[j] = (n < p.V ? n : p.V - 1) * p.wld;
    }

    // A rows without a source (their outputs are written as NaN) and W rows
    // past the vocabulary (their columns are never stored) read a clamped,
    // valid row; only a chunk that runs past the hidden size needs zeros.
    // KFULL (the hidden size is a multiple of KC) compiles the loads without
    // any k guard, which keeps the memory counters exact across the loop.
    auto load_a = [&](int c, u32x4 (&r)[AV]) {
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int64_t k = (int64_t)c * KC + a_kv[j];
            if (KFULL) {
                r[j] = *reinterpret_cast<const u32x4*>(p.hidden + a_off[j] + k);
            } else {
                const bool ok = k < p.H;
                const u32x4 v = *reinterpret_cast<const u32x4*>(p.hidden + a_off[j] + (ok ? k : 0));
                r[j] = ok ? v : zero4;
            }
        }
    };
    auto store_a = [&](int buf, const u32x4 (&r)[AV]) {
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int idx = j * TPB + tid;
            if (AVN % TPB == 0 || idx < AVN) {
                const int row = idx / (KC / 8);
                const int kv = idx % (KC / 8);
                *reinterpret_cast<u32x4*>(&sA[buf][row][kv * 8]) = r[j];
            }
        }
    };
    auto load_w = [&](int c, u32x4 (&r)[KS][NT]) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t k = (int64_t)c * KC + s * 32 + kq;
                if (KFULL) {
                    r[s][j] = *reinterpret_cast<const u32x4*>(p.W + w_off[j] + k);
                } else {
                    const bool ok = k < p.H;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(p.W + w_off[j] + (ok ? k : 0));
                    r[s][j] = ok ? v : zero4;
                }
            }
        }
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 areg[AV];
    u32x4 w0[KS][NT], w1[KS][NT];
    load_a(0, areg);
    store_a(0, areg);
    load_w(0, w0);
    __syncthreads();

    // one k-chunk: prefetch the next chunk's A and W (PF: every step but the
    // last), multiply this one
    auto step = [&](auto PF, int c, const u32x4 (&wc)[KS][NT], u32x4 (&wn)[KS][NT]) {
        const int buf = c & 1;
        if constexpr (decltype(PF)::value) {
            // A first: its loads are consumed at the end of this step, and
            // memory counters retire in issue order, so waiting for them must
            // not also wait for the weight prefetch issued after them
            load_a(c + 1, areg);
            __builtin_amdgcn_sched_barrier(0);
            load_w(c + 1, wn);
            // keep the whole prefetch at the top of the step, A first
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (KFULL || c * KS + s < ksteps) {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(&sA[buf][i * 16 + l16][s * 32 + kq]);
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] = mfma16(a, wc[s][j], acc[i][j]);
                }
            }
        }
        if constexpr (decltype(PF)::value) store_a(buf ^ 1, areg);
        __syncthreads();
    };
    chunk_loop(nchunks, step, w0, w1);

    // whole row segments (aligned rows)
    if (rows_vec_ok<OUT_BF16>(p)) {
        static_assert(sizeof(sA) >= (size_t)ROWS * (TPB / 4 * NT + 4) * 4, "the staging fits sA");
        store_rows_staged<MT, NT, TPB, OUT_BF16>(p, reinterpret_cast<float*>(&sA[0][0][0]), acc, sIdx);
        return;
    }
    // D fragment: lane holds rows 4*(lane/16)+e of column lane%16
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t v = nbase + j * 16 + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = i * 16 + (lane >> 4) * 4 + e;
                if (r < p.R && v < p.V) {
                    const float val = sIdx[r] < 0 ? kNaN : scale_logit(acc[i][j][e], p.scale_mode, p.scale);
                    store_out<OUT_BF16>(p.out, (int64_t)r * p.old + v, val);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel for quantised weights: the structure of k_head_stream
// (MT row tiles, 16*NT W rows per wave, k in chunks of KC staged through LDS
// for the hidden rows) with the weights read as codes, one 16-byte run per
// lane per QB hidden elements plus the lane's group scale and bias, and
// dequantised to bf16 in registers right before their MFMAs. The hidden size
// is a multiple of 128, so every run is whole; runs past the hidden size (in
// the last chunk) are skipped. The logits leave as in k_head_stream.
// ---------------------------------------------------------------------------
// NG > 0: the chunk's NG group scales (and biases) of a W row are read with
// one vector load per lane (the hidden size is a multiple of KC = NG * group
// and the scale row pitch is even); NG = 0: one 2-byte load per run and lane.
template <int MT, int NT, int BITS, int NG, bool OUT_BF16>
__global__ __launch_bounds__(kStreamQThreads) void k_head_stream_q(HeadParams p) {
    using O = QOrder<BITS>;
    constexpr int KC = kStreamQKC;      // hidden elements per chunk
    constexpr int RPC = KC / O::QB;     // code runs per chunk
    constexpr int ND = NG > 0 ? NG / 2 : 1;   // scale dwords per chunk and row
    constexpr int AP = KC + 8;          // LDS row pitch (elements)
    constexpr int ROWS = MT * 16;
    constexpr int AVN = ROWS * KC / 8;
    constexpr int TPB = kStreamQThreads;
    constexpr int AV = (AVN + TPB - 1) / TPB;
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][ROWS][AP];
    __shared__ int32_t sIdx[ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t nbase = (int64_t)blockIdx.x * (TPB / 4 * NT) + wave * (16 * NT);
    const int l16 = lane & 15;
    const int qd = lane >> 4;           // lane quarter

    if (tid < ROWS)
        sIdx[tid] = (tid < p.R) ? row_source(p.row0 + tid, p.cu, p.num_decode, p.num_tokens, p.ex) : -1;
    __syncthreads();

    const int nchunks = (int)((p.H + KC - 1) / KC);
    const int nruns = (int)(p.H / O::QB);

    int64_t a_off[AV];
    int a_kv[AV];
#pragma unroll
    for (int j = 0; j < AV; ++j) {
        const int idx = j * TPB + tid;
        const bool in = (AVN % TPB == 0) || idx < AVN;
        const int row = in ? idx / (KC / 8) : 0;
        const int32_t t = sIdx[row];
        a_off[j] = (int64_t)(t >= 0 ? t : 0) * p.hld;
        a_kv[j] = in ? (idx % (KC / 8)) * 8 : 0;
    }
    int64_t q_off[NT], s_off[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int64_t n = nbase + j * 16 + l16;
        const int64_t nc = n < p.V ? n : p.V - 1;
        q_off[j] = nc * p.qw.qld + 4 * qd;
        s_off[j] = nc * p.qw.sld;
    }

    // hidden elements past H (last chunk) read element 0; their steps are skipped
    auto load_a = [&](int c, u32x4 (&r)[AV]) {
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int64_t k = (int64_t)c * KC + a_kv[j];
            r[j] = *reinterpret_cast<const u32x4*>(p.hidden + a_off[j] + (k < p.H ? k : 0));
        }
    };
    auto store_a = [&](int buf, const u32x4 (&r)[AV]) {
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int idx = j * TPB + tid;
            if (AVN % TPB == 0 || idx < AVN) {
                const int row = idx / (KC / 8);
                const int kv = idx % (KC / 8);
                *reinterpret_cast<u32x4*>(&sA[buf][row][kv * 8]) = r[j];
            }
        }
    };
    // scale and bias stay 16-bit (or packed pairs) until used: a widening at
    // the loop back-edge would wait for the prefetch
    typedef uint32_t u32v __attribute__((ext_vector_type(ND), aligned(4)));
    struct WChunk {
        u32x4 q[RPC][NT];
        uint16_t sc[RPC][NT], bi[RPC][NT];      // NG == 0
        u32v sv[NT], bv[NT];                    // NG > 0: groups c*NG .. c*NG+NG-1
    };
    // runs past H read run 0 (NG == 0 only; with NG > 0 every chunk is whole)
    auto load_w = [&](int c, WChunk& w) {
#pragma unroll
        for (int u = 0; u < RPC; ++u) {
            const int run = c * RPC + u;
            const int rc = NG > 0 ? run : (run < nruns ? run : 0);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                w.q[u][j] = *reinterpret_cast<const u32x4*>(p.qw.q + q_off[j] + (int64_t)rc * 16);
            if constexpr (NG == 0) {
                const int g = (rc * O::QB + qd * O::QQ) >> p.qw.gshift;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    w.sc[u][j] = p.qw.scales[s_off[j] + g];
                    w.bi[u][j] = p.qw.biases[s_off[j] + g];
                }
            }
        }
        if constexpr (NG > 0) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                w.sv[j] = *reinterpret_cast<const u32v*>(p.qw.scales + s_off[j] + c * NG);
                w.bv[j] = *reinterpret_cast<const u32v*>(p.qw.biases + s_off[j] + c * NG);
            }
        }
    };
    // fp32 value of the group scale (or bias) of run u for this lane
    auto pick = [&](const u32v& v, int u) -> float {
        constexpr int G = NG > 0 ? KC / NG : 1;
        const int e = (u * O::QB + qd * O::QQ) / G;     // group within the chunk
        uint32_t d = v[0];
#pragma unroll
        for (int i = 1; i < ND; ++i) d = (e >> 1) == i ? v[i] : d;
        return __uint_as_float((e & 1) ? (d & 0xFFFF0000u) : (d << 16));
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 areg[AV];
    WChunk w0, w1;
    load_a(0, areg);
    store_a(0, areg);
    load_w(0, w0);
    __syncthreads();

    // PF: this step prefetches the next chunk (every step but the last)
    auto step = [&](auto PF, int c, const WChunk& wc, WChunk& wn) {
        const int buf = c & 1;
        if constexpr (decltype(PF)::value) {
            load_a(c + 1, areg);
            __builtin_amdgcn_sched_barrier(0);
            load_w(c + 1, wn);
            // keep the whole prefetch at the top of the step, A first
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int u = 0; u < RPC; ++u) {
            if (c * RPC + u < nruns) {
                float sf[NT], bf[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    if constexpr (NG > 0) {
                        sf[j] = pick(wc.sv[j], u);
                        bf[j] = pick(wc.bv[j], u);
                    } else {
                        sf[j] = __uint_as_float((uint32_t)wc.sc[u][j] << 16);
                        bf[j] = __uint_as_float((uint32_t)wc.bi[u][j] << 16);
                    }
                }
#pragma unroll
                for (int st = 0; st < O::SPB; ++st) {
                    u32x4 fb[NT];
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const u32x4 qv = wc.q[u][j];
                        if constexpr (BITS == 4)
                            fb[j] = dequant8<4>(qv[st], 0u, sf[j], bf[j]);
                        else
                            fb[j] = dequant8<8>(qv[2 * st], qv[2 * st + 1], sf[j], bf[j]);
                    }
                    const int ka = u * O::QB + qd * O::QQ + 8 * st;
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        const u32x4 a = *reinterpret_cast<const u32x4*>(&sA[buf][i * 16 + l16][ka]);
#pragma unroll
                        for (int j = 0; j < NT; ++j) acc[i][j] = mfma16(a, fb[j], acc[i][j]);
                    }
                }
            }
        }
        if constexpr (decltype(PF)::value) store_a(buf ^ 1, areg);
        __syncthreads();
    };
    chunk_loop(nchunks, step, w0, w1);

    // whole row segments (aligned rows)
    if (rows_vec_ok<OUT_BF16>(p)) {
        static_assert(sizeof(sA) >= (size_t)ROWS * (TPB / 4 * NT + 4) * 4, "the staging fits sA");
        store_rows_staged<MT, NT, TPB, OUT_BF16>(p, reinterpret_cast<float*>(&sA[0][0][0]), acc, sIdx);
        return;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t v = nbase + j * 16 + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = i * 16 + (lane >> 4) * 4 + e;
                if (r < p.R && v < p.V) {
                    const float val = sIdx[r] < 0 ? kNaN : scale_logit(acc[i][j][e], p.scale_mode, p.scale);
                    store_out<OUT_BF16>(p.out, (int64_t)r * p.old + v, val);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel: a 256 x 256 output tile per workgroup of 8 waves, one 128 x 64
// eighth per wave (8 x 4 MFMA tiles). k advances in stages of 32 (one MFMA
// k-step). Each stage's A (gathered hidden rows) and B (W rows) slices, 256 x
// 64 B each, pass through registers into one of two LDS buffers: loads of stage
// s+3 are issued while stage s is multiplied (three register sets in
// flight) and stage s+1 is written to LDS at the end of stage s; the A
// fragments are read one 16-row group ahead of their MFMAs. One workgroup
// (two waves per SIMD) per CU. The 16-byte chunks of a
// 64-byte LDS row are XOR-swizzled with bits 1..2 of the row, so the fragment
// reads (16 rows, one chunk each) and the staging writes (consecutive chunks)
// are free of bank conflicts. Loads are branch-free: rows past R or with no
// source read row 0 (their outputs are never written or are NaN), W rows past
// V read row V-1, and the chunks past H (the stage count is rounded up to a
// multiple of 3) read k = 0 and are zeroed on their way into LDS.
// ---------------------------------------------------------------------------
constexpr int kTileM = 256, kTileN = 256, kTileK = 32;
constexpr int kTileThreads = 512;
constexpr int kWaveN = 64;                                     // columns per wave
constexpr int kTileLA = kTileM * 4 / kTileThreads;             // A chunks per thread per stage
constexpr int kTileLB = kTileN * 4 / kTileThreads;             // B chunks per thread per stage
constexpr int kTileStage = (kTileM + kTileN) * kTileK * 2;     // bytes per LDS stage
constexpr int kTileLds = 72 * 1024 + kTileM * 4;               // 2 stages / epilogue staging + row sources

// Staging registers of one stage's B slice: bf16 chunks, or the codes of the
// same elements with their group's scale and bias (dequantised on the way
// into LDS).
template <int BITS>
struct TileB {
    u32x4 v[kTileLB];
};
template <>
struct TileB<4> {
    uint32_t q[kTileLB];
    uint16_t sc[kTileLB], bi[kTileLB];
    uint32_t sb[kTileLB];          // (scale, bias) from the LDS table
};
template <>
struct TileB<8> {
    uint32_t q0[kTileLB], q1[kTileLB];
    uint16_t sc[kTileLB], bi[kTileLB];
    uint32_t sb[kTileLB];
};

// Largest group count per row for which the quantised tiled kernel keeps its
// tile's scale/bias table in LDS (256 rows x (groups + 1) dwords after the
// stage buffers, within the 160 KB of a CU).
constexpr int kTileMaxTableGroups = (160 * 1024 - kTileLds) / (kTileN * 4) - 1;

// BITS = 16: bf16 weights; 4 or 8: quantised weights (hidden size a multiple
// of 128), whose stages follow the quantised k order: stage st is k-step
// st % SPB of code run st / SPB, and LDS chunk c of a row holds the 8
// elements of lane quarter c. STAB (quantised only): the scale and bias of
// every group of the tile's 256 W rows are loaded once into an LDS table of
// (scale, bias) dwords; otherwise each stage loads the two values it needs.
template <bool OUT_BF16, int BITS, bool STAB>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_head_tiled(HeadParams p, int32_t mtiles, int32_t ntiles) {
    constexpr bool QUANT = BITS != 16;
    using O = QOrder<QUANT ? BITS : 4>;
    constexpr int NF = kWaveN / 16;                 // B fragments (16-column groups) per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int32_t* sIdx = reinterpret_cast<int32_t*>(lds + 72 * 1024);

    // XCD-aware order (tile_of)
    const int32_t total = mtiles * ntiles;
    const int32_t per_xcd = (int32_t)((gridDim.x + 7) / 8);
    const int32_t logical = (int32_t)(blockIdx.x % 8) * per_xcd + (int32_t)(blockIdx.x / 8);
    if (logical >= total) return;
    int32_t mt, nt;
    tile_of(logical, mtiles, ntiles, mt, nt);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave >> 2) * 128;
    const int wn = (wave & 3) * kWaveN;
    const int32_t m0 = mt * kTileM;
    const int64_t n0 = (int64_t)nt * kTileN;

    if (tid < kTileM) {
        const int32_t r = m0 + tid;
        sIdx[tid] = (r < p.R) ? row_source(p.row0 + r, p.cu, p.num_decode, p.num_tokens, p.ex) : -1;
    }
    uint32_t* tab = reinterpret_cast<uint32_t*>(lds + kTileLds);
    const int tsp = STAB ? (int)(p.H >> p.qw.gshift) + 1 : 0;   // table row pitch (dwords)
    if constexpr (STAB) {
        const int ng = tsp - 1;
        for (int e = tid; e < kTileN * ng; e += kTileThreads) {
            const int row = e / ng;
            const int g = e - row * ng;
            const int64_t n = n0 + row < p.V ? n0 + row : p.V - 1;
            const uint32_t sv = p.qw.scales[n * p.qw.sld + g];
            const uint32_t bv = p.qw.biases[n * p.qw.sld + g];
            tab[row * tsp + g] = sv | (bv << 16);
        }
    }
    __syncthreads();

    // this thread's staging chunks: rows tid/4 + 128j, chunk tid%4
    const int c = tid & 3;
    int64_t ga[kTileLA], gb[kTileLB], gs[kTileLB];  // offsets of the chunks at k = 0
    uint32_t wofs[kTileLA];                         // LDS byte offsets within a stage's A slice
#pragma unroll
    for (int j = 0; j < kTileLA; ++j) {
        const int row = (tid >> 2) + 128 * j;
        const int32_t t = sIdx[row];
        ga[j] = (int64_t)(t < 0 ? 0 : t) * p.hld + (QUANT ? c * O::QQ : c * 8);
        wofs[j] = (uint32_t)(row * 64 + ((c ^ ((row >> 1) & 3)) << 4));
    }
#pragma unroll
    for (int j = 0; j < kTileLB; ++j) {
        const int row = (tid >> 2) + 128 * j;
        const int64_t n = n0 + row < p.V ? n0 + row : p.V - 1;
        if constexpr (QUANT) {
            gb[j] = n * p.qw.qld + 4 * c;           // words of lane quarter c in run 0
            gs[j] = n * p.qw.sld;
        } else {
            gb[j] = n * p.wld + c * 8;
            gs[j] = 0;
        }
    }
    // fragment read offset: row l%16 of a 16-row group, chunk l/16
    const int fr = lane & 15;
    const uint32_t rofs = (uint32_t)(fr * 64 + (((lane >> 4) ^ ((fr >> 1) & 3)) << 4));
    const uint32_t aofs = (uint32_t)(wm * 64) + rofs;
    const uint32_t bofs = (uint32_t)((kTileM + wn) * 64) + rofs;

    // a multiple of 3 stages; the chunks past H load zeros
    const int nst = (int)((p.H + 3 * kTileK - 1) / (3 * kTileK)) * 3;

    // chunks past H (the padding stages, or the tail of a last partial one)
    // load from k = 0 and are zeroed when written to LDS
    auto gload = [&](int st, u32x4 (&ra)[kTileLA], TileB<BITS>& rb) {
        if constexpr (!QUANT) {
            const int64_t k0 = (int64_t)st * kTileK;
            const int64_t k = k0 + c * 8 + 8 <= p.H ? k0 : 0;
#pragma unroll
            for (int j = 0; j < kTileLA; ++j) ra[j] = *reinterpret_cast<const u32x4*>(p.hidden + ga[j] + k);
#pragma unroll
            for (int j = 0; j < kTileLB; ++j) rb.v[j] = *reinterpret_cast<const u32x4*>(p.W + gb[j] + k);
        } else {
            // whole stages only (H is a multiple of 128); stages past H read run 0
            const bool in = (int64_t)st * kTileK < p.H;
            const int run = in ? st / O::SPB : 0;
            const int sub = st % O::SPB;
            const int64_t k = (int64_t)run * O::QB + 8 * sub;
            const int g = (run * O::QB + c * O::QQ) >> p.qw.gshift;
#pragma unroll
            for (int j = 0; j < kTileLA; ++j) ra[j] = *reinterpret_cast<const u32x4*>(p.hidden + ga[j] + k);
#pragma unroll
            for (int j = 0; j < kTileLB; ++j) {
                const uint32_t* qp = p.qw.q + gb[j] + (int64_t)run * 16;
                if constexpr (BITS == 4) {
                    rb.q[j] = qp[sub];
                } else {
                    const uint2 w = *reinterpret_cast<const uint2*>(qp + 2 * sub);
                    rb.q0[j] = w.x;
                    rb.q1[j] = w.y;
                }
                if constexpr (STAB) {
                    rb.sb[j] = tab[((tid >> 2) + 128 * j) * tsp + g];
                } else {
                    rb.sc[j] = p.qw.scales[gs[j] + g];
                    rb.bi[j] = p.qw.biases[gs[j] + g];
                }
            }
        }
    };
    // chunk j of a stage's A slice (j < kTileLA) or W slice (j - kTileLA),
    // dequantised for quantised weights, zero past H
    auto wchunk = [&](uint8_t* __restrict__ base, int st, int j, const u32x4 (&ra)[kTileLA], const TileB<BITS>& rb) {
        const bool z = QUANT ? (int64_t)st * kTileK >= p.H : (int64_t)st * kTileK + c * 8 + 8 > p.H;
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
        if (j < kTileLA) {
            *reinterpret_cast<u32x4*>(base + wofs[j]) = z ? zero : ra[j];
            return;
        }
        const int jb = j - kTileLA;
        u32x4 b;
        if constexpr (!QUANT) {
            b = rb.v[jb];
        } else {
            float sf, bf;
            if constexpr (STAB) {
                sf = __uint_as_float(rb.sb[jb] << 16);
                bf = __uint_as_float(rb.sb[jb] & 0xFFFF0000u);
            } else {
                sf = __uint_as_float((uint32_t)rb.sc[jb] << 16);
                bf = __uint_as_float((uint32_t)rb.bi[jb] << 16);
            }
            if constexpr (BITS == 4)
                b = dequant8<4>(rb.q[jb], 0u, sf, bf);
            else
                b = dequant8<8>(rb.q0[jb], rb.q1[jb], sf, bf);
        }
        *reinterpret_cast<u32x4*>(base + kTileM * 64 + wofs[jb]) = z ? zero : b;
    };
    f32x4 acc[8][NF];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One stage: its MFMAs from rd; stage sw's chunks (wa, wb) written to wr,
    // one per 16-row group, and the loads of stage sl into (la, lb) issued
    // after the first group, held there by scheduling barriers (the compiler
    // otherwise gathers the writes, with their dequantisation, after the last
    // MFMA). The first MFMA's two fragments are read first; A fragments two
    // 16-row groups ahead of their MFMAs. rd and wr are the two LDS buffers.
    static_assert(kTileLA + kTileLB <= 8, "one chunk write per 16-row group");
    auto step = [&](const uint8_t* __restrict__ rd, uint8_t* __restrict__ wr, int sw, const u32x4 (&wa)[kTileLA],
                    const TileB<BITS>& wb, int sl, u32x4 (&la)[kTileLA], TileB<BITS>& lb) {
        __builtin_amdgcn_sched_barrier(0);
        u32x4 fb[NF];
        u32x4 fa0 = *reinterpret_cast<const u32x4*>(rd + aofs);
#pragma unroll
        for (int j = 0; j < NF; ++j) fb[j] = *reinterpret_cast<const u32x4*>(rd + bofs + j * 16 * 64);
        u32x4 fa1 = *reinterpret_cast<const u32x4*>(rd + aofs + 16 * 64);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x4 cur = fa0;
            fa0 = fa1;
            if (i < 6) fa1 = *reinterpret_cast<const u32x4*>(rd + aofs + (i + 2) * 16 * 64);
#pragma unroll
            for (int j = 0; j < NF; ++j) acc[i][j] = mfma16(cur, fb[j], acc[i][j]);
            if (i < kTileLA + kTileLB) wchunk(wr, sw, i, wa, wb);
            if (i == 0) gload(sl, la, lb);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // stage s is multiplied from LDS buffer s%2 while stage s+1 is written to
    // the other buffer from register set (s+1)%3 and stage s+3 is loaded into
    // set s%3
    u32x4 ra0[kTileLA], ra1[kTileLA], ra2[kTileLA];
    TileB<BITS> rb0, rb1, rb2;
    gload(0, ra0, rb0);
    gload(1, ra1, rb1);
    gload(2, ra2, rb2);
#pragma unroll
    for (int j = 0; j < kTileLA + kTileLB; ++j) wchunk(lds, 0, j, ra0, rb0);
    __syncthreads();
    int cur = 0;                                    // LDS buffer of stage s
    for (int s = 0; s < nst; s += 3) {
        step(lds + cur * kTileStage, lds + (cur ^ 1) * kTileStage, s + 1, ra1, rb1, s + 3, ra0, rb0);
        __syncthreads();
        cur ^= 1;
        step(lds + cur * kTileStage, lds + (cur ^ 1) * kTileStage, s + 2, ra2, rb2, s + 4, ra1, rb1);
        __syncthreads();
        cur ^= 1;
        step(lds + cur * kTileStage, lds + (cur ^ 1) * kTileStage, s + 3, ra0, rb0, s + 5, ra2, rb2);
        __syncthreads();
        cur ^= 1;
    }

    // Epilogue through LDS (free after the last barrier): per pass, each wave
    // stages 32 rows x 64 columns of its quarter (fp32, rows padded by 16 B),
    // then stores whole 16-byte row segments, non-temporal. The scale mode is
    // resolved once per launch; a wave whose 128 x 64 block lies inside the
    // logits matrix with every row sourced stores with no per-element checks.
    const int lq = lane >> 4;
    float* stg = reinterpret_cast<float*>(lds) + wave * (32 * 68);
    const bool vec_ok = !OUT_BF16 && (p.old % 4 == 0) &&
                        ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
    // bf16 logits: four per 8-byte store
    const bool bf_ok = OUT_BF16 && (p.old % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.out) & 7) == 0);
    const bool rows_sourced = __all(sIdx[wm + lane] >= 0 && sIdx[wm + 64 + lane] >= 0);
    const bool fast = vec_ok && rows_sourced && m0 + wm + 128 <= p.R && n0 + wn + kWaveN <= p.V;
    float* const wout = reinterpret_cast<float*>(p.out) + (int64_t)(m0 + wm) * p.old + (n0 + wn);
    const int64_t lofs = (int64_t)lq * p.old + 4 * fr;
    auto epilogue = [&](auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = h * 2 + ii;
#pragma unroll
                for (int j = 0; j < NF; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) stg[(ii * 16 + lq * 4 + e) * 68 + j * 16 + fr] = acc[i][j][e];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lane l stores columns 4*(l%16) .. +3 of rows l/16 + 4q, q = 0..7
            f32x4 val[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                val[q] = *reinterpret_cast<const f32x4*>(&stg[(lq + 4 * q) * 68 + 4 * fr]);
#pragma unroll
                for (int e = 0; e < 4; ++e) val[q][e] = scale_logit(val[q][e], MODE, p.scale);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (fast) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    __builtin_nontemporal_store(val[q], reinterpret_cast<f32x4*>(wout + (int64_t)(h * 32 + 4 * q) * p.old + lofs));
                continue;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int rl = wm + h * 32 + lq + 4 * q;
                const int32_t r = m0 + rl;
                const int64_t v = n0 + wn + 4 * fr;
                if (r < p.R) {
                    const bool valid = sIdx[rl] >= 0;
                    const f32x4 ov = valid ? val[q] : f32x4{kNaN, kNaN, kNaN, kNaN};
                    if (vec_ok && v + 4 <= p.V) {
                        __builtin_nontemporal_store(ov, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + (int64_t)r * p.old + v));
                    } else if (bf_ok && v + 4 <= p.V) {
                        store_bf16x4(p.out, (int64_t)r * p.old + v, ov);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (v + e < p.V) store_out<OUT_BF16>(p.out, (int64_t)r * p.old + v + e, ov[e]);
                    }
                }
            }
        }
    };
    if (p.scale_mode == 1)
        epilogue(std::integral_constant<int, 1>{});
    else if (p.scale_mode == 2)
        epilogue(std::integral_constant<int, 2>{});
    else
        epilogue(std::integral_constant<int, 0>{});
}

// The reduction partial of one 64-logit block of logits row r, from the 16
// lanes of a DPP row that hold its columns (4 each, lane order = column
// order): the block maximum M (exact), S = the sum of exp(x - M) computed as
// in the reduction's stream (2^(x log2e + c) with c = -RN(M log2e), scaled
// once by 2^-e, e = M log2e + c exactly), the four terms of a lane added in
// column order and the lanes by a fixed pairwise tree. Columns past the
// vocabulary count as -inf. A row without a source (NaN logits) gives M =
// -inf and S = NaN, and the key of NaN, as the stream does on NaN logits.
// Called by every lane (the DPP exchanges need the whole row); one lane writes.
__device__ inline void block_partial(const HeadParams& p, int32_t r, bool has_src, int64_t v, const f32x4& val,
                                     int64_t blk) {
    constexpr float kLog2eF = 1.4426950408889634f;
    constexpr float kNegInfF = -__builtin_inff();
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v + e < p.V ? val[e] : kNegInfF;
    auto dpp = [](float a, auto ctl) {
        constexpr int C = decltype(ctl)::value;
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), C, 0xF, 0xF, false));
    };
    using q1 = std::integral_constant<int, 0xB1>;    // quad_perm [1,0,3,2]
    using q2 = std::integral_constant<int, 0x4E>;    // quad_perm [2,3,0,1]
    using hm = std::integral_constant<int, 0x141>;   // row_half_mirror
    using rm = std::integral_constant<int, 0x140>;   // row_mirror
    float m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    m = fmaxf(m, dpp(m, q1{}));
    m = fmaxf(m, dpp(m, q2{}));
    m = fmaxf(m, dpp(m, hm{}));
    m = fmaxf(m, dpp(m, rm{}));
    const float mr = m == kNegInfF ? 0.f : m;
    const float c = -(mr * kLog2eF);
    const float ee = fmaf(mr, kLog2eF, c);
    float sm = (__builtin_amdgcn_exp2f(fmaf(x[0], kLog2eF, c)) + __builtin_amdgcn_exp2f(fmaf(x[1], kLog2eF, c))) +
               (__builtin_amdgcn_exp2f(fmaf(x[2], kLog2eF, c)) + __builtin_amdgcn_exp2f(fmaf(x[3], kLog2eF, c)));
    sm += dpp(sm, q1{});
    sm += dpp(sm, q2{});
    sm += dpp(sm, hm{});
    sm += dpp(sm, rm{});
    sm *= __builtin_amdgcn_exp2f(-ee);
    if ((threadIdx.x & 15) == 0 && r < p.R && blk < p.nb) {
        const float nan = __builtin_nanf("");
        p.part[(int64_t)r * p.nb + blk] = has_src ? make_float2(m, sm) : make_float2(kNegInfF, nan);
        p.bkeys[(int64_t)r * p.kld + blk] = f32_key(has_src ? m : nan);
    }
}

// ---------------------------------------------------------------------------
// bf16 tiled kernel with 64-wide k stages (hidden size a multiple of 128):
// the same 256 x 256 tile, waves, MFMA sequence and epilogue as k_head_tiled,
// but each stage carries two MFMA k-steps (a whole 128-byte row of A and of
// W per stage), so a tile takes half the barriers and every row load is a
// full cache line. Two register sets keep the loads two stages ahead of
// double-buffered LDS (2 x 64 KB). The 16-byte chunks of a 128-byte LDS row
// are XOR-swizzled with bits 0..2 of the row.
// ---------------------------------------------------------------------------
constexpr int kT64K = 64;
constexpr int kT64Stage = (kTileM + kTileN) * kT64K * 2;         // 64 KB
constexpr int kT64Lds = 2 * kT64Stage + 2 * kTileM * 4;   // two stages, two row-source lists
// eight waves: four (one per SIMD, 128 x 128 each) measured 1.23 ms against
// 0.76 ms on the 2048-row Qwen3-0.6B projection

// Staging registers of one 64-wide stage's W chunks (four per thread): bf16
// chunks, or the 4-bit codes of the same elements with their group's
// (scale, bias) pair from the tile's LDS table, dequantised on the LDS write.
template <int BITS> struct T64B { u32x4 v[4]; };
template <> struct T64B<4> { uint32_t q[4]; uint32_t sb[4]; };

// Eight waves (two per SIMD), each 128 x 64 of the tile. The workgroups of an
// XCD take its share of the tiles in the banded order (tile_of): with as many
// workgroups as tiles each takes one; with PERSIST and fewer workgroups (one
// per CU), each walks its XCD's share, and the last two stages of a tile load
// the next tile's first two stages (its row sources resolved at the start of
// the tile), so those loads overlap the tile's epilogue and no workgroup is
// dispatched per tile (measured 726 -> 685 us on the 2048-row Qwen3-0.6B
// projection). The epilogue stages 16 rows per pass in the LDS buffer the
// last stage was read from.
// FUSED (fp32 logits): each wave's 64 columns are one 64-logit block of the
// vocabulary, and the epilogue also writes, per row, that block's maximum as
// a key and its (max, sum of exp(x - max)) partial -- the reduction's
// streaming pass, done on the values while they are in registers (MTPLX PR
// #532, Motivation: no second pass over a chunk's logits).
template <bool OUT_BF16, bool FUSED, bool PERSIST, int BITS = 16>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_head_tiled64(HeadParams p, int32_t mtiles, int32_t ntiles) {
    constexpr int NW = 8;
    constexpr int NTH = NW * 64;
    constexpr int WN = kTileN / (NW / 2);              // columns per wave
    constexpr int NF = WN / 16;                         // B fragments per wave
    static_assert(NF == 4, "a wave's 64 columns are one 64-logit block");
    static_assert(!FUSED || !OUT_BF16, "partials of fp32 logits");
    constexpr bool QUANT = BITS != 16;
    static_assert(!QUANT || (BITS == 4 && !FUSED && !PERSIST), "4-bit weights: plain logits, one tile per workgroup");
    using O = QOrder<QUANT ? BITS : 4>;
    constexpr int L = kTileM * (kT64K / 8) / NTH;       // chunks per thread per stage (A and B each)
    static_assert(L == 4, "eight chunk writes per stage, one per 16-row group of its first k-step");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int32_t* const sIdx2 = reinterpret_cast<int32_t*>(lds + 2 * kT64Stage);   // [2][kTileM] with PERSIST
    // quantised: the tile's (scale, bias) pairs, [kTileN][groups + 1] dwords
    uint32_t* const tab = reinterpret_cast<uint32_t*>(lds + 2 * kT64Stage + 2 * kTileM * 4);
    const int tsp = QUANT ? (int)(p.H >> p.qw.gshift) + 1 : 0;

    const int32_t total = mtiles * ntiles;
    const int32_t per_xcd = (total + 7) / 8;
    const int32_t xcd = (int32_t)(blockIdx.x % 8);
    const int32_t wgs = (int32_t)(gridDim.x / 8);       // workgroups per XCD
    const int32_t lo = xcd * per_xcd;
    const int32_t hi = lo + per_xcd < total ? lo + per_xcd : total;
    int32_t logical = lo + (int32_t)(blockIdx.x / 8);
    if (logical >= hi) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave / (NW / 2)) * 128;
    const int wn = (wave % (NW / 2)) * WN;
    const int c = tid & 7;
    const int fr = lane & 15;
    const int lq = lane >> 4;
    const uint32_t rofs0 = (uint32_t)(fr * 128 + ((((lane >> 4) + 0) ^ (fr & 7)) << 4));
    const uint32_t rofs1 = (uint32_t)(fr * 128 + ((((lane >> 4) + 4) ^ (fr & 7)) << 4));
    const int nst = (int)(p.H / kT64K);                  // even: H is a multiple of 128
    uint32_t wofs[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int row = (tid >> 3) + (NTH / 8) * j;
        wofs[j] = (uint32_t)(row * 128 + ((c ^ (row & 7)) << 4));
    }
    auto sources = [&](int32_t lg, int32_t* dst) {
        int32_t mt_, nt_;
        tile_of(lg, mtiles, ntiles, mt_, nt_);
        for (int t = tid; t < kTileM; t += NTH) {
            const int32_t r = mt_ * kTileM + t;
            dst[t] = (r < p.R) ? row_source(p.row0 + r, p.cu, p.num_decode, p.num_tokens, p.ex) : -1;
        }
    };
    // this thread's staging chunks of tile lg (rows tid/8 + 64j, chunk tid%8)
    // as 32-bit byte offsets from the hidden matrix and from the tile's first
    // W row
    // quantised: chunk c holds the 8 elements of lane quarter c % 4 for the
    // stage's k-step c / 4, in the quantised order (step s of a code run
    // gives lane quarter j the elements QB/4 j + 8 s of the run)
    const int hc = QUANT ? c >> 2 : 0, jq = QUANT ? c & 3 : 0;
    uint32_t ga[L], gb[L];
    const uint8_t* wtile;
    auto addresses = [&](int32_t lg, const int32_t* src) {
        int32_t mt_, nt_;
        tile_of(lg, mtiles, ntiles, mt_, nt_);
        const int64_t nb0 = (int64_t)nt_ * kTileN;
        if constexpr (QUANT)
            wtile = reinterpret_cast<const uint8_t*>(p.qw.q + nb0 * p.qw.qld);
        else
            wtile = reinterpret_cast<const uint8_t*>(p.W + nb0 * p.wld);
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int row = (tid >> 3) + (NTH / 8) * j;
            const int32_t t = src[row];
            if constexpr (QUANT) {
                const int64_t n = nb0 + row < p.V ? row : p.V - 1 - nb0;
                ga[j] = (uint32_t)(((int64_t)(t < 0 ? 0 : t) * p.hld + O::QQ * jq) * 2);
                gb[j] = (uint32_t)((n * p.qw.qld + 4 * jq) * 4);
            } else {
                ga[j] = (uint32_t)(((int64_t)(t < 0 ? 0 : t) * p.hld + c * 8) * 2);
                const int64_t n = nb0 + row < p.V ? row : p.V - 1 - nb0;
                gb[j] = (uint32_t)((n * p.wld + c * 8) * 2);
            }
        }
    };
    // stage st of the tile whose addresses are set (st >= nst: stage st - nst)
    auto gload = [&](int st, u32x4 (&ra)[L], T64B<BITS>& rb) {
        const int stt = st < nst ? st : st - nst;
        if constexpr (!QUANT) {
            const int64_t kb = (int64_t)stt * kT64K * 2;
            const uint8_t* const hk = reinterpret_cast<const uint8_t*>(p.hidden) + kb;
            const uint8_t* const wk = wtile + kb;
#pragma unroll
            for (int j = 0; j < L; ++j) ra[j] = *reinterpret_cast<const u32x4*>(hk + ga[j]);
#pragma unroll
            for (int j = 0; j < L; ++j) rb.v[j] = *reinterpret_cast<const u32x4*>(wk + gb[j]);
        } else {
            const int ks = 2 * stt + hc;                 // this thread's k-step
            const int run = ks / O::SPB, sub = ks - run * O::SPB;
            const uint8_t* const hk = reinterpret_cast<const uint8_t*>(p.hidden) + (run * O::QB + 8 * sub) * 2;
            const uint8_t* const wk = wtile + (run * 16 + sub) * 4;
            const int g = (run * O::QB + O::QQ * jq) >> p.qw.gshift;
#pragma unroll
            for (int j = 0; j < L; ++j) ra[j] = *reinterpret_cast<const u32x4*>(hk + ga[j]);
#pragma unroll
            for (int j = 0; j < L; ++j) {
                rb.q[j] = *reinterpret_cast<const uint32_t*>(wk + gb[j]);
                rb.sb[j] = tab[((tid >> 3) + (NTH / 8) * j) * tsp + g];
            }
        }
    };
    // W chunk j of a stage, as written to LDS
    auto wchunk = [&](const T64B<BITS>& rb, int j) -> u32x4 {
        if constexpr (!QUANT) {
            return rb.v[j];
        } else {
            const float sf = __uint_as_float(rb.sb[j] << 16);
            const float bf = __uint_as_float(rb.sb[j] & 0xFFFF0000u);
            return dequant8<4>(rb.q[j], 0u, sf, bf);
        }
    };
    f32x4 acc[8][NF];
    auto step = [&](const uint8_t* __restrict__ rd, uint8_t* __restrict__ wr, int st, u32x4 (&la)[L],
                    T64B<BITS>& lb, const u32x4 (&wa)[L], const T64B<BITS>& wb) {
        __builtin_amdgcn_sched_barrier(0);
        // the second k-step's first two fragments, read during the first
        // k-step's seventh 16-row group (2 % on the 2048-row projection)
        u32x4 pa, pb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t rofs = h == 0 ? rofs0 : rofs1;
            const uint32_t aofs = (uint32_t)(wm * 128) + rofs;
            const uint32_t bofs = (uint32_t)((kTileM + wn) * 128) + rofs;
            // the first MFMA's two fragments first, so that it waits on two
            // reads rather than five (3 % on the 2048-row projection); A
            // fragments two 16-row groups ahead of their MFMAs (one ahead
            // measured 2-3 % slower)
            u32x4 fb[NF];
            u32x4 fa0;
            if (h == 1) {
                fa0 = pa;
                fb[0] = pb;
            } else {
                fa0 = *reinterpret_cast<const u32x4*>(rd + aofs);
                fb[0] = *reinterpret_cast<const u32x4*>(rd + bofs);
            }
#pragma unroll
            for (int j = 1; j < NF; ++j) fb[j] = *reinterpret_cast<const u32x4*>(rd + bofs + j * 16 * 128);
            u32x4 fa1 = *reinterpret_cast<const u32x4*>(rd + aofs + 16 * 128);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 cur = fa0;
                fa0 = fa1;
                if (i < 6) fa1 = *reinterpret_cast<const u32x4*>(rd + aofs + (i + 2) * 16 * 128);
#pragma unroll
                for (int j = 0; j < NF; ++j) acc[i][j] = mfma16(cur, fb[j], acc[i][j]);
                if (h == 0) {
                    if (i < L)
                        *reinterpret_cast<u32x4*>(wr + wofs[i]) = wa[i];
                    else
                        *reinterpret_cast<u32x4*>(wr + kTileM * 128 + wofs[i - L]) = wchunk(wb, i - L);
                    if (i == 0) gload(st, la, lb);
                    if (i == 6) {
                        pa = *reinterpret_cast<const u32x4*>(rd + (uint32_t)(wm * 128) + rofs1);
                        pb = *reinterpret_cast<const u32x4*>(rd + (uint32_t)((kTileM + wn) * 128) + rofs1);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // the first tile: its row sources (and, quantised, its scale/bias
    // table), its first two stages
    int cur = 0;
    sources(logical, sIdx2);
    if constexpr (QUANT) {
        int32_t mt_, nt_;
        tile_of(logical, mtiles, ntiles, mt_, nt_);
        const int64_t nb0 = (int64_t)nt_ * kTileN;
        const int ng = tsp - 1;
        for (int e = tid; e < kTileN * ng; e += NTH) {
            const int row = e / ng;
            const int g = e - row * ng;
            const int64_t n = nb0 + row < p.V ? nb0 + row : p.V - 1;
            tab[row * tsp + g] = (uint32_t)p.qw.scales[n * p.qw.sld + g] | ((uint32_t)p.qw.biases[n * p.qw.sld + g] << 16);
        }
    }
    __syncthreads();
    addresses(logical, sIdx2);
    u32x4 ra0[L], ra1[L];
    T64B<BITS> rb0, rb1;
    gload(0, ra0, rb0);
    gload(1, ra1, rb1);
#pragma unroll
    for (int j = 0; j < L; ++j) *reinterpret_cast<u32x4*>(lds + wofs[j]) = ra0[j];
#pragma unroll
    for (int j = 0; j < L; ++j) *reinterpret_cast<u32x4*>(lds + kTileM * 128 + wofs[j]) = wchunk(rb0, j);
    __syncthreads();

    while (true) {
        int32_t mt, nt;
        tile_of(logical, mtiles, ntiles, mt, nt);
        const int32_t m0 = mt * kTileM;
        const int64_t n0 = (int64_t)nt * kTileN;
        const int32_t next = logical + wgs;
        const bool has_next = PERSIST && next < hi;
        int32_t* const sIdx = sIdx2 + cur * kTileM;
        int32_t* const sIdxN = sIdx2 + (cur ^ 1) * kTileM;
        if (has_next) sources(next, sIdxN);   // visible after the first step's barrier
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < nst; s += 2) {
            if (s == nst - 2 && has_next) {
                if (nst == 2) __syncthreads();
                addresses(next, sIdxN);   // the loads of stages nst, nst + 1: the next tile's 0, 1
            }
            step(lds, lds + kT64Stage, s + 2, ra0, rb0, ra1, rb1);
            __syncthreads();
            step(lds + kT64Stage, lds, s + 3, ra1, rb1, ra0, rb0);
            __syncthreads();
        }
        // buffer 0 now holds the next tile's first stage; the epilogue stages
        // through buffer 1 (16 rows x 64 columns per wave and pass, rows
        // padded by 16 B)
        float* stg = reinterpret_cast<float*>(lds + kT64Stage) + wave * (16 * 68);
        const bool vec_ok = !OUT_BF16 && (p.old % 4 == 0) &&
                            ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
        // bf16 logits: four per 8-byte store
        const bool bf_ok = OUT_BF16 && (p.old % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.out) & 7) == 0);
        const bool rows_sourced = __all(sIdx[wm + lane] >= 0 && sIdx[wm + 64 + lane] >= 0);
        const bool fast = vec_ok && rows_sourced && m0 + wm + 128 <= p.R && n0 + wn + WN <= p.V;
        float* const wout = reinterpret_cast<float*>(p.out) + (int64_t)(m0 + wm) * p.old + (n0 + wn);
        const int64_t lofs = (int64_t)lq * p.old + 4 * fr;
        auto epilogue = [&](auto mode_c) {
            constexpr int MODE = decltype(mode_c)::value;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) stg[(lq * 4 + e) * 68 + j * 16 + fr] = acc[i][j][e];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // lane l: columns 4*(l%16) .. +3 of rows l/16 + 4q, q = 0..3
                f32x4 val[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    val[q] = *reinterpret_cast<const f32x4*>(&stg[(lq + 4 * q) * 68 + 4 * fr]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) val[q][e] = scale_logit(val[q][e], MODE, p.scale);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (fast && !FUSED) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        __builtin_nontemporal_store(val[q], reinterpret_cast<f32x4*>(wout + (int64_t)(i * 16 + 4 * q) * p.old + lofs));
                    continue;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rl = wm + i * 16 + lq + 4 * q;
                    const int32_t r = m0 + rl;
                    const int64_t v = n0 + wn + 4 * fr;
                    const bool valid = sIdx[rl] >= 0;
                    if constexpr (FUSED) block_partial(p, r, valid, v, val[q], (n0 + wn) >> 6);
                    const f32x4 ov = valid ? val[q] : f32x4{kNaN, kNaN, kNaN, kNaN};
                    float* o = reinterpret_cast<float*>(p.out) + (int64_t)r * p.old + v;
                    if (fast) {
                        __builtin_nontemporal_store(ov, reinterpret_cast<f32x4*>(o));
                    } else if (r < p.R) {
                        if (vec_ok && v + 4 <= p.V) {
                            __builtin_nontemporal_store(ov, reinterpret_cast<f32x4*>(o));
                        } else if (bf_ok && v + 4 <= p.V) {
                            store_bf16x4(p.out, (int64_t)r * p.old + v, ov);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (v + e < p.V) store_out<OUT_BF16>(p.out, (int64_t)r * p.old + v + e, ov[e]);
                        }
                    }
                }
            }
        };
        if (p.scale_mode == 1)
            epilogue(std::integral_constant<int, 1>{});
        else if (p.scale_mode == 2)
            epilogue(std::integral_constant<int, 2>{});
        else
            epilogue(std::integral_constant<int, 0>{});
        if (!has_next) break;
        __syncthreads();   // staging done before the next tile writes buffer 1
        logical = next;
        cur ^= 1;
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: 8 rows x 256 vocab columns per workgroup; hidden rows staged in
// LDS by k-chunks of 128; one fp32 FMA per (row, column, k), k ascending.
// ---------------------------------------------------------------------------
struct HeadParamsF32 {
    int32_t scale_mode;
    float scale;
    const float* hidden;
    int64_t num_tokens, H, hld;
    const float* W;
    int64_t V, wld;
    const int32_t* cu;
    int32_t num_decode;
    const int32_t* ex;
    int32_t row0, R;
    void* out;
    int64_t old;
};

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void k_head_f32(HeadParamsF32 p) {
    constexpr int RB = 8, KC = 128;
    __shared__ float sA[RB][KC];
    __shared__ int32_t sIdx[RB];
    const int tid = threadIdx.x;
    const int32_t m0 = blockIdx.y * RB;
    const int64_t v = (int64_t)blockIdx.x * kThreads + tid;
    if (tid < RB) {
        const int32_t r = m0 + tid;
        sIdx[tid] = (r < p.R) ? row_source(p.row0 + r, p.cu, p.num_decode, p.num_tokens, p.ex) : -1;
    }
    __syncthreads();
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = 0.f;
    for (int64_t k0 = 0; k0 < p.H; k0 += KC) {
        for (int j = tid; j < RB * KC; j += kThreads) {
            const int r = j / KC;
            const int64_t k = k0 + j % KC;
            const int32_t t = sIdx[r];
            sA[r][j % KC] = (t >= 0 && k < p.H) ? p.hidden[(int64_t)t * p.hld + k] : 0.f;
        }
        __syncthreads();
        if (v < p.V) {
            const int kn = (int)((p.H - k0) < KC ? (p.H - k0) : KC);
            const float* wr = p.W + v * p.wld + k0;
            for (int k = 0; k < kn; ++k) {
                const float w = wr[k];
#pragma unroll
                for (int i = 0; i < RB; ++i) acc[i] = fmaf(sA[i][k], w, acc[i]);
            }
        }
        __syncthreads();
    }
    if (v < p.V) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int32_t r = m0 + i;
            if (r < p.R)
                store_out<OUT_BF16>(p.out, (int64_t)r * p.old + v,
                                    sIdx[i] < 0 ? kNaN : scale_logit(acc[i], p.scale_mode, p.scale));
        }
    }
}


}  // namespace

template <int MT, bool OUT_BF16>
hipError_t launch_stream_mt(const HeadParams& p, hipStream_t s) {
    constexpr int NT = kStreamNT;
    constexpr int SLAB = kStreamThreads / 4 * NT;    // W rows per workgroup
    const dim3 grid((unsigned)((p.V + SLAB - 1) / SLAB));
    if (p.H % kStreamKC == 0)
        hipLaunchKernelGGL((k_head_stream<MT, NT, true, OUT_BF16>), grid, dim3(kStreamThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_head_stream<MT, NT, false, OUT_BF16>), grid, dim3(kStreamThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_head_stream_bf16(const HeadArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (a.rows > kStreamMaxRows) return hipErrorInvalidValue;
    const HeadParams p = to_params(a);
    switch ((a.rows + 15) / 16) {
        case 1: return a.out_bf16 ? launch_stream_mt<1, true>(p, s) : launch_stream_mt<1, false>(p, s);
        case 2: return a.out_bf16 ? launch_stream_mt<2, true>(p, s) : launch_stream_mt<2, false>(p, s);
        case 3: return a.out_bf16 ? launch_stream_mt<3, true>(p, s) : launch_stream_mt<3, false>(p, s);
        case 4: return a.out_bf16 ? launch_stream_mt<4, true>(p, s) : launch_stream_mt<4, false>(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool OUT_BF16, int BITS, bool STAB>
hipError_t launch_tiled(const HeadParams& p, int32_t mtiles, int32_t ntiles, hipStream_t s) {
    const void* fn = (const void*)k_head_tiled<OUT_BF16, BITS, STAB>;
    const int ng = STAB ? (int)(p.H >> p.qw.gshift) : 0;
    const size_t lds = kTileLds + (STAB ? (size_t)kTileN * (ng + 1) * 4 : 0);
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)mtiles * ntiles;
    const dim3 grid((unsigned)(((total + 7) / 8) * 8));
    hipLaunchKernelGGL((k_head_tiled<OUT_BF16, BITS, STAB>), grid, dim3(kTileThreads), lds, s, p,
                       mtiles, ntiles);
    return hipGetLastError();
}

template <bool OUT_BF16, int BITS>
hipError_t launch_tiled_q(const HeadParams& p, int32_t mtiles, int32_t ntiles, hipStream_t s) {
    if ((p.H >> p.qw.gshift) <= kTileMaxTableGroups) return launch_tiled<OUT_BF16, BITS, true>(p, mtiles, ntiles, s);
    return launch_tiled<OUT_BF16, BITS, false>(p, mtiles, ntiles, s);
}

// Persistent walk when every CU gets at least four tiles, for plain fp32
// logits (the bf16-output and partials epilogues do not fit the registers
// beside the next tile's state); otherwise one workgroup per tile.
template <bool OUT_BF16, bool FUSED = false, int BITS = 16>
hipError_t launch_tiled64(const HeadParams& p, int32_t mtiles, int32_t ntiles, hipStream_t s) {
    const int64_t total = (int64_t)mtiles * ntiles;
    const int cus = cu_count();
    if constexpr (BITS != 16) {
        // one tile per workgroup; the tile's (scale, bias) table after the
        // row-source lists
        const size_t lds = (size_t)kT64Lds + (size_t)kTileN * (size_t)((p.H >> p.qw.gshift) + 1) * 4;
        const void* fn = (const void*)k_head_tiled64<OUT_BF16, false, false, BITS>;
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        const dim3 grid((unsigned)(((total + 7) / 8) * 8));
        hipLaunchKernelGGL((k_head_tiled64<OUT_BF16, false, false, BITS>), grid, dim3(512), lds, s, p, mtiles, ntiles);
        return hipGetLastError();
    }
    if constexpr (!OUT_BF16 && !FUSED) {
        if (cus > 0 && total >= 4 * (int64_t)cus) {
            const void* fn = (const void*)k_head_tiled64<false, false, true>;
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kT64Lds);
            if (e != hipSuccess) return e;
            const dim3 grid((unsigned)((cus + 7) / 8 * 8));
            hipLaunchKernelGGL((k_head_tiled64<false, false, true>), grid, dim3(512), kT64Lds, s, p, mtiles, ntiles);
            return hipGetLastError();
        }
    }
    const void* fn = (const void*)k_head_tiled64<OUT_BF16, FUSED, false>;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kT64Lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)(((total + 7) / 8) * 8));
    hipLaunchKernelGGL((k_head_tiled64<OUT_BF16, FUSED, false>), grid, dim3(512), kT64Lds, s, p, mtiles, ntiles);
    return hipGetLastError();
}

hipError_t launch_head_tiled_bf16(const HeadArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    const HeadParams p = to_params(a);
    const int32_t mtiles = (a.rows + kTileM - 1) / kTileM;
    const int32_t ntiles = (int32_t)((a.vocab + kTileN - 1) / kTileN);
    if (tiled64_fits(p.num_tokens, p.hld, p.H, p.wld)) {
        if (a.part != nullptr)
            return a.out_bf16 ? hipErrorInvalidValue : launch_tiled64<false, true>(p, mtiles, ntiles, s);
        return a.out_bf16 ? launch_tiled64<true>(p, mtiles, ntiles, s) : launch_tiled64<false>(p, mtiles, ntiles, s);
    }
    if (a.part != nullptr) return hipErrorInvalidValue;
    return a.out_bf16 ? launch_tiled<true, 16, false>(p, mtiles, ntiles, s)
                      : launch_tiled<false, 16, false>(p, mtiles, ntiles, s);
}

template <int MT, int BITS, bool OUT_BF16>
hipError_t launch_stream_q_mt(const HeadParams& p, hipStream_t s) {
    constexpr int NT = kStreamQNT;
    constexpr int SLAB = kStreamQThreads / 4 * NT;   // W rows per workgroup
    const dim3 grid((unsigned)((p.V + SLAB - 1) / SLAB));
    // vector scale loads: whole chunks, even scale pitch, 4-byte aligned rows
    const int group = 1 << p.qw.gshift;
    const bool vec = p.H % kStreamQKC == 0 && p.qw.sld % 2 == 0 &&
                     (reinterpret_cast<uintptr_t>(p.qw.scales) & 3) == 0 &&
                     (reinterpret_cast<uintptr_t>(p.qw.biases) & 3) == 0;
    if (vec && group == kStreamQKC / 8)
        hipLaunchKernelGGL((k_head_stream_q<MT, NT, BITS, 8, OUT_BF16>), grid, dim3(kStreamQThreads), 0, s, p);
    else if (vec && group == kStreamQKC / 4)
        hipLaunchKernelGGL((k_head_stream_q<MT, NT, BITS, 4, OUT_BF16>), grid, dim3(kStreamQThreads), 0, s, p);
    else if (vec && group == kStreamQKC / 2)
        hipLaunchKernelGGL((k_head_stream_q<MT, NT, BITS, 2, OUT_BF16>), grid, dim3(kStreamQThreads), 0, s, p);
    else
        hipLaunchKernelGGL((k_head_stream_q<MT, NT, BITS, 0, OUT_BF16>), grid, dim3(kStreamQThreads), 0, s, p);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_stream_q_bits(const HeadArgs& a, const HeadParams& p, hipStream_t s) {
    switch ((a.rows + 15) / 16) {
        case 1: return a.out_bf16 ? launch_stream_q_mt<1, BITS, true>(p, s) : launch_stream_q_mt<1, BITS, false>(p, s);
        case 2: return a.out_bf16 ? launch_stream_q_mt<2, BITS, true>(p, s) : launch_stream_q_mt<2, BITS, false>(p, s);
        case 3: return a.out_bf16 ? launch_stream_q_mt<3, BITS, true>(p, s) : launch_stream_q_mt<3, BITS, false>(p, s);
        case 4: return a.out_bf16 ? launch_stream_q_mt<4, BITS, true>(p, s) : launch_stream_q_mt<4, BITS, false>(p, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_head_stream_q(const HeadArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (a.rows > kStreamMaxRows || a.hidden_dim % 128) return hipErrorInvalidValue;
    const HeadParams p = to_params(a);
    if (a.bits == 4) return launch_stream_q_bits<4>(a, p, s);
    if (a.bits == 8) return launch_stream_q_bits<8>(a, p, s);
    return hipErrorInvalidValue;
}

// The 4-bit tiled head takes the 64-wide-stage kernel when the tile's
// (scale, bias) table fits beside its stage buffers (at most 29 groups per
// row: hidden 1856 at group 64) and the hidden offsets fit 32 bits.
bool tiled64_q_ok(const HeadParams& p) {
    const int64_t groups = p.H >> p.qw.gshift;
    return tiled64_fits(p.num_tokens, p.hld, p.H, 0) &&
           (int64_t)kT64Lds + (int64_t)kTileN * (groups + 1) * 4 <= 160 * 1024;
}

hipError_t launch_head_tiled_q(const HeadArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (a.hidden_dim % 128) return hipErrorInvalidValue;
    const HeadParams p = to_params(a);
    // 4-bit codes (2048-row Qwen3-0.6B projection: 830 -> 790 us); 8-bit codes
    // keep the 32-wide kernel, whose registers hold their second code word
    // without spilling (the 64-wide form measured 851 against 828 us)
    if (a.bits == 4 && tiled64_q_ok(p)) {
        const int32_t mtiles = (a.rows + kTileM - 1) / kTileM;
        const int32_t ntiles = (int32_t)((a.vocab + kTileN - 1) / kTileN);
        return a.out_bf16 ? launch_tiled64<true, false, 4>(p, mtiles, ntiles, s)
                          : launch_tiled64<false, false, 4>(p, mtiles, ntiles, s);
    }
    const int32_t mtiles = (a.rows + kTileM - 1) / kTileM;
    const int32_t ntiles = (int32_t)((a.vocab + kTileN - 1) / kTileN);
    if (a.bits == 4)
        return a.out_bf16 ? launch_tiled_q<true, 4>(p, mtiles, ntiles, s) : launch_tiled_q<false, 4>(p, mtiles, ntiles, s);
    if (a.bits == 8)
        return a.out_bf16 ? launch_tiled_q<true, 8>(p, mtiles, ntiles, s) : launch_tiled_q<false, 8>(p, mtiles, ntiles, s);
    return hipErrorInvalidValue;
}

hipError_t launch_head_f32(const HeadArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    HeadParamsF32 p;
    p.scale_mode = a.scale_mode;
    p.scale = a.scale;
    p.hidden = static_cast<const float*>(a.hidden);
    p.num_tokens = a.num_tokens;
    p.H = a.hidden_dim;
    p.hld = a.hidden_ld;
    p.W = static_cast<const float*>(a.weight);
    p.V = a.vocab;
    p.wld = a.weight_ld;
    p.cu = a.cu;
    p.num_decode = a.num_decode;
    p.ex = a.ex;
    p.row0 = a.row0;
    p.R = a.rows;
    p.out = a.out;
    p.old = a.out_ld;
    const dim3 grid((unsigned)((a.vocab + kThreads - 1) / kThreads), (unsigned)((a.rows + 7) / 8));
    if (a.out_bf16)
        hipLaunchKernelGGL(k_head_f32<true>, grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(k_head_f32<false>, grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace lmh
