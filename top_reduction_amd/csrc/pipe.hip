// pipe.hip -- k-pipelined weight-streaming head for a few gathered rows
// (vllm-metal release v0.4.0, Summary: project only the sampled rows;
// mlxcel PR #1969: the head acts per position).
//
//   logits[r][v] = sum_k hidden[src(r)][k] * W[v][k]
//
// Each workgroup owns a contiguous run of 16-row W tiles (the runs of all
// workgroups differ by at most one tile). Its 16 waves form a chain over the
// hidden dimension: wave w owns the k-steps w*KSW .. w*KSW+KSW-1 and keeps the
// gathered hidden rows' fragments of those steps in registers for the whole
// launch. At stage s, wave w works on tile s - w of the run: it takes the
// tile's partial sums from wave w-1 through LDS, adds its k-steps with the
// MFMAs and hands the sums on to wave w+1; the last wave stores the logits.
// Every output therefore sees the same MFMA sequence as in the streaming and
// tiled kernels of head.hip (the same k order, no split), every wave streams
// an equal slice of every tile, and the workgroups' loads stay balanced until
// the launch ends. Each wave keeps the weight fragments of its next D tiles
// in flight in a register ring; past the end of the run the ring re-reads the
// run's last tile (an L2 hit).
//
// bf16 weights only: the same chain over group-quantised weights was
// measured slower than their weight-streaming kernel (the per-tile scale and
// bias loads of every wave throttle the memory pipe, and without them it only
// matched it), so quantised heads keep that kernel.
#include "head_common.h"

namespace lmh {
namespace {

#ifndef LMH_PIPE_INFLIGHT
#define LMH_PIPE_INFLIGHT 8
#endif
constexpr int kPipeWaves = 16;                   // waves per chain (one workgroup per CU)
constexpr int kPipeInflight = LMH_PIPE_INFLIGHT; // k-steps of weight fragments in flight per wave
// Cache policy of the logits stores: non-temporal (the logits are not read
// again by this launch; measured 2-5 % faster than default stores at 40 and
// 64 rows of the Qwen3-0.6B head)
constexpr int kNT = 2;
// Logits go out in groups of tiles that make whole 128-byte rows: two tiles
// of fp32, four of bf16 (fp32: 68.2 against 70.2 us for 64-byte row pieces
// at 40 rows of the Qwen3-0.6B head; groups of four 68.0, of eight 72.7)
template <bool OUT_BF16> constexpr int store_tiles() { return OUT_BF16 ? 4 : 2; }

// Logits output: the last wave stages each tile's logits in LDS and stores
// every aligned group of tiles as whole 128-byte rows with 16-byte stores
// (VEC: a vocabulary that is a multiple of 4 for fp32 logits, of 8 for
// bf16), or stores each tile right away with 4-byte (2-byte for bf16)
// stores. Head output scaling: x /
// scale (DIV), else x * smul (1 without scaling: exact); the mode is a
// template parameter because a branch around the stores would cost the
// compiler its exact wait counts.
template <int MT, int KSW, int D, bool OUT_BF16, bool DIV, bool VEC>
__global__ __launch_bounds__(64 * kPipeWaves) void k_head_pipe(HeadParams p, int32_t ntiles) {
    constexpr int WAVES = kPipeWaves;
    struct F {
        u32x4 v[KSW];            // the 16-byte B operand of each of the wave's k-steps
    };
    constexpr int SLOT = (WAVES - 1) * MT * 64;                    // f32x4 per stage parity
    constexpr int ES = OUT_BF16 ? 2 : 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char pipe_smem[];
    f32x4* slot = reinterpret_cast<f32x4*>(pipe_smem);                        // [2][WAVES-1][MT][64]
    int32_t* sIdx = reinterpret_cast<int32_t*>(pipe_smem + 2 * SLOT * 16);    // [MT*16]
    float* stage_out = reinterpret_cast<float*>(pipe_smem + 2 * SLOT * 16 + MT * 16 * 4);   // [MT*16][16*store_tiles]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int qd = lane >> 4;                   // lane quarter
    const int32_t G = (int32_t)gridDim.x;
    const int32_t t0 = (int32_t)(((int64_t)blockIdx.x * ntiles) / G);
    const int32_t n = (int32_t)(((int64_t)(blockIdx.x + 1) * ntiles) / G) - t0;   // >= 1

    if (tid < MT * 16)
        sIdx[tid] = (tid < p.R) ? row_source(p.row0 + tid, p.cu, p.num_decode, p.num_tokens, p.ex) : -1;
    __syncthreads();

    // hidden element of k-step s (of this wave) for this lane
    const int gs0 = wave * KSW;                 // the wave's first k-step
    auto hidden_k = [&](int s) -> int { return (gs0 + s) * 32 + qd * 8; };
    const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
    u32x4 a[MT][KSW];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int32_t t = sIdx[i * 16 + l16];
        const uint16_t* src = p.hidden + (int64_t)(t >= 0 ? t : 0) * p.hld;
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src + hidden_k(s));
            a[i][s] = t >= 0 ? v : zero4;
        }
    }

    // weight fragments of local tile j (clamped to the run and to the vocabulary)
    auto load_w = [&](int32_t j, F& f) {
        const int32_t jj = j < n ? j : n - 1;
        int64_t v = (int64_t)(t0 + jj) * 16 + l16;
        v = v < p.V ? v : p.V - 1;
        const uint16_t* src = p.W + v * p.wld;
#pragma unroll
        for (int s = 0; s < KSW; ++s) f.v[s] = *reinterpret_cast<const u32x4*>(src + hidden_k(s));
    };

    // output: lane holds rows 4*(lane/16)+e of column l16 of each 16-row group
    const float smul = p.scale_mode == 1 ? p.scale : 1.0f;
    const int64_t out_bytes = (int64_t)p.R * p.old * ES;
    const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(p.out, (uint32_t)out_bytes);   // < 2^31 (host check)
    const uint32_t rowbytes = (uint32_t)(p.old * ES);
    const int rl = qd * 4;                      // this lane's first row in each 16-row group
    uint32_t nan_rows = 0;                      // bit 4i+e: row 16i+rl+e has no source
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = i * 16 + rl + e;
            if (r < p.R && sIdx[r] < 0) nan_rows |= 1u << (4 * i + e);
        }

    // the last wave's logits of local tile j
    auto emit = [&](int32_t j, const f32x4 (&acc)[MT]) {
        const int64_t c0 = (int64_t)(t0 + j) * 16;          // first column of the tile
        auto value = [&](int i, int e) {
            const float x = acc[i][e];
            const float sc = DIV ? x / p.scale : x * smul;
            return (nan_rows >> (4 * i + e)) & 1u ? kNaN : sc;
        };
        if constexpr (VEC) {
            // the P tiles of an aligned group are staged side by side and
            // stored as whole 64 * P-byte rows once the group's last tile of
            // this run is in (the run's first and last groups may be partial)
            constexpr int P = store_tiles<OUT_BF16>();
            constexpr int CW = 16 * P;                       // staged columns
            const int32_t tg = t0 + j;
            const int part = tg % P;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) stage_out[(i * 16 + rl + e) * CW + part * 16 + l16] = value(i, e);
            if (part == P - 1 || j == n - 1) {
                const int32_t g0 = tg - part;                // the group's first tile
                constexpr int EPL = OUT_BF16 ? 8 : 4;        // logits per 16-byte store
                constexpr int LPR = CW / EPL;                // lanes per row
                constexpr int RPI = 64 / LPR;                // rows per store instruction
                const int cq = (lane % LPR) * EPL;
                const int32_t tq = g0 + cq / 16;             // the tile of this lane's columns
                const bool part_ok = tq >= t0 && tq <= tg;
                const int64_t col = (int64_t)g0 * 16 + cq;
#pragma unroll
                for (int i2 = 0; i2 < MT * 16 / RPI; ++i2) {
                    const int r = i2 * RPI + lane / LPR;
                    const bool ok = part_ok && col < p.V && r < p.R;
                    const uint32_t off = ok ? (uint32_t)r * rowbytes + (uint32_t)col * ES : 0x80000000u;
                    u32x4 word;
                    if constexpr (OUT_BF16) {
                        const f32x4 v0 = *reinterpret_cast<const f32x4*>(&stage_out[r * CW + cq]);
                        const f32x4 v1 = *reinterpret_cast<const f32x4*>(&stage_out[r * CW + cq + 4]);
                        word = u32x4{(uint32_t)f32_to_bf16_rne(v0[0]) | ((uint32_t)f32_to_bf16_rne(v0[1]) << 16),
                                     (uint32_t)f32_to_bf16_rne(v0[2]) | ((uint32_t)f32_to_bf16_rne(v0[3]) << 16),
                                     (uint32_t)f32_to_bf16_rne(v1[0]) | ((uint32_t)f32_to_bf16_rne(v1[1]) << 16),
                                     (uint32_t)f32_to_bf16_rne(v1[2]) | ((uint32_t)f32_to_bf16_rne(v1[3]) << 16)};
                    } else {
                        word = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4*>(&stage_out[r * CW + cq]));
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(word, orsrc, off, 0, kNT);
                }
            }
        } else {
            const bool vok = c0 + l16 < p.V;
            const uint32_t toff = (uint32_t)rl * rowbytes + (uint32_t)(c0 + l16) * ES;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float val = value(i, e);
                    const bool ok = vok && i * 16 + rl + e < p.R;
                    const uint32_t off = ok ? toff + (uint32_t)(i * 16 + e) * rowbytes : 0x80000000u;
                    if (OUT_BF16)
                        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(val), orsrc, off, 0, kNT);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), orsrc, off, 0, kNT);
                }
        }
    };

    // one stage of this wave: partial sums of tile j in, its k-steps, out
    auto stage = [&](auto LAST, int32_t j, F& wr, bool refill) {
        const int32_t st = j + wave;
        f32x4 acc[MT];
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
            const f32x4* in = slot + ((st - 1) & 1) * SLOT + (wave - 1) * MT * 64;
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[i] = in[i * 64 + lane];
        }
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[i] = mfma16(a[i][s], wr.v[s], acc[i]);
        }
        if (refill) load_w(j + D, wr);
        if constexpr (decltype(LAST)::value) {
            emit(j, acc);
        } else {
            f32x4* out = slot + (st & 1) * SLOT + wave * MT * 64;
#pragma unroll
            for (int i = 0; i < MT; ++i) out[i * 64 + lane] = acc[i];
        }
        __syncthreads();
    };

    // The wave's whole run: the first D tiles' loads, the stages before its
    // first tile, its tiles D per ring turn (the tail of fewer than D tiles
    // neither refills nor reads past the run), the stages after its last one.
    // The last wave runs its own copy, so no code path mixes the logits
    // stores into the other waves' memory counters; and the first ring turn
    // is peeled, so the loop is entered with the memory operations in flight
    // in the same order as on its back edge and the compiler's wait counts
    // stay exact (the last wave's stores would otherwise make the loop's
    // first stage wait for the whole ring).
    auto run = [&](auto LAST) {
        F w[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load_w(d, w[d]);
        for (int b = 0; b < wave; ++b) __syncthreads();
        auto turn = [&](int32_t j) {
#pragma unroll
            for (int d = 0; d < D; ++d) stage(LAST, j + d, w[d], true);
        };
        auto tail = [&](int32_t j) {
#pragma unroll
            for (int d = 0; d < D - 1; ++d)
                if (j + d < n) stage(LAST, j + d, w[d], false);
        };
        if (n >= D) {
            turn(0);
            int32_t j = D;
            for (; j + D <= n; j += D) turn(j);
            tail(j);
        } else {
            tail(0);
        }
        for (int b = wave + 1; b < WAVES; ++b) __syncthreads();
    };
    if (wave == WAVES - 1)
        run(std::integral_constant<bool, true>{});
    else
        run(std::integral_constant<bool, false>{});
}

template <int MT, int KSW, bool OUT_BF16, bool DIV, bool VEC>
hipError_t launch_pipe_k(const HeadParams& p, hipStream_t s) {
    constexpr int W = kPipeWaves;
    // ring depth: up to kPipeInflight k-steps in flight per wave (at most 4
    // tiles), fewer when the hidden fragments and sums leave no room in the
    // 128 registers of a wave (16 waves per CU)
    constexpr int kRingRegs = 128 - 4 * MT * KSW - 4 * MT - 56 - (DIV ? 8 : 0);
    constexpr int D0 = kPipeInflight / KSW > 4 ? 4 : (kPipeInflight / KSW > 0 ? kPipeInflight / KSW : 1);
    constexpr int D1 = kRingRegs / (4 * KSW);
    constexpr int D = D1 < 1 ? 1 : (D1 < D0 ? D1 : D0);
    const int32_t ntiles = (int32_t)((p.V + 15) / 16);
    // one workgroup (a 16-wave chain) per CU, never more than there are tiles
    int64_t g = (int64_t)cu_count();
    if (g <= 0) return hipErrorInvalidDevice;
    if (g > ntiles) g = ntiles;
    const size_t lds = (size_t)2 * (W - 1) * MT * 64 * 16 + (size_t)MT * 16 * 4 + (VEC ? (size_t)MT * 16 * 16 * store_tiles<OUT_BF16>() * 4 : 0);
    const void* fn = (const void*)k_head_pipe<MT, KSW, D, OUT_BF16, DIV, VEC>;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_head_pipe<MT, KSW, D, OUT_BF16, DIV, VEC>), dim3((unsigned)g), dim3(64 * W), lds, s, p,
                       ntiles);
    return hipGetLastError();
}

template <int MT, bool OUT_BF16, bool DIV, bool VEC>
hipError_t launch_pipe_ksw(const HeadParams& p, int ksw, hipStream_t s) {
    switch (ksw) {
        case 1: return launch_pipe_k<MT, 1, OUT_BF16, DIV, VEC>(p, s);
        case 2: return launch_pipe_k<MT, 2, OUT_BF16, DIV, VEC>(p, s);
        case 3: return launch_pipe_k<MT, 3, OUT_BF16, DIV, VEC>(p, s);
        case 4: return launch_pipe_k<MT, 4, OUT_BF16, DIV, VEC>(p, s);
        default: return hipErrorInvalidValue;
    }
}

// 16 bytes per lane when the vocabulary is a multiple of 4 fp32 or 8 bf16
// logits (the row pitch and base are 16-byte aligned by contract)
template <int MT, bool OUT_BF16>
hipError_t launch_pipe_mt(const HeadParams& p, int ksw, hipStream_t s) {
    const bool div = p.scale_mode == 2;
    if (p.V % (OUT_BF16 ? 8 : 4) == 0)
        return div ? launch_pipe_ksw<MT, OUT_BF16, true, true>(p, ksw, s)
                   : launch_pipe_ksw<MT, OUT_BF16, false, true>(p, ksw, s);
    return div ? launch_pipe_ksw<MT, OUT_BF16, true, false>(p, ksw, s)
               : launch_pipe_ksw<MT, OUT_BF16, false, false>(p, ksw, s);
}

}  // namespace

bool head_pipe_ok(const HeadArgs& a) {
    if (a.bits != 16 || a.rows <= 0 || a.rows > kStreamMaxRows) return false;
    const int64_t kw = 32 * (int64_t)kPipeWaves;           // hidden elements per k-step across the chain
    if (a.hidden_dim % kw != 0 || a.hidden_dim / kw > 4) return false;
    const int64_t out_bytes = (int64_t)a.rows * a.out_ld * (a.out_bf16 ? 2 : 4);
    return out_bytes < ((int64_t)1 << 31) && cu_count() > 0;
}

hipError_t launch_head_pipe(const HeadArgs& a, hipStream_t s) {
    if (!head_pipe_ok(a)) return hipErrorInvalidValue;
    const HeadParams p = to_params(a);
    const int ksw = (int)(a.hidden_dim / (32 * kPipeWaves));
    switch ((a.rows + 15) / 16) {
        case 1: return a.out_bf16 ? launch_pipe_mt<1, true>(p, ksw, s) : launch_pipe_mt<1, false>(p, ksw, s);
        case 2: return a.out_bf16 ? launch_pipe_mt<2, true>(p, ksw, s) : launch_pipe_mt<2, false>(p, ksw, s);
        case 3: return a.out_bf16 ? launch_pipe_mt<3, true>(p, ksw, s) : launch_pipe_mt<3, false>(p, ksw, s);
        case 4: return a.out_bf16 ? launch_pipe_mt<4, true>(p, ksw, s) : launch_pipe_mt<4, false>(p, ksw, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lmh
