// lmh_internal.h -- launchers and small device helpers shared by the HIP
// translation units of liblmhead (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lmhead.h"

namespace lmh {

constexpr int kBlock = LMH_BLOCK;                // logits per prefilter block
constexpr int kMaxCandidates = LMH_MAX_CANDIDATES;
constexpr int kStreamMaxRows = 64;               // weight-streaming head limit

// ----------------------------------------------------------------------------
// Row source of logits row r (vllm-metal release, Summary). Sampled mode:
// the last row of segment r, valid only when the segment is non-empty and,
// for a decode segment, exactly one token long. Explicit mode: ex[r].
// Returns -1 when the row has no valid source in [0, num_tokens).
// ----------------------------------------------------------------------------
__device__ inline int32_t row_source(int32_t r, const int32_t* cu, int32_t num_decode,
                                     int64_t num_tokens, const int32_t* ex) {
    int32_t t;
    if (ex != nullptr) {
        t = ex[r];
    } else {
        const int32_t lo = cu[r], hi = cu[r + 1];
        const int32_t len = hi - lo;
        if (len <= 0 || (r < num_decode && len != 1)) return -1;
        t = hi - 1;
    }
    return (t < 0 || (int64_t)t >= num_tokens) ? -1 : t;
}

// Monotone 32-bit key of a float: a < b  <=>  key(a) < key(b) for non-NaN
// values, with -0 and +0 mapped to the same key.
__device__ inline uint32_t f32_key(float x) {
    uint32_t u = __float_as_uint(x);
    u = (x == 0.0f) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ----------------------------------------------------------------------------
// Launchers (host side, enqueue only; return hipSuccess or the launch error)
// ----------------------------------------------------------------------------
struct RowsArgs {
    const int32_t* cu;
    int32_t num_segments;
    int32_t num_decode;
    int64_t num_tokens;
    const int32_t* ex;   // explicit indices or nullptr
    int32_t rows;        // R
    int32_t* gather_out; // may be nullptr
    int32_t* lcu_out;    // may be nullptr
    int32_t* err;        // may be nullptr
};
hipError_t launch_rows(const RowsArgs& a, hipStream_t s);

struct HeadArgs {
    const void* hidden;
    int64_t num_tokens, hidden_dim, hidden_ld;
    const void* weight;
    int64_t vocab, weight_ld;
    const int32_t* cu;
    int32_t num_decode;
    const int32_t* ex;
    int32_t row0;        // first logits row of this launch (chunking)
    int32_t rows;        // rows in this launch
    void* out;           // points at logits row `row0`
    int64_t out_ld;
    bool out_bf16;
    int32_t* err;
    // affine group-quantised weights (weight is then unused): codes of `bits`
    // bits packed in 32-bit words [vocab][q_ld], bf16 scale and bias per group
    // [vocab][s_ld], group = 1 << gshift
    int32_t bits = 16;
    const uint32_t* q = nullptr;
    int64_t q_ld = 0;
    const uint16_t* scales = nullptr;
    const uint16_t* biases = nullptr;
    int64_t s_ld = 0;
    int32_t gshift = 0;
    // output scaling on the fp32 accumulator: 0 none, 1 multiply, 2 divide
    int32_t scale_mode = 0;
    float scale = 1.0f;
    // the reduction's first pass done by the tiled kernel's epilogue (fp32
    // logits, hidden size a multiple of 128, more than kStreamMaxRows rows):
    // per row and 64-logit block, (max, sum of exp(x - max)) at
    // part[row * part_nb + b] and the block-max key at bkeys[row * keys_ld + b]
    float2* part = nullptr;
    uint32_t* bkeys = nullptr;
    int32_t part_nb = 0;
    int32_t keys_ld = 0;
};
// Compute units of the current device (0 if it cannot be queried).
int cu_count();

// The tiled kernel with 64-wide stages (and the reduction partials in its
// epilogue) takes a dense bf16 head whose hidden size is a multiple of 128
// and whose operand offsets fit 32 bits: the hidden matrix (num_tokens rows
// of pitch hidden_ld) and 256 weight rows of pitch weight_ld, in bytes.
inline bool tiled64_fits(int64_t num_tokens, int64_t hidden_ld, int64_t hidden_dim, int64_t weight_ld) {
    constexpr int64_t kMax = (int64_t)1 << 32;
    return hidden_dim % 128 == 0 && num_tokens * hidden_ld * 2 <= kMax && 256 * weight_ld * 2 <= kMax;
}

// bf16 MFMA heads. stream: R <= kStreamMaxRows; tiled: any R.
hipError_t launch_head_stream_bf16(const HeadArgs& a, hipStream_t s);
// The k-pipelined weight stream (bf16 or quantised weights), for the shapes
// head_pipe_ok accepts.
bool head_pipe_ok(const HeadArgs& a);
hipError_t launch_head_pipe(const HeadArgs& a, hipStream_t s);
hipError_t launch_head_tiled_bf16(const HeadArgs& a, hipStream_t s);
// The same two kernels over quantised weights (bits 4 or 8, hidden size a
// multiple of 128, group 32, 64 or 128), dequantised to bf16 on the fly.
hipError_t launch_head_stream_q(const HeadArgs& a, hipStream_t s);
hipError_t launch_head_tiled_q(const HeadArgs& a, hipStream_t s);
// fp32 FMA head.
hipError_t launch_head_f32(const HeadArgs& a, hipStream_t s);

// Bitwise comparison of R selective logits rows `sel` [R][sel_ld] (fp32)
// with the rows of `full` [num_tokens][full_ld] they were projected from
// (row r against full row src(r); rows with no valid source are skipped):
// res[0] = number of differing logits, res[1] = smallest r * vocab + v that
// differs (INT64_MAX if none). `res` is initialised by the launch.
hipError_t launch_selfcheck(const float* sel, int64_t sel_ld, const float* full, int64_t full_ld,
                            int32_t rows, int64_t vocab, const int32_t* cu, int32_t num_decode,
                            int64_t num_tokens, const int32_t* ex, int64_t* res, hipStream_t s);

// Token bitmask on compacted logits rows (see mask.hip).
struct MaskArgs {
    void* logits;
    int32_t dt;           // LMH_F32, LMH_BF16 or LMH_F16
    int64_t rows, vocab, ld;
    const int32_t* mask;  // [segments][mask_ld] 32-bit words
    int64_t mask_ld;
    const int32_t* lcu;   // [segments + 1] or nullptr (segment s is row s)
    int32_t segments;
    int32_t* err;         // may be nullptr
    // the buffer's rows are compacted rows win0 .. win0 + rows - 1 of
    // total_rows (0: the buffer holds them all)
    int64_t win0 = 0;
    int64_t total_rows = 0;
};
hipError_t launch_apply_bitmask(const MaskArgs& a, hipStream_t s);

struct ReducePlan {
    int64_t rows, vocab;
    int32_t k;
    int32_t nb;          // ceil(vocab / 64)
    int32_t kpt;         // block keys per stage-2 thread (4, 8, 16 or 32)
    int32_t kld;         // row pitch of the block-key array (elements)
    int32_t splits;      // (max, sum-exp) partials per row: one per 4096-logit segment
    int64_t nitems;      // rows * splits stage-1 work items, one per wave
    int64_t wgs;         // stage-1 workgroups
    size_t part_off, keys_off, bytes;  // workspace layout
};
ReducePlan plan_reduce(int64_t rows, int64_t vocab, int32_t k);

struct ReduceArgs {
    const void* logits;
    int32_t dt;          // LMH_F32, LMH_BF16 or LMH_F16
    int64_t ld;
    const int32_t* sel;  // may be nullptr
    float* lse;
    float* sel_lp;       // may be nullptr
    int32_t* topk_ids;
    float* topk_lp;
    void* ws;
    int32_t* err;
};
hipError_t launch_reduce_stage1(const ReducePlan& p, const ReduceArgs& a, hipStream_t s);
hipError_t launch_reduce_stage2(const ReducePlan& p, const ReduceArgs& a, hipStream_t s);
// Stage 2 on partials written by the tiled head's epilogue: one (max, sum)
// per 64-logit block (p.splits == p.nb), merged in their own fixed order
// (partial i to thread i mod 256 in ascending order, each wave's lanes as a
// pairwise tree, then the four waves in order); fp32 logits.
hipError_t launch_reduce_stage2_blocks(const ReducePlan& p, const ReduceArgs& a, hipStream_t s);
// True when the one-workgroup-per-row kernel serves this plan on the current
// device (rows fill the CUs evenly); the split path otherwise. Both give
// bitwise-identical results.
bool reduce_row_path(const ReducePlan& p);
// The whole reduction (either path).
hipError_t launch_reduce(const ReducePlan& p, const ReduceArgs& a, hipStream_t s);
// Full-vocabulary logprobs out[r][v] = fp32(x[r][v]) - lse[r] (out pitch:
// vocab), after a reduction has written lse.
hipError_t launch_full_logprobs(const void* logits, int32_t dt, int64_t rows, int64_t vocab, int64_t ld,
                                const float* lse, float* out, hipStream_t s);

// Single-launch path for a few rows (k_single): rows that take the split
// path, K <= LMH_SINGLE_MAX_K, at most 64 items per row, at most
// LMH_SINGLE_MAX_ROWS rows. It needs `counters`, one 32-bit word per row
// (LMH_SINGLE_MAX_ROWS words) that are zero before the launch and that the
// launch leaves zero; launches sharing counters must not overlap. Its scratch
// (a.ws) takes single_bytes(p) bytes, never more than p.bytes.
#define LMH_SINGLE_MAX_K 32
#define LMH_SINGLE_MAX_ROWS 4096
bool single_ok(const ReducePlan& p);
size_t single_bytes(const ReducePlan& p);
hipError_t launch_reduce_single(const ReducePlan& p, const ReduceArgs& a, uint32_t* counters, hipStream_t s);

// logprob_reduce's host-side checks (everything but the workspace), in its
// order; *workspace_bytes gets the workspace the shape needs. Then the
// enqueue of the reduction on a workspace of at least that size.
lmh_status reduce_validate(const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                           int64_t logits_ld, const int32_t* selected_ids, int32_t k, const float* lse,
                           const float* selected_logprob, const int32_t* topk_ids,
                           const float* topk_logprobs, size_t* workspace_bytes);
// With counters (see launch_reduce_single): single = 0 routes the shapes
// that single_ok accepts with K <= kSingleRouteK to the single-launch path
// (where it measured faster than the split path), single = 1 sends every
// shape that single_ok accepts there.
constexpr int32_t kSingleRouteK = 0;
lmh_status reduce_enqueue(const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                          int64_t logits_ld, const int32_t* selected_ids, int32_t k, float* lse,
                          float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                          void* workspace, int32_t* device_error, hipStream_t s,
                          uint32_t* single_counters = nullptr, int single = 0);

}  // namespace lmh
