// api.hip -- the C ABI of liblmhead (declared in include/lmhead.h): host-side
// argument checks, workspace layout and kernel dispatch. Every check that can
// be made on the host returns before the first HIP call; no entry point
// allocates, synchronises or copies to the host.
#include <climits>
#include <cmath>

#include "lmh_internal.h"

using namespace lmh;

namespace {

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline bool valid_dtype(lmh_dtype d) { return d == LMH_F32 || d == LMH_BF16; }
inline bool valid_logits_dtype(lmh_dtype d) { return valid_dtype(d) || d == LMH_F16; }   // reduction input
inline size_t esize(lmh_dtype d) { return d == LMH_F32 ? 4 : 2; }
inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct ProjectCheck {
    lmh_status st;
    int32_t rows;
};

// The head's weights: dense (fp32 or bf16, like the hidden states) or affine
// group-quantised (bits != 0).
struct WeightSpec {
    const void* dense;
    lmh_dtype dt;
    int64_t ld;
    const uint32_t* q;
    int64_t q_ld;
    const uint16_t* scales;
    const uint16_t* biases;
    int64_t s_ld;
    int32_t bits;     // 0: dense
    int32_t group;
    int32_t scale_mode;
    float scale;
};

WeightSpec dense_weight(const void* w, lmh_dtype dt, int64_t ld) {
    return WeightSpec{w, dt, ld, nullptr, 0, nullptr, nullptr, 0, 0, 0, LMH_SCALE_NONE, 1.0f};
}
WeightSpec quant_weight(const uint32_t* q, int64_t q_ld, const uint16_t* scales,
                        const uint16_t* biases, int64_t s_ld, int32_t bits, int32_t group) {
    return WeightSpec{nullptr, LMH_BF16, 0, q, q_ld, scales, biases, s_ld, bits, group,
                      LMH_SCALE_NONE, 1.0f};
}
WeightSpec head_weight(const lmh_head& h) {
    return WeightSpec{h.weight, h.weight_dt, h.weight_ld, h.weight_q, h.weight_q_ld, h.scales,
                      h.biases, h.scales_ld, h.bits, h.group_size, h.scale_mode, h.scale};
}

int32_t log2_exact(int32_t g) {
    int32_t s = 0;
    while ((1 << s) < g) ++s;
    return s;
}

// Checks shared by the projection entry points (everything but the output).
ProjectCheck check_project_inputs(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                                  int64_t hidden_dim, int64_t hidden_ld, const WeightSpec& w,
                                  int64_t vocab, const int32_t* cu_seqlens, int32_t num_segments,
                                  int32_t num_decode, const int32_t* logits_indices,
                                  int32_t num_indices) {
    if (!hidden || !cu_seqlens) return {LMH_ERR_NULL, 0};
    if (w.bits == 0 ? !w.dense : (!w.q || !w.scales || !w.biases)) return {LMH_ERR_NULL, 0};
    if (num_tokens <= 0 || num_tokens > INT32_MAX || hidden_dim <= 0 || vocab <= 0 ||
        vocab > INT32_MAX || num_segments < 0 || num_decode < 0 || num_decode > num_segments)
        return {LMH_ERR_SHAPE, 0};
    if (logits_indices != nullptr && num_indices < 0) return {LMH_ERR_SHAPE, 0};
    if (hidden_ld < hidden_dim) return {LMH_ERR_SHAPE, 0};
    if (w.scale_mode != LMH_SCALE_NONE &&
        ((w.scale_mode != LMH_SCALE_MUL && w.scale_mode != LMH_SCALE_DIV) || !std::isfinite(w.scale) ||
         w.scale == 0.0f))
        return {LMH_ERR_SHAPE, 0};
    if (w.bits == 0) {
        if (w.ld < hidden_dim) return {LMH_ERR_SHAPE, 0};
        if (!valid_dtype(hidden_dt) || w.dt != hidden_dt) return {LMH_ERR_DTYPE, 0};
    } else {
        if (hidden_dt != LMH_BF16 || (w.bits != 4 && w.bits != 8)) return {LMH_ERR_DTYPE, 0};
        if (w.group != 32 && w.group != 64 && w.group != 128) return {LMH_ERR_SHAPE, 0};
        if (hidden_dim % 128 || w.q_ld < hidden_dim * w.bits / 32 || w.s_ld < hidden_dim / w.group)
            return {LMH_ERR_SHAPE, 0};
        if (!aligned(w.q, 16) || w.q_ld % 4 || !aligned(w.scales, 2) || !aligned(w.biases, 2))
            return {LMH_ERR_ALIGN, 0};
    }
    if (hidden_dt == LMH_BF16) {
        if (!aligned(hidden, 16) || hidden_dim % 8 || hidden_ld % 8) return {LMH_ERR_ALIGN, 0};
        if (w.bits == 0 && (!aligned(w.dense, 16) || w.ld % 8)) return {LMH_ERR_ALIGN, 0};
    } else {
        if (!aligned(hidden, 4) || !aligned(w.dense, 4)) return {LMH_ERR_ALIGN, 0};
    }
    const int32_t rows = logits_indices ? num_indices : num_segments;
    return {LMH_OK, rows};
}

// Shape, dtype, pitch and K rules of the reduction (pointer alignment is
// checked by the callers).
lmh_status check_reduce_shape(lmh_dtype dt, int64_t rows, int64_t vocab, int64_t ld, int32_t k) {
    if (rows < 0 || rows > INT32_MAX || vocab <= 0 || vocab > INT32_MAX || ld < vocab)
        return LMH_ERR_SHAPE;
    if (!valid_logits_dtype(dt)) return LMH_ERR_DTYPE;
    if (((size_t)ld * esize(dt)) % 16) return LMH_ERR_ALIGN;
    const int64_t nb = ceil_div(vocab, kBlock);
    if (k < LMH_K_FULL || k > vocab) return LMH_ERR_K;
    if ((k < nb ? k : nb) * (int64_t)kBlock > kMaxCandidates) return LMH_ERR_K;
    if (k > 0 && nb > kMaxCandidates) return LMH_ERR_SHAPE;
    const ReducePlan p = plan_reduce(rows, vocab, k > 0 ? k : 0);
    if (p.wgs >= ((int64_t)1 << 30)) return LMH_ERR_SHAPE;   // stage-1 item index fits 32 bits
    return LMH_OK;
}

lmh_status from_hip(hipError_t e) { return e == hipSuccess ? LMH_OK : LMH_ERR_HIP; }

HeadArgs head_args(const void* hidden, int64_t num_tokens, int64_t hidden_dim, int64_t hidden_ld,
                   const WeightSpec& w, int64_t vocab, const int32_t* cu_seqlens, int32_t num_decode,
                   const int32_t* logits_indices, int32_t row0, int32_t rows, void* out,
                   int64_t out_ld, bool out_bf16, int32_t* device_error) {
    HeadArgs h{hidden, num_tokens, hidden_dim, hidden_ld, w.dense, vocab, w.ld, cu_seqlens,
               num_decode, logits_indices, row0, rows, out, out_ld, out_bf16, device_error};
    h.scale_mode = w.scale_mode;
    h.scale = w.scale;
    if (w.bits != 0) {
        h.bits = w.bits;
        h.q = w.q;
        h.q_ld = w.q_ld;
        h.scales = w.scales;
        h.biases = w.biases;
        h.s_ld = w.s_ld;
        h.gshift = log2_exact(w.group);
    }
    return h;
}

lmh_status launch_head(const HeadArgs& h, bool bf16_inputs, int32_t variant, hipStream_t s) {
    if (!bf16_inputs) return from_hip(launch_head_f32(h, s));
    if (variant == LMH_HEAD_PIPE) return head_pipe_ok(h) ? from_hip(launch_head_pipe(h, s)) : LMH_ERR_SHAPE;
    // the pipelined stream pays off once there are two or more 16-row tiles
    // of hidden rows (measured: equal or slightly behind the plain stream for one)
    if (variant == LMH_HEAD_AUTO && h.rows > 16 && head_pipe_ok(h)) return from_hip(launch_head_pipe(h, s));
    const bool stream = variant == LMH_HEAD_STREAM || (variant == LMH_HEAD_AUTO && h.rows <= kStreamMaxRows);
    if (h.bits != 16) return from_hip(stream ? launch_head_stream_q(h, s) : launch_head_tiled_q(h, s));
    return from_hip(stream ? launch_head_stream_bf16(h, s) : launch_head_tiled_bf16(h, s));
}

lmh_status gather_project_impl(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                               int64_t hidden_dim, int64_t hidden_ld, const WeightSpec& w,
                               int64_t vocab, const int32_t* cu_seqlens, int32_t num_segments,
                               int32_t num_decode, const int32_t* logits_indices,
                               int32_t num_indices, void* logits, lmh_dtype logits_dt,
                               int64_t logits_ld, int32_t* logits_cu_seqlens,
                               int32_t* gather_indices, int32_t* device_error, void* stream,
                               int32_t variant) {
    const ProjectCheck c = check_project_inputs(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                                                w, vocab, cu_seqlens, num_segments, num_decode,
                                                logits_indices, num_indices);
    if (c.st != LMH_OK) return c.st;
    if (!logits && c.rows > 0) return LMH_ERR_NULL;
    if (logits_ld < vocab) return LMH_ERR_SHAPE;
    if (!valid_dtype(logits_dt)) return LMH_ERR_DTYPE;
    if (!aligned(logits, esize(logits_dt))) return LMH_ERR_ALIGN;
    if (variant < LMH_HEAD_AUTO || variant > LMH_HEAD_PIPE) return LMH_ERR_SHAPE;
    if (variant != LMH_HEAD_AUTO && hidden_dt != LMH_BF16) return LMH_ERR_SHAPE;
    if (variant == LMH_HEAD_STREAM && c.rows > kStreamMaxRows) return LMH_ERR_SHAPE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gather_indices || logits_cu_seqlens || device_error) {
        RowsArgs ra{cu_seqlens, num_segments, num_decode, num_tokens, logits_indices, c.rows,
                    gather_indices, logits_cu_seqlens, device_error};
        const lmh_status st = from_hip(launch_rows(ra, s));
        if (st != LMH_OK) return st;
    }
    if (c.rows == 0) return LMH_OK;
    const HeadArgs h = head_args(hidden, num_tokens, hidden_dim, hidden_ld, w, vocab, cu_seqlens,
                                 num_decode, logits_indices, 0, c.rows, logits, logits_ld,
                                 logits_dt == LMH_BF16, device_error);
    return launch_head(h, hidden_dt == LMH_BF16, variant, s);
}

// Workspace of the reduction when the tiled head's epilogue takes its
// streaming pass: per row of a chunk, one (max, sum) per 64-logit block and
// the block keys in the second kernel's layout.
size_t blocks_ws_bytes(int64_t chunk, int64_t vocab, int32_t k) {
    const ReducePlan p = plan_reduce(chunk, vocab, k > 0 ? k : 0);
    return up256((size_t)chunk * (size_t)p.nb * sizeof(float2)) + up256((size_t)chunk * (size_t)p.kld * 4);
}

lmh_status logprobs_impl(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                         int64_t hidden_dim, int64_t hidden_ld, const WeightSpec& w, int64_t vocab,
                         const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
                         const int32_t* logits_indices, int32_t num_indices,
                         const int32_t* selected_ids, int32_t k, float* lse,
                         float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                         int32_t* logits_cu_seqlens, int32_t* gather_indices, int32_t chunk_rows,
                         float* logits_debug, void* workspace, size_t workspace_bytes,
                         int32_t* device_error, void* stream, const uint32_t* vocab_mask = nullptr,
                         int64_t vocab_mask_ld = 0, bool allow_epilogue = true) {
    const ProjectCheck c = check_project_inputs(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                                                w, vocab, cu_seqlens, num_segments, num_decode,
                                                logits_indices, num_indices);
    if (c.st != LMH_OK) return c.st;
    if (c.rows > 0) {
        if (!lse) return LMH_ERR_NULL;
        if (selected_ids && !selected_logprob) return LMH_ERR_NULL;
        if (k > 0 && (!topk_ids || !topk_logprobs)) return LMH_ERR_NULL;
        if (k == LMH_K_FULL && !topk_logprobs) return LMH_ERR_NULL;
    }
    const int32_t kr = k > 0 ? k : 0;   // the top-K of the reduction (K = -1: none)
    if (vocab_mask != nullptr) {
        // explicit rows: the segment -> rows map is the logits_cu_seqlens
        // this call writes, so the caller must ask for it
        if (logits_indices != nullptr && !logits_cu_seqlens) return LMH_ERR_NULL;
        if (vocab_mask_ld < ceil_div(vocab, 32)) return LMH_ERR_SHAPE;
        if (!aligned(vocab_mask, 4)) return LMH_ERR_ALIGN;
    }
    if (chunk_rows < 0) return LMH_ERR_SHAPE;
    const int64_t R = c.rows;
    const int64_t chunk_cfg = chunk_rows > 0 ? chunk_rows : 256;
    const int64_t chunk = R < chunk_cfg ? (R > 0 ? R : 1) : chunk_cfg;
    const int64_t ld = ceil_div(vocab, 4) * 4;
    {
        // the reduction's rules, checked on the fp32 logits layout it will read
        const lmh_status st = check_reduce_shape(LMH_F32, chunk, vocab, ld, k);
        if (st != LMH_OK) return st;
    }
    const ReducePlan pc = plan_reduce(chunk, vocab, kr);
    const size_t logits_bytes = logits_debug ? 0 : up256((size_t)chunk * (size_t)ld * sizeof(float));
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < logits_bytes + pc.bytes)
        return LMH_ERR_WORKSPACE;
    // chunks of more rows than the weight-streaming kernels take run on the
    // tiled kernel; with a dense bf16 head of a hidden size it tiles in 64-wide
    // stages, its epilogue does the reduction's streaming pass (unless a token
    // mask must change the logits first, or the workspace has no room for the
    // per-block partials)
    const bool epi = allow_epilogue && hidden_dt == LMH_BF16 && w.bits == 0 &&
                     tiled64_fits(num_tokens, hidden_ld, hidden_dim, w.ld) &&
                     vocab_mask == nullptr && workspace_bytes >= logits_bytes + blocks_ws_bytes(chunk, vocab, kr);
    if (logits_debug && !aligned(logits_debug, 16)) return LMH_ERR_ALIGN;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gather_indices || logits_cu_seqlens || device_error) {
        RowsArgs ra{cu_seqlens, num_segments, num_decode, num_tokens, logits_indices, c.rows,
                    gather_indices, logits_cu_seqlens, device_error};
        const lmh_status st = from_hip(launch_rows(ra, s));
        if (st != LMH_OK) return st;
    }
    char* ws = static_cast<char*>(workspace);
    float* ws_logits = reinterpret_cast<float*>(ws);
    void* ws_reduce = ws + logits_bytes;
    for (int64_t r0 = 0; r0 < R; r0 += chunk) {
        const int32_t n = (int32_t)((R - r0) < chunk ? (R - r0) : chunk);
        float* out = logits_debug ? logits_debug + r0 * ld : ws_logits;
        HeadArgs h = head_args(hidden, num_tokens, hidden_dim, hidden_ld, w, vocab, cu_seqlens, num_decode,
                               logits_indices, (int32_t)r0, n, out, ld, false, device_error);
        if (epi && n > kStreamMaxRows) {
            // the head writes the logits and, per block, the partials and keys;
            // the second reduction kernel finishes each row from them
            ReducePlan q = plan_reduce(n, vocab, kr);
            q.splits = q.nb;
            q.part_off = 0;
            q.keys_off = up256((size_t)chunk * (size_t)q.nb * sizeof(float2));
            h.part = reinterpret_cast<float2*>(static_cast<char*>(ws_reduce) + q.part_off);
            h.bkeys = reinterpret_cast<uint32_t*>(static_cast<char*>(ws_reduce) + q.keys_off);
            h.part_nb = q.nb;
            h.keys_ld = q.kld;
            lmh_status st = launch_head(h, true, LMH_HEAD_AUTO, s);
            if (st != LMH_OK) return st;
            ReduceArgs a{out, LMH_F32, ld, selected_ids ? selected_ids + r0 : nullptr, lse + r0,
                         selected_ids ? selected_logprob + r0 : nullptr,
                         kr > 0 ? topk_ids + r0 * kr : nullptr, kr > 0 ? topk_logprobs + r0 * kr : nullptr,
                         ws_reduce, device_error};
            st = from_hip(launch_reduce_stage2_blocks(q, a, s));
            if (st != LMH_OK) return st;
            if (k == LMH_K_FULL) {
                st = from_hip(launch_full_logprobs(out, LMH_F32, n, vocab, ld, lse + r0, topk_logprobs + r0 * vocab, s));
                if (st != LMH_OK) return st;
            }
            continue;
        }
        lmh_status st = launch_head(h, hidden_dt == LMH_BF16, LMH_HEAD_AUTO, s);
        if (st != LMH_OK) return st;
        if (vocab_mask != nullptr && num_segments > 0) {
            // each segment's mask on this chunk's rows, before they are reduced
            MaskArgs m{out, LMH_F32, n, vocab, ld, reinterpret_cast<const int32_t*>(vocab_mask),
                       vocab_mask_ld, logits_indices ? logits_cu_seqlens : nullptr, num_segments,
                       device_error};
            m.win0 = r0;
            m.total_rows = R;
            st = from_hip(launch_apply_bitmask(m, s));
            if (st != LMH_OK) return st;
        }
        // this chunk's decomposition, inside the workspace layout sized for a full chunk
        ReducePlan q = plan_reduce(n, vocab, kr);
        q.part_off = pc.part_off;
        q.keys_off = pc.keys_off;
        q.bytes = pc.bytes;
        ReduceArgs a{out, LMH_F32, ld, selected_ids ? selected_ids + r0 : nullptr, lse + r0,
                     selected_ids ? selected_logprob + r0 : nullptr,
                     kr > 0 ? topk_ids + r0 * kr : nullptr, kr > 0 ? topk_logprobs + r0 * kr : nullptr,
                     ws_reduce, device_error};
        st = from_hip(launch_reduce(q, a, s));
        if (st != LMH_OK) return st;
        if (k == LMH_K_FULL) {
            st = from_hip(launch_full_logprobs(out, LMH_F32, n, vocab, ld, lse + r0, topk_logprobs + r0 * vocab, s));
            if (st != LMH_OK) return st;
        }
    }
    return LMH_OK;
}

}  // namespace

namespace lmh {

lmh_status reduce_validate(const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                           int64_t logits_ld, const int32_t* selected_ids, int32_t k, const float* lse,
                           const float* selected_logprob, const int32_t* topk_ids,
                           const float* topk_logprobs, size_t* workspace_bytes) {
    const lmh_status st = check_reduce_shape(logits_dt, rows, vocab, logits_ld, k);
    if (st != LMH_OK) return st;
    *workspace_bytes = plan_reduce(rows, vocab, k > 0 ? k : 0).bytes;
    if (rows == 0) return LMH_OK;
    if (!logits || !lse) return LMH_ERR_NULL;
    if (selected_ids && !selected_logprob) return LMH_ERR_NULL;
    if (k > 0 && (!topk_ids || !topk_logprobs)) return LMH_ERR_NULL;
    if (k == LMH_K_FULL && !topk_logprobs) return LMH_ERR_NULL;
    if (!aligned(logits, 16)) return LMH_ERR_ALIGN;
    return LMH_OK;
}

lmh_status reduce_enqueue(const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                          int64_t logits_ld, const int32_t* selected_ids, int32_t k, float* lse,
                          float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                          void* workspace, int32_t* device_error, hipStream_t s, uint32_t* single_counters,
                          int single) {
    const int32_t kr = k > 0 ? k : 0;   // K = -1: lse first, then every logprob
    const ReducePlan p = plan_reduce(rows, vocab, kr);
    ReduceArgs a{logits, (int32_t)logits_dt, logits_ld, selected_ids, lse, selected_logprob,
                 kr > 0 ? topk_ids : nullptr, kr > 0 ? topk_logprobs : nullptr, workspace, device_error};
    const bool one = single_counters != nullptr && single_ok(p) && single_bytes(p) <= p.bytes &&
                     (single == 1 || p.k <= kSingleRouteK);
    const lmh_status st = from_hip(one ? launch_reduce_single(p, a, single_counters, s) : launch_reduce(p, a, s));
    if (st != LMH_OK || k != LMH_K_FULL) return st;
    return from_hip(launch_full_logprobs(logits, (int32_t)logits_dt, rows, vocab, logits_ld, lse, topk_logprobs, s));
}

}  // namespace lmh

extern "C" {

const char* lmh_status_string(lmh_status st) {
    switch (st) {
        case LMH_OK: return "LMH_OK";
        case LMH_ERR_NULL: return "LMH_ERR_NULL: a required pointer is NULL";
        case LMH_ERR_SHAPE: return "LMH_ERR_SHAPE: invalid size, pitch or size limit";
        case LMH_ERR_K: return "LMH_ERR_K: k < -1, k > vocab or min(k, blocks) * 64 > 8192";
        case LMH_ERR_DTYPE: return "LMH_ERR_DTYPE: unsupported dtype";
        case LMH_ERR_ALIGN: return "LMH_ERR_ALIGN: pointer or row pitch not aligned";
        case LMH_ERR_WORKSPACE: return "LMH_ERR_WORKSPACE: workspace missing or too small";
        case LMH_ERR_HIP: return "LMH_ERR_HIP: a HIP launch failed";
    }
    return "unknown lmh_status";
}

lmh_status lmhead_gather_project(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                                 int64_t hidden_dim, int64_t hidden_ld, const void* weight,
                                 lmh_dtype weight_dt, int64_t vocab, int64_t weight_ld,
                                 const int32_t* cu_seqlens, int32_t num_segments,
                                 int32_t num_decode, const int32_t* logits_indices,
                                 int32_t num_indices, void* logits, lmh_dtype logits_dt,
                                 int64_t logits_ld, int32_t* logits_cu_seqlens,
                                 int32_t* gather_indices, int32_t* device_error, void* stream) {
    return gather_project_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                               dense_weight(weight, weight_dt, weight_ld), vocab, cu_seqlens,
                               num_segments, num_decode, logits_indices, num_indices, logits,
                               logits_dt, logits_ld, logits_cu_seqlens, gather_indices,
                               device_error, stream, LMH_HEAD_AUTO);
}

lmh_status lmh_debug_gather_project(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                                    int64_t hidden_dim, int64_t hidden_ld, const void* weight,
                                    lmh_dtype weight_dt, int64_t vocab, int64_t weight_ld,
                                    const int32_t* cu_seqlens, int32_t num_segments,
                                    int32_t num_decode, const int32_t* logits_indices,
                                    int32_t num_indices, void* logits, lmh_dtype logits_dt,
                                    int64_t logits_ld, int32_t* logits_cu_seqlens,
                                    int32_t* gather_indices, int32_t* device_error, void* stream,
                                    int32_t variant) {
    return gather_project_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                               dense_weight(weight, weight_dt, weight_ld), vocab, cu_seqlens,
                               num_segments, num_decode, logits_indices, num_indices, logits,
                               logits_dt, logits_ld, logits_cu_seqlens, gather_indices,
                               device_error, stream, variant);
}

lmh_status lmhead_gather_project_q(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                                   int64_t hidden_dim, int64_t hidden_ld, const uint32_t* weight_q,
                                   int64_t weight_q_ld, const uint16_t* scales,
                                   const uint16_t* biases, int64_t scales_ld, int32_t bits,
                                   int32_t group_size, int64_t vocab, const int32_t* cu_seqlens,
                                   int32_t num_segments, int32_t num_decode,
                                   const int32_t* logits_indices, int32_t num_indices,
                                   void* logits, lmh_dtype logits_dt, int64_t logits_ld,
                                   int32_t* logits_cu_seqlens, int32_t* gather_indices,
                                   int32_t* device_error, void* stream) {
    return gather_project_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                               quant_weight(weight_q, weight_q_ld, scales, biases, scales_ld, bits,
                                            group_size),
                               vocab, cu_seqlens, num_segments, num_decode, logits_indices,
                               num_indices, logits, logits_dt, logits_ld, logits_cu_seqlens,
                               gather_indices, device_error, stream, LMH_HEAD_AUTO);
}

lmh_status lmh_debug_gather_project_q(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                                      int64_t hidden_dim, int64_t hidden_ld,
                                      const uint32_t* weight_q, int64_t weight_q_ld,
                                      const uint16_t* scales, const uint16_t* biases,
                                      int64_t scales_ld, int32_t bits, int32_t group_size,
                                      int64_t vocab, const int32_t* cu_seqlens,
                                      int32_t num_segments, int32_t num_decode,
                                      const int32_t* logits_indices, int32_t num_indices,
                                      void* logits, lmh_dtype logits_dt, int64_t logits_ld,
                                      int32_t* logits_cu_seqlens, int32_t* gather_indices,
                                      int32_t* device_error, void* stream, int32_t variant) {
    return gather_project_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                               quant_weight(weight_q, weight_q_ld, scales, biases, scales_ld, bits,
                                            group_size),
                               vocab, cu_seqlens, num_segments, num_decode, logits_indices,
                               num_indices, logits, logits_dt, logits_ld, logits_cu_seqlens,
                               gather_indices, device_error, stream, variant);
}

size_t logprob_reduce_workspace_size(int64_t rows, int64_t vocab, int32_t k) {
    if (rows < 0 || vocab <= 0) return 256;
    return plan_reduce(rows, vocab, k < 0 ? 0 : k).bytes;
}

lmh_status logprob_reduce(const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                          int64_t logits_ld, const int32_t* selected_ids, int32_t k, float* lse,
                          float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                          void* workspace, size_t workspace_bytes, int32_t* device_error,
                          void* stream) {
    size_t need = 0;
    const lmh_status st = lmh::reduce_validate(logits, logits_dt, rows, vocab, logits_ld, selected_ids, k,
                                               lse, selected_logprob, topk_ids, topk_logprobs, &need);
    if (st != LMH_OK) return st;
    if (rows == 0) return LMH_OK;   // nothing is read or written
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return LMH_ERR_WORKSPACE;
    return lmh::reduce_enqueue(logits, logits_dt, rows, vocab, logits_ld, selected_ids, k, lse,
                               selected_logprob, topk_ids, topk_logprobs, workspace, device_error,
                               static_cast<hipStream_t>(stream));
}

lmh_status lmh_debug_reduce_single(const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                                   int64_t logits_ld, const int32_t* selected_ids, int32_t k, float* lse,
                                   float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                                   void* workspace, size_t workspace_bytes, uint32_t* counters,
                                   int32_t* device_error, void* stream) {
    size_t need = 0;
    const lmh_status st = lmh::reduce_validate(logits, logits_dt, rows, vocab, logits_ld, selected_ids, k,
                                               lse, selected_logprob, topk_ids, topk_logprobs, &need);
    if (st != LMH_OK) return st;
    if (rows == 0) return LMH_OK;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return LMH_ERR_WORKSPACE;
    if (!counters) return LMH_ERR_NULL;
    if (!single_ok(plan_reduce(rows, vocab, k > 0 ? k : 0))) return LMH_ERR_SHAPE;
    return lmh::reduce_enqueue(logits, logits_dt, rows, vocab, logits_ld, selected_ids, k, lse,
                               selected_logprob, topk_ids, topk_logprobs, workspace, device_error,
                               static_cast<hipStream_t>(stream), counters, 1);
}

lmh_status lmh_debug_reduce_stage1(const void* logits, lmh_dtype logits_dt, int64_t rows,
                                   int64_t vocab, int64_t logits_ld, int32_t k, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (!logits) return LMH_ERR_NULL;
    const lmh_status st = check_reduce_shape(logits_dt, rows, vocab, logits_ld, k);
    if (st != LMH_OK) return st;
    if (!aligned(logits, 16)) return LMH_ERR_ALIGN;
    const ReducePlan p = plan_reduce(rows, vocab, k > 0 ? k : 0);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.bytes) return LMH_ERR_WORKSPACE;
    if (rows == 0) return LMH_OK;
    ReduceArgs a{logits, (int32_t)logits_dt, logits_ld, nullptr, nullptr, nullptr,
                 nullptr, nullptr, workspace, nullptr};
    return from_hip(launch_reduce_stage1(p, a, static_cast<hipStream_t>(stream)));
}

lmh_status lmhead_apply_bitmask(void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab,
                                int64_t logits_ld, const int32_t* bitmask, int64_t bitmask_ld,
                                const int32_t* logits_cu_seqlens, int32_t num_segments,
                                int32_t* device_error, void* stream) {
    if (rows < 0 || rows > INT32_MAX || vocab <= 0 || vocab > INT32_MAX || logits_ld < vocab ||
        num_segments < 0)
        return LMH_ERR_SHAPE;
    const int64_t words = ceil_div(vocab, 32);
    if (bitmask_ld < words) return LMH_ERR_SHAPE;
    if (logits_cu_seqlens == nullptr && num_segments != rows) return LMH_ERR_SHAPE;
    if (ceil_div(ceil_div(vocab, 4), 256) * (int64_t)num_segments >= ((int64_t)1 << 31)) return LMH_ERR_SHAPE;
    if (!valid_logits_dtype(logits_dt)) return LMH_ERR_DTYPE;
    if (num_segments == 0) return LMH_OK;   // nothing is read or written
    if (!logits || !bitmask) return LMH_ERR_NULL;
    if (!aligned(logits, 16) || ((size_t)logits_ld * esize(logits_dt)) % 16 || !aligned(bitmask, 4))
        return LMH_ERR_ALIGN;
    MaskArgs a{logits, (int32_t)logits_dt, rows, vocab, logits_ld, bitmask, bitmask_ld,
               logits_cu_seqlens, num_segments, device_error};
    return from_hip(launch_apply_bitmask(a, static_cast<hipStream_t>(stream)));
}

int32_t lmh_debug_reduce_path(int64_t rows, int64_t vocab, int32_t k) {
    if (rows <= 0 || vocab <= 0 || k < LMH_K_FULL) return 0;
    return reduce_row_path(plan_reduce(rows, vocab, k > 0 ? k : 0)) ? 1 : 0;
}

size_t lmhead_logprobs_workspace_size(int64_t rows, int64_t vocab, int32_t k, int32_t chunk_rows) {
    if (rows < 0 || vocab <= 0) return 256;
    const int64_t chunk_cfg = chunk_rows > 0 ? chunk_rows : 256;
    const int64_t chunk = rows < chunk_cfg ? (rows > 0 ? rows : 1) : chunk_cfg;
    const int64_t ld = ceil_div(vocab, 4) * 4;
    const size_t red = plan_reduce(chunk, vocab, k < 0 ? 0 : k).bytes;
    const size_t blk = blocks_ws_bytes(chunk, vocab, k);
    return up256((size_t)chunk * (size_t)ld * sizeof(float)) + (red > blk ? red : blk);
}

lmh_status lmhead_logprobs(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                           int64_t hidden_dim, int64_t hidden_ld, const void* weight,
                           lmh_dtype weight_dt, int64_t vocab, int64_t weight_ld,
                           const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
                           const int32_t* logits_indices, int32_t num_indices,
                           const int32_t* selected_ids, int32_t k, float* lse,
                           float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                           int32_t* logits_cu_seqlens, int32_t* gather_indices, int32_t chunk_rows,
                           float* logits_debug, void* workspace, size_t workspace_bytes,
                           int32_t* device_error, void* stream) {
    return logprobs_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                         dense_weight(weight, weight_dt, weight_ld), vocab, cu_seqlens,
                         num_segments, num_decode, logits_indices, num_indices, selected_ids, k,
                         lse, selected_logprob, topk_ids, topk_logprobs, logits_cu_seqlens,
                         gather_indices, chunk_rows, logits_debug, workspace, workspace_bytes,
                         device_error, stream);
}

lmh_status lmhead_logprobs_q(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                             int64_t hidden_dim, int64_t hidden_ld, const uint32_t* weight_q,
                             int64_t weight_q_ld, const uint16_t* scales, const uint16_t* biases,
                             int64_t scales_ld, int32_t bits, int32_t group_size, int64_t vocab,
                             const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
                             const int32_t* logits_indices, int32_t num_indices,
                             const int32_t* selected_ids, int32_t k, float* lse,
                             float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
                             int32_t* logits_cu_seqlens, int32_t* gather_indices,
                             int32_t chunk_rows, float* logits_debug, void* workspace,
                             size_t workspace_bytes, int32_t* device_error, void* stream) {
    return logprobs_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                         quant_weight(weight_q, weight_q_ld, scales, biases, scales_ld, bits,
                                      group_size),
                         vocab, cu_seqlens, num_segments, num_decode, logits_indices, num_indices,
                         selected_ids, k, lse, selected_logprob, topk_ids, topk_logprobs,
                         logits_cu_seqlens, gather_indices, chunk_rows, logits_debug, workspace,
                         workspace_bytes, device_error, stream);
}

lmh_status lmhead_gather_project_ex(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                                    int64_t hidden_dim, int64_t hidden_ld, const lmh_head* head,
                                    int64_t vocab, const int32_t* cu_seqlens, int32_t num_segments,
                                    int32_t num_decode, const int32_t* logits_indices,
                                    int32_t num_indices, void* logits, lmh_dtype logits_dt,
                                    int64_t logits_ld, int32_t* logits_cu_seqlens,
                                    int32_t* gather_indices, int32_t* device_error, void* stream,
                                    int32_t variant) {
    if (!head) return LMH_ERR_NULL;
    return gather_project_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                               head_weight(*head), vocab, cu_seqlens, num_segments, num_decode,
                               logits_indices, num_indices, logits, logits_dt, logits_ld,
                               logits_cu_seqlens, gather_indices, device_error, stream, variant);
}

lmh_status lmhead_logprobs_ex(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                              int64_t hidden_dim, int64_t hidden_ld, const lmh_head* head,
                              int64_t vocab, const int32_t* cu_seqlens, int32_t num_segments,
                              int32_t num_decode, const int32_t* logits_indices,
                              int32_t num_indices, const int32_t* selected_ids, int32_t k,
                              float* lse, float* selected_logprob, int32_t* topk_ids,
                              float* topk_logprobs, int32_t* logits_cu_seqlens,
                              int32_t* gather_indices, int32_t chunk_rows, float* logits_debug,
                              const uint32_t* vocab_mask, int64_t vocab_mask_ld, void* workspace,
                              size_t workspace_bytes, int32_t* device_error, void* stream) {
    if (!head) return LMH_ERR_NULL;
    return logprobs_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld, head_weight(*head),
                         vocab, cu_seqlens, num_segments, num_decode, logits_indices, num_indices,
                         selected_ids, k, lse, selected_logprob, topk_ids, topk_logprobs,
                         logits_cu_seqlens, gather_indices, chunk_rows, logits_debug, workspace,
                         workspace_bytes, device_error, stream, vocab_mask, vocab_mask_ld);
}

lmh_status lmh_debug_logprobs_ex(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                                 int64_t hidden_dim, int64_t hidden_ld, const lmh_head* head,
                                 int64_t vocab, const int32_t* cu_seqlens, int32_t num_segments,
                                 int32_t num_decode, const int32_t* logits_indices,
                                 int32_t num_indices, const int32_t* selected_ids, int32_t k,
                                 float* lse, float* selected_logprob, int32_t* topk_ids,
                                 float* topk_logprobs, int32_t* logits_cu_seqlens,
                                 int32_t* gather_indices, int32_t chunk_rows, float* logits_debug,
                                 const uint32_t* vocab_mask, int64_t vocab_mask_ld, void* workspace,
                                 size_t workspace_bytes, int32_t* device_error, void* stream,
                                 int32_t epilogue) {
    if (!head) return LMH_ERR_NULL;
    if (epilogue != 0 && epilogue != 1) return LMH_ERR_SHAPE;
    return logprobs_impl(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld, head_weight(*head),
                         vocab, cu_seqlens, num_segments, num_decode, logits_indices, num_indices,
                         selected_ids, k, lse, selected_logprob, topk_ids, topk_logprobs,
                         logits_cu_seqlens, gather_indices, chunk_rows, logits_debug, workspace,
                         workspace_bytes, device_error, stream, vocab_mask, vocab_mask_ld, epilogue == 0);
}

size_t lmhead_selfcheck_workspace_size(int64_t rows, int64_t vocab) {
    if (rows <= 0 || vocab <= 0) return 256;
    return up256((size_t)rows * (size_t)(ceil_div(vocab, 4) * 4) * sizeof(float));
}

lmh_status lmhead_selfcheck(const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens,
                            int64_t hidden_dim, int64_t hidden_ld, const lmh_head* head,
                            int64_t vocab, const int32_t* cu_seqlens, int32_t num_segments,
                            int32_t num_decode, const int32_t* logits_indices, int32_t num_indices,
                            const float* full_logits, int64_t full_ld, void* workspace,
                            size_t workspace_bytes, int64_t* result, int32_t* device_error,
                            void* stream) {
    if (!head || !full_logits || !result) return LMH_ERR_NULL;
    const WeightSpec w = head_weight(*head);
    const ProjectCheck c = check_project_inputs(hidden, hidden_dt, num_tokens, hidden_dim, hidden_ld,
                                                w, vocab, cu_seqlens, num_segments, num_decode,
                                                logits_indices, num_indices);
    if (c.st != LMH_OK) return c.st;
    if (full_ld < vocab) return LMH_ERR_SHAPE;
    if (!aligned(full_logits, 4) || !aligned(result, 8)) return LMH_ERR_ALIGN;
    const int64_t ld = ceil_div(vocab, 4) * 4;
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < lmhead_selfcheck_workspace_size(c.rows, vocab))
        return LMH_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (device_error) {
        RowsArgs ra{cu_seqlens, num_segments, num_decode, num_tokens, logits_indices, c.rows,
                    nullptr, nullptr, device_error};
        const lmh_status st = from_hip(launch_rows(ra, s));
        if (st != LMH_OK) return st;
    }
    float* sel = static_cast<float*>(workspace);
    if (c.rows > 0) {
        const HeadArgs h = head_args(hidden, num_tokens, hidden_dim, hidden_ld, w, vocab, cu_seqlens,
                                     num_decode, logits_indices, 0, c.rows, sel, ld, false,
                                     device_error);
        const lmh_status st = launch_head(h, hidden_dt == LMH_BF16, LMH_HEAD_AUTO, s);
        if (st != LMH_OK) return st;
    }
    return from_hip(launch_selfcheck(sel, ld, full_logits, full_ld, c.rows, vocab, cu_seqlens,
                                     num_decode, num_tokens, logits_indices, result, s));
}

}  // extern "C"
