/*
 * lmhead.h -- C ABI of the selective LM head and the on-device logprob
 * reduction for AMD Instinct MI355X (gfx950).
 *
 * Two stages, each callable alone, plus a fused call:
 *
 *   lmhead_gather_project  gathers the sampled rows of a packed batch (the
 *                          last row of every segment, which includes every
 *                          decode row, or an explicit row list) and projects
 *                          only those rows through the head
 *                          [rows x hidden] . [hidden x vocab].
 *   logprob_reduce         reduces each logits row on the device to a compact
 *                          O(K+1) result: the row logsumexp, the selected
 *                          token's logprob and the exact top-K ids and
 *                          logprobs, exact ties listed by ascending id.
 *   lmhead_logprobs        both, chunked, with the fp32 logits kept in a
 *                          caller-provided workspace.
 *
 * Sources (the pages this implements):
 *   [vllm-metal]  vllm-metal release v0.4.0.dev20260831001336 (selective
 *                 logits for the paged text path), Summary: the sampled row
 *                 of prefill segment j is cu_seqlens[num_decode + j + 1] - 1;
 *                 decode rows are the leading one-token segments; an
 *                 optional logits_indices replaces the sampled rows; pure
 *                 decode is unchanged; logits_cu_seqlens describes the
 *                 compacted logits layout.
 *   [mlxcel]      mlxcel PR #1969, description: the head acts per position,
 *                 so the row projected from a gathered hidden row equals the
 *                 same row of the full projection.
 *   [MTPLX]       MTPLX PR #532, Change: an fp32 logsumexp per row; a
 *                 prefilter over 64-logit blocks that keeps the K blocks
 *                 with the largest maxima and takes the exact top-K among
 *                 what they hold; logprobs formed for the K results and the
 *                 scored token alone; equal values ordered by token id,
 *                 lowest first.
 *   [openinfer]   openinfer issue #719, Suggested direction and Acceptance
 *                 criteria: logsumexp, selected logprob and top-k computed
 *                 while the logits stay on the GPU, returned as an O(k+1)
 *                 result per row; no full-row device-to-host copy.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller. The library
 *     allocates nothing, keeps no state between calls, never synchronises and
 *     never copies to the host: all work is enqueued on `stream` (a
 *     hipStream_t; NULL is the null stream) and the caller keeps every buffer
 *     alive until that work completes. Calls on distinct outputs and
 *     workspaces may run concurrently.
 *   - Row pitches (`*_ld`) are in elements. Matrices are row-major.
 *   - Argument errors visible on the host return a status BEFORE any HIP
 *     call, so nothing is enqueued. A failed launch returns LMH_ERR_HIP.
 *   - Errors that depend on device data are OR-ed into *device_error (an
 *     int32 the caller zeroes beforehand; may be NULL) with the LMH_DEVERR_*
 *     bits; the affected outputs are NaN (logits, logprobs) or -1 (indices).
 *   - Logprob results are fp32: lse is an fp32 logsumexp of the row, and a
 *     logprob is float32(logit) - lse rounded once. Top-K ids are exact:
 *     order is value descending with exact ties (IEEE equality: -0 == +0,
 *     -inf == -inf) by ascending token id. Rows containing +inf or NaN are
 *     outside the contract.
 */
#ifndef LMHEAD_H
#define LMHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LMH_OK = 0,
    LMH_ERR_NULL = 1,      /* a required pointer is NULL                        */
    LMH_ERR_SHAPE = 2,     /* a size is negative/zero where it must not be, a   */
                           /* row pitch is below the row width, or a size limit */
                           /* below is exceeded                                 */
    LMH_ERR_K = 3,         /* K < -1, K > vocab, or min(K, nb) * 64 > 8192      */
    LMH_ERR_DTYPE = 4,     /* unsupported dtype or dtype combination           */
    LMH_ERR_ALIGN = 5,     /* a base pointer or row pitch is not 16-B aligned   */
    LMH_ERR_WORKSPACE = 6, /* workspace NULL or smaller than the size function  */
    LMH_ERR_HIP = 7        /* a HIP launch failed                               */
} lmh_status;

/* LMH_F16 (IEEE binary16) is accepted for the logits of logprob_reduce only
 * [MTPLX PR #532, Tests: bf16/f16 logits]; every other dtype argument takes
 * LMH_F32 or LMH_BF16. */
typedef enum {
    LMH_F32 = 0,
    LMH_BF16 = 1,
    LMH_F16 = 2,
    /* not a dtype: makes every 32-bit value a value of the type, so an
     * unknown code from a caller is checked (LMH_ERR_DTYPE), not undefined */
    LMH_DTYPE_MAX_ENUM = 0x7FFFFFFF
} lmh_dtype;

/* device_error bits */
#define LMH_DEVERR_INDEX 1  /* a row index or selected id outside its range            */
#define LMH_DEVERR_LAYOUT 2 /* cu_seqlens[0] != 0, cu_seqlens decreasing, cu_seqlens[S] */
                            /* beyond num_tokens, a decode segment not one token long,   */
                            /* or an empty segment in sampled mode                       */

/* k = LMH_K_FULL asks for every token's logprob instead of a top-K
 * [openinfer, Acceptance criteria: -1 = full vocabulary] */
#define LMH_K_FULL (-1)

/* logits per prefilter block [MTPLX, Change] and the candidate bound */
#define LMH_BLOCK 64
#define LMH_MAX_CANDIDATES 8192
/* largest vocabulary the reduction accepts when K > 0 (block maxima of a row
 * are resolved in on-chip memory) */
#define LMH_MAX_VOCAB_TOPK (8192 * LMH_BLOCK)

/*
 * lmhead_gather_project -- row gather + head projection [vllm-metal, mlxcel].
 *
 * hidden  [num_tokens][hidden_dim], pitch hidden_ld, dtype hidden_dt: the
 *         packed, final-normed hidden states of one step.
 * weight  [vocab][hidden_dim], pitch weight_ld, dtype weight_dt == hidden_dt:
 *         the head, one row per token id (the transpose of the
 *         [hidden x vocab] operand).
 * cu_seqlens [num_segments + 1] int32: segment boundaries; the first
 *         num_decode segments are decode rows (one token each).
 * logits_indices [num_indices] int32 or NULL. NULL selects sampled mode:
 *         R = num_segments rows, row s is cu_seqlens[s+1] - 1. Otherwise
 *         R = num_indices rows taken as given (e.g. every prompt position).
 * logits  [R][vocab], pitch logits_ld, dtype logits_dt (fp32, or bf16 rounded
 *         to nearest even from the fp32 accumulator):
 *         logits[r][v] = sum_k hidden[idx[r]][k] * weight[v][k].
 *         bf16 inputs run on MFMA with fp32 accumulation; fp32 inputs on fp32
 *         FMA. The result for a row does not depend on which other rows are
 *         projected with it (bitwise).
 * logits_cu_seqlens [num_segments + 1] int32 or NULL: sampled mode writes
 *         0..num_segments; explicit mode writes, per segment s, the number of
 *         logits rows whose source row lies before cu_seqlens[s].
 * gather_indices [R] int32 or NULL: the source row of each logits row (-1 if
 *         invalid).
 * Requirements: num_tokens, hidden_dim, vocab > 0; num_segments >= 0;
 *   0 <= num_decode <= num_segments; pitches >= widths. For bf16: hidden and
 *   weight 16-B aligned, hidden_dim, hidden_ld and weight_ld multiples of 8.
 *   logits 4-B (fp32) / 2-B (bf16) aligned.
 * A row whose source index is outside [0, num_tokens) (or, in sampled mode,
 * whose segment is malformed) is written as NaN and flagged.
 */
lmh_status lmhead_gather_project(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld,
    const void* weight, lmh_dtype weight_dt, int64_t vocab, int64_t weight_ld,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    void* logits, lmh_dtype logits_dt, int64_t logits_ld,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t* device_error, void* stream);

/*
 * logprob_reduce_workspace_size -- bytes of device workspace logprob_reduce
 * needs for this shape (0 never; always a multiple of 256).
 */
size_t logprob_reduce_workspace_size(int64_t rows, int64_t vocab, int32_t k);

/*
 * logprob_reduce -- per-row logsumexp, selected logprob and exact top-K
 * [MTPLX, openinfer].
 *
 * logits  [rows][vocab], pitch logits_ld, fp32, bf16 or f16; 16-B aligned
 *         base and pitch. f16 and bf16 values are widened to fp32 exactly.
 * selected_ids [rows] int32 or NULL (then selected_logprob is not written).
 * k       0 <= k <= vocab and min(k, ceil(vocab/64)) * 64 <= 8192 (so k <= 128
 *         at vocabularies above 8192). k = 0 computes lse and the selected
 *         logprob only; topk_* may then be NULL. k = LMH_K_FULL (-1) writes
 *         every token's logprob instead of a top-K: topk_logprobs is then
 *         [rows][vocab] fp32 (row pitch vocab, element v the logprob of
 *         token v, float32(logit) - lse like every other logprob) and
 *         topk_ids is not used (may be NULL).
 * lse [rows], selected_logprob [rows], topk_ids [rows][k] (int32),
 * topk_logprobs [rows][k] (fp32): outputs, written in full.
 * Method: one coalesced pass over each row produces online (max, sum-exp)
 * partials per 4096-logit segment and the maximum of every 64-logit block;
 * the partials are combined in one fixed order, the min(k, nb) blocks with
 * the largest maxima (equal maxima by ascending block index) are kept and the
 * exact top-K is taken among the entries of those blocks that are not below
 * the k-th kept block maximum. No full-vocabulary log-softmax is formed.
 * When the rows fill the device's compute units evenly (see
 * lmh_debug_reduce_path) one workgroup reduces each row in a single launch
 * with the block maxima in LDS; otherwise a streaming launch over all rows
 * writes partials and block maxima to the workspace and a second launch
 * finishes each row. Both give bitwise-identical results, so a row's
 * results do not depend on the rows around it.
 * An all -inf row gives lse = -inf and NaN logprobs (ids 0..k-1); a selected
 * id outside [0, vocab) gives NaN and LMH_DEVERR_INDEX. rows = 0 is a no-op
 * (pointers may then be NULL) once the shape and K rules pass.
 */
lmh_status logprob_reduce(
    const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab, int64_t logits_ld,
    const int32_t* selected_ids, int32_t k,
    float* lse, float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream);

/*
 * logprob_reduce_noalloc -- logprob_reduce for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc. There is no workspace argument; the
 * scratch (LMH_NOALLOC_SCRATCH_BYTES of workspace plus one 32-bit counter
 * per row for up to 4096 rows) lives in a static device array per GPU that
 * the library holds until the process ends (its device address is looked up
 * on the first call on each device, with that device current, and that call
 * also enqueues a small kernel on `stream` that clears the counters).
 * The call allocates and frees nothing.
 * Arguments, outputs, results (bitwise) and status codes are those of
 * logprob_reduce; a shape whose logprob_reduce_workspace_size exceeds
 * LMH_NOALLOC_SCRATCH_BYTES returns LMH_ERR_WORKSPACE before any HIP call.
 * Few rows (decode steps, openinfer issue #719, Description: rows that leave
 * most compute units idle) with K = 0 (or -1) and vocab <= 262,144 take a
 * single launch: each row is spread over several workgroups that each reduce
 * a slice, and the last workgroup of the row to arrive (a per-row counter in
 * the array, back at zero when the launch ends) merges the slices; K >= 1
 * takes the two launches, which measured faster there. All calls on one GPU
 * share that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and must be ordered by the caller. Nothing in the
 * array needs clearing between calls.
 */
#define LMH_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
lmh_status logprob_reduce_noalloc(
    const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab, int64_t logits_ld,
    const int32_t* selected_ids, int32_t k,
    float* lse, float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
    int32_t* device_error, void* stream);

/*
 * lmhead_apply_bitmask -- token bitmask on the compacted logits, in place
 * [vllm-metal, Testing: bitmask application under the compacted layout].
 *
 * logits  [rows][vocab], pitch logits_ld, fp32, bf16 or f16; 16-B aligned
 *         base and pitch (the layout logprob_reduce takes).
 * bitmask [num_segments][bitmask_ld] 32-bit words, bitmask_ld >=
 *         ceil(vocab/32), 4-B aligned: bit v % 32 of word v / 32 of row s set
 *         keeps token v in segment s's rows; clear sets it to -inf. Bits past
 *         vocab are ignored.
 * logits_cu_seqlens [num_segments + 1] or NULL: segment s owns the logits
 *         rows logits_cu_seqlens[s] .. logits_cu_seqlens[s+1]-1 (the array
 *         lmhead_gather_project writes); NULL requires num_segments == rows
 *         and gives segment s the row s.
 * Only masked entries are written (no logits are read); padding between
 * vocab and logits_ld is never touched. A segment whose bounds decrease or
 * leave [0, rows] is skipped and sets LMH_DEVERR_LAYOUT in *device_error.
 * num_segments = 0 is a no-op (pointers may then be NULL).
 */
lmh_status lmhead_apply_bitmask(
    void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab, int64_t logits_ld,
    const int32_t* bitmask, int64_t bitmask_ld,
    const int32_t* logits_cu_seqlens, int32_t num_segments,
    int32_t* device_error, void* stream);

/*
 * lmhead_logprobs_workspace_size -- bytes of device workspace lmhead_logprobs
 * needs: room for one chunk of fp32 logits (chunk_rows x vocab, chunk_rows = 0
 * meaning 256) plus the reduction's workspace for that chunk.
 */
size_t lmhead_logprobs_workspace_size(int64_t rows, int64_t vocab, int32_t k, int32_t chunk_rows);

/*
 * lmhead_logprobs -- fused gather + projection + reduction
 * [vllm-metal, mlxcel, MTPLX, openinfer].
 *
 * Arguments as in lmhead_gather_project and logprob_reduce. The R selected
 * rows are processed in chunks of chunk_rows (0 => 256, the chunk size of
 * MTPLX PR #532, Motivation): each chunk is projected to fp32 logits in the
 * workspace and reduced there, so no logits row leaves the device and at
 * most one chunk of logits is resident. selected_ids is indexed by logits
 * row (R entries). logits_debug, when not NULL, is an [R][vocab] fp32 buffer
 * that receives the logits that were reduced (tests use it); the workspace
 * then only holds the reduction's part. Chunks of more than 64 rows of a dense
 * bf16 head whose hidden size is a multiple of 128 (hidden matrix and 256
 * weight rows each at most 4 GiB) are projected by the tiled kernel, whose
 * epilogue also writes, per row and 64-logit block, the
 * block maximum and its (max, sum of exp) partial [MTPLX PR #532,
 * Motivation: no second full pass over a chunk's logits]; the reduction then
 * merges those partials (one per block: partial i to thread i mod 256 in
 * ascending order, each wave's lanes as a pairwise tree, then the four waves
 * in order) and takes the top-K from them, with no pass of its own over the
 * logits. Ids and selected values are those of the unfused reduction of the
 * same logits; lse may differ from it in the last bits (another summation
 * order). k = LMH_K_FULL writes every token's
 * logprob of each logits row into topk_logprobs [R][vocab] (row pitch vocab),
 * as logprob_reduce does. A row without a valid source (flagged
 * in device_error) has NaN logits, so its lse, selected logprob and top-K
 * logprobs come out NaN and its top-K ids -1.
 */
lmh_status lmhead_logprobs(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld,
    const void* weight, lmh_dtype weight_dt, int64_t vocab, int64_t weight_ld,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    const int32_t* selected_ids, int32_t k,
    float* lse, float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t chunk_rows, float* logits_debug,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream);

/*
 * Quantised head weights [mlxcel: the measured models are 4-bit].
 *
 * The head may be given as affine group-quantised codes instead of dense
 * weights: for token v and hidden index k, with g = k / group_size,
 *     weight[v][k] = scales[v][g] * q(v, k) + biases[v][g],
 * where q(v, k) is the unsigned `bits`-bit code (bits 4 or 8) stored
 * little-endian in the 32-bit words of row v of weight_q: word
 * (k * bits) / 32, starting at bit (k * bits) % 32.
 *
 * weight_q  [vocab][weight_q_ld] uint32 words, 16-B aligned, weight_q_ld a
 *           multiple of 4 and >= hidden_dim * bits / 32.
 * scales, biases [vocab][scales_ld] bf16 (raw uint16 bits), 2-B aligned,
 *           scales_ld >= hidden_dim / group_size.
 * bits 4 or 8 (else LMH_ERR_DTYPE); group_size 32, 64 or 128; hidden_dim a
 *           multiple of 128 (else LMH_ERR_SHAPE). hidden_dt must be LMH_BF16.
 * Each weight is formed on the device as fma(scale, q, bias) in fp32 (the
 * product is exact) and rounded once to bf16 (nearest even), then enters the
 * same bf16 MFMA path with fp32 accumulation as dense bf16 weights, so a
 * row's logits do not depend on the rows projected with it (bitwise). The
 * hidden index is summed in an order of the library's own (runs of
 * 512 / bits elements, one run per lane and MFMA group), so results equal
 * the dense path's on the dequantised weights up to fp32 summation order.
 * All other arguments, outputs and rules are those of lmhead_gather_project
 * and lmhead_logprobs (workspace: lmhead_logprobs_workspace_size).
 */
lmh_status lmhead_gather_project_q(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld,
    const uint32_t* weight_q, int64_t weight_q_ld, const uint16_t* scales, const uint16_t* biases,
    int64_t scales_ld, int32_t bits, int32_t group_size, int64_t vocab,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    void* logits, lmh_dtype logits_dt, int64_t logits_ld,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t* device_error, void* stream);

lmh_status lmhead_logprobs_q(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld,
    const uint32_t* weight_q, int64_t weight_q_ld, const uint16_t* scales, const uint16_t* biases,
    int64_t scales_ld, int32_t bits, int32_t group_size, int64_t vocab,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    const int32_t* selected_ids, int32_t k,
    float* lse, float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t chunk_rows, float* logits_debug,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream);

/* ---------------------------------------------------------------------------
 * Head descriptor and extended entry points.
 *
 * Head output scaling [vllm-metal, Summary: some heads scale their logits
 * outside the projection -- Cohere's logit_scale, Granite's logits_scaling --
 * and a selective path that leaves the scaling out gives wrong logits without
 * failing]. scale_mode LMH_SCALE_MUL multiplies every fp32 logit by `scale`,
 * LMH_SCALE_DIV divides it by `scale` (IEEE fp32 division, correctly
 * rounded); the scaling is applied to the fp32 accumulator before any bf16
 * rounding of the output, on every head kernel alike.
 * ------------------------------------------------------------------------- */
#define LMH_SCALE_NONE 0
#define LMH_SCALE_MUL 1
#define LMH_SCALE_DIV 2

typedef struct lmh_head {
    /* dense weights (bits == 0): [vocab][weight_ld], weight_dt == hidden_dt */
    const void* weight;
    lmh_dtype weight_dt;
    int64_t weight_ld;
    /* affine group-quantised weights (bits 4 or 8), as for lmhead_gather_project_q */
    int32_t bits;
    int32_t group_size;
    const uint32_t* weight_q;
    int64_t weight_q_ld;
    const uint16_t* scales;
    const uint16_t* biases;
    int64_t scales_ld;
    /* output scaling */
    int32_t scale_mode;   /* LMH_SCALE_NONE, LMH_SCALE_MUL or LMH_SCALE_DIV */
    float scale;          /* finite and nonzero when scale_mode != LMH_SCALE_NONE */
} lmh_head;

/*
 * lmhead_gather_project_ex -- lmhead_gather_project / lmhead_gather_project_q
 * with the head given by `head` (NULL is LMH_ERR_NULL) and output scaling.
 * `variant` is LMH_HEAD_AUTO or forces a kernel as in
 * lmh_debug_gather_project. An unknown scale_mode, or a zero or non-finite
 * scale with a mode set, returns LMH_ERR_SHAPE.
 */
lmh_status lmhead_gather_project_ex(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld, const lmh_head* head, int64_t vocab,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    void* logits, lmh_dtype logits_dt, int64_t logits_ld,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t* device_error, void* stream, int32_t variant);

/*
 * lmhead_logprobs_ex -- lmhead_logprobs with the head given by `head` (dense
 * or quantised, with output scaling: the reduction sees the scaled logits)
 * and an optional token bitmask [vllm-metal, Testing: bitmask application
 * under the compacted layout].
 * vocab_mask [num_segments][vocab_mask_ld] 32-bit words or NULL (no mask):
 *         the layout lmhead_apply_bitmask takes (bit v % 32 of word v / 32 of
 *         row s set keeps token v in segment s's logits rows, clear makes it
 *         -inf; bits past vocab ignored), vocab_mask_ld >= ceil(vocab/32),
 *         4-B aligned. Each chunk's fp32 logits are masked before they are
 *         reduced, so lse, the selected logprob and the top-K are those of
 *         the masked rows (a fully masked row: lse -inf, NaN logprobs; a
 *         masked selected token: logprob -inf). Segment s owns the logits
 *         rows logits_cu_seqlens[s] .. [s+1]-1: with logits_indices the call
 *         computes those bounds into logits_cu_seqlens, which must then be
 *         non-NULL (else LMH_ERR_NULL); in sampled mode segment s is row s.
 *         A segment whose bounds are malformed is left unmasked and sets
 *         LMH_DEVERR_LAYOUT. vocab_mask_ld is ignored when vocab_mask is NULL.
 */
lmh_status lmhead_logprobs_ex(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld, const lmh_head* head, int64_t vocab,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    const int32_t* selected_ids, int32_t k,
    float* lse, float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t chunk_rows, float* logits_debug,
    const uint32_t* vocab_mask, int64_t vocab_mask_ld,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream);

/*
 * lmhead_selfcheck_workspace_size -- bytes of device workspace
 * lmhead_selfcheck needs: rows x roundup(vocab, 4) fp32.
 */
size_t lmhead_selfcheck_workspace_size(int64_t rows, int64_t vocab);

/*
 * lmhead_selfcheck -- bit-exact check of the selective path against a head's
 * own full output [vllm-metal, Summary: selective logits are used only where
 * the selected rows equal the model's own output bit for bit; Testing: a
 * scaled head the selective path does not reproduce is rejected].
 *
 * Projects the R selected rows (sampled or explicit mode, as in
 * lmhead_gather_project) through `head` into the workspace as fp32 and
 * compares each with row src(r) of full_logits [num_tokens][full_ld] fp32 --
 * the logits the model's own forward produced for every position -- as bit
 * patterns. result is a DEVICE int64[2]: result[0] = number of differing
 * logits, result[1] = the smallest r * vocab + v that differs (INT64_MAX when
 * none). Rows without a valid source are skipped (and flagged in
 * device_error). result is written by the call (no need to clear it).
 */
lmh_status lmhead_selfcheck(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld, const lmh_head* head, int64_t vocab,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    const float* full_logits, int64_t full_ld,
    void* workspace, size_t workspace_bytes, int64_t* result,
    int32_t* device_error, void* stream);

/* lmh_status_string -- static, human-readable name of a status code. */
const char* lmh_status_string(lmh_status status);

/* ---------------------------------------------------------------------------
 * Diagnostic entry points (tests and measurement). Same contracts as above.
 * ------------------------------------------------------------------------- */

/* Head kernel choices for lmh_debug_gather_project's `variant`. */
#define LMH_HEAD_AUTO 0   /* k-pipelined streaming where it applies and R >  */
                          /* 16, weight streaming for other R <= 64, tiled    */
                          /* otherwise                                        */
#define LMH_HEAD_STREAM 1 /* weight-streaming kernel (requires R <= 64)      */
#define LMH_HEAD_TILED 2  /* LDS-tiled kernel                                */
#define LMH_HEAD_PIPE 3   /* k-pipelined weight streaming: bf16 weights,      */
                          /* R <= 64, hidden 512, 1024, 1536 or 2048, and     */
                          /* R * logits_ld * element size below 2^31 bytes    */

/*
 * lmh_debug_gather_project -- lmhead_gather_project with the bf16 head kernel
 * forced (tests use it to show the kernels give bitwise-identical rows).
 * LMH_HEAD_STREAM with R > 64, LMH_HEAD_PIPE outside its shapes, or any
 * non-auto variant with fp32 inputs, returns LMH_ERR_SHAPE.
 */
lmh_status lmh_debug_gather_project(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld,
    const void* weight, lmh_dtype weight_dt, int64_t vocab, int64_t weight_ld,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    void* logits, lmh_dtype logits_dt, int64_t logits_ld,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t* device_error, void* stream, int32_t variant);

/*
 * lmh_debug_gather_project_q -- lmhead_gather_project_q with the head kernel
 * forced (LMH_HEAD_STREAM with R > 64 returns LMH_ERR_SHAPE).
 */
lmh_status lmh_debug_gather_project_q(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld,
    const uint32_t* weight_q, int64_t weight_q_ld, const uint16_t* scales, const uint16_t* biases,
    int64_t scales_ld, int32_t bits, int32_t group_size, int64_t vocab,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    void* logits, lmh_dtype logits_dt, int64_t logits_ld,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t* device_error, void* stream, int32_t variant);

/*
 * lmh_debug_logprobs_ex -- lmhead_logprobs_ex with the reduction's first pass
 * chosen: epilogue 0 lets chunks of more than 64 rows of a dense bf16 head
 * (hidden size a multiple of 128, hidden matrix and 256 weight rows each at
 * most 4 GiB, no vocab_mask) take it in the tiled head's epilogue, as
 * lmhead_logprobs_ex does; 1 always runs it as its own pass over
 * the chunk's logits (tests and measurement compare the two). Any other
 * value returns LMH_ERR_SHAPE.
 */
lmh_status lmh_debug_logprobs_ex(
    const void* hidden, lmh_dtype hidden_dt, int64_t num_tokens, int64_t hidden_dim,
    int64_t hidden_ld, const lmh_head* head, int64_t vocab,
    const int32_t* cu_seqlens, int32_t num_segments, int32_t num_decode,
    const int32_t* logits_indices, int32_t num_indices,
    const int32_t* selected_ids, int32_t k,
    float* lse, float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
    int32_t* logits_cu_seqlens, int32_t* gather_indices,
    int32_t chunk_rows, float* logits_debug,
    const uint32_t* vocab_mask, int64_t vocab_mask_ld,
    void* workspace, size_t workspace_bytes, int32_t* device_error, void* stream,
    int32_t epilogue);

/*
 * lmh_debug_reduce_single -- logprob_reduce through the single-launch path
 * that logprob_reduce_noalloc takes for few rows, at any k it supports
 * (-1 <= k <= 32; logprob_reduce_noalloc takes it only for k <= 0, where it
 * measured faster than the two launches), on a caller workspace (the size
 * logprob_reduce_workspace_size gives) and caller counters: 4096 32-bit
 * words, zero before the first call, which every call leaves zero. Shapes
 * the path does not take (rows that fill the compute units, k > 32, vocab >
 * 64 * 4096 or rows > 4096) return LMH_ERR_SHAPE; counters NULL returns
 * LMH_ERR_NULL. Results are bitwise those of logprob_reduce. Calls sharing
 * counters must not overlap.
 */
lmh_status lmh_debug_reduce_single(
    const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab, int64_t logits_ld,
    const int32_t* selected_ids, int32_t k,
    float* lse, float* selected_logprob, int32_t* topk_ids, float* topk_logprobs,
    void* workspace, size_t workspace_bytes, uint32_t* counters, int32_t* device_error, void* stream);

/*
 * lmh_debug_reduce_stage1 -- only the streaming pass of logprob_reduce
 * (partials and block maxima into the workspace); used to time that kernel
 * alone. Same argument rules as logprob_reduce.
 */
lmh_status lmh_debug_reduce_stage1(
    const void* logits, lmh_dtype logits_dt, int64_t rows, int64_t vocab, int64_t logits_ld,
    int32_t k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lmh_debug_reduce_path -- 1 when logprob_reduce with these sizes runs as one
 * workgroup per row on the current HIP device (rows fill its compute units
 * evenly and, for k > 0, vocab <= 4096 * 64), 0 when it runs as the two-launch
 * split path. No device work; rows, vocab and k are not validated.
 */
int32_t lmh_debug_reduce_path(int64_t rows, int64_t vocab, int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_H */
