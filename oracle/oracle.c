/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the selective
 * LM head and the per-row logprob reduction.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path (the
 * HIP library) shares no source, header, table or helper with this file.
 *
 * Everything is computed in f64. Every bf16 or fp32 input widens to f64
 * exactly, so the only roundings are those of f64 arithmetic.
 *
 * Sources (the pages):
 *   - vllm-metal release v0.4.0 "selective logits", Summary: the sampled row
 *     of prefill segment j is cu_seqlens[num_decode + j + 1] - 1; decode
 *     rows are the leading one-token segments; an optional logits_indices
 *     list replaces the sampled rows; logits_cu_seqlens describes the
 *     compacted logits layout.
 *   - mlxcel PR #1969, description: the head acts per position, so the
 *     projected row of a gathered hidden row equals the full forward's row.
 *   - MTPLX PR #532, Motivation and Change: the result equals the full
 *     log-softmax read at the top-K entries and at the scored token;
 *     exact ties list by ascending token id; the 64-logit block-max
 *     prefilter keeps the K blocks with the largest maxima.
 *   - openinfer issue #719, Description: the host routine makes a
 *     full-vocabulary max pass, an f64 exp-sum pass and a top-k pass.
 *   - mlxcel PR #1969, description: the measured models are 4-bit; the
 *     quantised head weights are read as MLX-style affine groups
 *     (orc_dequant), then used by the same f64 head.
 *
 * The reduction here is the plain definition (max, f64 exp-sum, full sort),
 * not the prefilter: the prefilter is an acceleration that must reach the
 * same result. orc_prefilter_check() tests that claim on given rows.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes of this library (independent of the product's enum) */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2
#define ORC_F16 3

/* status codes */
#define ORC_OK 0
#define ORC_ERR_LAYOUT 1 /* cu_seqlens malformed (see orc_rows) */
#define ORC_ERR_INDEX 2  /* a row index outside [0, num_tokens) */

static double widen(const void* base, int dt, int64_t i) {
    if (dt == ORC_F32) return (double)((const float*)base)[i];
    if (dt == ORC_F64) return ((const double*)base)[i];
    if (dt == ORC_F16) {
        /* IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction */
        const uint16_t h = ((const uint16_t*)base)[i];
        const int e = (h >> 10) & 0x1F;
        const int m = h & 0x3FF;
        double v;
        if (e == 0)
            v = ldexp((double)m, -24);                 /* subnormal: m * 2^-14 * 2^-10 */
        else if (e == 31)
            v = m ? NAN : INFINITY;
        else
            v = ldexp((double)(m | 0x400), e - 25);    /* (1 + m/1024) * 2^(e-15) */
        return (h & 0x8000) ? -v : v;
    }
    /* bf16: the top 16 bits of an IEEE binary32 */
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* f64 values of n elements of dtype dt (exposed for the pins of widen). */
void orc_widen(const void* base, int dt, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = widen(base, dt, i);
}

/*
 * Row targets (vllm-metal release, Summary).
 *
 * cu[0..S] are segment boundaries of a packed batch of num_tokens rows; the
 * first num_decode segments are decode rows of exactly one token.
 *
 * Sampled mode (explicit == NULL): R = S rows, idx[s] = cu[s+1] - 1 (the last
 * row of each segment; for a decode segment d that is row d), and
 * logits_cu[s] = s because every segment contributes exactly one logits row.
 *
 * Explicit mode: R = n_explicit rows, idx = explicit, and logits_cu[s] is the
 * number of logits rows whose source row lies before segment s begins,
 * i.e. #{r : explicit[r] < cu[s]}.
 *
 * Layout requirements: cu[0] == 0, cu non-decreasing, cu[S] <= num_tokens,
 * each decode segment exactly one token long, and (sampled mode only) no
 * empty segment, since an empty segment has no last row. Violations return
 * ORC_ERR_LAYOUT; an explicit index outside [0, num_tokens) ORC_ERR_INDEX.
 * idx_out has R entries, logits_cu_out S + 1 entries (either may be NULL).
 */
int orc_rows(const int32_t* cu, int32_t S, int32_t num_decode, int64_t num_tokens,
             const int32_t* explicit_idx, int32_t n_explicit,
             int32_t* idx_out, int32_t* logits_cu_out) {
    if (S < 0 || num_decode < 0 || num_decode > S) return ORC_ERR_LAYOUT;
    if (cu[0] != 0) return ORC_ERR_LAYOUT;
    for (int32_t s = 0; s < S; ++s) {
        if (cu[s + 1] < cu[s]) return ORC_ERR_LAYOUT;
        if (s < num_decode && cu[s + 1] - cu[s] != 1) return ORC_ERR_LAYOUT;
        if (explicit_idx == NULL && cu[s + 1] == cu[s]) return ORC_ERR_LAYOUT;
    }
    if ((int64_t)cu[S] > num_tokens) return ORC_ERR_LAYOUT;

    if (explicit_idx == NULL) {
        for (int32_t s = 0; s < S; ++s) {
            if (idx_out) idx_out[s] = cu[s + 1] - 1;
        }
        if (logits_cu_out)
            for (int32_t s = 0; s <= S; ++s) logits_cu_out[s] = s;
        return ORC_OK;
    }
    for (int32_t r = 0; r < n_explicit; ++r) {
        if (explicit_idx[r] < 0 || (int64_t)explicit_idx[r] >= num_tokens) return ORC_ERR_INDEX;
        if (idx_out) idx_out[r] = explicit_idx[r];
    }
    if (logits_cu_out) {
        for (int32_t s = 0; s <= S; ++s) {
            int32_t c = 0;
            for (int32_t r = 0; r < n_explicit; ++r)
                if (explicit_idx[r] < cu[s]) ++c;
            logits_cu_out[s] = c;
        }
    }
    return ORC_OK;
}

/*
 * Token bitmask on the compacted logits (vllm-metal release, Testing:
 * bitmask application under the compacted layout). Segment s owns the logits
 * rows lcu[s] .. lcu[s+1]-1 (the logits_cu_seqlens of orc_rows; lcu NULL:
 * S == rows and segment s owns row s alone). Token v of those rows keeps its
 * value when bit v % 32 of word v / 32 of mask row s is set and becomes -inf
 * otherwise (bits past V are ignored). Z is f64 [rows][ld], changed in
 * place. A segment whose bounds decrease or leave [0, rows] is left alone
 * and the call returns ORC_ERR_LAYOUT.
 */
int orc_apply_bitmask(double* Z, int64_t rows, int64_t V, int64_t ld, const uint32_t* mask,
                      int64_t mask_ld, const int32_t* lcu, int32_t S) {
    int st = ORC_OK;
    for (int32_t s = 0; s < S; ++s) {
        const int64_t r0 = lcu ? lcu[s] : s;
        const int64_t r1 = lcu ? lcu[s + 1] : s + 1;
        if (r0 < 0 || r1 < r0 || r1 > rows) {
            st = ORC_ERR_LAYOUT;
            continue;
        }
        for (int64_t r = r0; r < r1; ++r) {
            for (int64_t v = 0; v < V; ++v) {
                const uint32_t word = mask[s * mask_ld + v / 32];
                if (((word >> (v % 32)) & 1u) == 0) Z[r * ld + v] = -INFINITY;
            }
        }
    }
    return st;
}

/*
 * Head projection on gathered rows (vllm-metal release, Summary; mlxcel
 * PR #1969): Z[r][v] = sum_{k=0}^{H-1} hidden[idx[r]][k] * W[v][k], summed in
 * ascending k, in f64. hidden is [num_tokens][H] with row pitch hld; W is
 * [V][H] with row pitch wld (one row per token id). Z is [R][V], dense.
 * A row whose index is outside [0, num_tokens) is filled with NaN.
 */
void orc_head(const void* hidden, int hdt, int64_t num_tokens, int64_t H, int64_t hld,
              const void* W, int wdt, int64_t V, int64_t wld,
              const int32_t* idx, int32_t R, double* Z) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t v = 0; v < V; ++v) {
            int64_t t = idx[r];
            if (t < 0 || t >= num_tokens) {
                Z[r * V + v] = NAN;
                continue;
            }
            double acc = 0.0;
            for (int64_t k = 0; k < H; ++k)
                acc += widen(hidden, hdt, t * hld + k) * widen(W, wdt, v * wld + k);
            Z[r * V + v] = acc;
        }
    }
}

/*
 * Head output scaling (vllm-metal release, Summary: some heads scale their
 * logits outside the projection, Cohere's logit_scale and Granite's
 * logits_scaling). Reading taken: mode 1 multiplies every logit by `value`,
 * mode 2 divides it by `value`, mode 0 leaves it; applied to the exact f64
 * logits in place.
 */
void orc_scale_logits(double* Z, int64_t n, int mode, double value) {
    if (mode == 1) {
        for (int64_t i = 0; i < n; ++i) Z[i] = Z[i] * value;
    } else if (mode == 2) {
        for (int64_t i = 0; i < n; ++i) Z[i] = Z[i] / value;
    }
}

/*
 * Quantised head weights (the pages' measured models are 4-bit MLX models:
 * mlxcel PR #1969, description). Reading taken for the format: MLX-style
 * affine groups -- for token v and hidden index k, with g = k / group,
 *     W[v][k] = scale[v][g] * q(v, k) + bias[v][g],
 * q(v, k) an unsigned `bits`-bit integer (bits 4 or 8) stored little-endian
 * in 32-bit words: word (k * bits) / 32 of row v, starting at bit
 * (k * bits) % 32. scale and bias are bf16, [V][groups] with row pitch
 * s_ld; q rows have pitch q_ld words. Output W64 is [V][H] f64, exact (a bf16
 * times a small integer plus a bf16 is exactly representable in f64).
 */
void orc_dequant(const uint32_t* q, int64_t q_ld, const uint16_t* scales, const uint16_t* biases,
                 int64_t s_ld, int bits, int group, int64_t V, int64_t H, double* W64) {
    const uint32_t mask = (bits == 32) ? 0xFFFFFFFFu : ((1u << bits) - 1u);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t k = 0; k < H; ++k) {
            const int64_t bit = k * bits;
            const uint32_t word = q[v * q_ld + bit / 32];
            const uint32_t qv = (word >> (bit % 32)) & mask;
            const int64_t g = k / group;
            W64[v * H + k] = widen(scales, ORC_BF16, v * s_ld + g) * (double)qv +
                             widen(biases, ORC_BF16, v * s_ld + g);
        }
    }
}

typedef struct {
    double x;
    int32_t id;
} orc_entry;

/* the total order of the top-K: larger value first; equal values (IEEE
 * equality, so -0 == +0 and -inf == -inf) by ascending token id */
static int orc_cmp(const void* pa, const void* pb) {
    const orc_entry* a = (const orc_entry*)pa;
    const orc_entry* b = (const orc_entry*)pb;
    if (a->x > b->x) return -1;
    if (a->x < b->x) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id ? 1 : 0);
}

/*
 * Per-row reduction (openinfer issue #719, Description and Suggested
 * direction; MTPLX PR #532, Change):
 *   m    = max_v x_v
 *   lse  = -inf if m == -inf, else m + log(sum_v exp(x_v - m)), summed in v order
 *   logprob(v) = x_v - lse
 *   selected   = logprob(sel[r])   (NaN if sel[r] is outside [0, V))
 *   top-K      = the first K ids after a full sort under orc_cmp, with
 *                their logprobs
 * logits is [rows][V] with row pitch ld, dtype dt. sel may be NULL (then
 * sel_lp is not written); K may be 0 (then topk_* are not touched).
 * Outputs: lse[rows], sel_lp[rows], topk_ids[rows][K], topk_lp[rows][K].
 * Inputs with +inf or NaN are outside the contract.
 */
void orc_reduce(const void* logits, int dt, int64_t rows, int64_t V, int64_t ld,
                const int32_t* sel, int32_t K,
                double* lse, double* sel_lp, int32_t* topk_ids, double* topk_lp) {
#pragma omp parallel
    {
        orc_entry* e = (K > 0) ? (orc_entry*)malloc(sizeof(orc_entry) * (size_t)V) : NULL;
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t base = r * ld;
            double m = -INFINITY;
            for (int64_t v = 0; v < V; ++v) {
                double x = widen(logits, dt, base + v);
                if (x > m) m = x;
            }
            double l;
            if (m == -INFINITY) {
                l = -INFINITY;
            } else {
                double s = 0.0;
                for (int64_t v = 0; v < V; ++v) s += exp(widen(logits, dt, base + v) - m);
                l = m + log(s);
            }
            lse[r] = l;
            if (sel != NULL && sel_lp != NULL) {
                int32_t t = sel[r];
                sel_lp[r] = (t < 0 || (int64_t)t >= V) ? NAN : widen(logits, dt, base + t) - l;
            }
            if (K > 0) {
                for (int64_t v = 0; v < V; ++v) {
                    e[v].x = widen(logits, dt, base + v);
                    e[v].id = (int32_t)v;
                }
                qsort(e, (size_t)V, sizeof(orc_entry), orc_cmp);
                for (int32_t i = 0; i < K; ++i) {
                    topk_ids[r * K + i] = e[i].id;
                    topk_lp[r * K + i] = e[i].x - l;
                }
            }
        }
        free(e);
    }
}

/*
 * Prefilter invariant checker (MTPLX PR #532, Change), test use only.
 *
 * For each row: view the row as nb = ceil(V / block) blocks (the last one
 * partial when block does not divide V; its maximum is over valid entries
 * only); order the blocks by (block max descending, block index ascending);
 * mark the first min(K, nb) of them. Let T be the max of the K-th marked
 * block when K <= nb (T = -inf when K > nb: then fewer than K maxima bound
 * the top-K from below). Then check that every one of the exact top-K ids
 * (orc_cmp order, full sort)
 *   (a) lies in a marked block, and
 *   (b) has a value >= T (the threshold filter),
 * and count the candidates that survive the threshold filter (entries of
 * marked blocks with value >= T).
 * block_ties_descending = 1 swaps the block tie-break to descending block
 * index, a deliberately wrong rule: tests use it to show that the ascending
 * rule is the one the invariant needs.
 * Returns the number of rows on which the invariant fails (0 = holds).
 * n_candidates (optional, [rows]) receives each row's candidate count.
 */
int64_t orc_prefilter_check(const void* logits, int dt, int64_t rows, int64_t V, int64_t ld,
                            int32_t K, int32_t block, int32_t block_ties_descending,
                            int64_t* n_candidates) {
    int64_t fails = 0;
    const int64_t nb = (V + block - 1) / block;
#pragma omp parallel reduction(+ : fails)
    {
        orc_entry* e = (orc_entry*)malloc(sizeof(orc_entry) * (size_t)(V > nb ? V : nb));
        orc_entry* bm = (orc_entry*)malloc(sizeof(orc_entry) * (size_t)nb);
        unsigned char* marked = (unsigned char*)malloc((size_t)nb);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t base = r * ld;
            for (int64_t b = 0; b < nb; ++b) {
                double mx = -INFINITY;
                int64_t hi = (b + 1) * block < V ? (b + 1) * block : V;
                for (int64_t v = b * block; v < hi; ++v) {
                    double x = widen(logits, dt, base + v);
                    if (x > mx) mx = x;
                }
                bm[b].x = mx;
                bm[b].id = block_ties_descending ? (int32_t)(nb - 1 - b) : (int32_t)b;
            }
            qsort(bm, (size_t)nb, sizeof(orc_entry), orc_cmp);
            memset(marked, 0, (size_t)nb);
            int64_t nsel = K < nb ? K : nb;
            for (int64_t i = 0; i < nsel; ++i)
                marked[block_ties_descending ? nb - 1 - bm[i].id : bm[i].id] = 1;
            /* the threshold needs K marked maxima: with K > nb there are
             * fewer, and every entry stays a candidate */
            double T = (K == 0) ? INFINITY : (K <= nb ? bm[K - 1].x : -INFINITY);

            int64_t cand = 0;
            for (int64_t v = 0; v < V; ++v) {
                double x = widen(logits, dt, base + v);
                if (marked[v / block] && x >= T) ++cand;
            }
            if (n_candidates) n_candidates[r] = cand;

            for (int64_t v = 0; v < V; ++v) {
                e[v].x = widen(logits, dt, base + v);
                e[v].id = (int32_t)v;
            }
            qsort(e, (size_t)V, sizeof(orc_entry), orc_cmp);
            int ok = 1;
            for (int32_t i = 0; i < K && i < V; ++i) {
                if (!marked[e[i].id / block]) ok = 0;
                if (!(e[i].x >= T)) ok = 0;
            }
            if (!ok) ++fails;
        }
        free(e);
        free(bm);
        free(marked);
    }
    return fails;
}

/* number of OpenMP threads the oracle will use (for reporting) */
int orc_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
