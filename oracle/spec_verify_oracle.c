/*
 * spec_verify_oracle.c -- plain CPU oracle for batched draft-token verification.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark load this file's library.  It shares no
 * code, header, table or helper with the HIP path, and the HIP path never
 * calls it.
 *
 * Everything here is written for a reader checking it against the pages by eye:
 * scalar loops, all arithmetic in double precision (fp64), one full softmax per
 * row, one left-to-right scan per request.  Nothing is blocked, fused or
 * reordered.
 *
 * Sources (page title, then section):
 *   [ANATOMY]  "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
 *              (bilingual copy), section "Speculative Decoding": the
 *              draft / verify / accept-reject steps and the residual and bonus
 *              rules.
 *   [BOOK]     "02. Speculative Decoding" (vLLM learning book), section 2
 *              "Algorithm (Leviathan 2023)" flowchart, and the FAQ entry on why
 *              a bonus token can be sampled when every draft is accepted.
 *   [TRTLLM]   "TensorRT-LLM source teardown (10): speculative decoding",
 *              section "Rejection sampling: an optional, stricter acceptance
 *              path" (output layout [batch, D+1] padded with -1, per-request
 *              length; target and draft must be filtered identically) and
 *              section "MTP mechanism background" (the "Generation phase 1"
 *              worked example: inputs E+FGH, target tokens FGXY, accepted FGX).
 *   [KESTREL]  "Kestrel_VLLM - 32: anchoring of a speculative round", section 2
 *              (acceptance: count leading drafts equal to the target argmax,
 *              emit the argmax at the first mismatch) and section 3.3 (every
 *              emitted token lies on the target's own argmax chain).
 *   [EAGLE]    "05 - TensorRT-LLM speculative decoding and auto-deploy",
 *              sections "Eagle-2 multi-level tree drafting" (the
 *              paths[batch, max_decoding_tokens, max_path_len] table) and
 *              "Target-model verification: tree attention and batched
 *              parallelism" (each tree token is compared against the target
 *              logits of its parent; the accepted branch is chosen).
 *
 * Readings where the pages leave a step open (all follow the plainest reading):
 *   - Row i of target_logits and row i of draft_logits are both distributions
 *     over draft token i (0-based); target row k is the bonus row.
 *   - The acceptance test is strict: accept iff P >= Q, otherwise iff u < P/Q.
 *     So Q == 0 always accepts.
 *   - uniforms[b, i] (i < k) drives test i; uniforms[b, k] drives the one final
 *     sample (residual or bonus).
 *   - Inverse-CDF sampling walks the vocabulary in ascending index order and
 *     picks the smallest j whose running sum exceeds u * Z.  If rounding leaves
 *     no such j, it takes the last j with positive weight.
 *   - If the residual mass is zero (p == q exactly at a rejected row, which a
 *     strict test with u < 1 cannot produce), it samples from p instead.
 *   - Temperature divides both target and draft logits.
 *   - Argmax uses the raw logits and takes the lowest index among equal maxima.
 *   - A draft token outside [0, V) is rejected (P and Q are reported as 0); a
 *     path entry outside [0, N] ends the path like -1.
 *
 * parity unpinned: none of the pages prints numeric logits or probabilities,
 * so exact probability values are pinned only by closed forms and by a library
 * softmax in the tests, never by a printed example.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types of the logits tensors (same integer meaning as the library's
 * public enum; written out again here, not shared). */
#define ORACLE_DTYPE_F32 0
#define ORACLE_DTYPE_BF16 1

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARGUMENT 1
#define ORACLE_NO_MEMORY 2

/* One logit as a double.  bf16 is the top half of an IEEE fp32 word, so the
 * conversion is exact. */
static double logit_at(const void *base, int dtype, size_t index)
{
    if (dtype == ORACLE_DTYPE_F32)
        return (double)((const float *)base)[index];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[index] << 16;
    float value;
    memcpy(&value, &bits, sizeof value);
    return (double)value;
}

/* probs[j] = softmax(row / temperature)[j], in fp64, subtracting the row
 * maximum first.  A logit of -inf gets probability exactly 0.
 * [ANATOMY] "Speculative Decoding": the verifier turns each of the k+1 target
 * rows (and each draft row) into a probability distribution.  [TRTLLM]
 * "Rejection sampling": temperature is applied identically to both sides. */
static void softmax_row(const void *logits, int dtype, size_t row_offset, int V,
                        double temperature, double *probs)
{
    double zmax = -INFINITY;
    for (int j = 0; j < V; ++j) {
        double z = logit_at(logits, dtype, row_offset + (size_t)j) / temperature;
        probs[j] = z;
        if (z > zmax)
            zmax = z;
    }
    double total = 0.0;
    for (int j = 0; j < V; ++j) {
        probs[j] = exp(probs[j] - zmax);
        total += probs[j];
    }
    for (int j = 0; j < V; ++j)
        probs[j] /= total;
}

/* Inverse-CDF draw from the unnormalised weights w[0..V-1] with the uniform u:
 * the smallest j with w[0] + ... + w[j] > u * Z, Z = sum of all weights.
 * *margin receives the distance from u * Z to the nearer edge of the chosen
 * token's CDF interval, divided by Z.
 * [ANATOMY] "Speculative Decoding": normalise the weights to sum to 1 and
 * sample one token from them. */
static int32_t inverse_cdf(const double *w, int V, double u, double *margin)
{
    double Z = 0.0;
    for (int j = 0; j < V; ++j)
        Z += w[j];
    double target = u * Z;
    double below = 0.0; /* running sum before token j */
    for (int j = 0; j < V; ++j) {
        double above = below + w[j];
        if (above > target) {
            double lo = target - below;
            double hi = above - target;
            *margin = (lo < hi ? lo : hi) / Z;
            return (int32_t)j;
        }
        below = above;
    }
    /* Rounding left u * Z at or past the total: the last positive weight. */
    *margin = 0.0;
    for (int j = V - 1; j >= 0; --j)
        if (w[j] > 0.0)
            return (int32_t)j;
    return 0;
}

/*
 * Symmetric filtering of a row's distribution ([TRTLLM] "Rejection sampling":
 * the sampling filters -- temperature, top-k, top-p, min_p -- must be applied
 * to the target and the draft side identically).  The pages name the filters
 * but do not define them; readings (standard definitions, all thresholds on
 * the raw logit x, which orders tokens exactly as p does):
 *   top-k (0 < top_k < V): keep x >= the top_k-th largest logit, counting
 *         repeated values (every token tied with it is kept);
 *   top-p (0 < top_p < 1): among the top-k survivors, in descending logit
 *         order, keep the smallest run of distinct logit values whose mass
 *         reaches top_p times the survivors' mass (ties kept);
 *   min_p (0 < min_p <= 1): keep p >= min_p * max p, i.e.
 *         x >= max x + T * ln(min_p);
 * applied in this order; the kept tokens' probabilities are renormalised and
 * every other token gets probability 0.
 */
struct oracle_filter {
    int top_k;
    double top_p;
    double min_p;
};

static int cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

/* probs[] (the row's softmax) is filtered in place.  *margin receives how far
 * the top-p decision was from flipping (distance of the target mass to the
 * nearer cumulative edge, relative to the survivors' mass) and how close any
 * logit lies to the min_p threshold (absolute, in logit units); +inf when
 * neither filter is active. */
static void filter_row(const void *logits, int dtype, size_t row_offset, int V,
                       double temperature, const struct oracle_filter *f, double *probs,
                       double *scratch, double *margin)
{
    *margin = INFINITY;
    double thr = -INFINITY;
    double xmax = -INFINITY;
    for (int j = 0; j < V; ++j) {
        double x = logit_at(logits, dtype, row_offset + (size_t)j);
        scratch[j] = x;
        if (x > xmax)
            xmax = x;
    }
    qsort(scratch, (size_t)V, sizeof(double), cmp_desc);
    if (f->top_k > 0 && f->top_k < V)
        thr = scratch[f->top_k - 1];
    if (f->top_p > 0.0 && f->top_p < 1.0) {
        double mass1 = 0.0;
        for (int j = 0; j < V; ++j)
            if (logit_at(logits, dtype, row_offset + (size_t)j) >= thr)
                mass1 += probs[j];
        double target = f->top_p * mass1;
        /* walk the distinct survivor values in descending order */
        double cum = 0.0;
        int g = 0;
        while (g < V && scratch[g] >= thr) {
            double value = scratch[g];
            double group = 0.0;
            for (int j = 0; j < V; ++j)
                if (logit_at(logits, dtype, row_offset + (size_t)j) == value)
                    group += probs[j];
            double before = cum;
            cum += group;
            if (cum >= target) {
                double lo = target - before, hi = cum - target;
                double m = (lo < hi ? lo : hi) / mass1;
                if (m < *margin)
                    *margin = m;
                thr = value;
                break;
            }
            while (g < V && scratch[g] == value)
                ++g;
        }
    }
    if (f->min_p > 0.0) {
        double tmin = xmax + temperature * log(f->min_p);
        for (int j = 0; j < V; ++j) {
            double d = fabs(logit_at(logits, dtype, row_offset + (size_t)j) - tmin);
            if (d < *margin)
                *margin = d;
        }
        if (tmin > thr)
            thr = tmin;
    }
    if (thr == -INFINITY)
        return;
    double total = 0.0;
    for (int j = 0; j < V; ++j) {
        if (logit_at(logits, dtype, row_offset + (size_t)j) < thr)
            probs[j] = 0.0;
        total += probs[j];
    }
    for (int j = 0; j < V; ++j)
        probs[j] /= total;
}

/*
 * Stochastic verification of B linear drafts of length k.
 *
 *   target_logits [B, k+1, V]  (dtype)   draft_logits [B, k, V] (dtype)
 *   draft_tokens  [B, k] int32           uniforms [B, k+1] fp32
 *   out_tokens    [B, k+1] int32: accepted drafts, then the correction or bonus
 *                 token, then -1 padding        ([TRTLLM] "Rejection sampling")
 *   num_accepted  [B] int32: number of accepted draft tokens
 *   p_at_draft, q_at_draft [B, k] (may be NULL): p_i(x_i) and q_i(x_i), fp64
 *   margins [B, k+1] (may be NULL): for each decision actually taken, its
 *           distance from the decision boundary (test i: |u - min(1, P/Q)|;
 *           final sample: see inverse_cdf); +inf where no decision was taken.
 *
 * The steps follow [ANATOMY] "Speculative Decoding" and the [BOOK] section 2
 * flowchart, in their order:
 *   1. for i = 0, 1, ..., k-1 (left to right): with x = draft token i,
 *      P = p_i(x), Q = q_i(x): accept when P >= Q; otherwise accept when
 *      u_i < P / Q.  Stop at the first rejection.
 *   2. rejected at row s: sample from max(0, p_s - q_s), normalised;
 *      all k accepted: sample the bonus token from p_k ([BOOK] FAQ 2).
 */
static int verify_stochastic(const void *target_logits, const void *draft_logits, int dtype,
                             const int32_t *draft_tokens, const float *uniforms,
                             double temperature, int B, int k, int V,
                             int32_t *out_tokens, int32_t *num_accepted,
                             double *p_at_draft, double *q_at_draft, double *margins,
                             const struct oracle_filter *filter, double *filter_margins);

int oracle_verify_stochastic(const void *target_logits, const void *draft_logits, int dtype,
                             const int32_t *draft_tokens, const float *uniforms,
                             double temperature, int B, int k, int V,
                             int32_t *out_tokens, int32_t *num_accepted,
                             double *p_at_draft, double *q_at_draft, double *margins)
{
    return verify_stochastic(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                             temperature, B, k, V, out_tokens, num_accepted, p_at_draft,
                             q_at_draft, margins, NULL, NULL);
}

/*
 * Stochastic verification with every target and draft row filtered
 * (filter_row) before the tests and the final draw.  top_k = 0, top_p = 1 and
 * min_p = 0 switch the respective filter off.  filter_margins [B] (may be
 * NULL): the smallest filter margin over the request's rows.
 */
int oracle_verify_stochastic_filtered(const void *target_logits, const void *draft_logits,
                                      int dtype, const int32_t *draft_tokens,
                                      const float *uniforms, double temperature, int top_k,
                                      double top_p, double min_p, int B, int k, int V,
                                      int32_t *out_tokens, int32_t *num_accepted,
                                      double *p_at_draft, double *q_at_draft, double *margins,
                                      double *filter_margins)
{
    if (top_k < 0 || !(top_p > 0.0) || top_p > 1.0 || !(min_p >= 0.0) || min_p > 1.0)
        return ORACLE_BAD_ARGUMENT;
    struct oracle_filter f = {top_k, top_p, min_p};
    return verify_stochastic(target_logits, draft_logits, dtype, draft_tokens, uniforms,
                             temperature, B, k, V, out_tokens, num_accepted, p_at_draft,
                             q_at_draft, margins, &f, filter_margins);
}

static int verify_stochastic(const void *target_logits, const void *draft_logits, int dtype,
                             const int32_t *draft_tokens, const float *uniforms,
                             double temperature, int B, int k, int V,
                             int32_t *out_tokens, int32_t *num_accepted,
                             double *p_at_draft, double *q_at_draft, double *margins,
                             const struct oracle_filter *filter, double *filter_margins)
{
    if (B < 0 || k < 0 || V < 1 || !(temperature > 0.0) || isinf(temperature))
        return ORACLE_BAD_ARGUMENT;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_BAD_ARGUMENT;
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    double *scratch = (double *)malloc(sizeof(double) * (size_t)V);
    if (!p || !q || !w || !scratch) {
        free(p);
        free(q);
        free(w);
        free(scratch);
        return ORACLE_NO_MEMORY;
    }
    double fmargin;
/* One row's distribution: softmax, then the filter when there is one. */
#define ROW_DIST(logits, offset, out)                                                   \
    do {                                                                                \
        softmax_row((logits), dtype, (offset), V, temperature, (out));                  \
        if (filter) {                                                                   \
            filter_row((logits), dtype, (offset), V, temperature, filter, (out), scratch, \
                       &fmargin);                                                       \
            if (fmargin < request_fmargin)                                              \
                request_fmargin = fmargin;                                              \
        }                                                                               \
    } while (0)

    for (int b = 0; b < B; ++b) {
        const int32_t *x = draft_tokens + (size_t)b * k;
        const float *u = uniforms + (size_t)b * (k + 1);
        int32_t *out = out_tokens + (size_t)b * (k + 1);
        double *margin = margins ? margins + (size_t)b * (k + 1) : NULL;
        double request_fmargin = INFINITY;
        if (margin)
            for (int i = 0; i <= k; ++i)
                margin[i] = INFINITY;

        /* Step 1: left-to-right accept/reject, stop at the first rejection. */
        int s = k;
        for (int i = 0; i < k; ++i) {
            size_t t_row = ((size_t)b * (k + 1) + i) * (size_t)V;
            size_t d_row = ((size_t)b * k + i) * (size_t)V;
            ROW_DIST(target_logits, t_row, p);
            ROW_DIST(draft_logits, d_row, q);
            int in_range = x[i] >= 0 && x[i] < V;
            double P = in_range ? p[x[i]] : 0.0;
            double Q = in_range ? q[x[i]] : 0.0;
            if (p_at_draft)
                p_at_draft[(size_t)b * k + i] = P;
            if (q_at_draft)
                q_at_draft[(size_t)b * k + i] = Q;

            int accepted;
            if (!in_range)
                accepted = 0;
            else if (P >= Q)
                accepted = 1;
            else
                accepted = (double)u[i] < P / Q;
            if (margin) {
                double threshold = (P >= Q) ? 1.0 : P / Q;
                margin[i] = in_range ? fabs((double)u[i] - threshold) : INFINITY;
            }
            if (!accepted) {
                s = i;
                break;
            }
        }
        /* Remaining p_at_draft / q_at_draft entries (after the stop row) are
         * still defined: they are the same per-row probabilities. */
        for (int i = s + 1; i < k; ++i) {
            size_t t_row = ((size_t)b * (k + 1) + i) * (size_t)V;
            size_t d_row = ((size_t)b * k + i) * (size_t)V;
            int in_range = x[i] >= 0 && x[i] < V;
            if (p_at_draft) {
                ROW_DIST(target_logits, t_row, p);
                p_at_draft[(size_t)b * k + i] = in_range ? p[x[i]] : 0.0;
            }
            if (q_at_draft) {
                ROW_DIST(draft_logits, d_row, q);
                q_at_draft[(size_t)b * k + i] = in_range ? q[x[i]] : 0.0;
            }
        }

        /* Step 2: the one final token. */
        ROW_DIST(target_logits, ((size_t)b * (k + 1) + s) * (size_t)V, p);
        if (s < k) {
            ROW_DIST(draft_logits, ((size_t)b * k + s) * (size_t)V, q);
            double Z = 0.0;
            for (int j = 0; j < V; ++j) {
                double d = p[j] - q[j];
                w[j] = d > 0.0 ? d : 0.0;
                Z += w[j];
            }
            if (!(Z > 0.0)) /* p_s == q_s: sample from p_s */
                memcpy(w, p, sizeof(double) * (size_t)V);
        } else {
            memcpy(w, p, sizeof(double) * (size_t)V);
        }
        double final_margin;
        int32_t token = inverse_cdf(w, V, (double)u[k], &final_margin);
        if (margin)
            margin[k] = final_margin;

        for (int i = 0; i < s; ++i)
            out[i] = x[i];
        out[s] = token;
        for (int i = s + 1; i <= k; ++i)
            out[i] = -1;
        num_accepted[b] = s;
        if (filter_margins)
            filter_margins[b] = request_fmargin;
    }
#undef ROW_DIST
    free(p);
    free(q);
    free(w);
    free(scratch);
    return ORACLE_OK;
}

/* Bytes of one logit of `dtype`. */
static size_t elem_bytes(int dtype)
{
    return dtype == ORACLE_DTYPE_BF16 ? 2 : 4;
}

/* Draft length of request b under the ragged layout: draft_lens[b] clamped to
 * [0, k] (k when draft_lens is NULL). */
static int ragged_len(const int32_t *draft_lens, int b, int k)
{
    if (!draft_lens)
        return k;
    int kb = draft_lens[b];
    return kb < 0 ? 0 : (kb > k ? k : kb);
}

/*
 * Stochastic verification with per-request draft lengths ([TRTLLM] section on
 * the acceptance pipeline, step 2: ragged verification, where each request is
 * verified over its own window while buffers stay padded to the static
 * maximum k).  Request b uses only its first k_b = draft_lens[b] drafts
 * (clamped to [0, k]): it is verified exactly as a request of length k_b on
 * its own -- target rows 0..k_b, draft rows 0..k_b-1, uniforms[b, 0..k_b-1]
 * for the tests and uniforms[b, k_b] for the final token.  Layouts stay padded
 * to k: out_tokens[b, k_b+1..k] = -1, p/q_at_draft[b, k_b..k-1] = 0 and
 * margins[b, k_b+1..k] = +inf.
 */
int oracle_verify_stochastic_ragged(const void *target_logits, const void *draft_logits,
                                    int dtype, const int32_t *draft_tokens,
                                    const int32_t *draft_lens, const float *uniforms,
                                    double temperature, int B, int k, int V,
                                    int32_t *out_tokens, int32_t *num_accepted,
                                    double *p_at_draft, double *q_at_draft, double *margins)
{
    if (B < 0 || k < 0 || V < 1)
        return ORACLE_BAD_ARGUMENT;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_BAD_ARGUMENT;
    const size_t eb = elem_bytes(dtype);
    int32_t *out1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k + 1));
    double *p1 = (double *)malloc(sizeof(double) * (size_t)(k + 1));
    double *q1 = (double *)malloc(sizeof(double) * (size_t)(k + 1));
    double *m1 = (double *)malloc(sizeof(double) * (size_t)(k + 1));
    if (!out1 || !p1 || !q1 || !m1) {
        free(out1);
        free(p1);
        free(q1);
        free(m1);
        return ORACLE_NO_MEMORY;
    }
    int rc = ORACLE_OK;
    for (int b = 0; b < B && rc == ORACLE_OK; ++b) {
        const int kb = ragged_len(draft_lens, b, k);
        const char *t = (const char *)target_logits + eb * (size_t)b * (k + 1) * (size_t)V;
        const char *d = draft_logits
            ? (const char *)draft_logits + eb * (size_t)b * k * (size_t)V : NULL;
        int32_t acc;
        rc = oracle_verify_stochastic(t, d, dtype, draft_tokens + (size_t)b * k,
                                      uniforms + (size_t)b * (k + 1), temperature, 1, kb, V,
                                      out1, &acc, p1, q1, m1);
        for (int i = 0; i <= k; ++i) {
            out_tokens[(size_t)b * (k + 1) + i] = i <= kb ? out1[i] : -1;
            if (margins)
                margins[(size_t)b * (k + 1) + i] = i <= kb ? m1[i] : INFINITY;
        }
        for (int i = 0; i < k; ++i) {
            if (p_at_draft)
                p_at_draft[(size_t)b * k + i] = i < kb ? p1[i] : 0.0;
            if (q_at_draft)
                q_at_draft[(size_t)b * k + i] = i < kb ? q1[i] : 0.0;
        }
        num_accepted[b] = acc;
    }
    free(out1);
    free(p1);
    free(q1);
    free(m1);
    return rc;
}

/*
 * Counter-based uniforms.  [TRTLLM] "Rejection sampling" draws its uniforms
 * from Philox with a per-call (seed, offset) instead of taking them as an
 * input.  Generator: Philox4x64-10 as published by Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): ten rounds of
 * two 64x64->128-bit multiplications by fixed odd constants, the high halves
 * XORed with the other two counter words and the key, the key advanced by two
 * Weyl constants between rounds.
 * Reading (the pages fix no layout): the uniform of request b, draw i comes
 * from the block at counter (offset, b, i / 4, 0) with key (seed, 0), word
 * i % 4, as (word >> 40) * 2^-24 (24 random bits: exact in float32, in
 * [0, 1)).  Draws i = 0..k-1 drive the tests, draw k (k_b with ragged lengths)
 * the final token, exactly like the uniforms[b, i] input of the other calls.
 */
static void philox_round(uint64_t ctr[4], const uint64_t key[2])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    unsigned __int128 p0 = (unsigned __int128)M0 * ctr[0];
    unsigned __int128 p1 = (unsigned __int128)M1 * ctr[2];
    uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    uint64_t c1 = ctr[1], c3 = ctr[3];
    ctr[0] = hi1 ^ c1 ^ key[0];
    ctr[1] = lo1;
    ctr[2] = hi0 ^ c3 ^ key[1];
    ctr[3] = lo0;
}

void oracle_philox4x64_10(const uint64_t counter[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c[4] = {counter[0], counter[1], counter[2], counter[3]};
    uint64_t k[2] = {key[0], key[1]};
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k[0] += W0;
            k[1] += W1;
        }
        philox_round(c, k);
    }
    for (int i = 0; i < 4; ++i)
        out[i] = c[i];
}

/* uniforms[b, i] for b < B, i < n under the layout above. */
void oracle_philox_uniforms(uint64_t seed, uint64_t offset, int B, int n, float *uniforms)
{
    const uint64_t key[2] = {seed, 0};
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < n; ++i) {
            const uint64_t ctr[4] = {offset, (uint64_t)b, (uint64_t)(i / 4), 0};
            uint64_t block[4];
            oracle_philox4x64_10(ctr, key, block);
            uniforms[(size_t)b * n + i] = (float)((double)(block[i % 4] >> 40) * 0x1p-24);
        }
}

/* Index of the largest raw logit of one row; the lowest index wins a tie. */
static int32_t argmax_row(const void *logits, int dtype, size_t row_offset, int V)
{
    int32_t best = 0;
    double best_value = logit_at(logits, dtype, row_offset);
    for (int j = 1; j < V; ++j) {
        double v = logit_at(logits, dtype, row_offset + (size_t)j);
        if (v > best_value) {
            best_value = v;
            best = (int32_t)j;
        }
    }
    return best;
}

/*
 * Greedy verification ([KESTREL] section 2, acceptance and emit steps;
 * section 3.3): a_i = argmax of target row i for i = 0..k; the accepted count
 * s is the number of leading draft tokens equal to a_0, a_1, ...; the output is
 * draft[0..s-1], then a_s, then -1 padding.  When s == 0 the only token is
 * a_0 (no row before 0 is ever read).
 *   argmax_out [B, k+1] (may be NULL) receives every a_i.
 */
int oracle_verify_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens,
                         int B, int k, int V, int32_t *out_tokens, int32_t *num_accepted,
                         int32_t *argmax_out)
{
    if (B < 0 || k < 0 || V < 1)
        return ORACLE_BAD_ARGUMENT;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_BAD_ARGUMENT;
    for (int b = 0; b < B; ++b) {
        const int32_t *x = draft_tokens + (size_t)b * k;
        int32_t *out = out_tokens + (size_t)b * (k + 1);
        int32_t a[1024 + 1];
        int32_t *arg = (k + 1 <= 1025) ? a : (int32_t *)malloc(sizeof(int32_t) * (size_t)(k + 1));
        if (!arg)
            return ORACLE_NO_MEMORY;
        for (int i = 0; i <= k; ++i)
            arg[i] = argmax_row(target_logits, dtype, ((size_t)b * (k + 1) + i) * (size_t)V, V);
        int s = 0;
        while (s < k && x[s] == arg[s])
            ++s;
        for (int i = 0; i < s; ++i)
            out[i] = x[i];
        out[s] = arg[s];
        for (int i = s + 1; i <= k; ++i)
            out[i] = -1;
        num_accepted[b] = s;
        if (argmax_out)
            memcpy(argmax_out + (size_t)b * (k + 1), arg, sizeof(int32_t) * (size_t)(k + 1));
        if (arg != a)
            free(arg);
    }
    return ORACLE_OK;
}

/*
 * Greedy verification with per-request draft lengths (same reading as
 * oracle_verify_stochastic_ragged): request b is verified as a request of
 * length k_b = draft_lens[b] (clamped to [0, k]) on its own, target rows
 * 0..k_b; out_tokens[b, k_b+1..k] = -1.  argmax_out[b, i] for i > k_b is -1.
 */
int oracle_verify_greedy_ragged(const void *target_logits, int dtype,
                                const int32_t *draft_tokens, const int32_t *draft_lens, int B,
                                int k, int V, int32_t *out_tokens, int32_t *num_accepted,
                                int32_t *argmax_out)
{
    if (B < 0 || k < 0 || V < 1)
        return ORACLE_BAD_ARGUMENT;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_BAD_ARGUMENT;
    const size_t eb = elem_bytes(dtype);
    int32_t *out1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k + 1));
    int32_t *arg1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k + 1));
    if (!out1 || !arg1) {
        free(out1);
        free(arg1);
        return ORACLE_NO_MEMORY;
    }
    int rc = ORACLE_OK;
    for (int b = 0; b < B && rc == ORACLE_OK; ++b) {
        const int kb = ragged_len(draft_lens, b, k);
        const char *t = (const char *)target_logits + eb * (size_t)b * (k + 1) * (size_t)V;
        int32_t acc;
        rc = oracle_verify_greedy(t, dtype, draft_tokens + (size_t)b * k, 1, kb, V, out1, &acc,
                                  arg1);
        for (int i = 0; i <= k; ++i) {
            out_tokens[(size_t)b * (k + 1) + i] = i <= kb ? out1[i] : -1;
            if (argmax_out)
                argmax_out[(size_t)b * (k + 1) + i] = i <= kb ? arg1[i] : -1;
        }
        num_accepted[b] = acc;
    }
    free(out1);
    free(arg1);
    return rc;
}

/*
 * Tree (EAGLE-style) greedy verification ([EAGLE] both sections named above).
 *
 *   target_logits [B, N+1, V]: row n holds the target's distribution after
 *                 tree node n (node 0 is the root, the last committed token).
 *   node_tokens   [B, N+1] int32: the draft token at each node; [b, 0] unused.
 *   paths         [B, P, L] int32: each row lists node indices from the root
 *                 down one branch, padded with -1; a row whose first entry is
 *                 not a node index is unused.
 *   out_tokens    [B, L]: tokens of the accepted nodes, then the argmax at the
 *                 last accepted node, then -1 padding.
 *   num_accepted  [B]: accepted node count.
 *   best_path     [B] (may be NULL): the chosen path row, -1 if none is used.
 *   accepted_nodes [B, L] (may be NULL): the accepted node indices, -1 padded.
 *
 * A node is accepted when its token equals the argmax of its parent's row, and
 * a path's accepted length m is the number of nodes accepted in a row from the
 * root.  The chosen path has the largest m; among equal m the lowest row index.
 */
int oracle_verify_tree(const void *target_logits, int dtype, const int32_t *node_tokens,
                       const int32_t *paths, int B, int N, int P, int L, int V,
                       int32_t *out_tokens, int32_t *num_accepted, int32_t *best_path,
                       int32_t *accepted_nodes)
{
    if (B < 0 || N < 0 || P < 0 || L < 1 || V < 1)
        return ORACLE_BAD_ARGUMENT;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_BAD_ARGUMENT;
    int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N + 1));
    if (!a)
        return ORACLE_NO_MEMORY;
    for (int b = 0; b < B; ++b) {
        for (int n = 0; n <= N; ++n)
            a[n] = argmax_row(target_logits, dtype, ((size_t)b * (N + 1) + n) * (size_t)V, V);
        const int32_t *tok = node_tokens + (size_t)b * (N + 1);

        int best = -1, best_m = -1;
        for (int p = 0; p < P; ++p) {
            const int32_t *row = paths + ((size_t)b * P + p) * (size_t)L;
            if (row[0] < 0 || row[0] > N)
                continue; /* unused row */
            int m = 0;
            while (m + 1 < L) {
                int32_t child = row[m + 1];
                if (child < 0 || child > N)
                    break;
                if (tok[child] != a[row[m]])
                    break;
                ++m;
            }
            if (m > best_m) { /* strictly longer: lower rows win ties */
                best_m = m;
                best = p;
            }
        }

        int32_t *out = out_tokens + (size_t)b * L;
        int32_t *nodes = accepted_nodes ? accepted_nodes + (size_t)b * L : NULL;
        for (int t = 0; t < L; ++t) {
            out[t] = -1;
            if (nodes)
                nodes[t] = -1;
        }
        if (best < 0) { /* no usable path: the tree is the root alone */
            out[0] = a[0];
            num_accepted[b] = 0;
        } else {
            const int32_t *row = paths + ((size_t)b * P + best) * (size_t)L;
            for (int t = 1; t <= best_m; ++t) {
                out[t - 1] = tok[row[t]];
                if (nodes)
                    nodes[t - 1] = row[t];
            }
            out[best_m] = a[row[best_m]];
            num_accepted[b] = best_m;
        }
        if (best_path)
            best_path[b] = best;
    }
    free(a);
    return ORACLE_OK;
}

/*
 * Stochastic tree verification.
 *
 * The pages verify a draft tree against the target's rows in one pass by
 * "rejection sampling" ([EAGLE] "Target-model verification: tree attention and
 * batched parallelism"; the paths tensor [batch, max_decoding_tokens,
 * max_path_len] of "Eagle-2 multi-level tree drafting") without stating the
 * rule for several candidate children.  Reading: the linear rule of verify_stochastic
 * applied to the children of each accepted node in turn, in the form of
 * multi-candidate speculative sampling (SpecInfer, Miao et al., ASPLOS 2024):
 *
 *   target_logits [B, N+1, V]: row n is the target distribution after node n
 *                 (node 0 is the root, the last committed token).
 *   draft_logits  [B, N+1, V]: row n is the draft distribution that node n's
 *                 children were drawn from (rows of leaves are not read).
 *   node_tokens [B, N+1]: node n's token ([b, 0] ignored).
 *   paths [B, P, L]: node indices root-first, -1 padded; node paths[t] is a
 *                 child of node paths[t-1] (the first row that names a node
 *                 fixes its parent); rows whose first entry is not in [0, N]
 *                 are unused, and an entry outside [0, N] ends a row.
 *   uniforms [B, N+1]: uniforms[b, c-1] drives the test of node c (c >= 1);
 *                 uniforms[b, N] drives the final draw.
 *
 *   n = 0; p = softmax(target row n / T); q = softmax(draft row n / T).
 *   For each child c of n, in ascending node order: with x = token of c,
 *   P = p(x), Q = q(x): accept when P >= Q or u * Q < P, and reject an x
 *   outside [0, V) (as verify_stochastic does).  On acceptance: n = c and start again one level down.
 *   On rejection: p = max(0, p - q) renormalised (left as it is if that mass is
 *   0), and the next child is tried against it.  When no child of n is
 *   accepted (or n has none), the final token is drawn from p by inverse CDF
 *   with uniforms[b, N].
 *
 *   out_tokens [B, L]: the accepted nodes' tokens, the final token, then -1.
 *   num_accepted [B]: accepted nodes.  accepted_nodes [B, L]: their indices,
 *   then -1.  margins [B, N+1] (may be NULL): for each test taken, |u - t|
 *   with t = min(1, P/Q) (as verify_stochastic; +inf for an id outside the
 *   vocabulary and for tests not taken), and the final draw's margin
 *   (inverse_cdf) at index N.
 *
 * A tree that is a single chain 0 -> 1 -> ... -> k is verify_stochastic with
 * k drafts (draft row i of the linear call = row i here).
 */
int oracle_verify_tree_stochastic(const void *target_logits, const void *draft_logits, int dtype,
                                  const int32_t *node_tokens, const int32_t *paths,
                                  const float *uniforms, double temperature, int B, int N, int P,
                                  int L, int V, int32_t *out_tokens, int32_t *num_accepted,
                                  int32_t *accepted_nodes, double *margins)
{
    if (B < 0 || N < 0 || P < 0 || L < 1 || V < 1 || !(temperature > 0.0) || isinf(temperature))
        return ORACLE_BAD_ARGUMENT;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return ORACLE_BAD_ARGUMENT;
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    int32_t *parent = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N + 1));
    if (!p || !q || !w || !parent) {
        free(p);
        free(q);
        free(w);
        free(parent);
        return ORACLE_NO_MEMORY;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *tok = node_tokens + (size_t)b * (N + 1);
        const float *u = uniforms + (size_t)b * (N + 1);
        double *margin = margins ? margins + (size_t)b * (N + 1) : NULL;
        if (margin)
            for (int i = 0; i <= N; ++i)
                margin[i] = INFINITY;
        for (int n = 0; n <= N; ++n)
            parent[n] = -1;
        for (int r = 0; r < P; ++r) {
            const int32_t *row = paths + ((size_t)b * P + r) * (size_t)L;
            if (row[0] < 0 || row[0] > N)
                continue;
            for (int t = 1; t < L; ++t) {
                int32_t c = row[t];
                if (c < 0 || c > N)
                    break;
                if (c != 0 && parent[c] < 0)
                    parent[c] = row[t - 1];
            }
        }

        int32_t *out = out_tokens + (size_t)b * L;
        int32_t *nodes = accepted_nodes ? accepted_nodes + (size_t)b * L : NULL;
        for (int t = 0; t < L; ++t) {
            out[t] = -1;
            if (nodes)
                nodes[t] = -1;
        }
        int n = 0, depth = 0;
        for (;;) {
            softmax_row(target_logits, dtype, ((size_t)b * (N + 1) + n) * (size_t)V, V,
                        temperature, p);
            int has_child = 0;
            for (int c = 1; c <= N; ++c)
                if (parent[c] == n)
                    has_child = 1;
            if (has_child)
                softmax_row(draft_logits, dtype, ((size_t)b * (N + 1) + n) * (size_t)V, V,
                            temperature, q);
            int next = -1, rejected = 0;
            for (int c = 1; c <= N && next < 0 && depth + 1 < L; ++c) {
                if (parent[c] != n)
                    continue;
                int32_t x = tok[c];
                int in_range = x >= 0 && x < V;
                double P_ = in_range ? p[x] : 0.0;
                double Q_ = in_range ? q[x] : 0.0;
                int accepted;
                if (!in_range)
                    accepted = 0; /* an id outside the vocabulary is rejected */
                else if (P_ >= Q_)
                    accepted = 1;
                else
                    accepted = (double)u[c - 1] < P_ / Q_;
                if (margin) {
                    double threshold = (P_ >= Q_) ? 1.0 : P_ / Q_;
                    margin[c - 1] = in_range ? fabs((double)u[c - 1] - threshold) : INFINITY;
                }
                if (accepted) {
                    next = c;
                    break;
                }
                /* w: the residual, kept unnormalised for the final draw (as
                 * verify_stochastic draws from it); p: its normalised form for
                 * the next sibling's test. */
                double Z = 0.0;
                for (int j = 0; j < V; ++j) {
                    const double excess = p[j] - q[j];
                    w[j] = excess > 0.0 ? excess : 0.0;
                    Z += w[j];
                }
                if (Z > 0.0)
                    for (int j = 0; j < V; ++j)
                        p[j] = w[j] / Z;
                else
                    memcpy(w, p, sizeof(double) * (size_t)V);
                rejected = 1;
            }
            if (next < 0) {
                double final_margin;
                out[depth] = inverse_cdf(rejected ? w : p, V, (double)u[N], &final_margin);
                if (margin)
                    margin[N] = final_margin;
                break;
            }
            out[depth] = tok[next];
            if (nodes)
                nodes[depth] = next;
            ++depth;
            n = next;
        }
        num_accepted[b] = depth;
    }
    free(p);
    free(q);
    free(w);
    free(parent);
    return ORACLE_OK;
}
