/*
 * spec_verify.h -- C ABI of the batched draft-token verification library
 * (speculative decoding) for AMD Instinct MI355X (gfx950).
 *
 * Three verification calls, one per mode, plus sizing and status helpers.
 * Every pointer argument named *_logits, *_tokens, uniforms, paths, out_*,
 * num_accepted, best_path, accepted_nodes, p_at_draft, q_at_draft and
 * workspace is a DEVICE pointer owned by the caller.  The library never
 * allocates, frees or synchronises; it never reads device data on the host.
 * Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 * default stream); outputs are valid once the stream has reached that point.
 * Inputs are never modified.  Shapes are plain integers, layouts are dense and
 * row-major with the vocabulary innermost.
 *
 * Errors are fail-closed: every argument is checked on the host before any
 * launch; on an error nothing is launched and no output is touched.
 *
 * Data preconditions (documented, not checked on the device): logits hold no
 * NaN and each row has at least one finite value (-inf is allowed); uniforms lie
 * in [0, 1).  Out-of-range ids are tolerated with a defined result: a draft
 * token outside [0, V) is rejected (stochastic) or never matches (greedy); a
 * path entry outside [0, N] ends that path like -1.
 *
 * Sources (page title, section):
 *   "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
 *     "Speculative Decoding" -- the accept / reject / residual / bonus rules.
 *   "02. Speculative Decoding" (vLLM learning book), section 2 flowchart -- the
 *     test r < min(1, p(x_i) / q(x_i)) and the residual (p - q)+ / Z.
 *   "TensorRT-LLM source teardown (10): speculative decoding", "Rejection
 *     sampling" -- accepted_tokens [batch, D+1] (accepted drafts, correction or
 *     bonus token, then -1 padding) plus a per-request count; host-side
 *     fail-closed shape guards that never read device values.
 *   "Kestrel_VLLM - 32", section 2 -- greedy acceptance by argmax match.
 *   "05 - TensorRT-LLM speculative decoding and auto-deploy", "Eagle-2
 *     multi-level tree drafting" -- paths[batch, max_decoding_tokens,
 *     max_path_len].
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stable integer enums: values are never renumbered. */
enum spec_verify_dtype {
    SPEC_VERIFY_F32 = 0,  /* IEEE binary32 logits */
    SPEC_VERIFY_BF16 = 1  /* bfloat16 logits (upper half of a binary32) */
};

enum spec_verify_mode {
    SPEC_VERIFY_MODE_STOCHASTIC = 0,
    SPEC_VERIFY_MODE_GREEDY = 1,
    SPEC_VERIFY_MODE_TREE = 2,
    /* Sizing only: the stochastic workspace plus a buffer in which the
     * filtered call (with top-k or top-p on) collects, per logits row, the
     * logits within 16 octaves of weight of the row's maximum (up to 16384
     * slots of 4 bytes per row) and the mass of the others, in one parallel
     * pass, so that its per-row selection reads those instead of the row.
     * spec_verify_stochastic_filtered accepts a workspace of either size and
     * gives the same bits with both; this one is faster. */
    SPEC_VERIFY_MODE_STOCHASTIC_FILTERED = 3,
    /* Sizing only: the exchange areas (3328 bytes per request) that let
     * spec_verify_tree_stochastic split each request's walk over several
     * workgroups (rows_per_request = N + 1). */
    SPEC_VERIFY_MODE_TREE_STOCHASTIC = 4
};

enum spec_verify_status {
    SPEC_VERIFY_OK = 0,
    SPEC_VERIFY_INVALID_ARGUMENT = 1,   /* null pointer, bad size, bad temperature */
    SPEC_VERIFY_UNSUPPORTED_DTYPE = 2,
    SPEC_VERIFY_WORKSPACE_TOO_SMALL = 3,
    SPEC_VERIFY_LIMIT_EXCEEDED = 4,     /* k, N, P, L or V beyond the limits below */
    SPEC_VERIFY_HIP_ERROR = 5           /* a launch failed; see hipGetLastError */
};

/* Limits checked on the host. */
#define SPEC_VERIFY_MAX_K 64          /* draft length of the linear modes */
#define SPEC_VERIFY_MAX_TREE_ROWS 1024 /* N + 1 */
#define SPEC_VERIFY_MAX_PATHS 1024    /* P */
#define SPEC_VERIFY_MAX_PATH_LEN 64   /* L */
#define SPEC_VERIFY_MAX_PATH_TABLE 16384 /* P * L */
#define SPEC_VERIFY_MAX_VOCAB (1 << 30)
#define SPEC_VERIFY_MAX_STOCHASTIC_VOCAB (1 << 22) /* V of the linear stochastic calls */
#define SPEC_VERIFY_MAX_FILTER_VOCAB (1 << 22) /* V of a filtered call with a filter on */
#define SPEC_VERIFY_MAX_TREE_SAMPLING_VOCAB (1 << 19) /* V of spec_verify_tree_stochastic */
#define SPEC_VERIFY_MIN_TEMPERATURE 1e-20f /* keeps log2(e)/T finite in fp32 */
#define SPEC_VERIFY_MAX_TEMPERATURE 1e20f

/* Library version as major * 10000 + minor * 100 + patch. */
int spec_verify_version(void);

/* Static, NUL-terminated description of a status code. */
const char *spec_verify_status_string(int status);

/*
 * Bytes of device workspace one call of `mode` needs for a batch of B
 * requests with `rows_per_request` target rows each (k + 1 for the linear
 * modes, N + 1 for the tree mode) over a vocabulary of V in `dtype`.
 * Returns 0 for arguments the corresponding call would reject.
 *
 * The workspace holds per-request arrival counters, per-chunk partial
 * reductions and per-request sampling state.  It must be zero-filled before
 * its first use (spec_verify_workspace_init does that); every call leaves all
 * of it zero-filled again when it completes, so one workspace serves any
 * number of later calls of any mode and shape whose size fits, provided calls
 * that share it are ordered on one stream.  (A call cut short by a device
 * fault leaves it undefined: zero it again.)  Its address must be 256-byte
 * aligned, as hipMalloc's and torch's allocations are; calls reject any other
 * with SPEC_VERIFY_INVALID_ARGUMENT.
 */
size_t spec_verify_workspace_bytes(int mode, int B, int rows_per_request, int V, int dtype);

/*
 * Waits inside a call are bounded.  Workgroups of a call wait only for
 * workgroups of the same launch that come before them in the grid, so the
 * bounds (tens of milliseconds) are reached only when other work holds the
 * device's compute units for that long.  A stochastic sampling workgroup, or a
 * greedy or tree epilogue, that reaches its bound computes what it waited for
 * itself (the same result) and marks the workspace stale: a late workgroup may
 * then still write into it, so every later call on a stale workspace computes
 * its statistics without reading them from the workspace (slower, same
 * results) until the workspace is zeroed again (spec_verify_workspace_init).
 */

/*
 * Zero-fill `workspace_bytes` bytes of a fresh workspace on `stream` with a fill
 * kernel (no memset node).  Call once after allocating it.
 */
int spec_verify_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stochastic schedule of the plain, ragged, counter-based and allocation-free
 * calls (process-wide, not thread-safe; default AUTO).  All schedules give
 * bit-identical results.
 *
 *   AUTO          rows 16-byte aligned (pointers and V * element size): one
 *                 launch whose grid holds each request's statistics
 *                 workgroups, with the sampling workgroups of request b after
 *                 those of request b + L; sampling workgroups wait (bounded
 *                 polling) for their request's statistics.  L = B (every
 *                 sampling workgroup last) when the call's logits fit the
 *                 256 MiB last-level cache; otherwise three times the
 *                 requests whose workgroups are resident at once, so that a
 *                 request's stop rows are read again while still cached.
 *                 Unaligned rows: TWO_KERNELS.
 *   TWO_KERNELS   a statistics kernel, then a sampling kernel.
 *   SELF_COMPUTE  the sampling kernel alone, every sampling workgroup
 *                 computing its request's statistics itself (slow; for
 *                 testing: the same bits with no statistics exchanged).
 *   INTERLEAVED   AUTO's one launch with L = 1 at every size (for testing:
 *                 sampling workgroups poll statistics still being computed).
 *
 * Returns INVALID_ARGUMENT for any other value.
 */
enum {
    SPEC_VERIFY_SCHEDULE_AUTO = 0,
    SPEC_VERIFY_SCHEDULE_TWO_KERNELS = 1,
    SPEC_VERIFY_SCHEDULE_SELF_COMPUTE = 2,
    SPEC_VERIFY_SCHEDULE_INTERLEAVED = 3
};
int spec_verify_set_schedule(int schedule);

/*
 * Profiling hook.  After this call, every verification call launches its
 * streaming kernel (the one that reads every logits row; under the one-launch
 * stochastic schedule, the whole call; for the filtered call, its per-row
 * selection kernel; for spec_verify_tree_stochastic, its one kernel) with
 * events[2 * i] and
 * events[2 * i + 1] attached as the kernel's start and stop events
 * (hipExtLaunchKernel: they take the kernel's own start and end timestamps),
 * with i advancing by one per call and wrapping at n_pairs.  The events are
 * hipEvent_t handles (passed as void*) that the caller created and destroys.
 * Pass NULL and 0 to switch the hook off.  The hook is process-wide and not
 * thread-safe; it exists so that a benchmark can time that kernel alone on the
 * stream it runs on.
 */
int spec_verify_profile_events(void *const *events, int n_pairs);

/*
 * Stochastic verification (speculative sampling) of B linear drafts of length k.
 *
 *   target_logits [B, k+1, V] dtype  -- row i (i < k) is the target distribution
 *                  for draft token i; row k is the bonus row.
 *   draft_logits  [B, k, V] dtype    -- row i is the draft distribution that
 *                  proposed draft token i (may be NULL when k == 0).
 *   draft_tokens  [B, k] int32 (may be NULL when k == 0).
 *   uniforms      [B, k+1] float32 in [0, 1): uniforms[b, i] (i < k) drives test
 *                  i; uniforms[b, k] drives the one final (residual or bonus)
 *                  sample.
 *   temperature   in [SPEC_VERIFY_MIN_TEMPERATURE, SPEC_VERIFY_MAX_TEMPERATURE]
 *                  (else INVALID_ARGUMENT): both logits tensors are divided by
 *                  it before the softmax (the two sides are filtered
 *                  identically).
 *
 * Per request, with p_i = softmax(target row i / T), q_i = softmax(draft row
 * i / T), P = p_i(x_i), Q = q_i(x_i): test i accepts when P >= Q or
 * u_i * Q < P (the strict test u < min(1, P/Q)); s = the first rejected i, or
 * k.  The final token is the inverse-CDF draw with u_k over token ids in
 * ascending order (the smallest j whose running weight exceeds u_k * Z) from
 * the weights max(0, p_s - q_s) when s < k, or p_k when s == k.
 *
 * Outputs:
 *   out_tokens   [B, k+1] int32: draft[0..s-1], the final token, then -1.
 *   num_accepted [B] int32: s.
 *   p_at_draft, q_at_draft [B, k] float32 or NULL: P and Q of every draft
 *                 position (0 for an out-of-range draft id).
 *
 * Work: one streaming pass that reads every logits row once (softmax
 * statistics), then a sampler that reads only each request's stop row(s); in
 * one launch or two kernels (see spec_verify_set_schedule).
 * V <= SPEC_VERIFY_MAX_STOCHASTIC_VOCAB (else LIMIT_EXCEEDED).
 */
int spec_verify_stochastic(const void *target_logits, const void *draft_logits, int dtype,
                           const int32_t *draft_tokens, const float *uniforms,
                           float temperature, int B, int k, int V,
                           int32_t *out_tokens, int32_t *num_accepted,
                           float *p_at_draft, float *q_at_draft,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * spec_verify_stochastic without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, outputs and results are those
 * of spec_verify_stochastic; the workspace is a fixed array of
 * SPEC_VERIFY_NOALLOC_SCRATCH_BYTES in the library's device memory, one per
 * GPU, held until the process ends.  The call allocates and frees nothing.
 *
 *   - A shape whose workspace (spec_verify_workspace_bytes of MODE_STOCHASTIC)
 *     exceeds SPEC_VERIFY_NOALLOC_SCRATCH_BYTES is rejected on the host with
 *     SPEC_VERIFY_LIMIT_EXCEEDED; nothing is launched.
 *   - The array belongs to the current device; `stream` must belong to it too.
 *     The first call on a device looks up the array's address and zero-fills
 *     it with a fill kernel on `stream`; every completed call leaves it zero.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in time
 *     on one GPU (several streams, several host threads) race on it and give
 *     undefined results.  Order them on one stream.
 */
#define SPEC_VERIFY_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int spec_verify_stochastic_noalloc(const void *target_logits, const void *draft_logits,
                                   int dtype, const int32_t *draft_tokens,
                                   const float *uniforms, float temperature, int B, int k,
                                   int V, int32_t *out_tokens, int32_t *num_accepted,
                                   float *p_at_draft, float *q_at_draft, void *stream);

/*
 * Stochastic verification with a draft length per request (page "TensorRT-LLM
 * source teardown (10)", acceptance pipeline, step 2: ragged verification,
 * every request verified over its own window while buffers stay padded to the
 * static maximum k; padding never counts).
 *
 *   draft_lens [B] int32, device: request b uses its first
 *              k_b = clamp(draft_lens[b], 0, k) drafts (NULL: k_b = k for all).
 *
 * Request b gives exactly what spec_verify_stochastic gives for that request
 * alone with k = k_b: target rows 0..k_b, draft rows and tokens 0..k_b-1,
 * uniforms[b, i] for test i < k_b and uniforms[b, k_b] for the final token.
 * Rows past the window are not read.  The other arguments and layouts are those
 * of spec_verify_stochastic (padded to k): out_tokens[b, k_b+1..k] = -1,
 * p_at_draft / q_at_draft [b, k_b..k-1] = 0, num_accepted[b] <= k_b.
 */
int spec_verify_stochastic_ragged(const void *target_logits, const void *draft_logits,
                                  int dtype, const int32_t *draft_tokens,
                                  const int32_t *draft_lens, const float *uniforms,
                                  float temperature, int B, int k, int V,
                                  int32_t *out_tokens, int32_t *num_accepted,
                                  float *p_at_draft, float *q_at_draft,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stochastic verification with counter-based uniforms instead of an input
 * tensor (page "TensorRT-LLM source teardown (10)", "Rejection sampling": a
 * per-call seed and offset).  Draw i of request b (tests i < k_b, final token
 * k_b) is word i % 4 of the Philox4x64-10 block (Salmon et al., SC 2011) at
 * counter (offset, b, i / 4, 0) with key (seed, 0), as its top 24 bits times
 * 2^-24.  Otherwise identical to spec_verify_stochastic_ragged (draft_lens may
 * be NULL); a caller advances `offset` between calls to get fresh draws.
 */
int spec_verify_stochastic_philox(const void *target_logits, const void *draft_logits,
                                  int dtype, const int32_t *draft_tokens,
                                  const int32_t *draft_lens, uint64_t seed, uint64_t offset,
                                  float temperature, int B, int k, int V,
                                  int32_t *out_tokens, int32_t *num_accepted,
                                  float *p_at_draft, float *q_at_draft,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stochastic verification with sampling filters applied to every target and
 * every draft row alike (page "TensorRT-LLM source teardown (10)", "Rejection
 * sampling": both sides must be filtered identically -- temperature, top-k,
 * top-p, min-p -- or the acceptance test is wrong; page "Inside vLLM: Anatomy
 * of a High-Throughput LLM Inference System" sets top_p in its example).  The
 * pages name the filters without defining them; a row keeps the tokens whose
 * logit x is >= tau = the largest of
 *   top-k: the top_k-th largest logit of the row, counting repeated values
 *          (off when top_k == 0 or top_k >= V);
 *   top-p: the smallest logit value v such that the tokens x >= v among the
 *          top-k survivors hold at least top_p of the survivors' mass (every
 *          token tied with v kept; off when top_p == 1);
 *   min-p: max x + temperature * ln(min_p), i.e. p >= min_p * max p (off when
 *          min_p == 0);
 * and the kept tokens' probabilities are renormalised; every other token has
 * probability 0 in the tests (p_at_draft / q_at_draft report the filtered
 * values) and in the final draw.
 *
 *   top_k  >= 0;  top_p in (0, 1];  min_p in [0, 1].
 *
 * Other arguments, layouts and outputs as spec_verify_stochastic; every request
 * uses k drafts.  With every filter off this is spec_verify_stochastic.  With a
 * filter on, V <= SPEC_VERIFY_MAX_FILTER_VOCAB (else LIMIT_EXCEEDED), and the
 * call runs a per-row selection pass over the logits between the statistics
 * and the sampler.  The masses that decide top-p come from fast weights
 * (~1.5e-7 relative) when the boundary is more than 1e-6 (relative) from the
 * nearest edge between distinct logit values, otherwise from fp64 weights
 * (~1e-12 relative): only a boundary closer than that to an edge can come out
 * differently from exact arithmetic.
 */
int spec_verify_stochastic_filtered(const void *target_logits, const void *draft_logits,
                                    int dtype, const int32_t *draft_tokens,
                                    const float *uniforms, float temperature, int top_k,
                                    float top_p, float min_p, int B, int k, int V,
                                    int32_t *out_tokens, int32_t *num_accepted,
                                    float *p_at_draft, float *q_at_draft,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Greedy verification of B linear drafts of length k.
 *
 *   target_logits [B, k+1, V] dtype; draft_tokens [B, k] int32 (NULL if k == 0).
 *
 * a_i = argmax of raw target row i (lowest index among equal maxima);
 * s = number of leading i with draft_tokens[b, i] == a_i.
 *   out_tokens   [B, k+1] int32: draft[0..s-1], a_s, then -1.
 *   num_accepted [B] int32: s.
 */
int spec_verify_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens,
                       int B, int k, int V, int32_t *out_tokens, int32_t *num_accepted,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Greedy verification with a draft length per request (same reading as
 * spec_verify_stochastic_ragged): request b compares its first
 * k_b = clamp(draft_lens[b], 0, k) drafts with a_0..a_{k_b-1} and emits
 * draft[0..s-1], a_s, then -1 up to position k; rows past k_b are not read.
 * draft_lens [B] int32, device (NULL: k_b = k).
 */
int spec_verify_greedy_ragged(const void *target_logits, int dtype, const int32_t *draft_tokens,
                              const int32_t *draft_lens, int B, int k, int V,
                              int32_t *out_tokens, int32_t *num_accepted, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Tree (EAGLE-style) greedy verification.
 *
 *   target_logits [B, N+1, V] dtype -- row n: target distribution after node n
 *                  (node 0 is the root, the last committed token).
 *   node_tokens   [B, N+1] int32 -- draft token of node n; [b, 0] is ignored.
 *   paths         [B, P, L] int32 -- node indices from the root down one branch,
 *                  -1 padded; a row whose first entry is not in [0, N] is unused.
 *
 * A path's accepted length m is the number of its nodes, from the root down,
 * whose token equals the argmax of the previous node's row, counted until the
 * first mismatch.  The chosen row has the largest m, the lowest row index among
 * equal m.
 *   out_tokens     [B, L] int32: tokens of the m accepted nodes, the argmax of
 *                  the last accepted node's row, then -1.  With no usable row:
 *                  the root row's argmax, then -1.
 *   num_accepted   [B] int32: m.
 *   best_path      [B] int32 or NULL: the chosen row, -1 if no row is usable.
 *   accepted_nodes [B, L] int32 or NULL: the m accepted node indices, then -1
 *                  (the rows a caller keeps when it compacts its KV cache).
 */
int spec_verify_tree(const void *target_logits, int dtype, const int32_t *node_tokens,
                     const int32_t *paths, int B, int N, int P, int L, int V,
                     int32_t *out_tokens, int32_t *num_accepted, int32_t *best_path,
                     int32_t *accepted_nodes, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Stochastic verification of a draft tree.  The page "05 - TensorRT-LLM
 * speculative decoding and auto-deploy" ("Target-model verification: tree
 * attention and batched parallelism") checks every tree node against the
 * target in one pass by "rejection sampling", with the tree given as the paths
 * table of "Eagle-2 multi-level tree drafting", and states no rule for several
 * candidate children.  The rule used: starting at the root, the children of
 * the current node are tested in ascending node order as the linear call tests
 * one draft (accept child c when p(x) >= q(x) or u q(x) < p(x), x its token, p
 * the current target distribution, q the draft row the children were drawn
 * from); each rejection replaces p by max(0, p - q) renormalised; an accepted
 * child becomes the current node (one level down, at most L - 1 levels);
 * when no child is accepted, one token is drawn from the last residual
 * max(0, p - q) (from p when nothing was rejected at that node, or when the
 * residual has no mass) by inverse CDF, as in the linear call.  With children
 * drawn independently from q this emits tokens distributed as the target's
 * (multi-candidate speculative sampling, SpecInfer, Miao et al., ASPLOS 2024);
 * a single-chain tree gives exactly spec_verify_stochastic.
 *
 *   target_logits [B, N+1, V] dtype: row n, the target distribution after
 *                  node n (node 0 = the root, the last committed token).
 *   draft_logits  [B, N+1, V] dtype: row n, the draft distribution node n's
 *                  children were drawn from (rows of leaves are not read).
 *   node_tokens   [B, N+1] int32: node n's token ([b, 0] ignored).
 *   paths         [B, P, L] int32: node indices root-first, -1 padded; node
 *                  paths[t] is a child of paths[t-1], the first row (then the
 *                  first position) that names a node fixing its parent; a row
 *                  whose first entry is not in [0, N] is unused and an entry
 *                  outside [0, N] ends a row.
 *   uniforms      [B, N+1] fp32 in [0, 1): uniforms[b, c-1] drives node c's
 *                  test, uniforms[b, N] the final draw.
 *   out_tokens     [B, L] int32: the accepted nodes' tokens, the final token,
 *                  then -1.
 *   num_accepted   [B] int32: accepted nodes (tree depth reached).
 *   accepted_nodes [B, L] int32 or NULL: their node indices, then -1.
 *
 * Limits: N + 1 <= SPEC_VERIFY_MAX_TREE_ROWS, P <= SPEC_VERIFY_MAX_PATHS,
 * L <= SPEC_VERIFY_MAX_PATH_LEN, P * L <= SPEC_VERIFY_MAX_PATH_TABLE,
 * V <= SPEC_VERIFY_MAX_TREE_SAMPLING_VOCAB.  Draft ids outside [0, V) are
 * rejected.  Each request's walk reads, per visited node, its two rows once
 * for their statistics, once more per rejected child, and once for the final
 * draw.
 *
 *   workspace      device, zero-filled before first use (left zero), of at
 *                  least spec_verify_workspace_bytes(SPEC_VERIFY_MODE_TREE_-
 *                  STOCHASTIC, B, N + 1, V, dtype) bytes, or NULL.  With it,
 *                  each request's walk is split over up to 8 workgroups (the
 *                  row tiles shared out, their sums exchanged through it) when
 *                  all of them fit on the device at once (by the kernel's
 *                  occupancy); otherwise, or with NULL, one workgroup per
 *                  request walks its tree.  The two give the same tokens
 *                  except where a decision lies within rounding of its
 *                  boundary (the row statistics are merged in a different
 *                  order).  Calls sharing a workspace must be ordered on one
 *                  stream; calls with their own workspaces may run at once on
 *                  several streams.  A request's workgroups wait on each other
 *                  and are grouped by arrival, so only a kernel that holds
 *                  compute units for good on another stream can keep one from
 *                  starting; every wait is bounded, and num_accepted[b] = -2
 *                  then marks a request whose walk gave up waiting for one of
 *                  its workgroups (its outputs are not valid).
 */
int spec_verify_tree_stochastic(const void *target_logits, const void *draft_logits, int dtype,
                                const int32_t *node_tokens, const int32_t *paths,
                                const float *uniforms, float temperature, int B, int N, int P,
                                int L, int V, int32_t *out_tokens, int32_t *num_accepted,
                                int32_t *accepted_nodes, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Workgroups per request that spec_verify_tree_stochastic would use, with a
 * workspace of the right size and 16-byte aligned rows, for B requests over a
 * vocabulary of V on the current device: at most 8 and one per 8192-token row
 * tile, and B times it must fit on the device at once; 1 when the walk is not
 * split.  0 for arguments that call would reject.  Initialises the device's
 * HIP context if needed; no GPU work.
 */
int spec_verify_tree_stochastic_split(int B, int V, int dtype);

/*
 * Testing hook for the split walk's failure path: sets how many times a
 * workgroup polls one exchange word before it gives up and the request is
 * marked num_accepted = -2 (default 1048576; a negative value restores it),
 * for calls of spec_verify_tree_stochastic made from then on, process-wide.
 * Returns the previous value.  A tiny value makes split walks give up on
 * purpose, so tests can check that the kernel still ends, marks the requests
 * and clears its workspace; it has no use outside tests.
 */
int spec_verify_debug_tree_spin_limit(int polls);

/*
 * Testing hook for the bounded waits of the linear calls: sets how many times
 * a sampling workgroup of the stochastic calls, or an epilogue workgroup of
 * the greedy and tree calls, polls its request's published statistics before
 * it computes what is missing itself and marks the workspace stale (default
 * 65536; a negative value restores it), for calls made from then on,
 * process-wide.  Returns the previous value.  A tiny value makes waits give
 * up on purpose, so tests can check that results still match and that later
 * calls on the stale workspace do too; it has no use outside tests.
 */
int spec_verify_debug_spin_limit(int polls);

/*
 * Gather of the accepted rows (page "TensorRT-LLM source teardown (10)", KV
 * rewind, fourth step: the accepted draft tokens' KV rows, scattered when the
 * draft was a tree, are moved to contiguous logical positions):
 *   dst[b, j, :] = src[b, accepted_nodes[b, j], :] for j < num_accepted[b].
 *   src [B, N1, row_bytes] bytes, device; dst [B, L, row_bytes] bytes, device
 *   (must not overlap src); accepted_nodes [B, L] and num_accepted [B] int32,
 *   device (the outputs of spec_verify_tree or spec_verify_tree_stochastic).
 * Slots j >= num_accepted[b], and slots whose node is outside [0, N1), are
 * left as they are.  16-byte copies when row_bytes and both pointers allow.
 */
int spec_verify_gather_rows(const void *src, void *dst, size_t row_bytes,
                            const int32_t *accepted_nodes, const int32_t *num_accepted, int B,
                            int N1, int L, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
