// sv_api.hip -- the C ABI: host-side validation, launch geometry, launches.
//
// Every check runs on the host before anything is enqueued, and reads only
// shapes, pointers and scalars (never device data): a rejected call launches
// nothing and touches no output, so a caller can capture calls in a graph.
// Host-side, fail-closed validation follows the shape guards described on the
// page "TensorRT-LLM source teardown (10): speculative decoding", section
// "Rejection sampling".
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "spec_verify.h"
#include "sv_common.hpp"
#include "sv_launch.hpp"

// Workspace of spec_verify_stochastic_noalloc: a fixed device array, one copy
// per GPU (each device that loads the library holds its own), kept until the
// process ends.  Host code never passes the array's name to a kernel or a copy:
// it looks up each device's address once (hipGetSymbolAddress) and uses that.
static __device__ __align__(256) unsigned char scratch[SPEC_VERIFY_NOALLOC_SCRATCH_BYTES];

namespace {

int elem_bytes_of(int dtype) {
    if (dtype == SPEC_VERIFY_F32) return 4;
    if (dtype == SPEC_VERIFY_BF16) return 2;
    return 0;
}

// Rows are 16-byte aligned and hold whole 16-byte vectors.
bool vec_ok(const void* p, int V, int eb) {
    return p == nullptr || ((reinterpret_cast<uintptr_t>(p) % 16 == 0) &&
                            ((size_t)V * (size_t)eb) % 16 == 0);
}

// A workspace holds 8- and 16-byte words (counters, partials, exchange
// words): it must be 256-byte aligned, as every device allocation is.
bool ws_aligned(const void* p) { return reinterpret_cast<uintptr_t>(p) % 256 == 0; }

int finish(hipError_t e) { return e == hipSuccess ? SPEC_VERIFY_OK : SPEC_VERIFY_HIP_ERROR; }

constexpr size_t kNoAllocBytes = SPEC_VERIFY_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`: on the first call per device its
// address is looked up and the array zero-filled by a fill kernel on `st`
// (ordered before the call that follows on the same stream).
int noalloc_scratch(hipStream_t st, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return SPEC_VERIFY_HIP_ERROR;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return SPEC_VERIFY_HIP_ERROR;
        if (sv::run_fill_zero(p, kNoAllocBytes, st) != hipSuccess) return SPEC_VERIFY_HIP_ERROR;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPEC_VERIFY_OK;
}

// Profiling hook state (see spec_verify_profile_events).
void* const* g_events = nullptr;
int g_event_pairs = 0;
int g_event_next = 0;

sv::KernelEvents next_events() {
    sv::KernelEvents ev;
    if (g_events && g_event_pairs > 0) {
        const int i = g_event_next;
        g_event_next = (i + 1) % g_event_pairs;
        ev.begin = (hipEvent_t)g_events[2 * i];
        ev.end = (hipEvent_t)g_events[2 * i + 1];
    }
    return ev;
}

}  // namespace

extern "C" {

int spec_verify_version(void) { return 100; }

const char* spec_verify_status_string(int status) {
    switch (status) {
        case SPEC_VERIFY_OK: return "ok";
        case SPEC_VERIFY_INVALID_ARGUMENT: return "invalid argument";
        case SPEC_VERIFY_UNSUPPORTED_DTYPE: return "unsupported dtype";
        case SPEC_VERIFY_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SPEC_VERIFY_LIMIT_EXCEEDED: return "limit exceeded";
        case SPEC_VERIFY_HIP_ERROR: return "HIP launch error";
        default: return "unknown status";
    }
}

size_t spec_verify_workspace_bytes(int mode, int B, int rows_per_request, int V, int dtype) {
    const int eb = elem_bytes_of(dtype);
    if (eb == 0 || mode < 0 || mode > 4 || V > SPEC_VERIFY_MAX_VOCAB) return 0;
    const bool tree = mode == 2 || mode == 4;
    if (!tree && rows_per_request - 1 > SPEC_VERIFY_MAX_K) return 0;
    if (tree && rows_per_request > SPEC_VERIFY_MAX_TREE_ROWS) return 0;
    if (mode == 4 && V > SPEC_VERIFY_MAX_TREE_SAMPLING_VOCAB) return 0;
    if ((mode == 0 || mode == 3) && V > SPEC_VERIFY_MAX_STOCHASTIC_VOCAB) return 0;
    sv::Geometry g;
    if (!sv::make_geometry(mode, B, rows_per_request, V, eb, &g)) return 0;
    return g.bytes;
}

int spec_verify_set_schedule(int schedule) {
    if (schedule != SPEC_VERIFY_SCHEDULE_AUTO && schedule != SPEC_VERIFY_SCHEDULE_TWO_KERNELS &&
        schedule != SPEC_VERIFY_SCHEDULE_SELF_COMPUTE && schedule != SPEC_VERIFY_SCHEDULE_INTERLEAVED)
        return SPEC_VERIFY_INVALID_ARGUMENT;
    sv::g_stochastic_schedule = schedule;
    return SPEC_VERIFY_OK;
}

int spec_verify_profile_events(void* const* events, int n_pairs) {
    if (n_pairs < 0 || (n_pairs > 0 && events == nullptr)) return SPEC_VERIFY_INVALID_ARGUMENT;
    g_events = n_pairs > 0 ? events : nullptr;
    g_event_pairs = n_pairs;
    g_event_next = 0;
    return SPEC_VERIFY_OK;
}

int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (workspace == nullptr && workspace_bytes != 0) return SPEC_VERIFY_INVALID_ARGUMENT;
    return finish(sv::run_fill_zero(workspace, workspace_bytes, (hipStream_t)stream));
}

static int stochastic_impl(const void* target_logits, const void* draft_logits, int dtype,
                           const int32_t* draft_tokens, const int32_t* draft_lens,
                           const float* uniforms, bool counter_uniforms, uint64_t seed,
                           uint64_t offset, float temperature, int B, int k, int V,
                           int32_t* out_tokens, int32_t* num_accepted, float* p_at_draft,
                           float* q_at_draft, void* workspace, size_t workspace_bytes,
                           void* stream, const sv::FilterCall* filter = nullptr,
                           bool noalloc = false) {
    const int eb = elem_bytes_of(dtype);
    if (eb == 0) return SPEC_VERIFY_UNSUPPORTED_DTYPE;
    if (B < 1 || k < 0 || V < 1) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!(temperature >= SPEC_VERIFY_MIN_TEMPERATURE) ||
        !(temperature <= SPEC_VERIFY_MAX_TEMPERATURE))
        return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!target_logits || !out_tokens || !num_accepted)
        return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!noalloc && (!workspace || !ws_aligned(workspace))) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!counter_uniforms && !uniforms) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (k > 0 && (!draft_logits || !draft_tokens)) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (k > SPEC_VERIFY_MAX_K || V > SPEC_VERIFY_MAX_STOCHASTIC_VOCAB)
        return SPEC_VERIFY_LIMIT_EXCEEDED;
    if (filter && V > SPEC_VERIFY_MAX_FILTER_VOCAB) return SPEC_VERIFY_LIMIT_EXCEEDED;
    // A filtered call's sampler chunks are its own (geometry mode 5, or 3 when
    // the workspace also holds the candidates); mode 5 never needs more bytes
    // than mode 0.
    sv::Geometry g;
    if (!sv::make_geometry(filter ? 5 : 0, B, k + 1, V, eb, &g)) return SPEC_VERIFY_INVALID_ARGUMENT;
    if ((long long)B * g.R * g.S > 0x7fffffffLL || (long long)B * g.S2 > 0x7fffffffLL)
        return SPEC_VERIFY_LIMIT_EXCEEDED;
    if (noalloc) {
        // Every check above ran first: a rejected call launches nothing.
        if (g.bytes > kNoAllocBytes) return SPEC_VERIFY_LIMIT_EXCEEDED;
        const int st = noalloc_scratch((hipStream_t)stream, &workspace);
        if (st != SPEC_VERIFY_OK) return st;
        workspace_bytes = kNoAllocBytes;
    }
    if (workspace_bytes < g.bytes) return SPEC_VERIFY_WORKSPACE_TOO_SMALL;
    if (filter) {  // room for the filter candidates: the same layout plus their buffer
        sv::Geometry g3;
        if (sv::make_geometry(3, B, k + 1, V, eb, &g3) && workspace_bytes >= g3.bytes) g = g3;
    }

    sv::StochasticCall c;
    c.target = target_logits;
    c.draft = k > 0 ? draft_logits : nullptr;
    c.dtype = dtype;
    c.vec = vec_ok(target_logits, V, eb) && vec_ok(c.draft, V, eb);
    c.draft_tokens = draft_tokens;
    c.draft_lens = draft_lens;
    c.uniforms = counter_uniforms ? nullptr : uniforms;
    c.seed = seed;
    c.offset = offset;
    c.temperature = temperature;
    c.B = B;
    c.k = k;
    c.V = V;
    c.out_tokens = out_tokens;
    c.num_accepted = num_accepted;
    c.p_at_draft = p_at_draft;
    c.q_at_draft = q_at_draft;
    c.workspace = workspace;
    if (filter)
        return finish(sv::run_stochastic_filtered(c, *filter, g, (hipStream_t)stream, next_events()));
    return finish(sv::run_stochastic(c, g, (hipStream_t)stream, next_events()));
}

int spec_verify_stochastic_filtered(const void* target_logits, const void* draft_logits,
                                    int dtype, const int32_t* draft_tokens,
                                    const float* uniforms, float temperature, int top_k,
                                    float top_p, float min_p, int B, int k, int V,
                                    int32_t* out_tokens, int32_t* num_accepted,
                                    float* p_at_draft, float* q_at_draft, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (top_k < 0 || !(top_p > 0.0f) || !(top_p <= 1.0f) || !(min_p >= 0.0f) || !(min_p <= 1.0f))
        return SPEC_VERIFY_INVALID_ARGUMENT;
    sv::FilterCall f;
    f.top_k = top_k;
    f.top_p = top_p;
    f.min_p = min_p;
    const bool on = (top_k > 0 && top_k < V) || top_p < 1.0f || min_p > 0.0f;
    return stochastic_impl(target_logits, draft_logits, dtype, draft_tokens, nullptr, uniforms,
                           false, 0, 0, temperature, B, k, V, out_tokens, num_accepted,
                           p_at_draft, q_at_draft, workspace, workspace_bytes, stream,
                           on ? &f : nullptr);
}

int spec_verify_stochastic_ragged(const void* target_logits, const void* draft_logits,
                                  int dtype, const int32_t* draft_tokens,
                                  const int32_t* draft_lens, const float* uniforms,
                                  float temperature, int B, int k, int V, int32_t* out_tokens,
                                  int32_t* num_accepted, float* p_at_draft, float* q_at_draft,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    return stochastic_impl(target_logits, draft_logits, dtype, draft_tokens, draft_lens,
                           uniforms, false, 0, 0, temperature, B, k, V, out_tokens, num_accepted,
                           p_at_draft, q_at_draft, workspace, workspace_bytes, stream);
}

int spec_verify_stochastic(const void* target_logits, const void* draft_logits, int dtype,
                           const int32_t* draft_tokens, const float* uniforms,
                           float temperature, int B, int k, int V, int32_t* out_tokens,
                           int32_t* num_accepted, float* p_at_draft, float* q_at_draft,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return stochastic_impl(target_logits, draft_logits, dtype, draft_tokens, nullptr, uniforms,
                           false, 0, 0, temperature, B, k, V, out_tokens, num_accepted,
                           p_at_draft, q_at_draft, workspace, workspace_bytes, stream);
}

int spec_verify_stochastic_noalloc(const void* target_logits, const void* draft_logits,
                                   int dtype, const int32_t* draft_tokens, const float* uniforms,
                                   float temperature, int B, int k, int V, int32_t* out_tokens,
                                   int32_t* num_accepted, float* p_at_draft, float* q_at_draft,
                                   void* stream) {
    return stochastic_impl(target_logits, draft_logits, dtype, draft_tokens, nullptr, uniforms,
                           false, 0, 0, temperature, B, k, V, out_tokens, num_accepted,
                           p_at_draft, q_at_draft, nullptr, 0, stream, nullptr, true);
}

int spec_verify_stochastic_philox(const void* target_logits, const void* draft_logits, int dtype,
                                  const int32_t* draft_tokens, const int32_t* draft_lens,
                                  uint64_t seed, uint64_t offset, float temperature, int B, int k,
                                  int V, int32_t* out_tokens, int32_t* num_accepted,
                                  float* p_at_draft, float* q_at_draft, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return stochastic_impl(target_logits, draft_logits, dtype, draft_tokens, draft_lens, nullptr,
                           true, seed, offset, temperature, B, k, V, out_tokens, num_accepted,
                           p_at_draft, q_at_draft, workspace, workspace_bytes, stream);
}

int spec_verify_greedy_ragged(const void* target_logits, int dtype, const int32_t* draft_tokens,
                              const int32_t* draft_lens, int B, int k, int V,
                              int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                              size_t workspace_bytes, void* stream) {
    const int eb = elem_bytes_of(dtype);
    if (eb == 0) return SPEC_VERIFY_UNSUPPORTED_DTYPE;
    if (B < 1 || k < 0 || V < 1) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!target_logits || !out_tokens || !num_accepted || !workspace || !ws_aligned(workspace))
        return SPEC_VERIFY_INVALID_ARGUMENT;
    if (k > 0 && !draft_tokens) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (k > SPEC_VERIFY_MAX_K || V > SPEC_VERIFY_MAX_VOCAB) return SPEC_VERIFY_LIMIT_EXCEEDED;
    sv::Geometry g;
    if (!sv::make_geometry(1, B, k + 1, V, eb, &g)) return SPEC_VERIFY_INVALID_ARGUMENT;
    if ((long long)B * g.R * g.S > 0x7fffffffLL) return SPEC_VERIFY_LIMIT_EXCEEDED;
    if (workspace_bytes < g.bytes) return SPEC_VERIFY_WORKSPACE_TOO_SMALL;

    sv::GreedyCall c;
    c.target = target_logits;
    c.dtype = dtype;
    c.vec = vec_ok(target_logits, V, eb);
    c.draft_tokens = draft_tokens;
    c.draft_lens = draft_lens;
    c.B = B;
    c.k = k;
    c.V = V;
    c.out_tokens = out_tokens;
    c.num_accepted = num_accepted;
    c.workspace = workspace;
    return finish(sv::run_greedy(c, g, (hipStream_t)stream, next_events()));
}

int spec_verify_greedy(const void* target_logits, int dtype, const int32_t* draft_tokens, int B,
                       int k, int V, int32_t* out_tokens, int32_t* num_accepted,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return spec_verify_greedy_ragged(target_logits, dtype, draft_tokens, nullptr, B, k, V,
                                     out_tokens, num_accepted, workspace, workspace_bytes,
                                     stream);
}

int spec_verify_tree(const void* target_logits, int dtype, const int32_t* node_tokens,
                     const int32_t* paths, int B, int N, int P, int L, int V,
                     int32_t* out_tokens, int32_t* num_accepted, int32_t* best_path,
                     int32_t* accepted_nodes, void* workspace, size_t workspace_bytes,
                     void* stream) {
    const int eb = elem_bytes_of(dtype);
    if (eb == 0) return SPEC_VERIFY_UNSUPPORTED_DTYPE;
    if (B < 1 || N < 0 || P < 0 || L < 1 || V < 1) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!target_logits || !node_tokens || !out_tokens || !num_accepted || !workspace ||
        !ws_aligned(workspace))
        return SPEC_VERIFY_INVALID_ARGUMENT;
    if (P > 0 && !paths) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (N + 1 > SPEC_VERIFY_MAX_TREE_ROWS || P > SPEC_VERIFY_MAX_PATHS ||
        L > SPEC_VERIFY_MAX_PATH_LEN || (long long)P * L > SPEC_VERIFY_MAX_PATH_TABLE ||
        V > SPEC_VERIFY_MAX_VOCAB)
        return SPEC_VERIFY_LIMIT_EXCEEDED;
    sv::Geometry g;
    if (!sv::make_geometry(2, B, N + 1, V, eb, &g)) return SPEC_VERIFY_INVALID_ARGUMENT;
    if ((long long)B * g.R * g.S > 0x7fffffffLL) return SPEC_VERIFY_LIMIT_EXCEEDED;
    if (workspace_bytes < g.bytes) return SPEC_VERIFY_WORKSPACE_TOO_SMALL;

    sv::TreeCall c;
    c.target = target_logits;
    c.dtype = dtype;
    c.vec = vec_ok(target_logits, V, eb);
    c.node_tokens = node_tokens;
    c.paths = paths;
    c.B = B;
    c.N = N;
    c.P = P;
    c.L = L;
    c.V = V;
    c.out_tokens = out_tokens;
    c.num_accepted = num_accepted;
    c.best_path = best_path;
    c.accepted_nodes = accepted_nodes;
    c.workspace = workspace;
    return finish(sv::run_tree(c, g, (hipStream_t)stream, next_events()));
}

int spec_verify_tree_stochastic(const void* target_logits, const void* draft_logits, int dtype,
                                const int32_t* node_tokens, const int32_t* paths,
                                const float* uniforms, float temperature, int B, int N, int P,
                                int L, int V, int32_t* out_tokens, int32_t* num_accepted,
                                int32_t* accepted_nodes, void* workspace, size_t workspace_bytes,
                                void* stream) {
    const int eb = elem_bytes_of(dtype);
    if (eb == 0) return SPEC_VERIFY_UNSUPPORTED_DTYPE;
    if (B < 1 || N < 0 || P < 0 || L < 1 || V < 1) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!(temperature >= SPEC_VERIFY_MIN_TEMPERATURE) ||
        !(temperature <= SPEC_VERIFY_MAX_TEMPERATURE))
        return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!target_logits || !draft_logits || !node_tokens || !uniforms || !out_tokens ||
        !num_accepted || (workspace && !ws_aligned(workspace)))
        return SPEC_VERIFY_INVALID_ARGUMENT;
    if (P > 0 && !paths) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (N + 1 > SPEC_VERIFY_MAX_TREE_ROWS || P > SPEC_VERIFY_MAX_PATHS ||
        L > SPEC_VERIFY_MAX_PATH_LEN || (long long)P * L > SPEC_VERIFY_MAX_PATH_TABLE ||
        V > SPEC_VERIFY_MAX_TREE_SAMPLING_VOCAB)
        return SPEC_VERIFY_LIMIT_EXCEEDED;
    sv::TreeStochCall c;
    c.target = target_logits;
    c.draft = draft_logits;
    c.dtype = dtype;
    c.vec = vec_ok(target_logits, V, eb) && vec_ok(draft_logits, V, eb);
    c.node_tokens = node_tokens;
    c.paths = paths;
    c.uniforms = uniforms;
    c.temperature = temperature;
    c.B = B;
    c.N = N;
    c.P = P;
    c.L = L;
    c.V = V;
    c.out_tokens = out_tokens;
    c.num_accepted = num_accepted;
    c.accepted_nodes = accepted_nodes;
    c.workspace = workspace;
    c.workspace_bytes = workspace ? workspace_bytes : 0;
    return finish(sv::run_tree_stochastic(c, (hipStream_t)stream, next_events()));
}

int spec_verify_tree_stochastic_split(int B, int V, int dtype) {
    if (elem_bytes_of(dtype) == 0 || B < 1 || V < 1 || V > SPEC_VERIFY_MAX_TREE_SAMPLING_VOCAB)
        return 0;
    return sv::tree_stochastic_split(B, V, dtype);
}

int spec_verify_debug_tree_spin_limit(int polls) { return sv::tree_stochastic_spin_limit(polls); }

int spec_verify_debug_spin_limit(int polls) { return sv::set_debug_spin_limit(polls, 1 << 16); }

int spec_verify_gather_rows(const void* src, void* dst, size_t row_bytes,
                            const int32_t* accepted_nodes, const int32_t* num_accepted, int B,
                            int N1, int L, void* stream) {
    if (B < 1 || N1 < 1 || L < 1) return SPEC_VERIFY_INVALID_ARGUMENT;
    if (!src || !dst || !accepted_nodes || !num_accepted) return SPEC_VERIFY_INVALID_ARGUMENT;
    if ((long long)B * L > 0x7fffffffLL) return SPEC_VERIFY_LIMIT_EXCEEDED;
    if (row_bytes == 0) return SPEC_VERIFY_OK;
    sv::GatherCall c;
    c.src = src;
    c.dst = dst;
    c.row_bytes = row_bytes;
    c.accepted_nodes = accepted_nodes;
    c.num_accepted = num_accepted;
    c.B = B;
    c.N1 = N1;
    c.L = L;
    return finish(sv::run_gather_rows(c, (hipStream_t)stream));
}

}  // extern "C"
