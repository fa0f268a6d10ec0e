// sv_launch.hpp -- validated call descriptions passed from the C ABI layer to the
// kernel launchers (internal; not part of the public header).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

#include "sv_common.hpp"

namespace sv {

struct StochasticCall {
    const void* target;
    const void* draft;
    int dtype;  // 0 f32, 1 bf16
    bool vec;   // rows are 16-byte aligned and V is a whole number of vectors
    const int32_t* draft_tokens;
    const int32_t* draft_lens;  // [B] or null (every request uses k drafts)
    const float* uniforms;      // [B, k+1], or null: Philox draws from (seed, offset)
    unsigned long long seed, offset;
    float temperature;
    int B, k, V;
    int32_t* out_tokens;
    int32_t* num_accepted;
    float* p_at_draft;
    float* q_at_draft;
    void* workspace;
};

// Sampling filters of the filtered stochastic call (top_k 0 / top_p 1 /
// min_p 0: off).
struct FilterCall {
    int top_k;
    float top_p, min_p;
};

struct GreedyCall {
    const void* target;
    int dtype;
    bool vec;
    const int32_t* draft_tokens;
    const int32_t* draft_lens;  // [B] or null
    int B, k, V;
    int32_t* out_tokens;
    int32_t* num_accepted;
    void* workspace;
};

struct TreeCall {
    const void* target;
    int dtype;
    bool vec;
    const int32_t* node_tokens;
    const int32_t* paths;
    int B, N, P, L, V;
    int32_t* out_tokens;
    int32_t* num_accepted;
    int32_t* best_path;
    int32_t* accepted_nodes;
    void* workspace;
};

// Stochastic tree verification (no workspace).
struct TreeStochCall {
    const void* target;
    const void* draft;
    int dtype;
    bool vec;
    const int32_t* node_tokens;
    const int32_t* paths;
    const float* uniforms;
    float temperature;
    int B, N, P, L, V;
    int32_t* out_tokens;
    int32_t* num_accepted;
    int32_t* accepted_nodes;
    void* workspace;          // exchange areas (mode 4 size), or null: one workgroup per request
    size_t workspace_bytes;
};

// Accepted-row gather.
struct GatherCall {
    const void* src;
    void* dst;
    size_t row_bytes;
    const int32_t* accepted_nodes;
    const int32_t* num_accepted;
    int B, N1, L;
};

// Optional events recorded around the streaming kernel (both null = none).
struct KernelEvents {
    hipEvent_t begin = nullptr, end = nullptr;
};

// Stochastic schedule: 0 one launch where rows are 16-byte aligned (else two
// kernels), 1 two kernels, 2 one launch whose sampler items compute their
// request's statistics themselves instead of waiting (for tests).
extern int g_stochastic_schedule;
// Poll limit of the linear calls' bounded waits (testing hook; < 0: default).
int debug_spin_limit(int fallback);
int set_debug_spin_limit(int polls, int fallback);

hipError_t run_stochastic(const StochasticCall& call, const Geometry& g, hipStream_t st,
                          const KernelEvents& ev);
// Filtered call: statistics, then the per-row filter selection, then the
// sampler with every row's filter applied.
hipError_t run_stochastic_filtered(const StochasticCall& call, const FilterCall& f,
                                   const Geometry& g, hipStream_t st, const KernelEvents& ev);
hipError_t run_filter(const StochasticCall& call, const FilterCall& f, const Geometry& g,
                      hipStream_t st, const KernelEvents& ev);
hipError_t run_greedy(const GreedyCall& call, const Geometry& g, hipStream_t st,
                      const KernelEvents& ev);
hipError_t run_tree(const TreeCall& call, const Geometry& g, hipStream_t st,
                    const KernelEvents& ev);
hipError_t run_fill_zero(void* ptr, size_t bytes, hipStream_t st);
int tree_stochastic_split(int B, int V, int dtype);
int tree_stochastic_spin_limit(int polls);
hipError_t run_tree_stochastic(const TreeStochCall& c, hipStream_t st, const KernelEvents& ev);
hipError_t run_gather_rows(const GatherCall& c, hipStream_t st);

}  // namespace sv
