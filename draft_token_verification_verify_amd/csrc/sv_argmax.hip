// sv_argmax.hip -- greedy and tree (EAGLE-style) verification.
//
// Greedy (page "Kestrel_VLLM - 32", section 2, acceptance and emit steps; page
// "TensorRT-LLM source teardown (10)", section "Rejection sampling": an
// all-greedy batch gives the argmax result): a_i = argmax of target row i,
// accepted count s = leading drafts equal to a_0, a_1, ...; emit the accepted
// drafts, then a_s.
//
// Tree (page "05 - TensorRT-LLM speculative decoding and auto-deploy",
// sections "Eagle-2 multi-level tree drafting" and "Target-model
// verification"): every node's token is checked against the argmax of its
// parent's row; the branch of paths[b, P, L] with the most nodes accepted from
// the root down is kept (lowest path row on ties).
//
// One kernel per mode: one workgroup per (request, row, vocabulary chunk)
// streams its chunk once with 16-byte loads and reduces it to (max, lowest
// index of the max).  The last workgroup of each request (arrival ticket)
// merges the chunks of every row in chunk order and runs the mode's epilogue:
// the leading-match count (greedy), or the path walk with the path table, the
// node tokens and the argmax vector staged in LDS (tree).
#include <limits.h>

#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

struct ArgPartial {
    float v;
    int i;
};
static_assert(sizeof(ArgPartial) == 8, "ArgPartial layout");

struct ArgmaxArgs {
    const void* target;
    int B, R, V, S, chunk;
    ArgPartial* partials;  // [B, R, S]
    uint32_t* tickets;     // [B]
    // greedy
    const int32_t* draft_tokens;  // [B, k]
    int k;
    // tree
    const int32_t* node_tokens;  // [B, N+1]
    const int32_t* paths;        // [B, P, L]
    int N, P, L;
    int paths_in_lds;
    int32_t* out_tokens;
    int32_t* num_accepted;
    int32_t* best_path;
    int32_t* accepted_nodes;
};

__device__ inline ArgPartial merge_row(const ArgmaxArgs& a, int b, int r) {
    const ArgPartial* p = a.partials + ((size_t)b * a.R + r) * a.S;
    float v = -INFINITY;
    int i = INT_MAX;
    for (int ch = 0; ch < a.S; ++ch) {  // fixed chunk order
        ArgPartial q = p[ch];
        merge_argmax(v, i, q.v, q.i);
    }
    ArgPartial out;
    out.v = v;
    out.i = i;
    return out;
}

__device__ void greedy_epilogue(const ArgmaxArgs& a, int b) {
    __shared__ int sh_a[kMaxK + 1];
    const int k = a.k;
    for (int r = threadIdx.x; r <= k; r += kThreads) sh_a[r] = merge_row(a, b, r).i;
    __syncthreads();
    __shared__ int sh_s;
    if (threadIdx.x == 0) {
        int s = 0;
        while (s < k && a.draft_tokens[(size_t)b * k + s] == sh_a[s]) ++s;
        sh_s = s;
        a.num_accepted[b] = s;
    }
    __syncthreads();
    const int s = sh_s;
    for (int i = threadIdx.x; i <= k; i += kThreads) {
        int32_t v = -1;
        if (i < s) v = a.draft_tokens[(size_t)b * k + i];
        else if (i == s) v = sh_a[s];
        a.out_tokens[(size_t)b * (k + 1) + i] = v;
    }
}

__device__ void tree_epilogue(const ArgmaxArgs& a, int b) {
    extern __shared__ int dyn[];
    const int N = a.N, P = a.P, L = a.L;
    int* sh_a = dyn;             // [N+1] argmax of each node's row
    int* sh_tok = dyn + (N + 1); // [N+1] node tokens
    int* sh_paths = dyn + 2 * (N + 1);
    for (int n = threadIdx.x; n <= N; n += kThreads) {
        sh_a[n] = merge_row(a, b, n).i;
        sh_tok[n] = a.node_tokens[(size_t)b * (N + 1) + n];
    }
    const int32_t* gpaths = a.paths + (size_t)b * P * L;
    if (a.paths_in_lds)
        for (int q = threadIdx.x; q < P * L; q += kThreads) sh_paths[q] = gpaths[q];
    __syncthreads();
    const int32_t* paths = a.paths_in_lds ? (const int32_t*)sh_paths : gpaths;

    int best_m = -1, best_p = INT_MAX;
    for (int p = threadIdx.x; p < P; p += kThreads) {
        const int32_t* row = paths + (size_t)p * L;
        const int r0 = row[0];
        if (r0 < 0 || r0 > N) continue;  // unused row
        int m = 0;
        while (m + 1 < L) {
            const int child = row[m + 1];
            if (child < 0 || child > N) break;
            if (sh_tok[child] != sh_a[row[m]]) break;
            ++m;
        }
        if (m > best_m) {  // p ascends within a thread: strictly longer only
            best_m = m;
            best_p = p;
        }
    }
    // Workgroup reduction: longest m, then lowest path row.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        int m2 = __shfl_xor(best_m, off, 64);
        int p2 = __shfl_xor(best_p, off, 64);
        bool take = (m2 > best_m) || (m2 == best_m && p2 < best_p);
        best_m = take ? m2 : best_m;
        best_p = take ? p2 : best_p;
    }
    __shared__ int red_m[kWaves], red_p[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red_m[wave] = best_m;
        red_p[wave] = best_p;
    }
    __syncthreads();
    best_m = red_m[0];
    best_p = red_p[0];
    for (int w = 1; w < kWaves; ++w) {
        bool take = (red_m[w] > best_m) || (red_m[w] == best_m && red_p[w] < best_p);
        best_m = take ? red_m[w] : best_m;
        best_p = take ? red_p[w] : best_p;
    }
    const bool none = best_m < 0;
    const int m = none ? 0 : best_m;
    const int32_t* row = none ? nullptr : paths + (size_t)best_p * L;
    for (int t = threadIdx.x; t < L; t += kThreads) {
        int32_t tok = -1, node = -1;
        if (none) {
            if (t == 0) tok = sh_a[0];
        } else if (t < m) {
            node = row[t + 1];
            tok = sh_tok[node];
        } else if (t == m) {
            tok = sh_a[row[m]];
        }
        a.out_tokens[(size_t)b * L + t] = tok;
        if (a.accepted_nodes) a.accepted_nodes[(size_t)b * L + t] = node;
    }
    if (threadIdx.x == 0) {
        a.num_accepted[b] = m;
        if (a.best_path) a.best_path[b] = none ? -1 : best_p;
    }
}

// MODE 1: greedy, MODE 2: tree.
template <typename T, int U, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void argmax_kernel(ArgmaxArgs a) {
    constexpr int EPV = Elem<T>::kPerVec;
    const int tile = blockIdx.x;
    const int ch = tile % a.S;
    const int rr = tile / a.S;
    const int b = rr / a.R;
    const T* row = static_cast<const T*>(a.target) + (size_t)rr * (size_t)a.V;
    const int lo = ch * a.chunk;
    const int hi = min(a.V, lo + a.chunk);

    float bv = -INFINITY;
    int bi = INT_MAX;
    if constexpr (VEC) {
        const int nvec = (hi - lo) / EPV;
        const uint4* base = reinterpret_cast<const uint4*>(row + lo);
        // All U loads issue back to back: slots past the chunk's end reload its
        // last vector (in bounds) and are masked afterwards.
        uint4 raw[U];
#pragma unroll
        for (int j = 0; j < U; ++j) raw[j] = base[min((int)threadIdx.x + j * kThreads, nvec - 1)];
        float x[U][EPV];
        int first[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int v = threadIdx.x + j * kThreads;
            Elem<T>::widen(raw[j], x[j]);
            first[j] = lo + v * EPV;
            if (v >= nvec) {
#pragma unroll
                for (int e = 0; e < EPV; ++e) x[j][e] = -INFINITY;
                first[j] = INT_MAX - EPV;
            }
        }
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) bv = fmaxf(bv, x[j][e]);
        // Lowest index holding the maximum: walk from the highest slot down.
#pragma unroll
        for (int j = U - 1; j >= 0; --j)
#pragma unroll
            for (int e = EPV - 1; e >= 0; --e) bi = (x[j][e] == bv) ? first[j] + e : bi;
    } else {
        for (int j = lo + threadIdx.x; j < hi; j += kThreads) {
            float x = Elem<T>::load(row, j);
            if (x > bv || bi == INT_MAX) {
                bv = x;
                bi = j;
            }
        }
    }

    wave_reduce_argmax(bv, bi);
    __shared__ float red_v[kWaves];
    __shared__ int red_i[kWaves];
    __shared__ int last_flag;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red_v[wave] = bv;
        red_i[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = red_v[0];
        int i = red_i[0];
        for (int w = 1; w < kWaves; ++w) merge_argmax(v, i, red_v[w], red_i[w]);
        ArgPartial p;
        p.v = v;
        p.i = i;
        a.partials[tile] = p;
    }
    if (arrive_last(a.tickets + b, (uint32_t)(a.R * a.S), &last_flag)) {
        if constexpr (MODE == 1) greedy_epilogue(a, b);
        else tree_epilogue(a, b);
    }
}

template <typename T, bool VEC, int MODE>
static hipError_t launch_argmax(const ArgmaxArgs& a, int U, size_t lds, hipStream_t st) {
    const dim3 grid((unsigned)((long long)a.B * a.R * a.S)), block(kThreads);
    switch (U) {
        case 8: argmax_kernel<T, 8, VEC, MODE><<<grid, block, lds, st>>>(a); break;
        case 4: argmax_kernel<T, 4, VEC, MODE><<<grid, block, lds, st>>>(a); break;
        case 2: argmax_kernel<T, 2, VEC, MODE><<<grid, block, lds, st>>>(a); break;
        default: argmax_kernel<T, 1, VEC, MODE><<<grid, block, lds, st>>>(a); break;
    }
    return hipGetLastError();
}

template <int MODE>
static hipError_t dispatch(const ArgmaxArgs& a, int dtype, bool vec, int U, size_t lds,
                           hipStream_t st) {
    if (dtype == 1)
        return vec ? launch_argmax<bf16_t, true, MODE>(a, U, lds, st)
                   : launch_argmax<bf16_t, false, MODE>(a, U, lds, st);
    return vec ? launch_argmax<float, true, MODE>(a, U, lds, st)
               : launch_argmax<float, false, MODE>(a, U, lds, st);
}

static ArgmaxArgs base_args(const void* target, int B, int R, int V, const Geometry& g,
                            void* workspace) {
    char* ws = static_cast<char*>(workspace);
    ArgmaxArgs a = {};
    a.target = target;
    a.B = B;
    a.R = R;
    a.V = V;
    a.S = g.S;
    a.chunk = g.chunk;
    a.partials = reinterpret_cast<ArgPartial*>(ws + g.off_partials);
    a.tickets = reinterpret_cast<uint32_t*>(ws + g.off_ticket_a);
    return a;
}

hipError_t run_greedy(const GreedyCall& c, const Geometry& g, hipStream_t st,
                      const KernelEvents& ev) {
    ArgmaxArgs a = base_args(c.target, c.B, c.k + 1, c.V, g, c.workspace);
    a.draft_tokens = c.draft_tokens;
    a.k = c.k;
    a.out_tokens = c.out_tokens;
    a.num_accepted = c.num_accepted;
    hipError_t e;
    if (ev.begin && (e = hipEventRecord(ev.begin, st)) != hipSuccess) return e;
    if ((e = dispatch<1>(a, c.dtype, c.vec, g.U, 0, st)) != hipSuccess) return e;
    return ev.end ? hipEventRecord(ev.end, st) : hipSuccess;
}

hipError_t run_tree(const TreeCall& c, const Geometry& g, hipStream_t st,
                    const KernelEvents& ev) {
    ArgmaxArgs a = base_args(c.target, c.B, c.N + 1, c.V, g, c.workspace);
    a.node_tokens = c.node_tokens;
    a.paths = c.paths;
    a.N = c.N;
    a.P = c.P;
    a.L = c.L;
    a.paths_in_lds = (c.P * c.L <= kTreeLdsPathEntries) ? 1 : 0;
    a.out_tokens = c.out_tokens;
    a.num_accepted = c.num_accepted;
    a.best_path = c.best_path;
    a.accepted_nodes = c.accepted_nodes;
    const size_t lds = sizeof(int) * (2 * (size_t)(c.N + 1) +
                                      (a.paths_in_lds ? (size_t)c.P * c.L : 0));
    hipError_t e;
    if (ev.begin && (e = hipEventRecord(ev.begin, st)) != hipSuccess) return e;
    if ((e = dispatch<2>(a, c.dtype, c.vec, g.U, lds, st)) != hipSuccess) return e;
    return ev.end ? hipEventRecord(ev.end, st) : hipSuccess;
}

// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(unsigned char* p, size_t bytes) {
    const size_t nvec = bytes / 16;
    const size_t stride = (size_t)gridDim.x * kThreads;
    uint4 z = make_uint4(0, 0, 0, 0);
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride)
        reinterpret_cast<uint4*>(p)[i] = z;
    for (size_t i = nvec * 16 + (size_t)blockIdx.x * kThreads + threadIdx.x; i < bytes;
         i += stride)
        p[i] = 0;
}

hipError_t run_fill_zero(void* ptr, size_t bytes, hipStream_t st) {
    if (bytes == 0) return hipSuccess;
    size_t blocks = (bytes / 16 + kThreads - 1) / kThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    fill_zero_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
        static_cast<unsigned char*>(ptr), bytes);
    return hipGetLastError();
}

}  // namespace sv
