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
// One kernel per call.  One workgroup per (request, row, vocabulary chunk)
// streams its chunk once with 16-byte loads and reduces it to (max, lowest
// index of the max), published as one tagged 64-bit word; these take no
// atomics and wait for nothing.  After them in the grid, one workgroup per
// request polls its request's words until all are published, merges them in
// chunk order and runs the mode's epilogue: the leading-match count (greedy),
// or the path walk with the path table, the node tokens and the argmax vector
// staged in LDS (tree); it is the words' only reader and clears them.  Its
// wait is bounded: past the bound it computes the missing rows' maxima itself
// and marks the workspace stale (a word no call clears), since a late word may
// then be left behind; from then on the epilogues of every call on that
// workspace compute the maxima themselves, until the workspace is zeroed.
#include <limits.h>

#include "sv_common.hpp"
#include "sv_launch.hpp"
#include "sv_stream.hpp"

namespace sv {

struct ArgmaxArgs {
    const void* target;
    int B, R, V, S, chunk;
    Partial16* partials;  // [B, R, S]: word 0 = 2^63 | lowest index << 32 | bits(chunk max)
    uint32_t* stale;      // nonzero: published words may be stale (see above)
    int spin_limit;       // polls before an epilogue computes missing maxima itself
    // greedy
    const int32_t* draft_tokens;  // [B, k]
    const int32_t* lens;          // [B] draft length per request, or null (all k)
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

// Streaming argmax of every target row (lowest index among equal maxima), then
// the greedy (MODE 1) or tree (MODE 2) epilogue per request.
template <typename T, int U, int MODE>
struct ArgmaxOp : ArgmaxArgs {
    __device__ const T* row(int b, int r) const {
        return static_cast<const T*>(target) + ((size_t)b * R + r) * (size_t)V;
    }

    // Greedy draft length of request b: lens[b] clamped to [0, k], or k.
    __device__ int kb_of(int b) const { return lens ? min(max(lens[b], 0), k) : k; }
    // Greedy rows past a request's draft window are not read.
    __device__ bool skip(int b, int r) const { return MODE == 1 && lens && r > kb_of(b); }
    __device__ void publish_skipped(Partial16* dst) const {
        publish(dst, -INFINITY, __int_as_float(INT_MAX), 0.0);
    }

    // One 64-bit word per chunk, stored at once: the tag bit tells a published
    // word from the cleared 0 (indices fit 31 bits).
    __device__ void publish(Partial16* dst, float f0, float f1, double) const {
        const unsigned long long w = (1ull << 63) |
                                     ((unsigned long long)(unsigned)__float_as_int(f1) << 32) |
                                     (unsigned long long)__float_as_uint(f0);
        store_coherent(reinterpret_cast<unsigned long long*>(dst), w);
    }

    __device__ void finish(float v, int i, float* f0, float* f1, double* d) const {
        wave_reduce_argmax(v, i);
        __shared__ float red_v[kWaves];
        __shared__ int red_i[kWaves];
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        if (lane == 0) {
            red_v[wave] = v;
            red_i[wave] = i;
        }
        __syncthreads();
        v = red_v[0];
        i = red_i[0];
        for (int w = 1; w < kWaves; ++w) merge_argmax(v, i, red_v[w], red_i[w]);
        __syncthreads();
        *f0 = v;
        *f1 = __int_as_float(i);
        *d = 0.0;
    }

    __device__ void tile(int, int, int lo, int, const uint4* raw, int nvec, float* f0, float* f1,
                         double* d) const {
        constexpr int EPV = Elem<T>::kPerVec;
        float x[U][EPV];
        int first[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int v = threadIdx.x + j * kThreads;
            Elem<T>::widen(raw[j], x[j]);
            first[j] = lo + v * EPV;
        }
        if (nvec < U * kThreads) {  // ragged last chunk of a row: mask the padding
#pragma unroll
            for (int j = 0; j < U; ++j)
                if ((int)threadIdx.x + j * kThreads >= nvec) {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) x[j][e] = -INFINITY;
                    first[j] = INT_MAX - EPV;
                }
        }
        float bv = -INFINITY;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) bv = fmaxf(bv, x[j][e]);
        // Lowest index holding the maximum: walk from the highest slot down.
        int bi = INT_MAX;
#pragma unroll
        for (int j = U - 1; j >= 0; --j)
#pragma unroll
            for (int e = EPV - 1; e >= 0; --e) bi = (x[j][e] == bv) ? first[j] + e : bi;
        finish(bv, bi, f0, f1, d);
    }

    __device__ void tile_scalar(int b, int r, int lo, int hi, float* f0, float* f1,
                                double* d) const {
        const T* p = row(b, r);
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int j = lo + threadIdx.x; j < hi; j += kThreads) {
            const float x = Elem<T>::load(p, j);
            if (x > bv || bi == INT_MAX) {
                bv = x;
                bi = j;
            }
        }
        finish(bv, bi, f0, f1, d);
    }

    __device__ int row_argmax(int b, int r) const {
        const unsigned long long* p =
            reinterpret_cast<const unsigned long long*>(partials + ((size_t)b * R + r) * S);
        float v = -INFINITY;
        int i = INT_MAX;
        for (int ch = 0; ch < S; ++ch) {  // fixed chunk order
            const unsigned long long w = load_coherent(p + 2 * ch);
            merge_argmax(v, i, __uint_as_float((unsigned)w), (int)((w >> 32) & 0x7fffffffu));
        }
        return i;
    }

    // Argmax of row r of request b computed by this workgroup alone (any order
    // gives the same maximum and lowest index).
    __device__ int row_argmax_here(int b, int r) const {
        const T* p = row(b, r);
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int j = threadIdx.x; j < V; j += kThreads) {
            const float x = Elem<T>::load(p, j);
            if (x > bv || bi == INT_MAX) {
                bv = x;
                bi = j;
            }
        }
        wave_reduce_argmax(bv, bi);
        __shared__ float red_v[kWaves];
        __shared__ int red_i[kWaves];
        if ((threadIdx.x & 63) == 0) {
            red_v[threadIdx.x >> 6] = bv;
            red_i[threadIdx.x >> 6] = bi;
        }
        __syncthreads();
        bv = red_v[0];
        bi = red_i[0];
        for (int w = 1; w < kWaves; ++w) merge_argmax(bv, bi, red_v[w], red_i[w]);
        __syncthreads();
        return bi;
    }

    // The epilogue workgroup of request b: the argmax of rows 0 .. rows-1 (into
    // sh_a), from the published words (all R * S of the request, skipped rows'
    // too, are awaited, so none is published after they are cleared), or, past
    // the poll limit or on a stale workspace, computed here.  Returns whether
    // the words were used.
    __device__ bool gather_argmax(int b, int rows, int* sh_a) const {
        __shared__ int sh_ok;
        const int n = R * S;
        const unsigned long long* p =
            reinterpret_cast<const unsigned long long*>(partials + (size_t)b * n);
        if (threadIdx.x == 0) sh_ok = load_coherent(stale) == 0u;
        __syncthreads();
        bool use = sh_ok != 0;
        for (int it = 0; use; ++it) {
            int ok = 1;
            for (int t = threadIdx.x; t < n; t += kThreads)
                ok &= (load_coherent(p + 2 * t) >> 63) != 0ull;
            if (__syncthreads_and(ok)) break;
            if (it >= spin_limit) {
                use = false;
                if (threadIdx.x == 0) store_coherent(stale, 1u);
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (use) {
            for (int r = threadIdx.x; r < rows; r += kThreads) sh_a[r] = row_argmax(b, r);
        } else {
            for (int r = 0; r < rows; ++r) {
                const int i = row_argmax_here(b, r);
                if (threadIdx.x == 0) sh_a[r] = i;
            }
        }
        __syncthreads();
        return use;
    }

    // After the epilogue: the request's words back to zero (this workgroup is
    // their only reader), unless the workspace is stale.
    __device__ void clear_words(int b, bool used) const {
        __syncthreads();
        if (used) clear_partials(partials + (size_t)b * R * S, R * S);
    }

    __device__ void greedy_epilogue(int b) const {
        __shared__ int sh_a[kMaxK + 1];
        __shared__ int sh_s;
        const int kb = kb_of(b);
        const bool used = gather_argmax(b, kb + 1, sh_a);
        if (threadIdx.x == 0) {
            int s = 0;
            while (s < kb && draft_tokens[(size_t)b * k + s] == sh_a[s]) ++s;
            sh_s = s;
            num_accepted[b] = s;
        }
        __syncthreads();
        const int s = sh_s;
        for (int i = threadIdx.x; i <= k; i += kThreads) {
            int32_t v = -1;
            if (i < s) v = draft_tokens[(size_t)b * k + i];
            else if (i == s) v = sh_a[s];
            out_tokens[(size_t)b * (k + 1) + i] = v;
        }
        clear_words(b, used);
    }

    __device__ void tree_epilogue(int b) const {
        extern __shared__ int dyn[];
        int* sh_a = dyn;              // [N+1] argmax of each node's row
        int* sh_tok = dyn + (N + 1);  // [N+1] node tokens
        int* sh_paths = dyn + 2 * (N + 1);
        for (int n = threadIdx.x; n <= N; n += kThreads)
            sh_tok[n] = node_tokens[(size_t)b * (N + 1) + n];
        const bool used = gather_argmax(b, N + 1, sh_a);
        const int32_t* gpaths = paths + (size_t)b * P * L;
        if (paths_in_lds)
            for (int q = threadIdx.x; q < P * L; q += kThreads) sh_paths[q] = gpaths[q];
        __syncthreads();
        const int32_t* pt = paths_in_lds ? (const int32_t*)sh_paths : gpaths;

        int best_m = -1, best_p = INT_MAX;
        for (int p = threadIdx.x; p < P; p += kThreads) {
            const int32_t* rowp = pt + (size_t)p * L;
            const int r0 = rowp[0];
            if (r0 < 0 || r0 > N) continue;  // unused row
            int m = 0;
            while (m + 1 < L) {
                const int child = rowp[m + 1];
                if (child < 0 || child > N) break;
                if (sh_tok[child] != sh_a[rowp[m]]) break;
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
            const int m2 = __shfl_xor(best_m, off, 64);
            const int p2 = __shfl_xor(best_p, off, 64);
            const bool take = (m2 > best_m) || (m2 == best_m && p2 < best_p);
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
            const bool take = (red_m[w] > best_m) || (red_m[w] == best_m && red_p[w] < best_p);
            best_m = take ? red_m[w] : best_m;
            best_p = take ? red_p[w] : best_p;
        }
        const bool none = best_m < 0;
        const int m = none ? 0 : best_m;
        const int32_t* rowp = none ? nullptr : pt + (size_t)best_p * L;
        for (int t = threadIdx.x; t < L; t += kThreads) {
            int32_t tok = -1, node = -1;
            if (none) {
                if (t == 0) tok = sh_a[0];
            } else if (t < m) {
                node = rowp[t + 1];
                tok = sh_tok[node];
            } else if (t == m) {
                tok = sh_a[rowp[m]];
            }
            out_tokens[(size_t)b * L + t] = tok;
            if (accepted_nodes) accepted_nodes[(size_t)b * L + t] = node;
        }
        if (threadIdx.x == 0) {
            num_accepted[b] = m;
            if (best_path) best_path[b] = none ? -1 : best_p;
        }
        clear_words(b, used);
    }
};

// Polls of an epilogue workgroup for one request's words before it computes
// the maxima itself: far above any wait seen when workgroups are dispatched in
// order.
constexpr int kEpilogueSpin = 1 << 16;

template <typename T, int U, bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void argmax_kernel(ArgmaxArgs a) {
    ArgmaxOp<T, U, MODE> op;
    static_cast<ArgmaxArgs&>(op) = a;
    const int n_tiles = a.B * a.R * a.S;
    if ((int)blockIdx.x < n_tiles) {
        // Rows are read once (the epilogues read only the published maxima).
        if constexpr (VEC) stream_tile_vec<T, U, true>(op, blockIdx.x);
        else stream_tile_scalar<T>(op, blockIdx.x);
        return;
    }
    const int b = (int)blockIdx.x - n_tiles;
    if constexpr (MODE == 1) op.greedy_epilogue(b);
    else op.tree_epilogue(b);
}

// One kernel: the streaming tiles, then one epilogue workgroup per request (the
// profiling events, when set, take its start and end).  `lds` is the tree
// epilogue's dynamic LDS.
template <typename T, int U, bool VEC, int MODE>
static hipError_t launch_argmax_u(const ArgmaxArgs& a, size_t lds, hipStream_t st,
                                  const KernelEvents& ev) {
    const unsigned grid = (unsigned)((long long)a.B * a.R * a.S + a.B);
    hipExtLaunchKernelGGL(argmax_kernel<T, U, VEC, MODE>, dim3(grid), dim3(kThreads), lds, st,
                          ev.begin, ev.end, 0, a);
    return hipGetLastError();
}

template <typename T, bool VEC, int MODE>
static hipError_t launch_argmax(const ArgmaxArgs& a, int U, size_t lds, hipStream_t st,
                                const KernelEvents& ev) {
    switch (U) {
        case 16: return launch_argmax_u<T, 16, VEC, MODE>(a, lds, st, ev);
        case 8: return launch_argmax_u<T, 8, VEC, MODE>(a, lds, st, ev);
        case 4: return launch_argmax_u<T, 4, VEC, MODE>(a, lds, st, ev);
        case 2: return launch_argmax_u<T, 2, VEC, MODE>(a, lds, st, ev);
        default: return launch_argmax_u<T, 1, VEC, MODE>(a, lds, st, ev);
    }
}

template <int MODE>
static hipError_t dispatch(const ArgmaxArgs& a, int dtype, bool vec, int U, size_t lds,
                           hipStream_t st, const KernelEvents& ev) {
    if (dtype == 1)
        return vec ? launch_argmax<bf16_t, true, MODE>(a, U, lds, st, ev)
                   : launch_argmax<bf16_t, false, MODE>(a, U, lds, st, ev);
    return vec ? launch_argmax<float, true, MODE>(a, U, lds, st, ev)
               : launch_argmax<float, false, MODE>(a, U, lds, st, ev);
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
    a.partials = reinterpret_cast<Partial16*>(ws + g.off_partials);
    a.stale = reinterpret_cast<uint32_t*>(ws + g.off_tickets) + 8;
    a.spin_limit = debug_spin_limit(kEpilogueSpin);
    return a;
}

hipError_t run_greedy(const GreedyCall& c, const Geometry& g, hipStream_t st,
                      const KernelEvents& ev) {
    ArgmaxArgs a = base_args(c.target, c.B, c.k + 1, c.V, g, c.workspace);
    a.draft_tokens = c.draft_tokens;
    a.lens = c.draft_lens;
    a.k = c.k;
    a.out_tokens = c.out_tokens;
    a.num_accepted = c.num_accepted;
    return dispatch<1>(a, c.dtype, c.vec, g.U, 0, st, ev);
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
    return dispatch<2>(a, c.dtype, c.vec, g.U, lds, st, ev);
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
