// sv_stochastic.hip -- stochastic verification (speculative sampling).
//
// Rule (page "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
// section "Speculative Decoding"; page "02. Speculative Decoding" of the vLLM
// learning book, section 2 flowchart): draft token i is accepted when
// p_i(x_i) >= q_i(x_i), otherwise with probability p_i(x_i) / q_i(x_i); the
// first rejection at row s ends the scan and one token is drawn from
// max(0, p_s - q_s) renormalised; if all k drafts pass, one bonus token is drawn
// from the extra target row p_k.
//
// Two kernels:
//   stats:   one workgroup per (request, logits row, vocabulary chunk).  Reads
//            its chunk once with 16-byte loads and reduces it to softmax
//            statistics: the chunk max m and s = sum of 2^((x - m) * log2(e)/T).
//            Each thread sums its own elements against its own maximum (so a
//            row's largest logits, each usually the maximum of its thread,
//            contribute an exact 1) in fp64, and threads are merged with fp64
//            scale factors.
//   sample:  one workgroup per (request, stop-row chunk).  Every workgroup of a
//            request first merges that request's partials (chunk order, fp64),
//            gathers the tested logits, computes p_i(x_i) and q_i(x_i), runs the
//            k tests (independent given the uniforms) and takes the first
//            failure as the stop row s; the chunk-0 workgroup writes the
//            accepted drafts, the -1 padding, num_accepted and the
//            probabilities.  Each workgroup then weighs its chunk of the final
//            distribution (residual max(0, p_s - q_s) or bonus p_k) in fp64 --
//            tokens within 2^-8 of the row maximum take an fp64 exponential,
//            the rest fp32 -- and stores the mass of every 64-token segment.
//            The last of the request's workgroups (arrival ticket) finds the
//            segment holding u_k * Z by a prefix sum over the segment masses,
//            then the token inside it by a wave-wide prefix sum (ascending
//            vocabulary order: the smallest j whose running mass exceeds
//            u_k * Z).
// The streaming kernel has no atomics or fences: the kernel boundary publishes
// its partials to the sampler.
//
// Accuracy matters beyond the decisions themselves: a vocabulary of ~10^5 has
// ~10^5 CDF edges, so a relative error e in the cumulative weights moves the
// drawn token on a fraction ~V * e of the draws.  The fp64 paths above keep e
// near 1e-10.
#include <algorithm>
#include <atomic>

#include "sv_common.hpp"
#include "sv_launch.hpp"
#include "sv_stream.hpp"

// Lookahead of the one-launch grid, fixed for tuning (< 0: chosen per call).
#ifndef SV_LOOKAHEAD
#define SV_LOOKAHEAD -1
#endif

namespace sv {

struct CallArgs {
    const void* target;
    const void* draft;
    const int32_t* draft_tokens;
    const int32_t* lens;     // [B] draft length per request, or null (all k)
    const float* uniforms;   // [B, k+1], or null: counter-based draws from (seed, offset)
    unsigned long long seed, offset;
    int B, k, V;
    int R, S, chunk;         // streaming geometry: rows per request, chunks per row
    int S2, chunk2;          // sampler geometry: chunks per stop row
    Scale sc;                // log2(e) / temperature
    Partial16* partials;     // [B, 2k+1, S]: f0 = chunk max, f1 = written flag, d = sum
    int spin_limit;          // polls of unpublished partials before computing them here
    uint32_t* tickets;       // per request (padded): sampler arrivals
    double* segs;            // per request: stop-row mass per 64-token segment, run-major
    int32_t* out_tokens;     // [B, k+1]
    int32_t* num_accepted;   // [B]
    float* p_at_draft;       // [B, k] or null
    float* q_at_draft;       // [B, k] or null
    RowFilter* rowf;         // [B, 2k+1] sampling filter per row (filtered call), else null
    unsigned long long* masses;   // [B, S2] stop-row chunk masses, bitwise complemented (0: none)
    int lookahead;           // one-launch grid: items of request b follow the tiles of b + lookahead
    int nontemporal;         // one-launch grid: tiles load with non-temporal hints
    int self_compute;        // items compute every partial themselves (no tiles in the grid)
};

// Draft length of request b: lens[b] clamped to [0, k] (per-request windows in
// buffers padded to k; page "TensorRT-LLM source teardown (10)", acceptance
// pipeline, step 2), or k.
__device__ inline int draft_len(const CallArgs& a, int b) {
    if (!a.lens) return a.k;
    return min(max(a.lens[b], 0), a.k);
}

// Whether logits row r of request b (r = 0..k target, k+1.. draft) lies past
// the request's draft window and is never read.
__device__ inline bool row_unused(const CallArgs& a, int b, int r) {
    if (!a.lens) return false;
    const int kb = draft_len(a, b);
    return (r <= a.k) ? (r > kb) : (r - a.k - 1 >= kb);
}

// Counter-based uniforms (page "TensorRT-LLM source teardown (10)", "Rejection
// sampling": a per-call seed and offset instead of an input tensor).
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC 2011): ten rounds, each multiplying counter words 0 and 2 by
// two odd 64-bit constants (128-bit products), XORing the high halves with the
// other two words and the key, and keeping the low halves; the key advances by
// two Weyl constants between rounds.  Draw i of request b is word i % 4 of the
// block at counter (offset, b, i / 4, 0) with key (seed, 0), as its top 24
// bits times 2^-24: exact in float32, in [0, 1).
__device__ inline float philox_uniform(unsigned long long seed, unsigned long long offset, int b,
                                       int i) {
    unsigned long long c0 = offset, c1 = (unsigned long long)b, c2 = (unsigned long long)(i / 4),
                       c3 = 0ull;
    unsigned long long k0 = seed, k1 = 0ull;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B97F4A7C15ull;
            k1 += 0xBB67AE8584CAA73Bull;
        }
        const unsigned long long m0 = 0xD2E7470EE14C6C93ull, m1 = 0xCA5A826395121157ull;
        const unsigned long long hi0 = __umul64hi(m0, c0), lo0 = m0 * c0;
        const unsigned long long hi1 = __umul64hi(m1, c2), lo1 = m1 * c2;
        const unsigned long long n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    const int w = i % 4;
    const unsigned long long word = w == 0 ? c0 : w == 1 ? c1 : w == 2 ? c2 : c3;
    return (float)(word >> 40) * 0x1p-24f;
}

// Draw i of request b: the input tensor's uniforms[b, i], or the counter-based one.
__device__ inline float uniform_at(const CallArgs& a, int b, int i) {
    if (a.uniforms) return a.uniforms[(size_t)b * (a.k + 1) + i];
    return philox_uniform(a.seed, a.offset, b, i);
}

// p(x) = 2^((x - M) * c) / S in fp64; 0 when x or the whole row is -inf.
__device__ inline double prob_of(float x, float M, double S, double c256, const double* tab) {
    if (M == -INFINITY || !(S > 0.0)) return 0.0;
    return exp2_table(x, M, c256, tab) / S;
}

// ---------------------------------------------------------------------------
// Streaming statistics.  Row order within request b: r = 0..k target rows,
// r = k+1..2k draft rows 0..k-1.
// ---------------------------------------------------------------------------
template <typename T, int U>
struct StatsOp : CallArgs {
    __device__ const T* row(int b, int r) const {
        if (r <= k) return static_cast<const T*>(target) + ((size_t)b * (k + 1) + r) * (size_t)V;
        return static_cast<const T*>(draft) + ((size_t)b * k + (r - k - 1)) * (size_t)V;
    }

    __device__ void publish(Partial16* dst, float f0, float f1, double d) const;
    // Rows past a request's draft window are not read; their partial is the
    // one of an all -inf chunk.
    __device__ bool skip(int b, int r) const { return row_unused(*this, b, r); }
    __device__ void publish_skipped(Partial16* dst) const {
        publish(dst, -INFINITY, kPartialWritten, 1.0);
    }

    // Workgroup reduction of per-thread (max m, fp64 sum s against m) into the
    // tile's (M, S): every thread's sum is rescaled to the common M with an fp64
    // exponential, then summed in fixed order.
    __device__ __forceinline__ void finish(float m, double s, float* f0, float* f1, double* d) const {
        __shared__ float red_f[kWaves];
        __shared__ double red_d[kWaves];
        const float M = block_max(m, red_f);
        const double f = (m == -INFINITY) ? 0.0 : exp2_accurate(m, M, sc);
        const double Ssum = block_sum(s * f, red_d);
        *f0 = M;
        *f1 = kPartialWritten;
        // A chunk with a finite max sums to >= 1 (its largest logit counts 1);
        // an all -inf chunk, whose weight in every merge is 0, stores 1.  So a
        // published partial never reads back as the cleared (all-zero) state.
        *d = (M == -INFINITY) ? 1.0 : Ssum;
    }

    __device__ __forceinline__ void tile(int b, int r, int lo, int hi, const uint4* raw, int nvec,
                                         float* f0, float* f1, double* d) const {
        constexpr int EPV = Elem<T>::kPerVec;
        float x[U][EPV];
#pragma unroll
        for (int j = 0; j < U; ++j) Elem<T>::widen(raw[j], x[j]);
        if (nvec < U * kThreads) {  // ragged last chunk of a row: mask the padding
#pragma unroll
            for (int j = 0; j < U; ++j)
                if ((int)threadIdx.x + j * kThreads >= nvec)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) x[j][e] = -INFINITY;
        }
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) m = fmaxf(m, x[j][e]);
        // The terms of each 16-byte vector are summed in fp32, the vectors' sums
        // in fp64.
        const float ms = (m == -INFINITY) ? 0.f : m;
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float g = 0.f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) g += fast_exp2(scaled(x[j][e] - ms, sc));
            s += (double)g;
        }
        finish(m, s, f0, f1, d);
    }

    __device__ __forceinline__ void tile_scalar(int b, int r, int lo, int hi, float* f0, float* f1,
                                                double* d) const {
        const T* p = row(b, r);
        float m = -INFINITY;
        for (int j = lo + threadIdx.x; j < hi; j += kThreads) m = fmaxf(m, Elem<T>::load(p, j));
        const float ms = (m == -INFINITY) ? 0.f : m;
        double s = 0.0;
        for (int j = lo + threadIdx.x; j < hi; j += kThreads)
            s += (double)fast_exp2(scaled(Elem<T>::load(p, j) - ms, sc));
        finish(m, s, f0, f1, d);
    }
};

// Publish a statistics partial for readers in the same launch: two 8-byte
// agent-coherent stores, each half carrying its own proof of publication
// (f1 == written flag; d != 0).
__device__ inline void publish_partial(Partial16* dst, float f0, float f1, double d) {
    unsigned long long* q = reinterpret_cast<unsigned long long*>(dst);
    store_coherent(q + 1, (unsigned long long)__double_as_longlong(d));
    store_coherent(q, ((unsigned long long)__float_as_uint(f1) << 32) | __float_as_uint(f0));
}

// Statistics tile t of a 16-byte aligned problem with a runtime vector count:
// the same element-to-thread mapping and the same operation order as
// StatsOp::tile (masked slots add exactly 0 there), hence the same bits.  Used
// by a sampler workgroup that computes partials itself instead of waiting.
template <typename T>
__device__ __forceinline__ void stats_tile_runtime(const CallArgs& a, int t, float* f0, float* f1, double* d) {
    constexpr int EPV = Elem<T>::kPerVec;
    StatsOp<T, 1> op;
    static_cast<CallArgs&>(op) = a;
    const int U = a.chunk / (kThreads * EPV);
    const int ch = t % a.S, rr = t / a.S;
    const int r = rr % a.R, b = rr / a.R;
    if (op.skip(b, r)) {
        *f0 = -INFINITY;
        *f1 = kPartialWritten;
        *d = 1.0;
        return;
    }
    const int lo = ch * a.chunk, hi = min(a.V, lo + a.chunk);
    const int nvec = (hi - lo) / EPV;
    const uint4* base = reinterpret_cast<const uint4*>(op.row(b, r) + lo);
    float m = -INFINITY;
    for (int j = 0; j < U; ++j) {
        const int v = (int)threadIdx.x + j * kThreads;
        if (v < nvec) {
            float x[EPV];
            Elem<T>::widen(base[v], x);
            for (int e = 0; e < EPV; ++e) m = fmaxf(m, x[e]);
        }
    }
    const float ms = (m == -INFINITY) ? 0.f : m;
    double s = 0.0;
    for (int j = 0; j < U; ++j) {
        const int v = (int)threadIdx.x + j * kThreads;
        if (v < nvec) {
            float x[EPV];
            Elem<T>::widen(base[v], x);
            float g = 0.f;
            for (int e = 0; e < EPV; ++e) g += fast_exp2(scaled(x[e] - ms, a.sc));
            s += (double)g;
        }
    }
    op.finish(m, s, f0, f1, d);
}

template <typename T, int U>
__device__ void StatsOp<T, U>::publish(Partial16* dst, float f0, float f1, double d) const {
    publish_partial(dst, f0, f1, d);
}

template <typename T, int U, bool VEC>
__global__ __launch_bounds__(kThreads) void stats_kernel(CallArgs a) {
    StatsOp<T, U> op;
    static_cast<CallArgs&>(op) = a;
    if constexpr (VEC) stream_tile_vec<T, U>(op, blockIdx.x);
    else stream_tile_scalar<T>(op, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Sampler: decision, stop-row mass, final draw.
// ---------------------------------------------------------------------------

// The request's decision, computed by every sampler workgroup of the request
// from the streaming partials (fixed chunk order, fp64).
struct Decision {
    int s, kb;  // stop row, draft length
    float mt, md;
    double st, sd;
    float taut, taud;  // filter thresholds of the stop rows (-inf: unfiltered)
};

static_assert(kMaxK < kThreads, "one test per thread");
constexpr int kMergeLds = 1024;  // partials per request staged in LDS for the merge

// Row statistics of request b from its n = R * S partials staged in LDS
// (pm[t] = chunk max, ps[t] = chunk sum): sh_m[r] = row max, sh_s[r] = sum of
// 2^((x - max) * c) in fp64, chunks merged in chunk order.  ps is overwritten.
__device__ __forceinline__ void merge_staged(const CallArgs& a, const float* pm, double* ps,
                                             float* sh_m, double* sh_s, const double* tab) {
    const int R = a.R, S = a.S, n = R * S;
    for (int r = threadIdx.x; r < R; r += kThreads) {
        float M = -INFINITY;
        for (int ch = 0; ch < S; ++ch) M = fmaxf(M, pm[r * S + ch]);
        sh_m[r] = M;
    }
    __syncthreads();
    // every thread takes a few partials: one fp64 exponential each
    for (int t = threadIdx.x; t < n; t += kThreads) {
        const float M = sh_m[t / S];
        ps[t] = (M == -INFINITY) ? 0.0 : ps[t] * exp2_table(pm[t], M, a.sc.c64 * 256.0, tab);
    }
    __syncthreads();
    for (int r = threadIdx.x; r < R; r += kThreads) {
        double acc = 0.0;
        for (int ch = 0; ch < S; ++ch) acc += ps[r * S + ch];  // fixed chunk order
        sh_s[r] = acc;
    }
    __syncthreads();
}

// The same from partials read in global memory (every one of which the caller
// has seen published), for requests of more than kMergeLds partials: the same
// values in the same order, so the same bits.
template <typename T>
__device__ __forceinline__ void merge_rows(const CallArgs& a, int b, float* sh_m, double* sh_s,
                                           const double* tab) {
    const int R = a.R, S = a.S, n = R * S;
    const Partial16* p = a.partials + (size_t)b * n;
    for (int r = threadIdx.x; r < R; r += kThreads) {
        const Partial16* q = p + (size_t)r * S;
        float M = -INFINITY;
        for (int ch = 0; ch < S; ++ch) M = fmaxf(M, read_partial(q + ch).f0);
        double acc = 0.0;
        if (M != -INFINITY)
            for (int ch = 0; ch < S; ++ch) {
                const PartialRead e = read_partial(q + ch);
                acc += e.d * exp2_table(e.f0, M, a.sc.c64 * 256.0, tab);
            }
        sh_m[r] = M;
        sh_s[r] = acc;
    }
    __syncthreads();
}

// Statistics tile t (request-major numbering) computed by this workgroup, with
// the element-to-thread mapping and operation order of the streaming tile, so
// the same bits as the partial its owner publishes.  Every thread gets them.
template <typename T, bool VEC>
__device__ __forceinline__ void stats_tile_any(const CallArgs& a, int t, float* m, double* s) {
    float f1;
    if constexpr (VEC) {
        stats_tile_runtime<T>(a, t, m, &f1, s);
    } else {
        StatsOp<T, 1> op;
        static_cast<CallArgs&>(op) = a;
        const int ch = t % a.S, rr = t / a.S;
        const int r = rr % a.R, b = rr / a.R;
        if (op.skip(b, r)) {
            *m = -INFINITY;
            *s = 1.0;
            return;
        }
        const int lo = ch * a.chunk, hi = min(a.V, lo + a.chunk);
        op.tile_scalar(b, r, lo, hi, m, &f1, s);
    }
}

// Partial t of request b as every thread sees it: the published one (when
// use_published), or, where it is not (yet, or any more) published, computed
// here.  Nothing is written.
template <typename T, bool VEC>
__device__ __forceinline__ void partial_here(const CallArgs& a, int b, int t, bool use_published, float* m,
                             double* s) {
    __shared__ float sh_pm;
    __shared__ double sh_ps;
    __shared__ int sh_ok;
    const int n = a.R * a.S;
    if (threadIdx.x == 0) {
        const PartialRead q = use_published ? read_partial(a.partials + (size_t)b * n + t)
                                            : PartialRead{0.f, false, 0.0};
        sh_ok = q.ok;
        sh_pm = q.f0;
        sh_ps = q.d;
    }
    __syncthreads();
    const bool ok = sh_ok != 0;
    *m = sh_pm;
    *s = sh_ps;
    __syncthreads();
    if (!ok) stats_tile_any<T, VEC>(a, b * n + t, m, s);
}

// merge_rows computed by one workgroup: the same maxima and sums in the same
// order, each partial taken as published (when use_published) or computed here
// (partial_here), so the same bits.  Slow (one partial at a time).
template <typename T, bool VEC>
__device__ __forceinline__ void merge_rows_here(const CallArgs& a, int b, float* sh_m, double* sh_s,
                                bool use_published, const double* tab) {
    const int R = a.R, S = a.S;
    for (int r = 0; r < R; ++r) {
        float M = -INFINITY, m;
        double s;
        for (int ch = 0; ch < S; ++ch) {
            partial_here<T, VEC>(a, b, r * S + ch, use_published, &m, &s);
            M = fmaxf(M, m);
        }
        double acc = 0.0;
        if (M != -INFINITY)
            for (int ch = 0; ch < S; ++ch) {
                partial_here<T, VEC>(a, b, r * S + ch, use_published, &m, &s);
                acc += s * exp2_table(m, M, a.sc.c64 * 256.0, tab);
            }
        if (threadIdx.x == 0) {
            sh_m[r] = M;
            sh_s[r] = acc;
        }
    }
    __syncthreads();
}

// Wave 1 loads the tested logits target[b, i, x_i] and draft[b, i, x_i]
// (i < kb) into sh_g[i] and sh_g[k + 1 + i]; they are read after the next
// barrier.  An id outside [0, V) leaves -inf (the test rejects it).
template <typename T>
__device__ inline void gather_tested(const CallArgs& a, int b, int kb, float* sh_g) {
    const int k = a.k;
    if (threadIdx.x >= 64 && threadIdx.x < 64 + kb) {
        const int i = threadIdx.x - 64;
        const int32_t x = a.draft_tokens[(size_t)b * k + i];
        float gt = -INFINITY, gd = -INFINITY;
        if (x >= 0 && x < a.V) {
            gt = Elem<T>::load(static_cast<const T*>(a.target) + ((size_t)b * (k + 1) + i) * (size_t)a.V, x);
            gd = Elem<T>::load(static_cast<const T*>(a.draft) + ((size_t)b * k + i) * (size_t)a.V, x);
        }
        sh_g[i] = gt;
        sh_g[k + 1 + i] = gd;
    }
}

// Test i's draft token and uniform, loaded by thread i (i < kb) ahead of the
// statistics they are compared with.
__device__ inline void load_test_inputs(const CallArgs& a, int b, int kb, int32_t* x, float* u) {
    const int i = threadIdx.x;
    *x = 0;
    *u = 0.f;
    if (i < kb) {
        *x = a.draft_tokens[(size_t)b * a.k + i];
        *u = uniform_at(a, b, i);
    }
}

// The tests of request b, all at once (thread i runs test i; they are
// independent given the uniforms), from its rows' maxima sh_m and masses sh_s
// (with FILT, thresholds sh_tau) and the tested logits sh_g.  Returns the stop
// row: the first rejected i, or kb.  With write_outputs it also writes the
// accepted drafts, the -1 padding, num_accepted, P and Q (out_tokens[b, s] is
// the final draw's).
template <bool FILT>
__device__ int run_tests(const CallArgs& a, int b, int kb, int32_t x, float u, const float* sh_m,
                         const double* sh_s, const float* sh_tau, const float* sh_g,
                         bool write_outputs, const double* tab) {
    __shared__ int sh_acc[kMaxK];
    __shared__ int sh_stop;
    const int k = a.k;
    const int i = threadIdx.x;
    if (i < k) {  // past the window (i >= kb): no test, P = Q = 0 reported
        double P = 0.0, Q = 0.0;
        int acc = 0;
        if (i < kb && x >= 0 && x < a.V) {
            const float gt = sh_g[i], gd = sh_g[k + 1 + i];
            // A token below its row's filter threshold has probability 0.
            const double c256 = a.sc.c64 * 256.0;
            if (!FILT || gt >= sh_tau[i]) P = prob_of(gt, sh_m[i], sh_s[i], c256, tab);
            if (!FILT || gd >= sh_tau[k + 1 + i]) Q = prob_of(gd, sh_m[k + 1 + i], sh_s[k + 1 + i], c256, tab);
            acc = (P >= Q) || ((double)u * Q < P);  // strict u < min(1, P/Q), no division
        }
        sh_acc[i] = acc;
        if (write_outputs) {
            if (a.p_at_draft) a.p_at_draft[(size_t)b * k + i] = (float)P;
            if (a.q_at_draft) a.q_at_draft[(size_t)b * k + i] = (float)Q;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = kb;
        for (int j = 0; j < kb; ++j)
            if (!sh_acc[j]) { s = j; break; }
        sh_stop = s;
        if (write_outputs) a.num_accepted[b] = s;
    }
    __syncthreads();
    const int s = sh_stop;
    if (write_outputs) {
        // Thread j holds draft token j (x, for j < kb) already: k < kThreads.
        const int j = threadIdx.x;
        if (j < s) a.out_tokens[(size_t)b * (k + 1) + j] = x;
        else if (j > s && j <= k) a.out_tokens[(size_t)b * (k + 1) + j] = -1;
    }
    __syncthreads();
    return s;
}

template <typename T, bool FILT>
__device__ void decide(const CallArgs& a, int b, bool write_outputs, Decision* out, const double* tab) {
    __shared__ float sh_m[2 * kMaxK + 1], sh_g[2 * kMaxK + 1], sh_tau[2 * kMaxK + 1];
    __shared__ double sh_s[2 * kMaxK + 1];
    const int k = a.k;
    const int kb = draft_len(a, b);
    // Wave 1 gathers the tested logits while wave 0 merges the partials.
    gather_tested<T>(a, b, kb, sh_g);
    int32_t x;
    float u;
    load_test_inputs(a, b, kb, &x, &u);
    if constexpr (FILT) {
        // Filtered rows: maximum, kept mass and threshold from the selection kernel.
        for (int r = threadIdx.x; r < a.R; r += kThreads) {
            const RowFilter f = a.rowf[(size_t)b * a.R + r];
            sh_m[r] = f.m;
            sh_s[r] = f.s;
            sh_tau[r] = f.tau;
        }
        __syncthreads();
    } else {
        merge_rows<T>(a, b, sh_m, sh_s, tab);
    }
    const int s = run_tests<FILT>(a, b, kb, x, u, sh_m, sh_s, sh_tau, sh_g, write_outputs, tab);
    out->s = s;
    out->kb = kb;
    out->mt = sh_m[s];
    out->st = sh_s[s];
    out->md = (s < kb) ? sh_m[k + 1 + s] : 0.f;
    out->sd = (s < kb) ? sh_s[k + 1 + s] : 1.0;
    out->taut = FILT ? sh_tau[s] : -INFINITY;
    out->taud = (FILT && s < kb) ? sh_tau[k + 1 + s] : -INFINITY;
    __syncthreads();
}

// Weight of one token in the final draw, in fp64, scaled by the target row's
// softmax sum S_t (the scale cancels against the total Z): the residual
// S_t * max(0, p - q) = max(0, e_t - r e_d) with r = S_t / S_d when the request
// stopped on a rejection, else S_t * p = e_t.  Here e = 2^((x - row max) * c).
// Tokens within 2^-8 of their row's maximum (the few that carry most of the
// mass) take the fp64 exponential; the others the fp32 one, whose error is
// then negligible against the total.  Filtered rows (FILT) weigh a token below
// the row's threshold as 0.
struct Weigher {
    float mt, md;
    double r;
    double c256;         // 256 log2(e) / T
    const double* tab;   // 2^(j / 256), j < 256 (exp2_table)
    float r32;     // r rounded to fp32
    float ad_big;  // draft exponent above which r e_d may pass 2^-8: -8 - log2(r)
    Scale sc;
    bool residual;
    float taut, taud;
    __device__ inline void set_ratio(double ratio) {
        r = ratio;
        r32 = (float)ratio;
        ad_big = -8.f - log2f(r32);
    }
    __device__ inline double e_of(float x, float m) const {
        const float a = scaled(x - m, sc);
        if (a > -8.f) return exp2_table(x, m, c256, tab);
        return (double)fast_exp2(a);
    }
    template <bool RESID, bool FILT>
    __device__ inline double w(float xt, float xd) const {
        const double et = (!FILT || xt >= taut) ? e_of(xt, mt) : 0.0;
        if constexpr (!RESID) return et;
        const double ed = (!FILT || xd >= taud) ? e_of(xd, md) : 0.0;
        return fmax(fma(-r, ed, et), 0.0);
    }
    template <bool FILT>
    __device__ inline double weigh(float xt, float xd) const {
        return residual ? w<true, FILT>(xt, xd) : w<false, FILT>(xt, xd);
    }
    // Add one token's weight to a segment sum: a token whose terms may pass
    // 2^-8 (of the target row's maximum weight) as w() gives it, in fp64;
    // every other token entirely in fp32 (its exponentials are the fp32 ones
    // of w() already), summed apart and added to the fp64 sum once.
    template <bool RESID, bool FILT>
    __device__ inline void add(float xt, float xd, double& big, float& small) const {
        const bool kt = !FILT || xt >= taut;
        const float at = scaled(xt - mt, sc);
        if constexpr (!RESID) {
            if (!kt) return;
            if (at > -8.f) big += exp2_table(xt, mt, c256, tab);
            else small += fast_exp2(at);
        } else {
            const bool kd = !FILT || xd >= taud;
            const float ad = scaled(xd - md, sc);
            if ((kt && at > -8.f) || (kd && ad > ad_big)) {
                big += w<true, FILT>(xt, xd);
            } else {
                const float et = kt ? fast_exp2(at) : 0.f;
                const float ed = kd ? fast_exp2(ad) : 0.f;
                small += fmaxf(fmaf(-r32, ed, et), 0.f);
            }
        }
    }
};

constexpr int kSub = 8;  // tokens per sampler sub-step

// Sum of the weights of this thread's segment of the chunk [lo, hi): the
// NSUB * 16 consecutive tokens from lo + t * NSUB * 16.  Each pass issues up to
// four 16-byte loads per row back to back (clamped in bounds; slots past hi are
// masked); the draft row is read only for a residual.  The per-token bound test
// stays a branch even in full chunks: it keeps the compiler from interleaving
// all of the segment's tokens, whose registers would cost occupancy.
template <typename T, bool VEC, int NSUB, bool RESID, bool FILT>
__device__ double segment_sum(const T* trow, const T* drow, const Weigher& W, int lo, int hi) {
    constexpr int SEG = NSUB * kSub;
    const int start = lo + (int)threadIdx.x * SEG;
    double seg = 0.0;
    float small = 0.f;
    if constexpr (VEC) {
        constexpr int EPV = Elem<T>::kPerVec;
        constexpr int NV = SEG / EPV;                  // vectors per row in the segment
        constexpr int NVP = NV < 4 ? NV : 4;           // vectors per row per pass
#pragma unroll 1
        for (int v0 = 0; v0 < NV; v0 += NVP) {
            uint4 rt[NVP], rd[NVP];
#pragma unroll
            for (int v = 0; v < NVP; ++v) {
                const int j = max(lo, min(start + (v0 + v) * EPV, hi - EPV));
                rt[v] = load16(trow + j);
                if constexpr (RESID) rd[v] = load16(drow + j);
            }
#pragma unroll
            for (int v = 0; v < NVP; ++v) {
                float xt[EPV], xd[EPV];
                Elem<T>::widen(rt[v], xt);
                if constexpr (RESID) Elem<T>::widen(rd[v], xd);
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    if (start + (v0 + v) * EPV + e < hi)
                        W.template add<RESID, FILT>(xt[e], RESID ? xd[e] : 0.f, seg, small);
            }
        }
    } else {
#pragma unroll 1
        for (int s0 = 0; s0 < SEG; s0 += kSub) {
            float xt[kSub], xd[kSub];
#pragma unroll
            for (int e = 0; e < kSub; ++e) {
                const int j = max(lo, min(start + s0 + e, hi - 1));
                xt[e] = Elem<T>::load(trow, j);
                xd[e] = RESID ? Elem<T>::load(drow, j) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < kSub; ++e)
                if (start + s0 + e < hi) W.template add<RESID, FILT>(xt[e], xd[e], seg, small);
        }
    }
    return seg + (double)small;
}

template <typename T, bool VEC, int NSUB, bool FILT>
__device__ inline double segment_sum_any(const T* trow, const T* drow, const Weigher& W, int lo,
                                         int hi) {
    return W.residual ? segment_sum<T, VEC, NSUB, true, FILT>(trow, drow, W, lo, hi)
                      : segment_sum<T, VEC, NSUB, false, FILT>(trow, drow, W, lo, hi);
}


// The stop row's mass is kept per 64-token segment (segment f covers tokens
// [64 f, 64 f + 64)).  A request's n segments are split into 256 runs of
// G = ceil(n / 256) consecutive segments; segment f is stored at
// (f % G) * 256 + f / G, so that the final draw's thread t, which owns run t,
// reads slot g of all runs with one coalesced load per g.
constexpr int kStoredSeg = 64;
constexpr int kRegSegs = 10;  // run slots a thread of the final draw keeps in registers

struct SegLayout {
    int n;  // stored segments per request
    int G;  // run length
    __device__ SegLayout(const CallArgs& a)
        : n(a.S2 * (a.chunk2 / kStoredSeg)), G((a.S2 * (a.chunk2 / kStoredSeg) + kThreads - 1) / kThreads) {}
    __device__ size_t per_request() const { return (size_t)G * kThreads; }
    __device__ size_t slot(int f) const { return (size_t)(f % G) * kThreads + f / G; }
};

// The 4 / NSUB threads that weigh one segment add their sums (in thread order;
// the partner lanes are in the same DPP row) and the first of them stores it.
template <int NSUB>
__device__ inline void store_segment(double* req_segs, const SegLayout& L, int ch, int chunk2,
                                     double seg) {
    constexpr int P = kStoredSeg / (NSUB * kSub);  // threads per stored segment
    static_assert(P >= 1 && P * NSUB * kSub == kStoredSeg, "segment split");
    if constexpr (P >= 2) seg += dpp_f64<dpp::kRowShl + 1>(seg);
    if constexpr (P >= 4) seg += dpp_f64<dpp::kRowShl + 2>(seg);
    if (threadIdx.x % P == 0) {
        const int f = ch * (chunk2 / kStoredSeg) + threadIdx.x / P;
        store_coherent(&req_segs[L.slot(f)], seg);
    }
}

// The last workgroup of request b draws the token: a prefix sum over the runs
// finds the run holding u_k * Z, its owner walks it to the segment, and wave 0
// walks that segment's tokens with a wave-wide prefix sum, one token per lane.
// Each level takes the first entry with positive weight whose running mass
// exceeds u_k * Z; where rounding leaves every running mass at or below it, the
// last entry with positive weight.
template <typename T, bool VEC, int NSUB, bool FILT>
__device__ void sample_final(const CallArgs& a, int b, int s_row, int kb, const T* trow,
                             const T* drow, Weigher W) {
    __shared__ double sh_wave[kWaves];
    __shared__ int sh_first[kWaves], sh_last[kWaves], sh_seg;
    __shared__ double sh_run0;
    const int k = a.k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const SegLayout L(a);
    const int n = L.n, G = L.G;
    const int first = tid * G;
    const int len = max(0, min(G, n - first));   // this thread's run: segments [first, first + len)
    double* segs = a.segs + (size_t)b * L.per_request();
    const double u = (double)uniform_at(a, b, kb);  // the final draw's uniform

    double v[kRegSegs];
    double grp, incl, Z;
    for (int pass = 0;; ++pass) {
        // Slot g of every run is one coalesced load; all loads issue together.
#pragma unroll
        for (int g = 0; g < kRegSegs; ++g)
            v[g] = load_coherent(segs + (size_t)min(g, G - 1) * kThreads + tid);
#pragma unroll
        for (int g = 0; g < kRegSegs; ++g) v[g] = (g < len) ? v[g] : 0.0;
        grp = 0.0;
#pragma unroll
        for (int g = 0; g < kRegSegs; ++g) grp += v[g];
        for (int g = kRegSegs; g < len; ++g) grp += load_coherent(segs + (size_t)g * kThreads + tid);
        incl = block_inclusive_scan(grp, sh_wave, &Z);
        if (Z > 0.0 || pass == 1) break;
        // The residual vanished (p_s == q_s): draw from p_s instead.
        W.residual = false;
        drow = trow;
        for (int c = 0; c < a.S2; ++c) {
            const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
            store_segment<NSUB>(segs, L, c, a.chunk2,
                                segment_sum<T, VEC, NSUB, false, FILT>(trow, drow, W, lo, hi));
        }
        wait_stores();
        __syncthreads();
    }
    const double tau = u * Z;
    // First run whose running mass exceeds tau, and last run with positive mass.
    {
        const unsigned long long over_m = __ballot(grp > 0.0 && incl > tau);
        const unsigned long long pos_m = __ballot(grp > 0.0);
        if (lane == 0) {
            sh_first[wave] = over_m ? wave * 64 + __ffsll((long long)over_m) - 1 : kThreads;
            sh_last[wave] = pos_m ? wave * 64 + 63 - __clzll((long long)pos_m) : -1;
        }
    }
    __syncthreads();
    int first_over = kThreads, last_pos = -1;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        first_over = min(first_over, sh_first[w]);
        last_pos = max(last_pos, sh_last[w]);
    }
    const bool over = first_over < kThreads;
    const int owner = over ? first_over : max(last_pos, 0);
    if (tid == owner) {
        double run = incl - grp, pick_base = 0.0, last_base = 0.0;
        int pick = -1, lastpos = -1;
#pragma unroll
        for (int g = 0; g < kRegSegs; ++g) {
            if (pick < 0) {
                const double w = v[g];  // zero past the run
                if (w > 0.0) {
                    lastpos = g;
                    last_base = run;
                    if (over && run + w > tau) { pick = g; pick_base = run; }
                }
                run += w;
            }
        }
        for (int g = kRegSegs; g < len && pick < 0; ++g) {
            const double w = load_coherent(segs + (size_t)g * kThreads + tid);
            if (w > 0.0) {
                lastpos = g;
                last_base = run;
                if (over && run + w > tau) { pick = g; pick_base = run; }
            }
            run += w;
        }
        if (pick < 0) { pick = max(lastpos, 0); pick_base = last_base; }
        sh_seg = min(first + pick, n - 1);
        sh_run0 = pick_base;
    }
    __syncthreads();

    // Token inside the segment: lane l of wave 0 weighs token 64 f + l.
    if (wave == 0) {
        const int base_tok = sh_seg * kStoredSeg;
        const int j = base_tok + lane;
        double w = 0.0;
        if (j < a.V) w = W.template weigh<FILT>(Elem<T>::load(trow, j), Elem<T>::load(drow, j));
        const double run = sh_run0 + wave_inclusive_scan(w);
        const unsigned long long hit = __ballot(over && w > 0.0 && run > tau);
        const unsigned long long pos = __ballot(w > 0.0);
        int sel;
        if (hit) sel = __ffsll((long long)hit) - 1;
        else if (pos) sel = 63 - __clzll((long long)pos);
        else sel = 0;  // no positive weight anywhere: unreachable with finite logits
        if (lane == 0) a.out_tokens[(size_t)b * (k + 1) + s_row] = base_tok + sel;
    }

    // Leave this request's part of the workspace zero for later calls (every
    // other workgroup of the request has finished reading and writing it before
    // taking its ticket).
    for (int g = 0; g < G; ++g) segs[(size_t)g * kThreads + tid] = 0.0;
    clear_partials(a.partials + (size_t)b * a.R * a.S, a.R * a.S);
    if constexpr (FILT)
        for (int r = tid; r < a.R; r += kThreads)
            *reinterpret_cast<uint4*>(a.rowf + (size_t)b * a.R + r) = make_uint4(0, 0, 0, 0);
}

// One sampler work item: chunk ch of request b's stop row.
template <typename T, bool VEC, int NSUB, bool FILT>
__device__ void sample_item(const CallArgs& a, int b, int ch) {
    const int k = a.k;
    __shared__ double exp_tab[256];
    fill_exp_table(exp_tab);
    __syncthreads();
    Decision dc;
    decide<T, FILT>(a, b, ch == 0, &dc, exp_tab);
    Weigher W;
    W.c256 = a.sc.c64 * 256.0;
    W.tab = exp_tab;
    W.mt = dc.mt;
    W.md = dc.md;
    W.set_ratio(dc.st / dc.sd);
    W.sc = a.sc;
    W.residual = dc.s < dc.kb;
    W.taut = dc.taut;
    W.taud = dc.taud;
    const T* trow = static_cast<const T*>(a.target) + ((size_t)b * (k + 1) + dc.s) * (size_t)a.V;
    const T* drow = W.residual
        ? static_cast<const T*>(a.draft) + ((size_t)b * k + dc.s) * (size_t)a.V
        : trow;
    __shared__ int last_flag;
    const int lo = ch * a.chunk2, hi = min(a.V, lo + a.chunk2);
    const double seg = segment_sum_any<T, VEC, NSUB, FILT>(trow, drow, W, lo, hi);
    const SegLayout L(a);
    store_segment<NSUB>(a.segs + (size_t)b * L.per_request(), L, ch, a.chunk2, seg);
    // Every thread's stores complete before the ticket is taken.
    wait_stores();
    __syncthreads();
    if (arrive_last(ticket_of(a.tickets, b), (uint32_t)a.S2, &last_flag))
        sample_final<T, VEC, NSUB, FILT>(a, b, dc.s, dc.kb, trow, drow, W);
}

template <typename T, bool VEC, int NSUB, bool FILT>
__global__ __launch_bounds__(kThreads) void sample_kernel(CallArgs a) {
    sample_item<T, VEC, NSUB, FILT>(a, blockIdx.x / a.S2, blockIdx.x % a.S2);
}

// ---------------------------------------------------------------------------
// The plain call.
//
// Tiles (one workgroup per (request, row, chunk)) compute the softmax
// statistics as above and publish their partials; they take no atomics and
// wait for nothing.
//
// Items (one workgroup per (request, stop-row chunk)) each read their
// request's partials (polling until all are published), merge them in chunk
// order and run the k tests, so every item of a request reaches the same
// decision (the chunk-0 item writes the accepted drafts, num_accepted, P and
// Q).  Each weighs its chunk of the final distribution (residual
// max(0, p_s - q_s) or bonus p_k, as Weigher does) into per-thread sums and
// publishes the chunk's mass; then reads every chunk mass of its request
// (computing here any that is late), and all find the same owner chunk: the
// first whose running mass exceeds u_k * Z.  The owner finds the token from
// its per-thread sums and one 64-lane scan of one thread's tokens.  Each item
// then takes its request's ticket; the last clears the partials and masses.
//
// Waits are bounded.  An item that gives up on a partial computes the
// request's statistics itself and marks the workspace stale (a word no call
// clears): a tile that publishes late may then leave a stale partial behind,
// so from then on every call on that workspace computes its statistics in the
// items and ignores published partials, until the workspace is zeroed again.
//
// One launch (rows 16-byte aligned): the grid holds the tiles request by
// request, and the items of request b follow the tiles of request
// b + lookahead (all items last when lookahead >= B).  Two kernels: all tiles,
// then all items.  Self-compute (testing): items alone, each computing its
// request's statistics.
// ---------------------------------------------------------------------------

__device__ inline unsigned long long enc_f64(double v) {
    return ~(unsigned long long)__double_as_longlong(v);
}
__device__ inline double dec_f64(unsigned long long w) {
    return __longlong_as_double((long long)~w);
}

// Per-request counters, each request on its own cache line: [0] item tickets.
// Word kStaleWord of request 0's line marks a stale workspace.
constexpr int kStaleWord = 8;
__device__ inline uint32_t* req_counter(const CallArgs& a, int b, int which) {
    return ticket_of(a.tickets, b) + which;
}
__device__ inline uint32_t* stale_word(const CallArgs& a) { return a.tickets + kStaleWord; }

// Request b's decision, in every item: the rows' statistics from the published
// partials (polled, bounded) merged in chunk order, or computed here (the
// self-compute schedule, a stale workspace, or a partial that never came: the
// workspace is then marked stale); then the tests.  With write_outputs the
// accepted drafts, num_accepted, P and Q are written.
template <typename T, bool VEC>
__device__ __forceinline__ void item_decide(const CallArgs& a, int b, int kb, bool write_outputs,
                                            Decision* out, const double* tab) {
    __shared__ float sh_m[2 * kMaxK + 1], sh_g[2 * kMaxK + 1];
    __shared__ double sh_s[2 * kMaxK + 1];
    __shared__ int sh_stale;
    const int k = a.k, n = a.R * a.S;
    gather_tested<T>(a, b, kb, sh_g);
    int32_t x;
    float u;
    load_test_inputs(a, b, kb, &x, &u);
    // The stale word is read alongside the first poll of the partials; up to
    // kMergeLds partials are kept in LDS as they are read.
    __shared__ float pm[kMergeLds];
    __shared__ double ps[kMergeLds];
    const bool staged = n <= kMergeLds;
    bool here = a.self_compute != 0;
    if (!here) {
        const Partial16* p = a.partials + (size_t)b * n;
        for (int it = 0;; ++it) {
            if (it == 0 && threadIdx.x == 0) sh_stale = load_coherent(stale_word(a)) != 0u;
            int ok = 1;
            for (int t = threadIdx.x; t < n; t += kThreads) {
                const PartialRead q = read_partial(p + t);
                ok &= q.ok;
                if (staged) {
                    pm[t] = q.f0;
                    ps[t] = q.d;
                }
            }
            ok = __syncthreads_and(ok);
            if (sh_stale) {
                here = true;
                break;
            }
            if (ok) break;
            if (it >= a.spin_limit) {
                here = true;
                if (threadIdx.x == 0) store_coherent(stale_word(a), 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    } else if (threadIdx.x == 0) {
        sh_stale = 1;
    }
    __syncthreads();
    if (here) merge_rows_here<T, VEC>(a, b, sh_m, sh_s, !a.self_compute && !sh_stale, tab);
    else if (staged) merge_staged(a, pm, ps, sh_m, sh_s, tab);
    else merge_rows<T>(a, b, sh_m, sh_s, tab);
    const int s = run_tests<false>(a, b, kb, x, u, sh_m, sh_s, nullptr, sh_g, write_outputs, tab);
    out->s = s;
    out->kb = kb;
    out->mt = sh_m[s];
    out->st = sh_s[s];
    out->md = (s < kb) ? sh_m[k + 1 + s] : 0.f;
    out->sd = (s < kb) ? sh_s[k + 1 + s] : 1.0;
    out->taut = -INFINITY;
    out->taud = -INFINITY;
    __syncthreads();
}

// Weights of request b's final draw (Weigher) and its stop rows.
template <typename T>
struct FinalRows {
    Weigher W;
    const T* trow;
    const T* drow;
};

// Workgroup-uniform values moved to scalar registers (every lane holds the
// same value): they then take no vector registers.
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline float uni(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }
__device__ inline double uni(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ inline Decision uni(const Decision& d) {
    Decision u;
    u.s = uni(d.s);
    u.kb = uni(d.kb);
    u.mt = uni(d.mt);
    u.md = uni(d.md);
    u.st = uni(d.st);
    u.sd = uni(d.sd);
    u.taut = uni(d.taut);
    u.taud = uni(d.taud);
    return u;
}

template <typename T>
__device__ inline FinalRows<T> final_rows(const CallArgs& a, int b, const Decision& d, const double* tab) {
    FinalRows<T> f;
    f.W.c256 = a.sc.c64 * 256.0;
    f.W.tab = tab;
    f.W.mt = d.mt;
    f.W.md = d.md;
    f.W.set_ratio(d.st / d.sd);
    f.W.sc = a.sc;
    f.W.residual = d.s < d.kb;
    f.W.taut = -INFINITY;
    f.W.taud = -INFINITY;
    f.trow = static_cast<const T*>(a.target) + ((size_t)b * (a.k + 1) + d.s) * (size_t)a.V;
    f.drow = f.W.residual
        ? static_cast<const T*>(a.draft) + ((size_t)b * a.k + d.s) * (size_t)a.V
        : f.trow;
    return f;
}

// Mass of chunk c of the final distribution: every thread's sum over its
// kSub * NSUB tokens (segment_sum), and their inclusive prefix in thread order;
// *total is the chunk's mass (the same additions as the last prefix).
template <typename T, bool VEC, int NSUB>
__device__ __forceinline__ double chunk_sums(const CallArgs& a, const FinalRows<T>& f, int c, double* incl,
                                    double* total) {
    __shared__ double sh_wave[kWaves];
    const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
    const double seg = segment_sum_any<T, VEC, NSUB, false>(f.trow, f.drow, f.W, lo, hi);
    *incl = block_inclusive_scan(seg, sh_wave, total);
    return seg;
}

// Across the workgroup: the first thread whose flag is set (kThreads if none)
// and the last thread whose second flag is set (-1 if none).
__device__ inline void block_first_last(bool first_flag, bool last_flag, int* first, int* last) {
    __shared__ int sh_first[kWaves], sh_last[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long fm = __ballot(first_flag);
    const unsigned long long lm = __ballot(last_flag);
    if (lane == 0) {
        sh_first[wave] = fm ? wave * 64 + __ffsll((long long)fm) - 1 : kThreads;
        sh_last[wave] = lm ? wave * 64 + 63 - __clzll((long long)lm) : -1;
    }
    __syncthreads();
    int fi = kThreads, la = -1;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        fi = min(fi, sh_first[w]);
        la = max(la, sh_last[w]);
    }
    __syncthreads();
    *first = fi;
    *last = la;
}

// The token inside chunk c: the first thread with positive mass whose running
// mass (prev + its inclusive prefix) exceeds tau, else the last with positive
// mass; then that thread's kSub * NSUB tokens, one per lane of wave 0, the first
// with positive weight whose running mass exceeds tau, else the last with
// positive weight.  Written to out_tokens[b, s_row] by lane 0 of wave 0.
template <typename T, bool VEC, int NSUB>
__device__ __forceinline__ void draw_in_chunk(const CallArgs& a, int b, int s_row, const FinalRows<T>& f, int c,
                              double seg, double incl, double prev, double tau) {
    __shared__ double sh_ti[kThreads];
    sh_ti[threadIdx.x] = incl;
    __syncthreads();
    int fi, la;
    block_first_last(seg > 0.0 && prev + incl > tau, seg > 0.0, &fi, &la);
    const bool over = fi < kThreads;
    const int tsel = over ? fi : max(la, 0);
    const double base_run = prev + (tsel > 0 ? sh_ti[tsel - 1] : 0.0);
    if (threadIdx.x < 64) {
        constexpr int SEG = NSUB * kSub;
        const int lane = threadIdx.x;
        const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
        const int j = lo + tsel * SEG + lane;
        double w = 0.0;
        if (lane < SEG && j < hi)
            w = f.W.template weigh<false>(Elem<T>::load(f.trow, j), Elem<T>::load(f.drow, j));
        const double run = base_run + wave_inclusive_scan(w);
        const unsigned long long hit = __ballot(over && w > 0.0 && run > tau);
        const unsigned long long pos = __ballot(w > 0.0);
        int sel;
        if (hit) sel = __ffsll((long long)hit) - 1;
        else if (pos) sel = 63 - __clzll((long long)pos);
        else sel = 0;
        if (lane == 0) a.out_tokens[(size_t)b * (a.k + 1) + s_row] = lo + tsel * SEG + sel;
    }
    __syncthreads();
}

// An arrival ticket on request b (thread 0's value; 0 elsewhere), taken once
// this workgroup has read all it needs and thread 0's stores (a published mass
// or partial) have completed, so that the last arrival's clearing cannot
// overtake them.
__device__ inline uint32_t take_ticket(const CallArgs& a, int b) {
    uint32_t prev = 0;
    if (threadIdx.x == 0) {
        wait_stores();
        prev = atomicAdd(req_counter(a, b, 0), 1u);
    }
    return prev;
}

// The last of the request's S2 arrivals (prev from take_ticket; a request of
// one item takes no ticket) clears both rounds' masses, the partials and the
// counter.  On a stale workspace a tile of this call may still publish after
// the clearing; later calls ignore published partials there in any case.
__device__ __forceinline__ void close_request(const CallArgs& a, int b, uint32_t prev) {
    __shared__ int sh_last;
    if (threadIdx.x == 0) sh_last = prev == (uint32_t)a.S2 - 1u;
    __syncthreads();
    if (sh_last) {
        for (int i = threadIdx.x; i < a.S2; i += kThreads) {
            store_coherent(&a.masses[(size_t)b * a.S2 + i], 0ull);
            store_coherent(&a.masses[(size_t)(a.B + b) * a.S2 + i], 0ull);
        }
        if (!a.self_compute) clear_partials(a.partials + (size_t)b * a.R * a.S, a.R * a.S);
        if (threadIdx.x == 0 && a.S2 > 1) atomicExch(req_counter(a, b, 0), 0u);
    }
}

// One item of the plain call: chunk c of request b's final draw.
template <typename T, bool VEC, int NSUB>
__device__ __forceinline__ void item_plain(const CallArgs& a, int b, int c) {
    __shared__ double sh_incl[kThreads];
    __shared__ double sh_scan[kWaves];
    // 1. The request's decision (the final draw's uniform is loaded first, so
    //    that its latency overlaps the decision's).
    const int kb = draft_len(a, b);
    const float u_final = uniform_at(a, b, kb);
    __shared__ double exp_tab[256];
    fill_exp_table(exp_tab);
    __syncthreads();
    Decision d;
    item_decide<T, VEC>(a, b, kb, c == 0, &d, exp_tab);
    d = uni(d);
    FinalRows<T> f = final_rows<T>(a, b, d, exp_tab);
    f.W.set_ratio(uni(f.W.r));
    const double u = uni((double)u_final);

    // Round 0 draws from the request's final distribution.  Its masses are all
    // zero only when the residual vanished (p_s == q_s exactly, which a strict
    // test with u < 1 never rejects); round 1 then draws from p_s instead, with
    // a second set of chunk masses.
    __shared__ int sh_miss[kMaxChunks2];
    __shared__ int sh_nmiss;
    int owner = -1;
    double seg = 0.0, incl = 0.0, Z = 0.0, prev_incl = 0.0;
    for (int round = 0; round < 2 && owner < 0; ++round) {
        if (round == 1) {
            f.W.residual = false;
            f.drow = f.trow;
        }
        unsigned long long* masses = a.masses + (size_t)(round * a.B + b) * a.S2;
        // 2. This chunk's sums and mass, published; then every chunk's mass,
        //    thread t holding chunk t's (at most kMaxChunks2 chunks): as
        //    published by its item, or, past the poll limit, weighed here by
        //    the same code (the same bits).
        double m = 0.0;
        int job = c, jn = 0;
        for (;;) {
            double incl_j, mass_j;
            const double seg_j = chunk_sums<T, VEC, NSUB>(a, f, job, &incl_j, &mass_j);
            if (job == c && jn == 0) {
                seg = seg_j;
                incl = incl_j;
                if (threadIdx.x == 0) {
                    sh_nmiss = 0;
                    if (a.S2 > 1) store_coherent(&masses[c], enc_f64(mass_j));
                }
                const int t = threadIdx.x;
                bool have = t >= a.S2 || t == c;
                if (t == c) m = mass_j;
                for (int it = 0; !have; ++it) {
                    const unsigned long long v = load_coherent(&masses[t]);
                    if (v != 0ull) {
                        m = dec_f64(v);
                        have = true;
                    } else if (it >= a.spin_limit) {
                        break;
                    } else {
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
                __syncthreads();
                if (!have) sh_miss[atomicAdd(&sh_nmiss, 1)] = t;
                __syncthreads();
            } else if ((int)threadIdx.x == job) {
                m = mass_j;
            }
            if (jn >= sh_nmiss) break;
            job = sh_miss[jn++];
        }

        // 3. Z and the owner chunk: the first with positive mass whose running
        //    mass (chunks in order, one workgroup-wide scan: the same values in
        //    every item) exceeds u Z, else the last with positive mass.
        const double ci = block_inclusive_scan(m, sh_scan, &Z);
        const double tau = u * Z;
        sh_incl[threadIdx.x] = ci;
        __syncthreads();
        int fi, la;
        block_first_last(m > 0.0 && ci > tau, m > 0.0, &fi, &la);
        owner = fi < kThreads ? fi : la;  // la: rounding left u Z at or past the total
        prev_incl = owner > 0 ? sh_incl[owner - 1] : 0.0;
        __syncthreads();
        owner = uni(owner);
        prev_incl = uni(prev_incl);
        Z = uni(Z);
    }

    // 4. Ticket (its value is used last): this item has read all it needs.
    const uint32_t prev = a.S2 > 1 ? take_ticket(a, b) : 0u;

    // 5. The owner draws.
    if (owner == c) draw_in_chunk<T, VEC, NSUB>(a, b, d.s, f, c, seg, incl, prev_incl, u * Z);

    // 6. The last arrival clears the request's part of the workspace.
    close_request(a, b, prev);
}

// Block index -> work of the one-launch grid: the tiles of requests
// 0 .. L-1, then for b = L .. B-1 the tiles of b followed by the items of
// b - L, then the items of the last L requests (L = min(lookahead, B)).
// Returns true for a tile (*idx its request-major tile index), false for an
// item (*idx = request * S2 + chunk).
__device__ inline bool plain_block(const CallArgs& a, int x, int* idx) {
    const int tpr = a.R * a.S, ipr = a.S2;
    const int L = min(a.lookahead, a.B);
    const int head = L * tpr;
    if (x < head) {
        *idx = x;
        return true;
    }
    x -= head;
    const int per = tpr + ipr, nmid = a.B - L;
    if (x < nmid * per) {
        const int seg = x / per, off = x % per;
        if (off < tpr) {
            *idx = (L + seg) * tpr + off;
            return true;
        }
        *idx = seg * ipr + (off - tpr);
        return false;
    }
    x -= nmid * per;
    *idx = nmid * ipr + x;
    return false;
}

#ifndef SV_PLAIN_WAVES
#define SV_PLAIN_WAVES 1
#endif
template <typename T, int U, int NSUB>
__global__ __launch_bounds__(kThreads, SV_PLAIN_WAVES) void plain_kernel(CallArgs a) {
    int idx;
    if (plain_block(a, (int)blockIdx.x, &idx)) {
        // Tiles issue ahead of the items that share their compute unit: an
        // item amid the stream then takes only the cycles the tiles leave.
        __builtin_amdgcn_s_setprio(3);
        StatsOp<T, U> op;
        static_cast<CallArgs&>(op) = a;
        // With non-temporal loads on, the rows a request most likely stops
        // at stay cached for the items' re-read: with per-position acceptance
        // a the stop row s has probability a^s (1 - a) below k and a^k at the
        // bonus row k, so target rows 0, 1 and k and draft rows 0 and 1.
        const int r = (idx / a.S) % a.R;
        const bool likely_stop = r <= 1 || r == a.k || r == a.k + 1 || r == a.k + 2;
        if (a.nontemporal && !likely_stop) stream_tile_vec<T, U, true>(op, idx);
        else stream_tile_vec<T, U, false>(op, idx);
    } else {
        item_plain<T, true, NSUB>(a, idx / a.S2, idx % a.S2);
    }
}

template <typename T, bool VEC, int NSUB>
__global__ __launch_bounds__(kThreads) void plain_items_kernel(CallArgs a) {
    item_plain<T, VEC, NSUB>(a, (int)blockIdx.x / a.S2, (int)blockIdx.x % a.S2);
}

// ---------------------------------------------------------------------------

template <typename T, int U, bool VEC>
static hipError_t launch_stats_u(const CallArgs& a, hipStream_t st, const KernelEvents& ev) {
    const unsigned n_tiles = (unsigned)((long long)a.B * a.R * a.S);
    // The events (when set) take the kernel's own start and end timestamps.
    hipExtLaunchKernelGGL(stats_kernel<T, U, VEC>, dim3(n_tiles), dim3(kThreads), 0, st, ev.begin,
                          ev.end, 0, a);
    return hipGetLastError();
}

template <typename T, bool VEC>
static hipError_t launch_stats(const CallArgs& a, int U, hipStream_t st, const KernelEvents& ev) {
    switch (U) {
        case 8: return launch_stats_u<T, 8, VEC>(a, st, ev);
        case 4: return launch_stats_u<T, 4, VEC>(a, st, ev);
        case 2: return launch_stats_u<T, 2, VEC>(a, st, ev);
        default: return launch_stats_u<T, 1, VEC>(a, st, ev);
    }
}

template <typename T, bool VEC>
static hipError_t launch_sample_filtered(const CallArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((long long)a.B * a.S2)), block(kThreads);
    switch (a.chunk2 / (kThreads * kSub)) {
        case 8: sample_kernel<T, VEC, 8, true><<<grid, block, 0, st>>>(a); break;
        case 4: sample_kernel<T, VEC, 4, true><<<grid, block, 0, st>>>(a); break;
        case 2: sample_kernel<T, VEC, 2, true><<<grid, block, 0, st>>>(a); break;
        default: sample_kernel<T, VEC, 1, true><<<grid, block, 0, st>>>(a); break;
    }
    return hipGetLastError();
}

// Workgroups of plain_kernel<T, U, NSUB> resident on the current device at
// once (cached per device); 0 when the runtime cannot say.
template <typename T, int U, int NSUB>
static int plain_resident() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(plain_kernel<T, U, NSUB>), kThreads, 0) !=
                hipSuccess)
            return 0;
        v = std::max(cus * per_cu, 1);
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// The one-launch grid's lookahead L (items of request b follow the tiles of
// request b + L).  A call whose logits fit the last-level cache (256 MiB)
// puts every item last (L = B): the stop rows are still resident when the
// stream ends, and items amid the stream would take ALU time from the tiles.
// A larger call would find its early stop rows evicted by then, so its items
// run amid the stream, three resident windows behind their tiles (a window is
// the requests whose workgroups are resident at once), late enough that the
// request's tiles have finished and its rows are still cached.
constexpr size_t kLastLevelCacheBytes = (size_t)256 << 20;

static bool beyond_last_level_cache(const CallArgs& a, size_t elem_bytes) {
    return (size_t)a.B * (size_t)a.R * (size_t)a.V * elem_bytes > kLastLevelCacheBytes;
}

static int plain_lookahead(const CallArgs& a, size_t elem_bytes, int resident) {
    if (SV_LOOKAHEAD >= 0) return std::min(SV_LOOKAHEAD, a.B);
    if (g_stochastic_schedule == 3) return 1;
    if (!beyond_last_level_cache(a, elem_bytes) || resident <= 0) return a.B;
    const long long per_request = (long long)a.R * a.S + a.S2;
    const long long L = (3LL * resident + per_request - 1) / per_request;
    return (int)std::min<long long>(std::max<long long>(L, 1), a.B);
}

// One launch: tiles and items in one grid.
template <typename T, int U, int NSUB>
static hipError_t launch_plain_u(const CallArgs& args, hipStream_t st, const KernelEvents& ev) {
    CallArgs a = args;
    a.lookahead = plain_lookahead(a, sizeof(T), plain_resident<T, U, NSUB>());
    // Tiles of a call beyond the last-level cache stream with non-temporal
    // loads (the faster choice there: most of their rows are never read
    // again); a smaller call's tiles leave their rows cached for the items,
    // which re-read the stop rows after the stream.
    a.nontemporal = beyond_last_level_cache(a, sizeof(T)) ? 1 : 0;
    const unsigned grid = (unsigned)((long long)a.B * a.R * a.S + (long long)a.B * a.S2);
    hipExtLaunchKernelGGL(plain_kernel<T, U, NSUB>, dim3(grid), dim3(kThreads), 0, st, ev.begin,
                          ev.end, 0, a);
    return hipGetLastError();
}

template <typename T, int NSUB>
static hipError_t launch_plain_n(const CallArgs& a, int U, hipStream_t st, const KernelEvents& ev) {
    switch (U) {
        case 8: return launch_plain_u<T, 8, NSUB>(a, st, ev);
        case 4: return launch_plain_u<T, 4, NSUB>(a, st, ev);
        case 2: return launch_plain_u<T, 2, NSUB>(a, st, ev);
        default: return launch_plain_u<T, 1, NSUB>(a, st, ev);
    }
}

template <typename T>
static hipError_t launch_plain(const CallArgs& a, int U, hipStream_t st, const KernelEvents& ev) {
    switch (a.chunk2 / (kThreads * kSub)) {
        case 8: return launch_plain_n<T, 8>(a, U, st, ev);
        case 4: return launch_plain_n<T, 4>(a, U, st, ev);
        case 2: return launch_plain_n<T, 2>(a, U, st, ev);
        default: return launch_plain_n<T, 1>(a, U, st, ev);
    }
}

// Items alone (after the statistics kernel, or computing the statistics
// themselves under the self-compute schedule).
template <typename T, bool VEC>
static hipError_t launch_plain_items(const CallArgs& a, hipStream_t st, const KernelEvents& ev) {
    const dim3 grid((unsigned)((long long)a.B * a.S2)), block(kThreads);
    switch (a.chunk2 / (kThreads * kSub)) {
        case 8:
            hipExtLaunchKernelGGL(plain_items_kernel<T, VEC, 8>, grid, block, 0, st, ev.begin,
                                  ev.end, 0, a);
            break;
        case 4:
            hipExtLaunchKernelGGL(plain_items_kernel<T, VEC, 4>, grid, block, 0, st, ev.begin,
                                  ev.end, 0, a);
            break;
        case 2:
            hipExtLaunchKernelGGL(plain_items_kernel<T, VEC, 2>, grid, block, 0, st, ev.begin,
                                  ev.end, 0, a);
            break;
        default:
            hipExtLaunchKernelGGL(plain_items_kernel<T, VEC, 1>, grid, block, 0, st, ev.begin,
                                  ev.end, 0, a);
            break;
    }
    return hipGetLastError();
}

// Two kernels: every tile, then every item (the events, when set, on the
// statistics kernel).
template <typename T, bool VEC>
static hipError_t launch_plain_two(const CallArgs& a, int U, hipStream_t st,
                                   const KernelEvents& ev) {
    const hipError_t e = launch_stats<T, VEC>(a, U, st, ev);
    if (e != hipSuccess) return e;
    return launch_plain_items<T, VEC>(a, st, KernelEvents{});
}

int g_stochastic_schedule = 0;

static std::atomic<int> g_debug_spin{-1};
int debug_spin_limit(int fallback) {
    const int v = g_debug_spin.load(std::memory_order_relaxed);
    return v < 0 ? fallback : v;
}
int set_debug_spin_limit(int polls, int fallback) {
    const int prev = g_debug_spin.exchange(polls < 0 ? -1 : polls);
    return prev < 0 ? fallback : prev;
}

// Polls of a decision record or chunk mass before an item derives it itself:
// far above any wait seen when workgroups are dispatched in order (a few
// microseconds).
constexpr int kSpinLimit = 1 << 16;

static CallArgs make_args(const StochasticCall& call, const Geometry& g) {
    char* ws = static_cast<char*>(call.workspace);
    CallArgs a;
    a.target = call.target;
    a.draft = call.draft;
    a.draft_tokens = call.draft_tokens;
    a.lens = call.draft_lens;
    a.uniforms = call.uniforms;
    a.seed = call.seed;
    a.offset = call.offset;
    a.B = call.B;
    a.k = call.k;
    a.V = call.V;
    a.R = g.R;
    a.S = g.S;
    a.chunk = g.chunk;
    a.S2 = g.S2;
    a.chunk2 = g.chunk2;
    a.sc = make_scale(call.temperature);
    a.partials = reinterpret_cast<Partial16*>(ws + g.off_partials);
    a.tickets = reinterpret_cast<uint32_t*>(ws + g.off_tickets);
    a.segs = reinterpret_cast<double*>(ws + g.off_segs);
    a.masses = reinterpret_cast<unsigned long long*>(ws + g.off_masses);
    a.out_tokens = call.out_tokens;
    a.num_accepted = call.num_accepted;
    a.p_at_draft = call.p_at_draft;
    a.q_at_draft = call.q_at_draft;
    a.rowf = nullptr;
    a.spin_limit = debug_spin_limit(kSpinLimit);
    a.self_compute = g_stochastic_schedule == 2;
    a.lookahead = call.B;  // the one-launch grid sets its own (plain_lookahead)
    a.nontemporal = 0;
    return a;
}

hipError_t run_stochastic(const StochasticCall& call, const Geometry& g, hipStream_t st,
                          const KernelEvents& ev) {
    const CallArgs a = make_args(call, g);
    if (a.self_compute)
        return call.dtype == 1 ? (call.vec ? launch_plain_items<bf16_t, true>(a, st, ev)
                                           : launch_plain_items<bf16_t, false>(a, st, ev))
                               : (call.vec ? launch_plain_items<float, true>(a, st, ev)
                                           : launch_plain_items<float, false>(a, st, ev));
    if (call.vec && g_stochastic_schedule != 1)
        return call.dtype == 1 ? launch_plain<bf16_t>(a, g.U, st, ev)
                               : launch_plain<float>(a, g.U, st, ev);
    if (call.dtype == 1)
        return call.vec ? launch_plain_two<bf16_t, true>(a, g.U, st, ev)
                        : launch_plain_two<bf16_t, false>(a, g.U, st, ev);
    return call.vec ? launch_plain_two<float, true>(a, g.U, st, ev)
                    : launch_plain_two<float, false>(a, g.U, st, ev);
}

hipError_t run_stochastic_filtered(const StochasticCall& call, const FilterCall& f,
                                   const Geometry& g, hipStream_t st, const KernelEvents& ev) {
    CallArgs a = make_args(call, g);
    a.rowf = reinterpret_cast<RowFilter*>(static_cast<char*>(call.workspace) + g.off_rowf);
    hipError_t e;
    const KernelEvents none;  // the events, when set, go to the selection kernel
    if (call.dtype == 1)
        e = call.vec ? launch_stats<bf16_t, true>(a, g.U, st, none)
                     : launch_stats<bf16_t, false>(a, g.U, st, none);
    else
        e = call.vec ? launch_stats<float, true>(a, g.U, st, none)
                     : launch_stats<float, false>(a, g.U, st, none);
    if (e != hipSuccess) return e;
    e = run_filter(call, f, g, st, ev);
    if (e != hipSuccess) return e;
    if (call.dtype == 1)
        return call.vec ? launch_sample_filtered<bf16_t, true>(a, st)
                        : launch_sample_filtered<bf16_t, false>(a, st);
    return call.vec ? launch_sample_filtered<float, true>(a, st)
                    : launch_sample_filtered<float, false>(a, st);
}

}  // namespace sv
