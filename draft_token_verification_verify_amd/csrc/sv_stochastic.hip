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
//            scale factors.  The last workgroup of a request to finish (arrival
//            ticket) merges the chunks of every row, computes p_i(x_i) and
//            q_i(x_i) in fp64, runs the k tests (independent given the
//            uniforms), takes the first failure as the stop row s and writes the
//            accepted drafts, the -1 padding and num_accepted.
//   sample:  one workgroup per (request, stop-row chunk).  Computes the chunk's
//            share of the final distribution's mass (residual max(0, p_s - q_s)
//            or bonus p_k) in fp64; tokens within 2^-8 of the row maximum take an
//            fp64 exponential, the rest fp32.  The last workgroup of a request
//            picks the chunk holding u_k * Z by a prefix sum over the chunk
//            masses, then the token inside that chunk by a prefix sum over
//            per-thread segments and a walk through one segment (ascending
//            vocabulary order: the smallest j whose running mass exceeds u_k * Z).
//
// Accuracy matters beyond the decisions themselves: a vocabulary of ~10^5 has
// ~10^5 CDF edges, so a relative error e in the cumulative weights moves the
// drawn token on a fraction ~V * e of the draws.  The fp64 paths above keep e
// near 1e-10.
#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

struct StatsArgs {
    const void* target;
    const void* draft;
    const int32_t* draft_tokens;
    const float* uniforms;
    int B, k, V, S, chunk;
    Scale sc;                // log2(e) / temperature
    StatPartial* partials;   // [B, 2k+1, S]
    uint32_t* tickets;       // [B]
    StopInfo* stop;          // [B]
    int32_t* out_tokens;     // [B, k+1]
    int32_t* num_accepted;   // [B]
    float* p_at_draft;       // [B, k] or null
    float* q_at_draft;       // [B, k] or null
};

// Row r of request b in the streaming order: rows 0..k are target rows, rows
// k+1..2k are draft rows 0..k-1.
template <typename T>
__device__ inline const T* stats_row(const StatsArgs& a, int b, int r) {
    if (r <= a.k)
        return static_cast<const T*>(a.target) + ((size_t)b * (a.k + 1) + r) * (size_t)a.V;
    return static_cast<const T*>(a.draft) + ((size_t)b * a.k + (r - a.k - 1)) * (size_t)a.V;
}

// p(x) = 2^((x - M) * c) / S in fp64; 0 when x or the whole row is -inf.
__device__ inline double prob_of(float x, float M, double S, const Scale& k) {
    if (M == -INFINITY || !(S > 0.0)) return 0.0;
    return exp2_accurate(x, M, k) / S;
}

// Per-request epilogue, run by the last workgroup of request b.
template <typename T>
__device__ void stats_epilogue(const StatsArgs& a, int b) {
    __shared__ float sh_m[2 * kMaxK + 1];
    __shared__ double sh_s[2 * kMaxK + 1];
    __shared__ int sh_acc[kMaxK];
    __shared__ int sh_stop;
    const int k = a.k, R = 2 * k + 1;
    for (int r = threadIdx.x; r < R; r += kThreads) {
        const StatPartial* p = a.partials + ((size_t)b * R + r) * a.S;
        float M = -INFINITY;
        for (int ch = 0; ch < a.S; ++ch) M = fmaxf(M, p[ch].m);
        double S = 0.0;
        if (M != -INFINITY)
            for (int ch = 0; ch < a.S; ++ch)  // fixed chunk order
                S += p[ch].s * exp2_accurate(p[ch].m, M, a.sc);
        sh_m[r] = M;
        sh_s[r] = S;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < k; i += kThreads) {
        const int32_t x = a.draft_tokens[(size_t)b * k + i];
        const float u = a.uniforms[(size_t)b * (k + 1) + i];
        double P = 0.0, Q = 0.0;
        int acc = 0;
        if (x >= 0 && x < a.V) {
            const float xt = Elem<T>::load(stats_row<T>(a, b, i), x);
            const float xd = Elem<T>::load(stats_row<T>(a, b, k + 1 + i), x);
            P = prob_of(xt, sh_m[i], sh_s[i], a.sc);
            Q = prob_of(xd, sh_m[k + 1 + i], sh_s[k + 1 + i], a.sc);
            acc = (P >= Q) || ((double)u * Q < P);  // strict u < min(1, P/Q), no division
        }
        sh_acc[i] = acc;
        if (a.p_at_draft) a.p_at_draft[(size_t)b * k + i] = (float)P;
        if (a.q_at_draft) a.q_at_draft[(size_t)b * k + i] = (float)Q;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = k;
        for (int i = 0; i < k; ++i)
            if (!sh_acc[i]) { s = i; break; }
        StopInfo si;
        si.s = s;
        si.mt = sh_m[s];
        si.st = sh_s[s];
        si.md = (s < k) ? sh_m[k + 1 + s] : 0.f;
        si.sd = (s < k) ? sh_s[k + 1 + s] : 1.0;
        si.pad = 0;
        a.stop[b] = si;
        a.num_accepted[b] = s;
        sh_stop = s;
    }
    __syncthreads();
    const int s = sh_stop;
    for (int i = threadIdx.x; i <= k; i += kThreads) {
        if (i < s) a.out_tokens[(size_t)b * (k + 1) + i] = a.draft_tokens[(size_t)b * k + i];
        else if (i > s) a.out_tokens[(size_t)b * (k + 1) + i] = -1;
        // out_tokens[b, s] is written by the sampler.
    }
}

template <typename T, int U, bool VEC>
__global__ __launch_bounds__(kThreads) void stats_kernel(StatsArgs a) {
    constexpr int EPV = Elem<T>::kPerVec;
    const int R = 2 * a.k + 1;
    const int tile = blockIdx.x;
    const int ch = tile % a.S;
    const int rr = tile / a.S;
    const int r = rr % R;
    const int b = rr / R;
    const T* row = stats_row<T>(a, b, r);
    const int lo = ch * a.chunk;
    const int hi = min(a.V, lo + a.chunk);

    // Each thread: its maximum m, then sum 2^((x - m) * c) over its elements in fp64.
    float m = -INFINITY;
    double s = 0.0;
    if constexpr (VEC) {
        // The chunk is whole 16-byte vectors (V % EPV == 0, rows 16-byte aligned).
        const int nvec = (hi - lo) / EPV;
        const uint4* base = reinterpret_cast<const uint4*>(row + lo);
        // All U loads issue back to back: slots past the chunk's end reload its
        // last vector (in bounds) and are masked to -inf afterwards.
        uint4 raw[U];
#pragma unroll
        for (int j = 0; j < U; ++j) raw[j] = base[min((int)threadIdx.x + j * kThreads, nvec - 1)];
        float x[U][EPV];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            Elem<T>::widen(raw[j], x[j]);
            if ((int)threadIdx.x + j * kThreads >= nvec)
#pragma unroll
                for (int e = 0; e < EPV; ++e) x[j][e] = -INFINITY;
        }
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) m = fmaxf(m, x[j][e]);
        const float ms = (m == -INFINITY) ? 0.f : m;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) s += (double)fast_exp2(scaled(x[j][e] - ms, a.sc));
    } else {
        for (int j = lo + threadIdx.x; j < hi; j += kThreads) m = fmaxf(m, Elem<T>::load(row, j));
        const float ms = (m == -INFINITY) ? 0.f : m;
        for (int j = lo + threadIdx.x; j < hi; j += kThreads)
            s += (double)fast_exp2(scaled(Elem<T>::load(row, j) - ms, a.sc));
    }

    // Workgroup: common maximum, then each thread's sum rescaled in fp64.
    __shared__ float red_f[kWaves];
    __shared__ double red_d[kWaves];
    __shared__ int last_flag;
    const float M = block_max(m, red_f);
    const double f = (m == -INFINITY) ? 0.0 : exp2_accurate(m, M, a.sc);
    const double S = block_sum(s * f, red_d);
    if (threadIdx.x == 0) {
        StatPartial p;
        p.m = M;
        p.pad = 0.f;
        p.s = S;
        a.partials[tile] = p;
    }
    if (arrive_last(a.tickets + b, (uint32_t)(R * a.S), &last_flag))
        stats_epilogue<T>(a, b);
}

// ---------------------------------------------------------------------------

struct SampleArgs {
    const void* target;
    const void* draft;
    const float* uniforms;
    int B, k, V, S2, chunk2;
    Scale sc;
    const StopInfo* stop;  // [B]
    double* mass;          // [B, S2]
    uint32_t* tickets;     // [B]
    int32_t* out_tokens;   // [B, k+1]
};

// Weight of one token in the final draw, in fp64: the residual max(0, p - q)
// when the request stopped on a rejection, else the target probability.  Tokens
// within 2^-8 of their row's maximum (the few that carry most of the mass) take
// the fp64 exponential; the others the fp32 one, whose error is then negligible
// against the total.
struct Weigher {
    float mt, md;
    double inv_st, inv_sd;
    Scale sc;
    bool residual;
    __device__ inline double e_of(float x, float m) const {
        const float a = scaled(x - m, sc);
        if (a > -8.f) return exp2_accurate(x, m, sc);
        return (double)fast_exp2(a);
    }
    __device__ inline double operator()(float xt, float xd) const {
        const double p = e_of(xt, mt) * inv_st;
        if (!residual) return p;
        const double q = e_of(xd, md) * inv_sd;
        return p > q ? p - q : 0.0;
    }
};

// Weights of this thread's segment (kSampleSeg consecutive tokens) of the chunk
// [lo, hi): w[] in ascending token order, first token id in *j0, count in *n.
template <typename T, bool VEC>
__device__ inline void segment_weights(const T* trow, const T* drow, const Weigher& W, int V,
                                       int lo, int hi, double* w, int* j0, int* n) {
    constexpr int EPV = Elem<T>::kPerVec;
    constexpr int SEG = kSampleSeg;
    constexpr int NV = SEG / EPV;
    const int start = lo + threadIdx.x * SEG;
    *j0 = start;
    *n = max(0, min(SEG, hi - start));
    // Loads issue back to back from in-bounds (clamped) positions; positions
    // past the chunk's end get weight 0.  drow == trow when there is no residual.
    if constexpr (VEC) {
        uint4 rt[NV], rd[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int j = min(start + v * EPV, hi - EPV);
            rt[v] = load16(trow + j);
            rd[v] = load16(drow + j);
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float xt[EPV], xd[EPV];
            Elem<T>::widen(rt[v], xt);
            Elem<T>::widen(rd[v], xd);
            const bool in = start + v * EPV < hi;
#pragma unroll
            for (int e = 0; e < EPV; ++e) w[v * EPV + e] = in ? W(xt[e], xd[e]) : 0.0;
        }
    } else {
        float xt[SEG], xd[SEG];
#pragma unroll
        for (int e = 0; e < SEG; ++e) {
            const int j = min(start + e, hi - 1);
            xt[e] = Elem<T>::load(trow, j);
            xd[e] = Elem<T>::load(drow, j);
        }
#pragma unroll
        for (int e = 0; e < SEG; ++e) w[e] = (start + e < hi) ? W(xt[e], xd[e]) : 0.0;
    }
    (void)V;
}

template <typename T, bool VEC>
__device__ double chunk_mass(const T* trow, const T* drow, const Weigher& W, int V, int lo,
                             int hi, double* red) {
    constexpr int SEG = kSampleSeg;
    double w[SEG];
    int j0, n;
    segment_weights<T, VEC>(trow, drow, W, V, lo, hi, w, &j0, &n);
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < SEG; ++e) acc += w[e];
    acc = wave_reduce_sum(acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) tot += red[q];
    __syncthreads();
    return tot;
}

template <typename T, bool VEC>
__device__ void sample_epilogue(const SampleArgs& a, int b, const T* trow, const T* drow,
                                Weigher W) {
    constexpr int SEG = kSampleSeg;
    __shared__ double sh_wave[kWaves];
    __shared__ double sh_red[kWaves];
    __shared__ int sh_first;
    __shared__ double sh_base, sh_tau;
    __shared__ int sh_chunk;
    const int k = a.k;
    double* mass = a.mass + (size_t)b * a.S2;
    const double u = (double)a.uniforms[(size_t)b * (k + 1) + k];

    // Chunk selection: thread t owns a contiguous group of chunk masses.
    const int G = (a.S2 + kThreads - 1) / kThreads;
    double Z = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
        double grp = 0.0;
        for (int g = 0; g < G; ++g) {
            const int c = threadIdx.x * G + g;
            if (c < a.S2) grp += mass[c];
        }
        double incl = block_inclusive_scan(grp, sh_wave, &Z);
        if (Z > 0.0 || pass == 1) {
            const double tau = u * Z;
            if (threadIdx.x == 0) sh_first = kThreads;
            __syncthreads();
            if (incl > tau) atomicMin(&sh_first, (int)threadIdx.x);
            __syncthreads();
            if (threadIdx.x == 0) {
                sh_tau = tau;
                sh_chunk = -1;
            }
            __syncthreads();
            int first = sh_first;
            if (first < kThreads && (int)threadIdx.x == first) {
                double run = incl - grp;
                int lastc = -1;
                double lastbase = 0.0;
                for (int g = 0; g < G; ++g) {
                    const int c = threadIdx.x * G + g;
                    if (c >= a.S2) break;
                    if (mass[c] > 0.0) { lastc = c; lastbase = run; }
                    if (run + mass[c] > tau) {
                        lastc = c;
                        lastbase = run;
                        break;
                    }
                    run += mass[c];
                }
                // Rounding can leave the walk short of tau: stay in this group.
                if (lastc >= 0) {
                    sh_chunk = lastc;
                    sh_base = lastbase;
                }
            }
            __syncthreads();
            if (sh_chunk < 0 && threadIdx.x == 0) {
                // u * Z at or past the total (rounding): the last chunk with mass.
                double run = 0.0;
                int lastc = 0;
                double lastbase = 0.0;
                for (int c = 0; c < a.S2; ++c) {
                    if (mass[c] > 0.0) { lastc = c; lastbase = run; }
                    run += mass[c];
                }
                sh_chunk = lastc;
                sh_base = lastbase;
            }
            __syncthreads();
            break;
        }
        // Z == 0: the residual vanished (p_s == q_s); draw from p_s instead.
        W.residual = false;
        for (int c = 0; c < a.S2; ++c) {
            const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
            double mc = chunk_mass<T, VEC>(trow, drow, W, a.V, lo, hi, sh_red);
            if (threadIdx.x == 0) mass[c] = mc;
            __syncthreads();
        }
        // Make thread 0's fresh masses visible to every wave before rereading.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }

    // Token selection inside the chosen chunk.
    const int c = sh_chunk;
    const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
    double w[SEG];
    int j0, n;
    segment_weights<T, VEC>(trow, drow, W, a.V, lo, hi, w, &j0, &n);
    double seg = 0.0;
#pragma unroll
    for (int e = 0; e < SEG; ++e) seg += w[e];
    double chunk_total;
    double incl = block_inclusive_scan(seg, sh_wave, &chunk_total);
    const double base = sh_base, tau = sh_tau;
    if (threadIdx.x == 0) sh_first = kThreads;
    __syncthreads();
    if (base + incl > tau) atomicMin(&sh_first, (int)threadIdx.x);
    __syncthreads();
    __shared__ int sh_token;
    if (threadIdx.x == 0) sh_token = -1;
    __syncthreads();
    if ((int)threadIdx.x == sh_first) {
        double run = base + (incl - seg);
        int tok = -1, last_pos = -1;
        for (int e = 0; e < SEG; ++e) {
            if (e >= n) break;
            if (w[e] > 0.0) last_pos = j0 + e;
            run += w[e];
            if (run > tau) { tok = j0 + e; break; }
        }
        sh_token = (tok >= 0) ? tok : last_pos;
    }
    __syncthreads();
    if (sh_token < 0) {
        // Rounding left u * Z past this chunk's total: the chunk's last positive weight.
        int last_pos = -1;
        for (int e = 0; e < SEG; ++e)
            if (e < n && w[e] > 0.0) last_pos = j0 + e;
        if (last_pos >= 0) atomicMax(&sh_token, last_pos);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        int tok = sh_token;
        if (tok < 0) tok = lo;  // no positive weight anywhere: unreachable with finite logits
        a.out_tokens[(size_t)b * (k + 1) + min(max(a.stop[b].s, 0), k)] = tok;
    }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_kernel(SampleArgs a) {
    const int tile = blockIdx.x;
    const int b = tile / a.S2;
    const int ch = tile % a.S2;
    StopInfo si = a.stop[b];
    const int k = a.k;
    si.s = min(max(si.s, 0), k);  // never index outside the request's rows
    Weigher W;
    W.mt = si.mt;
    W.inv_st = 1.0 / si.st;
    W.md = si.md;
    W.inv_sd = 1.0 / si.sd;
    W.sc = a.sc;
    W.residual = si.s < k;
    const T* trow = static_cast<const T*>(a.target) + ((size_t)b * (k + 1) + si.s) * (size_t)a.V;
    const T* drow = W.residual
        ? static_cast<const T*>(a.draft) + ((size_t)b * k + si.s) * (size_t)a.V
        : trow;
    __shared__ double red[kWaves];
    __shared__ int last_flag;
    const int lo = ch * a.chunk2, hi = min(a.V, lo + a.chunk2);
    double mc = chunk_mass<T, VEC>(trow, drow, W, a.V, lo, hi, red);
    if (threadIdx.x == 0) a.mass[(size_t)b * a.S2 + ch] = mc;
    if (arrive_last(a.tickets + b, (uint32_t)a.S2, &last_flag))
        sample_epilogue<T, VEC>(a, b, trow, drow, W);
}

// ---------------------------------------------------------------------------

template <typename T, bool VEC>
static hipError_t launch_stats(const StatsArgs& a, int U, hipStream_t st) {
    const int R = 2 * a.k + 1;
    const dim3 grid((unsigned)((long long)a.B * R * a.S)), block(kThreads);
    switch (U) {
        case 8: stats_kernel<T, 8, VEC><<<grid, block, 0, st>>>(a); break;
        case 4: stats_kernel<T, 4, VEC><<<grid, block, 0, st>>>(a); break;
        case 2: stats_kernel<T, 2, VEC><<<grid, block, 0, st>>>(a); break;
        default: stats_kernel<T, 1, VEC><<<grid, block, 0, st>>>(a); break;
    }
    return hipGetLastError();
}

template <typename T, bool VEC>
static hipError_t launch_sample(const SampleArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((long long)a.B * a.S2)), block(kThreads);
    sample_kernel<T, VEC><<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t run_stochastic(const StochasticCall& call, const Geometry& g, hipStream_t st,
                          const KernelEvents& ev) {
    char* ws = static_cast<char*>(call.workspace);
    StatsArgs a;
    a.target = call.target;
    a.draft = call.draft;
    a.draft_tokens = call.draft_tokens;
    a.uniforms = call.uniforms;
    a.B = call.B;
    a.k = call.k;
    a.V = call.V;
    a.S = g.S;
    a.chunk = g.chunk;
    a.sc = make_scale(call.temperature);
    a.partials = reinterpret_cast<StatPartial*>(ws + g.off_partials);
    a.tickets = reinterpret_cast<uint32_t*>(ws + g.off_ticket_a);
    a.stop = reinterpret_cast<StopInfo*>(ws + g.off_stop);
    a.out_tokens = call.out_tokens;
    a.num_accepted = call.num_accepted;
    a.p_at_draft = call.p_at_draft;
    a.q_at_draft = call.q_at_draft;

    SampleArgs s;
    s.target = call.target;
    s.draft = call.draft;
    s.uniforms = call.uniforms;
    s.B = call.B;
    s.k = call.k;
    s.V = call.V;
    s.S2 = g.S2;
    s.chunk2 = g.chunk2;
    s.sc = a.sc;
    s.stop = a.stop;
    s.mass = reinterpret_cast<double*>(ws + g.off_mass);
    s.tickets = reinterpret_cast<uint32_t*>(ws + g.off_ticket_b);
    s.out_tokens = call.out_tokens;

    hipError_t e;
    if (ev.begin && (e = hipEventRecord(ev.begin, st)) != hipSuccess) return e;
    if (call.dtype == 1)
        e = call.vec ? launch_stats<bf16_t, true>(a, g.U, st)
                     : launch_stats<bf16_t, false>(a, g.U, st);
    else
        e = call.vec ? launch_stats<float, true>(a, g.U, st)
                     : launch_stats<float, false>(a, g.U, st);
    if (e != hipSuccess) return e;
    if (ev.end && (e = hipEventRecord(ev.end, st)) != hipSuccess) return e;
    if (call.dtype == 1)
        return call.vec ? launch_sample<bf16_t, true>(s, st) : launch_sample<bf16_t, false>(s, st);
    return call.vec ? launch_sample<float, true>(s, st) : launch_sample<float, false>(s, st);
}

}  // namespace sv
