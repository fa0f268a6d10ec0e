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
//            statistics (max m, sum of exp2((x - m) * log2(e) / T)).  The last
//            workgroup of a request to finish (arrival ticket) merges the
//            chunks of every row, gathers p_i(x_i) and q_i(x_i), runs the k
//            tests (independent given the uniforms), takes the first failure as
//            the stop row s and writes the accepted drafts, the -1 padding and
//            num_accepted.
//   sample:  one workgroup per (request, stop-row chunk).  Computes the chunk's
//            share of the final distribution's mass (residual max(0, p_s - q_s)
//            or bonus p_k), in fp64.  The last workgroup of a request picks the
//            chunk holding u_k * Z by a prefix sum over the chunk masses, then
//            the token inside that chunk by a prefix sum over per-thread
//            segments and a walk through one segment (ascending vocabulary
//            order: the smallest j whose running mass exceeds u_k * Z).
#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

struct StatsArgs {
    const void* target;
    const void* draft;
    const int32_t* draft_tokens;
    const float* uniforms;
    int B, k, V, S, chunk;
    float c;                 // log2(e) / temperature
    float2* partials;        // [B, 2k+1, S]
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

// Per-request epilogue, run by the last workgroup of request b.
template <typename T>
__device__ void stats_epilogue(const StatsArgs& a, int b) {
    __shared__ float sh_m[2 * kMaxK + 1], sh_s[2 * kMaxK + 1];
    __shared__ int sh_acc[kMaxK];
    __shared__ int sh_stop;
    const int k = a.k, R = 2 * k + 1;
    for (int r = threadIdx.x; r < R; r += kThreads) {
        float m = -INFINITY, s = 0.f;
        const float2* p = a.partials + ((size_t)b * R + r) * a.S;
        for (int ch = 0; ch < a.S; ++ch) {  // fixed chunk order
            float2 v = p[ch];
            merge_ms(m, s, v.x, v.y, a.c);
        }
        sh_m[r] = m;
        sh_s[r] = s;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < k; i += kThreads) {
        const int32_t x = a.draft_tokens[(size_t)b * k + i];
        const float u = a.uniforms[(size_t)b * (k + 1) + i];
        float P = 0.f, Q = 0.f;
        int acc = 0;
        if (x >= 0 && x < a.V) {
            float xt = Elem<T>::load(stats_row<T>(a, b, i), x);
            float xd = Elem<T>::load(stats_row<T>(a, b, k + 1 + i), x);
            P = fast_exp2((xt - sh_m[i]) * a.c) / sh_s[i];
            Q = fast_exp2((xd - sh_m[k + 1 + i]) * a.c) / sh_s[k + 1 + i];
            acc = (P >= Q) || (u * Q < P);  // strict u < min(1, P/Q) without a division
        }
        sh_acc[i] = acc;
        if (a.p_at_draft) a.p_at_draft[(size_t)b * k + i] = P;
        if (a.q_at_draft) a.q_at_draft[(size_t)b * k + i] = Q;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = k;
        for (int i = 0; i < k; ++i)
            if (!sh_acc[i]) { s = i; break; }
        StopInfo si;
        si.s = s;
        si.pad = 0;
        si.mt = sh_m[s];
        si.st = sh_s[s];
        si.md = (s < k) ? sh_m[k + 1 + s] : 0.f;
        si.sd = (s < k) ? sh_s[k + 1 + s] : 1.f;
        si.pad2[0] = si.pad2[1] = 0.f;
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

    float m, s = 0.f;
    if constexpr (VEC) {
        // The chunk is whole 16-byte vectors (V % EPV == 0, rows 16-byte aligned).
        const int nvec = (hi - lo) / EPV;
        const uint4* base = reinterpret_cast<const uint4*>(row + lo);
        float x[U][EPV];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int v = threadIdx.x + j * kThreads;
            if (v < nvec) {
                Elem<T>::widen(base[v], x[j]);
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) x[j][e] = -INFINITY;
            }
        }
        m = -INFINITY;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) m = fmaxf(m, x[j][e]);
        const float ms = (m == -INFINITY) ? 0.f : m;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) s += fast_exp2((x[j][e] - ms) * a.c);
    } else {
        m = -INFINITY;
        for (int j = lo + threadIdx.x; j < hi; j += kThreads) {
            float x = Elem<T>::load(row, j);
            if (x > m) {
                s = s * fast_exp2((m - x) * a.c);
                m = x;
            }
            const float ms = (m == -INFINITY) ? 0.f : m;
            s += fast_exp2((x - ms) * a.c);
        }
    }

    wave_reduce_ms(m, s, a.c);
    __shared__ float red_m[kWaves], red_s[kWaves];
    __shared__ int last_flag;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float M = red_m[0], Ssum = red_s[0];
        for (int w = 1; w < kWaves; ++w) merge_ms(M, Ssum, red_m[w], red_s[w], a.c);
        a.partials[tile] = make_float2(M, Ssum);
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
    float c;
    const StopInfo* stop;  // [B]
    double* mass;          // [B, S2]
    uint32_t* tickets;     // [B]
    int32_t* out_tokens;   // [B, k+1]
};

// Weight of one token in the final draw: the residual max(0, p - q) when the
// request stopped on a rejection, else the target probability.
struct Weigher {
    float mt, inv_st, md, inv_sd, c;
    bool residual;
    __device__ inline float operator()(float xt, float xd) const {
        float p = fast_exp2((xt - mt) * c) * inv_st;
        if (!residual) return p;
        float q = fast_exp2((xd - md) * c) * inv_sd;
        return fmaxf(p - q, 0.f);
    }
};

// Weights of this thread's segment (kSampleSegVecs consecutive 16-byte vectors,
// or the scalar equivalent) of chunk `ch`: w[] in ascending token order,
// first token id in *j0, count in *n.
template <typename T, bool VEC>
__device__ inline void segment_weights(const T* trow, const T* drow, const Weigher& W, int V,
                                       int lo, int hi, float* w, int* j0, int* n) {
    constexpr int EPV = Elem<T>::kPerVec;
    constexpr int SEG = kSampleSegVecs * EPV;
    const int start = lo + threadIdx.x * SEG;
    *j0 = start;
    *n = max(0, min(SEG, hi - start));
    if constexpr (VEC) {
#pragma unroll
        for (int v = 0; v < kSampleSegVecs; ++v) {
            const int j = start + v * EPV;
            float xt[EPV], xd[EPV];
            if (j < hi) {
                Elem<T>::widen(load16(trow + j), xt);
                if (W.residual) Elem<T>::widen(load16(drow + j), xd);
                else
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xd[e] = 0.f;
#pragma unroll
                for (int e = 0; e < EPV; ++e) w[v * EPV + e] = W(xt[e], xd[e]);
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) w[v * EPV + e] = 0.f;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < SEG; ++e) {
            const int j = start + e;
            if (j < hi) {
                float xt = Elem<T>::load(trow, j);
                float xd = W.residual ? Elem<T>::load(drow, j) : 0.f;
                w[e] = W(xt, xd);
            } else {
                w[e] = 0.f;
            }
        }
    }
    (void)V;
}

template <typename T, bool VEC>
__device__ double chunk_mass(const T* trow, const T* drow, const Weigher& W, int V, int lo,
                             int hi, double* red) {
    constexpr int SEG = kSampleSegVecs * Elem<T>::kPerVec;
    float w[SEG];
    int j0, n;
    segment_weights<T, VEC>(trow, drow, W, V, lo, hi, w, &j0, &n);
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < SEG; ++e) acc += (double)w[e];
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
    constexpr int SEG = kSampleSegVecs * Elem<T>::kPerVec;
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
        __threadfence();
        __syncthreads();
        __threadfence();
    }

    // Token selection inside the chosen chunk.
    const int c = sh_chunk;
    const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
    float w[SEG];
    int j0, n;
    segment_weights<T, VEC>(trow, drow, W, a.V, lo, hi, w, &j0, &n);
    double seg = 0.0;
#pragma unroll
    for (int e = 0; e < SEG; ++e) seg += (double)w[e];
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
            if (w[e] > 0.f) last_pos = j0 + e;
            run += (double)w[e];
            if (run > tau) { tok = j0 + e; break; }
        }
        sh_token = (tok >= 0) ? tok : last_pos;
    }
    __syncthreads();
    if (sh_token < 0) {
        // Rounding left u * Z past this chunk's total: the chunk's last positive weight.
        int last_pos = -1;
        for (int e = 0; e < SEG; ++e)
            if (e < n && w[e] > 0.f) last_pos = j0 + e;
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
    W.inv_st = 1.f / si.st;
    W.md = si.md;
    W.inv_sd = 1.f / si.sd;
    W.c = a.c;
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
    a.c = kLog2e / call.temperature;
    a.partials = reinterpret_cast<float2*>(ws + g.off_partials);
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
    s.c = a.c;
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
