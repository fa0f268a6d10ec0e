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
//            scale factors.  A tile of a test row also publishes the raw logit
//            of the tested draft token when that token falls inside it.
//   sample:  one workgroup per (request, stop-row chunk).  Every workgroup of a
//            request first merges that request's partials (chunk order, fp64),
//            computes p_i(x_i) and q_i(x_i), runs the k tests (independent given
//            the uniforms) and takes the first failure as the stop row s; the
//            chunk-0 workgroup writes the accepted drafts, the -1 padding,
//            num_accepted and the probabilities.  Each workgroup then computes
//            its chunk's share of the final distribution's mass (residual
//            max(0, p_s - q_s) or bonus p_k) in fp64 -- tokens within 2^-8 of
//            the row maximum take an fp64 exponential, the rest fp32 -- and the
//            last of the request's workgroups (arrival ticket) picks the chunk
//            holding u_k * Z by a prefix sum over the chunk masses, then the
//            token inside that chunk by a prefix sum over per-thread segments
//            and a walk through one segment (ascending vocabulary order: the
//            smallest j whose running mass exceeds u_k * Z).
// The streaming kernel has no atomics or fences: the kernel boundary publishes
// its partials to the sampler.
//
// Accuracy matters beyond the decisions themselves: a vocabulary of ~10^5 has
// ~10^5 CDF edges, so a relative error e in the cumulative weights moves the
// drawn token on a fraction ~V * e of the draws.  The fp64 paths above keep e
// near 1e-10.
#include "sv_common.hpp"
#include "sv_launch.hpp"
#include "sv_stream.hpp"

namespace sv {

struct CallArgs {
    const void* target;
    const void* draft;
    const int32_t* draft_tokens;
    const float* uniforms;
    int B, k, V;
    int R, S, chunk;         // streaming geometry: rows per request, chunks per row
    int S2, chunk2;          // sampler geometry: chunks per stop row
    Scale sc;                // log2(e) / temperature
    Partial16* partials;     // [B, 2k+1, S]: f0 = chunk max, f1 = tested logit or NaN, d = sum
    uint32_t* tickets;       // per request (padded): sampler arrivals
    double* mass;            // [B, S2]
    int32_t* out_tokens;     // [B, k+1]
    int32_t* num_accepted;   // [B]
    float* p_at_draft;       // [B, k] or null
    float* q_at_draft;       // [B, k] or null
};

// p(x) = 2^((x - M) * c) / S in fp64; 0 when x or the whole row is -inf.
__device__ inline double prob_of(float x, float M, double S, const Scale& k) {
    if (M == -INFINITY || !(S > 0.0)) return 0.0;
    return exp2_accurate(x, M, k) / S;
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

    // Draft token tested on row r of request b, or -1 for the bonus row.
    __device__ int token_of_row(int b, int r) const {
        if (r == k) return -1;
        const int i = (r < k) ? r : r - k - 1;
        return draft_tokens[(size_t)b * k + i];
    }

    // Workgroup reduction of per-thread (max m, fp64 sum s against m) into the
    // tile's (M, S): every thread's sum is rescaled to the common M with an fp64
    // exponential, then summed in fixed order.
    __device__ void finish(float m, double s, float gx, float* f0, float* f1, double* d) const {
        __shared__ float red_f[kWaves];
        __shared__ double red_d[kWaves];
        const float M = block_max(m, red_f);
        const double f = (m == -INFINITY) ? 0.0 : exp2_accurate(m, M, sc);
        const double Ssum = block_sum(s * f, red_d);
        *f0 = M;
        *f1 = gx;
        *d = Ssum;
    }

    __device__ void tile(int b, int r, int lo, int hi, const uint4* raw, int nvec, float* f0,
                         float* f1, double* d) const {
        constexpr int EPV = Elem<T>::kPerVec;
        // Thread 0 fetches the tested token's logit early (it is in this tile's
        // lines, so the load overlaps the arithmetic).
        float gx = __builtin_nanf("");
        if (threadIdx.x == 0) {
            const int x = token_of_row(b, r);
            if (x >= lo && x < hi) gx = Elem<T>::load(row(b, r), x);
        }
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
        const float ms = (m == -INFINITY) ? 0.f : m;
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) s += (double)fast_exp2(scaled(x[j][e] - ms, sc));
        finish(m, s, gx, f0, f1, d);
    }

    __device__ void tile_scalar(int b, int r, int lo, int hi, float* f0, float* f1,
                                double* d) const {
        const T* p = row(b, r);
        float gx = __builtin_nanf("");
        if (threadIdx.x == 0) {
            const int x = token_of_row(b, r);
            if (x >= lo && x < hi) gx = Elem<T>::load(p, x);
        }
        float m = -INFINITY;
        for (int j = lo + threadIdx.x; j < hi; j += kThreads) m = fmaxf(m, Elem<T>::load(p, j));
        const float ms = (m == -INFINITY) ? 0.f : m;
        double s = 0.0;
        for (int j = lo + threadIdx.x; j < hi; j += kThreads)
            s += (double)fast_exp2(scaled(Elem<T>::load(p, j) - ms, sc));
        finish(m, s, gx, f0, f1, d);
    }
};

template <typename T, int U, bool VEC>
__global__ __launch_bounds__(kThreads) void stats_kernel(CallArgs a) {
    StatsOp<T, U> op;
    static_cast<CallArgs&>(op) = a;
    if constexpr (VEC) stream_tile_vec<T, U>(op);
    else stream_tile_scalar<T>(op);
}

// ---------------------------------------------------------------------------
// Sampler: decision, stop-row mass, final draw.
// ---------------------------------------------------------------------------

// The request's decision, computed by every sampler workgroup of the request
// from the streaming partials (fixed chunk order, fp64).
struct Decision {
    int s;
    float mt, md;
    double st, sd;
};

constexpr int kMergeLds = 1024;  // partials per request staged in LDS for the merge

// Row statistics of request b: sh_m[r] = row max, sh_s[r] = sum of
// 2^((x - max) * c) in fp64 (chunks merged in order), sh_g[r] = tested logit.
__device__ void merge_rows(const CallArgs& a, int b, float* sh_m, double* sh_s, float* sh_g) {
    const int R = a.R, S = a.S, n = R * S;
    const Partial16* p = a.partials + (size_t)b * n;
    for (int r = threadIdx.x; r < R; r += kThreads) sh_g[r] = __builtin_nanf("");
    __syncthreads();
    if (n <= kMergeLds) {
        // Every thread takes a few partials: one fp64 exponential each.
        __shared__ float pm[kMergeLds];
        __shared__ double ps[kMergeLds];
        for (int t = threadIdx.x; t < n; t += kThreads) {
            const Partial16 q = p[t];
            pm[t] = q.f0;
            ps[t] = q.d;
            if (!__builtin_isnan(q.f1)) sh_g[t / S] = q.f1;  // one chunk per row holds it
        }
        __syncthreads();
        for (int r = threadIdx.x; r < R; r += kThreads) {
            float M = -INFINITY;
            for (int ch = 0; ch < S; ++ch) M = fmaxf(M, pm[r * S + ch]);
            sh_m[r] = M;
        }
        __syncthreads();
        for (int t = threadIdx.x; t < n; t += kThreads) {
            const float M = sh_m[t / S];
            ps[t] = (M == -INFINITY) ? 0.0 : ps[t] * exp2_accurate(pm[t], M, a.sc);
        }
        __syncthreads();
        for (int r = threadIdx.x; r < R; r += kThreads) {
            double acc = 0.0;
            for (int ch = 0; ch < S; ++ch) acc += ps[r * S + ch];  // fixed chunk order
            sh_s[r] = acc;
        }
    } else {
        for (int r = threadIdx.x; r < R; r += kThreads) {
            const Partial16* q = p + (size_t)r * S;
            float M = -INFINITY;
            for (int ch = 0; ch < S; ++ch) {
                M = fmaxf(M, q[ch].f0);
                if (!__builtin_isnan(q[ch].f1)) sh_g[r] = q[ch].f1;
            }
            double acc = 0.0;
            if (M != -INFINITY)
                for (int ch = 0; ch < S; ++ch) acc += q[ch].d * exp2_accurate(q[ch].f0, M, a.sc);
            sh_m[r] = M;
            sh_s[r] = acc;
        }
    }
    __syncthreads();
}

__device__ void decide(const CallArgs& a, int b, bool write_outputs, Decision* out) {
    __shared__ float sh_m[2 * kMaxK + 1], sh_g[2 * kMaxK + 1];
    __shared__ double sh_s[2 * kMaxK + 1];
    __shared__ int sh_acc[kMaxK];
    __shared__ int sh_stop;
    const int k = a.k;
    merge_rows(a, b, sh_m, sh_s, sh_g);
    for (int i = threadIdx.x; i < k; i += kThreads) {
        const int32_t x = a.draft_tokens[(size_t)b * k + i];
        const float u = a.uniforms[(size_t)b * (k + 1) + i];
        double P = 0.0, Q = 0.0;
        int acc = 0;
        if (x >= 0 && x < a.V) {
            P = prob_of(sh_g[i], sh_m[i], sh_s[i], a.sc);
            Q = prob_of(sh_g[k + 1 + i], sh_m[k + 1 + i], sh_s[k + 1 + i], a.sc);
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
        int s = k;
        for (int i = 0; i < k; ++i)
            if (!sh_acc[i]) { s = i; break; }
        sh_stop = s;
        if (write_outputs) a.num_accepted[b] = s;
    }
    __syncthreads();
    const int s = sh_stop;
    if (write_outputs)
        for (int i = threadIdx.x; i <= k; i += kThreads) {
            if (i < s) a.out_tokens[(size_t)b * (k + 1) + i] = a.draft_tokens[(size_t)b * k + i];
            else if (i > s) a.out_tokens[(size_t)b * (k + 1) + i] = -1;
            // out_tokens[b, s] is written by the final draw.
        }
    out->s = s;
    out->mt = sh_m[s];
    out->st = sh_s[s];
    out->md = (s < k) ? sh_m[k + 1 + s] : 0.f;
    out->sd = (s < k) ? sh_s[k + 1 + s] : 1.0;
    __syncthreads();
}

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

constexpr int kSub = 16;  // tokens per sub-step of a sampler segment

// Visit this thread's contiguous segment of the chunk [lo, hi) -- tokens
// [lo + t * NSUB * 16, ...) -- in ascending order, 16 tokens per sub-step with
// all loads of a sub-step issued together (clamped in bounds); f(j, w) is
// called for every token of the segment inside the chunk.  drow == trow when
// there is no residual.
template <typename T, bool VEC, int NSUB, class F>
__device__ inline void visit_segment(const T* trow, const T* drow, const Weigher& W, int lo,
                                     int hi, F&& f) {
    constexpr int EPV = Elem<T>::kPerVec;
    constexpr int NV = kSub / EPV;
    const int start = lo + (int)threadIdx.x * (NSUB * kSub);
#pragma unroll 1
    for (int sub = 0; sub < NSUB; ++sub) {
        const int s0 = start + sub * kSub;
        if constexpr (VEC) {
            uint4 rt[NV], rd[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int j = max(lo, min(s0 + v * EPV, hi - EPV));
                rt[v] = load16(trow + j);
                rd[v] = load16(drow + j);
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float xt[EPV], xd[EPV];
                Elem<T>::widen(rt[v], xt);
                Elem<T>::widen(rd[v], xd);
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const int j = s0 + v * EPV + e;
                    if (j < hi) f(j, W(xt[e], xd[e]));
                }
            }
        } else {
            float xt[kSub], xd[kSub];
#pragma unroll
            for (int e = 0; e < kSub; ++e) {
                const int j = max(lo, min(s0 + e, hi - 1));
                xt[e] = Elem<T>::load(trow, j);
                xd[e] = Elem<T>::load(drow, j);
            }
#pragma unroll
            for (int e = 0; e < kSub; ++e)
                if (s0 + e < hi) f(s0 + e, W(xt[e], xd[e]));
        }
    }
}

// Sum of this thread's segment weights, and of the whole chunk (workgroup).
template <typename T, bool VEC, int NSUB>
__device__ double chunk_mass(const T* trow, const T* drow, const Weigher& W, int lo, int hi,
                             double* seg_out, double* red) {
    double seg = 0.0;
    visit_segment<T, VEC, NSUB>(trow, drow, W, lo, hi, [&](int, double w) { seg += w; });
    *seg_out = seg;
    return block_sum(seg, red);
}

// The last workgroup of request b: chunk holding u_k * Z, then the token in it.
template <typename T, bool VEC, int NSUB>
__device__ void sample_final(const CallArgs& a, int b, int s_row, const T* trow, const T* drow,
                             Weigher W) {
    __shared__ double sh_wave[kWaves];
    __shared__ double sh_red[kWaves];
    __shared__ int sh_first;
    __shared__ double sh_base, sh_tau;
    __shared__ int sh_chunk;
    __shared__ int sh_token;
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
            if (c < a.S2) grp += load_coherent(&mass[c]);
        }
        const double incl = block_inclusive_scan(grp, sh_wave, &Z);
        if (Z > 0.0 || pass == 1) {
            const double tau = u * Z;
            if (threadIdx.x == 0) {
                sh_first = kThreads;
                sh_tau = tau;
                sh_chunk = -1;
            }
            __syncthreads();
            if (incl > tau) atomicMin(&sh_first, (int)threadIdx.x);
            __syncthreads();
            if ((int)threadIdx.x == sh_first) {
                double run = incl - grp;
                int lastc = -1;
                double lastbase = 0.0;
                for (int g = 0; g < G; ++g) {
                    const int c = threadIdx.x * G + g;
                    if (c >= a.S2) break;
                    const double mc = load_coherent(&mass[c]);
                    if (mc > 0.0) { lastc = c; lastbase = run; }
                    if (run + mc > tau) {
                        lastc = c;
                        lastbase = run;
                        break;
                    }
                    run += mc;
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
                    const double mc = load_coherent(&mass[c]);
                    if (mc > 0.0) { lastc = c; lastbase = run; }
                    run += mc;
                }
                sh_chunk = lastc;
                sh_base = lastbase;
            }
            __syncthreads();
            break;
        }
        // Z == 0: the residual vanished (p_s == q_s); draw from p_s instead.
        W.residual = false;
        drow = trow;
        for (int c = 0; c < a.S2; ++c) {
            const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
            double seg;
            const double mc = chunk_mass<T, VEC, NSUB>(trow, drow, W, lo, hi, &seg, sh_red);
            if (threadIdx.x == 0) store_coherent(&mass[c], mc);
        }
        __syncthreads();
    }

    // Token selection inside the chosen chunk: prefix over the per-thread
    // segments, then one thread walks its segment.
    const int c = sh_chunk;
    const int lo = c * a.chunk2, hi = min(a.V, lo + a.chunk2);
    double seg = 0.0;
    visit_segment<T, VEC, NSUB>(trow, drow, W, lo, hi, [&](int, double w) { seg += w; });
    double chunk_total;
    const double incl = block_inclusive_scan(seg, sh_wave, &chunk_total);
    const double base = sh_base, tau = sh_tau;
    if (threadIdx.x == 0) {
        sh_first = kThreads;
        sh_token = -1;
    }
    __syncthreads();
    if (base + incl > tau) atomicMin(&sh_first, (int)threadIdx.x);
    __syncthreads();
    if ((int)threadIdx.x == sh_first) {
        double run = base + (incl - seg);
        int tok = -1, last_pos = -1;
        visit_segment<T, VEC, NSUB>(trow, drow, W, lo, hi, [&](int j, double w) {
            if (tok >= 0) return;
            if (w > 0.0) last_pos = j;
            run += w;
            if (run > tau) tok = j;
        });
        sh_token = (tok >= 0) ? tok : last_pos;
    }
    __syncthreads();
    if (sh_token < 0) {
        // Rounding left u * Z past this chunk's total: the chunk's last positive weight.
        int last_pos = -1;
        visit_segment<T, VEC, NSUB>(trow, drow, W, lo, hi, [&](int j, double w) {
            if (w > 0.0) last_pos = j;
        });
        if (last_pos >= 0) atomicMax(&sh_token, last_pos);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        int tok = sh_token;
        if (tok < 0) tok = lo;  // no positive weight anywhere: unreachable with finite logits
        a.out_tokens[(size_t)b * (k + 1) + s_row] = tok;
    }
    // Leave this request's part of the workspace zero for later calls (every
    // other workgroup of the request has read the partials and stored its mass
    // before taking its ticket).
    __syncthreads();
    for (int cc = threadIdx.x; cc < a.S2; cc += kThreads) mass[cc] = 0.0;
    clear_partials(a.partials + (size_t)b * a.R * a.S, a.R * a.S);
}

template <typename T, bool VEC, int NSUB>
__global__ __launch_bounds__(kThreads) void sample_kernel(CallArgs a) {
    const int tile = blockIdx.x;
    const int b = tile / a.S2;
    const int ch = tile % a.S2;
    const int k = a.k;
    Decision dc;
    decide(a, b, ch == 0, &dc);
    Weigher W;
    W.mt = dc.mt;
    W.inv_st = 1.0 / dc.st;
    W.md = dc.md;
    W.inv_sd = 1.0 / dc.sd;
    W.sc = a.sc;
    W.residual = dc.s < k;
    const T* trow = static_cast<const T*>(a.target) + ((size_t)b * (k + 1) + dc.s) * (size_t)a.V;
    const T* drow = W.residual
        ? static_cast<const T*>(a.draft) + ((size_t)b * k + dc.s) * (size_t)a.V
        : trow;
    __shared__ double red[kWaves];
    __shared__ int last_flag;
    const int lo = ch * a.chunk2, hi = min(a.V, lo + a.chunk2);
    double seg;
    const double mc = chunk_mass<T, VEC, NSUB>(trow, drow, W, lo, hi, &seg, red);
    if (threadIdx.x == 0) store_coherent(&a.mass[(size_t)b * a.S2 + ch], mc);
    if (arrive_last(ticket_of(a.tickets, b), (uint32_t)a.S2, &last_flag))
        sample_final<T, VEC, NSUB>(a, b, dc.s, trow, drow, W);
}

// ---------------------------------------------------------------------------

template <typename T, int U, bool VEC>
static hipError_t launch_stats_u(const CallArgs& a, hipStream_t st) {
    const unsigned n_tiles = (unsigned)((long long)a.B * a.R * a.S);
    stats_kernel<T, U, VEC><<<dim3(n_tiles), dim3(kThreads), 0, st>>>(a);
    return hipGetLastError();
}

template <typename T, bool VEC>
static hipError_t launch_stats(const CallArgs& a, int U, hipStream_t st) {
    switch (U) {
        case 8: return launch_stats_u<T, 8, VEC>(a, st);
        case 4: return launch_stats_u<T, 4, VEC>(a, st);
        case 2: return launch_stats_u<T, 2, VEC>(a, st);
        default: return launch_stats_u<T, 1, VEC>(a, st);
    }
}

template <typename T, bool VEC>
static hipError_t launch_sample(const CallArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((long long)a.B * a.S2)), block(kThreads);
    switch (a.chunk2 / (kThreads * kSub)) {
        case 4: sample_kernel<T, VEC, 4><<<grid, block, 0, st>>>(a); break;
        case 2: sample_kernel<T, VEC, 2><<<grid, block, 0, st>>>(a); break;
        default: sample_kernel<T, VEC, 1><<<grid, block, 0, st>>>(a); break;
    }
    return hipGetLastError();
}

hipError_t run_stochastic(const StochasticCall& call, const Geometry& g, hipStream_t st,
                          const KernelEvents& ev) {
    char* ws = static_cast<char*>(call.workspace);
    CallArgs a;
    a.target = call.target;
    a.draft = call.draft;
    a.draft_tokens = call.draft_tokens;
    a.uniforms = call.uniforms;
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
    a.mass = reinterpret_cast<double*>(ws + g.off_mass);
    a.out_tokens = call.out_tokens;
    a.num_accepted = call.num_accepted;
    a.p_at_draft = call.p_at_draft;
    a.q_at_draft = call.q_at_draft;

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
        return call.vec ? launch_sample<bf16_t, true>(a, st) : launch_sample<bf16_t, false>(a, st);
    return call.vec ? launch_sample<float, true>(a, st) : launch_sample<float, false>(a, st);
}

}  // namespace sv
