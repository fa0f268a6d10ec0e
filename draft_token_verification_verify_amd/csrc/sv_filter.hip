// sv_filter.hip -- the sampling filters of the filtered stochastic call (top-k,
// top-p, min-p), applied alike to every target and draft row.
//
// The target and the draft side of a verification must be filtered the same
// way (page "TensorRT-LLM source teardown (10)", "Rejection sampling": the
// temperature, top-k, top-p and min-p of the two sides must match, or the
// acceptance test compares distributions that were never sampled).  The pages
// name the filters without defining them; the definitions used, every
// threshold on the logit x (which orders tokens as p does):
//   top-k (0 < top_k < V): keep x >= the top_k-th largest logit (ties kept);
//   top-p (0 < top_p < 1): among the top-k survivors, in descending order,
//         keep the fewest distinct logit values whose mass reaches top_p times
//         the survivors' mass (ties kept);
//   min-p (0 < min_p <= 1): keep x >= max x + T ln(min_p), i.e. p >= min_p * max p;
// applied in that order.  A row keeps the tokens with x >= tau, tau the largest
// of the three thresholds, and its kept mass is renormalised.
//
// One workgroup of 1024 threads per logits row:
//   1. The row maximum m, from the streaming kernel's statistics partials.
//   2. With top-k or top-p on: a histogram of the row over bins of 1/16 octave
//      of weight below the maximum (bin = floor((m - x) * 16 c), the last bin
//      taking everything 128 octaves down): exact token counts and, for top-p,
//      masses as fixed-point integers (2^41 per unit of weight 2^((x-m)c));
//      integer sums do not depend on the order of the atomic adds, so every
//      run gives the same bits.
//   3. The bin holding the boundary is gathered into LDS and sorted; the
//      threshold is read off the sorted values.  A boundary bin larger than
//      the LDS buffer is first narrowed by 8-bit digits of the order-preserving
//      key of x (radix selection, one pass over the row per digit).
//   4. The kept mass s = sum over x >= tau of 2^((x - m) c), fp64, fixed order.
// The sampler then treats every token below its row's tau as probability 0 and
// normalises by s.
//
// Weights: 2^a for a = (x - m) c > -8 by the fp64 exponential; below, as 2^n
// times the fp32 exponential of the fraction, n = floor(a) (a computed in
// fp64), which keeps every weight within ~2^-22 relative.
#include "sv_common.hpp"
#include "sv_launch.hpp"
#include "sv_stream.hpp"

namespace sv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 2048;          // weight bins, 1/16 octave each
constexpr int kBinsPerOctave = 16;
constexpr int kDigitBits = 8;        // radix digit of the narrowing passes
constexpr int kDigits = 1 << kDigitBits;
constexpr int kCand = 8192;          // logits gathered into LDS for the exact selection
constexpr int kMassBits = 41;       // fixed-point mass: 2^41 units per octave-top weight
constexpr double kCertify = 1e-6;    // top-p margin (relative) the fast weights may decide

struct FilterArgs {
    const void* target;
    const void* draft;
    int B, k, V;
    int R, S;              // rows per request, statistics chunks per row
    double c64;            // log2(e) / temperature
    float bin_scale;       // bins per unit of logit: 16 c
    double temperature;
    int top_k;
    double top_p, min_p;
    const Partial16* partials;  // [B, R, S] statistics partials (f0 = chunk max)
    RowFilter* rowf;            // [B, R] output
};

template <typename T>
__device__ inline const T* filter_row(const FilterArgs& a, int b, int r) {
    if (r <= a.k) return static_cast<const T*>(a.target) + ((size_t)b * (a.k + 1) + r) * (size_t)a.V;
    return static_cast<const T*>(a.draft) + ((size_t)b * a.k + (r - a.k - 1)) * (size_t)a.V;
}

// Order-preserving unsigned key of a logit (larger x, larger key), restricted
// to the bits that can differ: all 32 for fp32, the top 16 for bf16 (whose
// widened values have zero low halves).
template <typename T> struct KeyBits { static constexpr int value = 32; };
template <> struct KeyBits<bf16_t> { static constexpr int value = 16; };

template <typename T>
__device__ inline uint32_t key_of(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return k >> (32 - KeyBits<T>::value);
}

template <typename T>
__device__ inline float value_of_key(uint32_t key) {
    uint32_t k = key << (32 - KeyBits<T>::value);
    if (KeyBits<T>::value < 32 && !(k & 0x80000000u)) k |= 0xffffffffu >> KeyBits<T>::value;
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// Weight bin of x below the row maximum m: monotone (a larger x never gets a
// larger bin), so every bin is an interval of logits.
__device__ inline int bin_of(float x, float m, float bin_scale) {
    const float t = fmaxf((m - x) * bin_scale, 0.f);
    return t < (float)(kBins - 1) ? (int)t : kBins - 1;
}

// Weights of bin b lie in (2^-(o+1), 2^-o], o its octave (the last bin shares
// octave 127).  Masses are kept in units of 2^-(o + 41) per bin: a weight is
// then at most 2^41 units and is rounded to within 2^-42 of itself, and a bin's
// sum of up to 2^22 weights fits 64 bits.
__device__ inline int octave_of(int bin) { return min(bin / kBinsPerOctave, 127); }
__device__ inline double unit_of(int bin) { return ldexp(1.0, -(octave_of(bin) + kMassBits)); }

// fp64 2^a, out of line: it sits on a rare branch of the per-logit loops.
__device__ __noinline__ double exp2_f64(double a) { return exp2(a); }

// 2^((x - m) c) for x <= m, fp64.  Accurate (acc): the fp64 exponential for
// every logit.  Otherwise the fp64 exponential above 2^-8 and below it 2^n
// times the fp32 exponential of the fractional part, n = floor of the fp64
// exponent: within ~1.5e-7 relative of the true weight.
__device__ inline double weight_of(float x, float m, double c64, bool acc) {
    if (x == -INFINITY) return 0.0;
    const double a = ((double)x - (double)m) * c64;
    if (a < -1100.0) return 0.0;
    if (acc || a > -8.0) return exp2_f64(a);
    const double n = floor(a);
    return ldexp((double)fast_exp2((float)(a - n)), (int)n);
}

__device__ inline unsigned long long qweight(float x, float m, double c64, int bin, bool acc) {
    return (unsigned long long)(ldexp(weight_of(x, m, c64, acc), octave_of(bin) + kMassBits) + 0.5);
}

// Every element of a row, in a fixed per-thread order (so per-thread sums are
// the same on every run).
template <typename T, bool VEC, class F>
__device__ inline void for_each_logit(const T* row, int V, F&& f) {
    if constexpr (VEC) {
        constexpr int EPV = Elem<T>::kPerVec;
        const int nvec = V / EPV;
        const uint4* p = reinterpret_cast<const uint4*>(row);
        int v = threadIdx.x;
        for (; v + 3 * kSelThreads < nvec; v += 4 * kSelThreads) {
            uint4 raw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) raw[j] = p[v + j * kSelThreads];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x[EPV];
                Elem<T>::widen(raw[j], x);
#pragma unroll
                for (int e = 0; e < EPV; ++e) f(x[e]);
            }
        }
        for (; v < nvec; v += kSelThreads) {
            float x[EPV];
            Elem<T>::widen(p[v], x);
#pragma unroll
            for (int e = 0; e < EPV; ++e) f(x[e]);
        }
    } else {
        for (int j = threadIdx.x; j < V; j += kSelThreads) f(Elem<T>::load(row, j));
    }
}

// ---------------------------------------------------------------------------
// Workgroup-wide steps (1024 threads).
// ---------------------------------------------------------------------------
struct SelLds {
    uint32_t cnt[kBins];  // weight-bin counts (inclusive prefix after the scan)
    union {
        unsigned long long q[kBins];  // per-bin fixed-point masses while counting
        double cum[kBins];            // inclusive running mass after the scan
    } mass;
    uint32_t dcnt[kDigits];           // digit histogram of a narrowing pass
    unsigned long long dmass[kDigits];
    float cand[kCand];                // gathered logits
    unsigned long long red_u[kSelWaves];
    double red_d[kSelWaves];
    float red_f[kSelWaves];
    unsigned long long bcast;
    int red_i;
    int n_gathered;
};

__device__ inline unsigned long long wave_inclusive_scan_u64(unsigned long long v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned long long o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive prefix over the workgroup in thread order; *total = the sum.
__device__ inline unsigned long long sel_exclusive_scan(unsigned long long v, SelLds& L,
                                                        unsigned long long* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long inc = wave_inclusive_scan_u64(v);
    if (lane == 63) L.red_u[wave] = inc;
    __syncthreads();
    unsigned long long before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const unsigned long long t = L.red_u[w];
        if (w < wave) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// fp64 exclusive prefix in thread order, fixed operation order.
__device__ inline double sel_exclusive_scan_f64(double v, SelLds& L) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const double inc = wave_inclusive_scan(v);
    if (lane == 63) L.red_d[wave] = inc;
    __syncthreads();
    double before = 0.0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w)
        if (w < wave) before += L.red_d[w];
    __syncthreads();
    return before + (inc - v);
}

__device__ inline unsigned long long sel_sum_u64(unsigned long long v, SelLds& L) {
    unsigned long long total;
    sel_exclusive_scan(v, L, &total);
    return total;
}

__device__ inline float sel_max(float v, SelLds& L) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) L.red_f[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = L.red_f[0];
#pragma unroll
    for (int w = 1; w < kSelWaves; ++w) r = fmaxf(r, L.red_f[w]);
    __syncthreads();
    return r;
}

// fp64 sum in a fixed order (same bits on every run).
__device__ inline double sel_sum_f64(double v, SelLds& L) {
    v = wave_reduce_sum(v);
    if ((threadIdx.x & 63) == 0) L.red_d[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = L.red_d[0];
#pragma unroll
    for (int w = 1; w < kSelWaves; ++w) r += L.red_d[w];
    __syncthreads();
    return r;
}

__device__ inline int sel_min_int(int v, SelLds& L) {
    if (threadIdx.x == 0) L.red_i = 0x7fffffff;
    __syncthreads();
    atomicMin(&L.red_i, v);
    __syncthreads();
    const int r = L.red_i;
    __syncthreads();
    return r;
}

// Weight bins: counts to an inclusive prefix in place and, with masses, the
// per-bin fixed-point sums to an fp64 inclusive running mass (bin units folded
// in; fixed order).
__device__ inline void scan_bins(SelLds& L, bool with_mass) {
    constexpr int kPer = kBins / kSelThreads;
    const int lo = threadIdx.x * kPer;
    unsigned long long c = 0;
    double md[kPer], msum = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        c += L.cnt[lo + i];
        md[i] = with_mass ? (double)L.mass.q[lo + i] * unit_of(lo + i) : 0.0;
        msum += md[i];
    }
    unsigned long long t;
    unsigned long long cx = sel_exclusive_scan(c, L, &t);
    double mx = with_mass ? sel_exclusive_scan_f64(msum, L) : 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        cx += L.cnt[lo + i];
        L.cnt[lo + i] = (uint32_t)cx;
        if (with_mass) {
            mx += md[i];
            L.mass.cum[lo + i] = mx;
        }
    }
    __syncthreads();
}

// In-place inclusive prefix of a digit histogram (counts, fixed-point masses).
__device__ inline void scan_digits(SelLds& L, int nd) {
    const int i = threadIdx.x;
    const unsigned long long c = i < nd ? L.dcnt[i] : 0ull;
    const unsigned long long q = i < nd ? L.dmass[i] : 0ull;
    unsigned long long t;
    const unsigned long long cx = sel_exclusive_scan(c, L, &t);
    const unsigned long long qx = sel_exclusive_scan(q, L, &t);
    if (i < nd) {
        L.dcnt[i] = (uint32_t)(cx + c);
        L.dmass[i] = qx + q;
    }
    __syncthreads();
}

// First bin whose inclusive count reaches r (nb when none does).
__device__ inline int first_bin_count(const uint32_t* incl, int nb, uint32_t r, SelLds& L) {
    unsigned long long below = 0;
    for (int i = threadIdx.x; i < nb; i += kSelThreads) below += incl[i] < r;
    return (int)sel_sum_u64(below, L);
}

// Descending bitonic sort of cand[0, n) (n <= kCand), padded with -inf.
__device__ inline void sort_desc(float* cand, int n) {
    int npad = 2;
    while (npad < n) npad <<= 1;
    for (int i = n + threadIdx.x; i < npad; i += kSelThreads) cand[i] = -INFINITY;
    __syncthreads();
    for (int size = 2; size <= npad; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < npad / 2; t += kSelThreads) {
                const int i = 2 * t - (t & (stride - 1)), j = i + stride;
                const float x = cand[i], y = cand[j];
                const bool desc = (i & size) == 0;
                if (desc ? (x < y) : (x > y)) {
                    cand[i] = y;
                    cand[j] = x;
                }
            }
            __syncthreads();
        }
}

struct SelectOut {
    float tau;
    double margin;  // mass mode: distance of the target from the nearer group edge
};

// Selection inside weight bin `bin` among the logits x >= floor_v (n_set of
// them, n_set >= 1):
//   rank mode: tau = the r-th largest (1 <= r <= n_set);
//   mass mode: tau = the largest distinct value v with
//              base + mass{x in the set, x >= v} >= target (base: the mass of
//              the bins before this one), or the smallest value of the set
//              when rounding leaves none; margin = the distance of the target
//              from the running mass at the two edges of v's group (0 when
//              none was found).
template <typename T, bool VEC>
__device__ SelectOut select_in_bin(const T* row, const FilterArgs& a, float m, int bin,
                                   float floor_v, uint32_t n_set, bool rank_mode, uint32_t r,
                                   double base, double target, bool acc, SelLds& L) {
    constexpr int KB = KeyBits<T>::value;
    const double unit = unit_of(bin);
    int done = 0;          // key bits fixed so far
    uint32_t prefix = 0;   // their value
    uint32_t n = n_set;    // set elements whose key starts with prefix
    unsigned long long mass_above = 0;  // fixed-point mass of the set above that interval
    auto in_set = [&](float x) {
        if (bin_of(x, m, a.bin_scale) != bin || !(x >= floor_v)) return false;
        return done == 0 || (key_of<T>(x) >> (KB - done)) == prefix;
    };
    // Narrow by key digits until the candidates fit in LDS.
    while (n > (uint32_t)kCand && done < KB) {
        const int w = min(kDigitBits, KB - done);
        const int shift = KB - done - w;
        const uint32_t mask = (1u << w) - 1;
        for (int i = threadIdx.x; i < kDigits; i += kSelThreads) {
            L.dcnt[i] = 0;
            L.dmass[i] = 0;
        }
        __syncthreads();
        for_each_logit<T, VEC>(row, a.V, [&](float x) {
            if (in_set(x)) {
                const int d = (int)(mask - ((key_of<T>(x) >> shift) & mask));  // 0: largest
                atomicAdd(&L.dcnt[d], 1u);
                if (!rank_mode) atomicAdd(&L.dmass[d], qweight(x, m, a.c64, bin, acc));
            }
        });
        __syncthreads();
        const int nd = 1 << w;
        scan_digits(L, nd);
        int d;
        if (rank_mode) {
            d = first_bin_count(L.dcnt, nd, r, L);
        } else {
            unsigned long long below = 0;
            for (int i = threadIdx.x; i < nd; i += kSelThreads)
                below += base + (double)(mass_above + L.dmass[i]) * unit < target;
            d = (int)sel_sum_u64(below, L);
            if (d == nd) d = first_bin_count(L.dcnt, nd, L.dcnt[nd - 1], L);  // last non-empty
        }
        d = min(d, nd - 1);
        const uint32_t c_ex = d ? L.dcnt[d - 1] : 0u;
        const unsigned long long m_ex = d ? L.dmass[d - 1] : 0ull;
        n = L.dcnt[d] - c_ex;
        mass_above += m_ex;
        if (rank_mode) r -= c_ex;
        prefix = (prefix << w) | (mask - (uint32_t)d);
        done += w;
        __syncthreads();
    }
    SelectOut out;
    if (n > (uint32_t)kCand) {  // one key left: every candidate has the same value
        out.tau = value_of_key<T>(prefix);
        const double before = base + (double)mass_above * unit;
        const double after =
            base + (double)(mass_above + (unsigned long long)n * qweight(out.tau, m, a.c64, bin, acc)) * unit;
        out.margin = fmin(after - target, target - before);
        return out;
    }
    // Gather the candidates and sort them.
    if (threadIdx.x == 0) L.n_gathered = 0;
    __syncthreads();
    for_each_logit<T, VEC>(row, a.V, [&](float x) {
        if (in_set(x)) {
            const int i = atomicAdd(&L.n_gathered, 1);
            if (i < kCand) L.cand[i] = x;
        }
    });
    __syncthreads();
    const int ng = min(L.n_gathered, kCand);
    __syncthreads();
    sort_desc(L.cand, ng);
    if (rank_mode) {
        out.tau = L.cand[max(min((int)r, ng), 1) - 1];
        out.margin = 0.0;
        __syncthreads();
        return out;
    }
    // Mass mode: running mass over the sorted values, each thread a run of
    // consecutive entries; the first group end (last entry of a run of equal
    // values) whose running mass reaches the target.
    const int per = (ng + kSelThreads - 1) / kSelThreads;
    const int lo = threadIdx.x * per;
    unsigned long long own = 0;
    for (int i = 0; i < per; ++i)
        if (lo + i < ng) own += qweight(L.cand[lo + i], m, a.c64, bin, acc);
    unsigned long long total;
    unsigned long long run = mass_above + sel_exclusive_scan(own, L, &total);
    int hit = 0x7fffffff;
    unsigned long long run_hit = 0;
    for (int i = 0; i < per; ++i) {
        const int j = lo + i;
        if (j < ng) {
            run += qweight(L.cand[j], m, a.c64, bin, acc);
            const bool group_end = (j == ng - 1) || (L.cand[j + 1] != L.cand[j]);
            if (group_end && base + (double)run * unit >= target && j < hit) {
                hit = j;
                run_hit = run;
            }
        }
    }
    const int h = sel_min_int(hit, L);
    if (hit == h && h < ng) L.bcast = run_hit;
    __syncthreads();
    if (h >= ng) {
        out.tau = L.cand[max(ng - 1, 0)];
        out.margin = 0.0;
        __syncthreads();
        return out;
    }
    out.tau = L.cand[h];
    const unsigned long long end = L.bcast;
    unsigned long long eq = 0;
    for (int j = threadIdx.x; j < ng; j += kSelThreads) eq += L.cand[j] == out.tau;
    eq = sel_sum_u64(eq, L);
    const unsigned long long start = end - eq * qweight(out.tau, m, a.c64, bin, acc);
    out.margin = fmin(base + (double)end * unit - target, target - (base + (double)start * unit));
    return out;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kSelThreads) void filter_kernel(FilterArgs a) {
    __shared__ SelLds L;
    const int row = blockIdx.x, b = row / a.R, r = row % a.R;
    const T* x = filter_row<T>(a, b, r);

    float mloc = -INFINITY;
    for (int ch = threadIdx.x; ch < a.S; ch += kSelThreads)
        mloc = fmaxf(mloc, read_partial(a.partials + (size_t)row * a.S + ch).f0);
    const float m = sel_max(mloc, L);

    float tau = -INFINITY;
    double s = 0.0;
    if (m != -INFINITY) {
        // min-p: the smallest float >= m + T ln(min_p) (x >= it exactly when
        // x >= the real threshold).
        if (a.min_p > 0.0) tau = __double2float_ru((double)m + a.temperature * log(a.min_p));
        float tau_k = -INFINITY, tau_p = -INFINITY;
        if (a.top_k > 0 && a.top_k < a.V) {
            for (int i = threadIdx.x; i < kBins; i += kSelThreads) L.cnt[i] = 0;
            __syncthreads();
            for_each_logit<T, VEC>(x, a.V, [&](float v) {
                atomicAdd(&L.cnt[bin_of(v, m, a.bin_scale)], 1u);
            });
            __syncthreads();
            scan_bins(L, false);
            const int bk = min(first_bin_count(L.cnt, kBins, (uint32_t)a.top_k, L), kBins - 1);
            const uint32_t ex = bk ? L.cnt[bk - 1] : 0u;
            tau_k = select_in_bin<T, VEC>(x, a, m, bk, -INFINITY, L.cnt[bk] - ex, true,
                                          (uint32_t)a.top_k - ex, 0.0, 0.0, false, L).tau;
        }
        if (a.top_p < 1.0) {
            // Over the top-k survivors: a pass with the fast weights, and a
            // second one with fp64 weights only when the first lands within
            // kCertify of a group edge (the fast masses are within ~1.5e-7
            // relative, so a wider margin decides the same way).
            for (int acc = 0; acc < 2; ++acc) {
                for (int i = threadIdx.x; i < kBins; i += kSelThreads) {
                    L.cnt[i] = 0;
                    L.mass.q[i] = 0;
                }
                __syncthreads();
                for_each_logit<T, VEC>(x, a.V, [&](float v) {
                    if (v >= tau_k) {
                        const int bn = bin_of(v, m, a.bin_scale);
                        atomicAdd(&L.cnt[bn], 1u);
                        atomicAdd(&L.mass.q[bn], qweight(v, m, a.c64, bn, acc != 0));
                    }
                });
                __syncthreads();
                scan_bins(L, true);
                const double mass1 = L.mass.cum[kBins - 1];
                const double target = a.top_p * mass1;
                unsigned long long below = 0;
                for (int i = threadIdx.x; i < kBins; i += kSelThreads)
                    below += L.mass.cum[i] < target;
                int bp = (int)sel_sum_u64(below, L);
                if (bp == kBins) bp = first_bin_count(L.cnt, kBins, L.cnt[kBins - 1], L);
                bp = min(bp, kBins - 1);
                const double base = bp ? L.mass.cum[bp - 1] : 0.0;
                const uint32_t n_set = L.cnt[bp] - (bp ? L.cnt[bp - 1] : 0u);
                const SelectOut o = select_in_bin<T, VEC>(x, a, m, bp, tau_k, n_set, false, 0u,
                                                          base, target, acc != 0, L);
                tau_p = o.tau;
                if (o.margin > kCertify * mass1) break;
            }
        }
        tau = fmaxf(tau, fmaxf(tau_k, tau_p));
        double acc = 0.0;
        for_each_logit<T, VEC>(x, a.V, [&](float v) {
            if (v >= tau) acc += weight_of(v, m, a.c64, false);
        });
        s = sel_sum_f64(acc, L);
    }
    if (threadIdx.x == 0) {
        RowFilter f;
        f.tau = tau;
        f.m = m;
        f.s = s;
        a.rowf[row] = f;
    }
}

template <typename T, bool VEC>
static hipError_t launch_filter(const FilterArgs& a, hipStream_t st) {
    filter_kernel<T, VEC><<<dim3((unsigned)(a.B * a.R)), dim3(kSelThreads), 0, st>>>(a);
    return hipGetLastError();
}

hipError_t run_filter(const StochasticCall& call, const FilterCall& f, const Geometry& g,
                      hipStream_t st) {
    char* ws = static_cast<char*>(call.workspace);
    FilterArgs a;
    a.target = call.target;
    a.draft = call.draft;
    a.B = call.B;
    a.k = call.k;
    a.V = call.V;
    a.R = g.R;
    a.S = g.S;
    a.c64 = 1.4426950408889634074 / (double)call.temperature;
    a.bin_scale = (float)(a.c64 * kBinsPerOctave);
    a.temperature = (double)call.temperature;
    a.top_k = f.top_k;
    a.top_p = (double)f.top_p;
    a.min_p = (double)f.min_p;
    a.partials = reinterpret_cast<const Partial16*>(ws + g.off_partials);
    a.rowf = reinterpret_cast<RowFilter*>(ws + g.off_rowf);
    if (call.dtype == 1)
        return call.vec ? launch_filter<bf16_t, true>(a, st) : launch_filter<bf16_t, false>(a, st);
    return call.vec ? launch_filter<float, true>(a, st) : launch_filter<float, false>(a, st);
}

}  // namespace sv
