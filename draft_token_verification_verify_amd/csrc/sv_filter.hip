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
// With a workspace sized for it and top-k or top-p on, a gather kernel first
// collects, in one parallel pass after the statistics, every logit less than
// 16 octaves of weight below its row's maximum and (top-p alone) the fp64 mass
// of the others; the selection below then reads those instead of its row.
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
constexpr int kBins = kFilterBins;   // weight bins, 1/16 octave each
constexpr int kBinsPerOctave = kFilterBinsPerOctave;
constexpr int kDigitBits = 8;        // radix digit of the narrowing passes
constexpr int kDigits = 1 << kDigitBits;
constexpr int kCand = 12288;         // LDS logit buffer
constexpr int kSortCap = 8192;       // general path: a bin is sorted in LDS up to this size
                                     // (a power of two <= kCand: the sort pads to one)
constexpr int kTop = 10240;          // fast path: the top of a row gathered into LDS
constexpr int kSub = kCand - kTop;   // fast path: one weight bin of it, to be sorted
static_assert((kSortCap & (kSortCap - 1)) == 0 && kSortCap <= kCand, "sorted buffer");
static_assert((kSub & (kSub - 1)) == 0, "sorted sub-buffer");
constexpr int kFirstLim = 128;       // fast path: first gather reaches 8 octaves down
static_assert(kCandMaxChunks <= kBins, "tail masses are staged in the bin arrays");
static_assert(kCandMaxChunks <= 4 * 64, "one wave turns the chunk counts into a prefix");
constexpr int kMassBits = 41;       // fixed-point mass: 2^41 units per octave-top weight
constexpr double kCertify = 1e-6;    // top-p margin (relative) the fast weights may decide
// Relative error bound of a row's mass from the streaming statistics (fp32
// exponentials, exponents rounded once in fp32; |exponent| weighted by mass is
// at most ~22 octaves for V <= 2^22), with a factor 3 to spare; a top-p edge
// decided against that mass must be this far from the target, and the gather
// overshoots the target by twice as much.
constexpr double kRowMassErr = 1e-5;

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
    float* cand;                // [B, R, S, seg] candidates of the gather kernel, or null
    uint32_t* ccount;           // [B, R, S] candidates found per chunk
    double* tails;              // [B, R, S] mass of the other logits, per chunk (top-p alone)
    int seg;                    // slots per chunk (a power of two)
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
    return filter_bin_of(x, m, bin_scale);
}

// The smallest logit whose bin is below lim (bins are monotone in x, so
// bin_of(x) < lim exactly when x >= it): a binary search over the
// order-preserving keys between -inf and the maximum.
__device__ inline float lowest_in_bins(int lim, float m, float bin_scale) {
    if (lim >= kBins) return -INFINITY;
    if (lim <= 0) return INFINITY;
    uint32_t lo = key_of<float>(-INFINITY), hi = key_of<float>(m);
    auto below = [&](uint32_t q) { return bin_of(value_of_key<float>(q), m, bin_scale) < lim; };
    // First single steps over the keys from m - lim / bin_scale, which lands
    // within a few keys of the answer (the answer is unique, so the steps and
    // the search agree); the binary search when they do not get there.
    const float guess = m - (float)lim / bin_scale;
    uint32_t q = guess >= -INFINITY ? min(max(key_of<float>(guess), lo), hi) : lo;
    for (int step = 0; step < 16; ++step) {
        if (!below(q)) {
            ++q;  // q < hi: below(hi) holds
        } else {
            if (q == lo || !below(q - 1)) return value_of_key<float>(q);
            --q;
        }
    }
    while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (bin_of(value_of_key<float>(mid), m, bin_scale) < lim) hi = mid;
        else lo = mid + 1;
    }
    return value_of_key<float>(lo);
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

// Weight of a logit at least 8 octaves below the maximum (a <= -8), with no
// call: the fast form of weight_of (acc false), or (acc) the fp64 exponential
// inlined, for loops over the tail of a row.
__device__ __attribute__((always_inline)) inline double tail_weight(float x, float m, double c64,
                                                                    bool acc) {
    if (x == -INFINITY) return 0.0;
    const double a = ((double)x - (double)m) * c64;
    if (a < -1100.0) return 0.0;
    if (acc) return exp2(a);
    const double n = floor(a);
    return ldexp((double)fast_exp2((float)(a - n)), (int)n);
}

__device__ inline unsigned long long qweight(float x, float m, double c64, int bin, bool acc) {
    return (unsigned long long)(ldexp(weight_of(x, m, c64, acc), octave_of(bin) + kMassBits) + 0.5);
}

// Every element of a row, in a fixed per-thread order (so per-thread sums are
// the same on every run).  Each thread keeps BATCH 16-byte loads in flight.
// Only one vector's elements are unrolled: the batch is walked by a loop that
// shifts the loaded vectors down one register slot per step, so the loop body
// holds EPV copies of f, not BATCH * EPV (the kernel's loops are otherwise
// larger than the instruction cache that two compute units share).
template <typename T, bool VEC, int BATCH = 4, class F>
__device__ inline void for_each_logit(const T* row, int V, F&& f) {
    if constexpr (VEC) {
        constexpr int EPV = Elem<T>::kPerVec;
        const int nvec = V / EPV;
        const uint4* p = reinterpret_cast<const uint4*>(row);
        for (int v0 = threadIdx.x; v0 < nvec; v0 += BATCH * kSelThreads) {
            uint4 raw[BATCH];
#pragma unroll
            for (int j = 0; j < BATCH; ++j) raw[j] = p[min(v0 + j * kSelThreads, nvec - 1)];
#pragma unroll 1
            for (int j = 0; j < BATCH; ++j) {
                if (v0 + j * kSelThreads < nvec) {
                    float x[EPV];
                    Elem<T>::widen(raw[0], x);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) f(x[e]);
                }
#pragma unroll
                for (int t = 0; t + 1 < BATCH; ++t) raw[t] = raw[t + 1];
            }
        }
    } else {
        for (int j = threadIdx.x; j < V; j += kSelThreads) f(Elem<T>::load(row, j));
    }
}

// ---------------------------------------------------------------------------
// Candidate gather (when the workspace has room for it): one 256-thread
// workgroup per statistics chunk, after the statistics, so every chunk knows
// its row's maximum m.  The logits of the chunk whose bin is below kCandBins
// go to the row's candidate buffer (one atomic per workgroup claims their
// slots; a row whose candidates outgrow the buffer keeps counting, and its
// filter then reads the row itself); the weights of the others are summed into
// the chunk's tail mass.  The selection then reads a few thousand candidates
// per row instead of the row, and has the mass below its first gather without
// another pass.
// ---------------------------------------------------------------------------
struct CandArgs {
    const void* target;
    const void* draft;
    int k, V, R;
    int S, chunk;       // streaming chunks per row, elements per chunk
    double c64;
    float bin_scale;
    const Partial16* partials;
    float* cand;        // [B, R, S, seg]: one segment per chunk
    uint32_t* ccount;   // [B, R, S]: candidates found per chunk (may exceed seg)
    double* tails;      // [B, R, S]: mass of the other logits per chunk
    int seg;
};

// TAIL: also sum the chunk's tail mass, with fp64 weights (the selection uses
// it for top-p without top-k only, and then decides against it as against the
// whole row's mass).
template <typename T, int U, bool TAIL>
__global__ __launch_bounds__(kThreads) void cand_kernel(CandArgs a) {
    constexpr int EPV = Elem<T>::kPerVec;
    static_assert(kThreads >= 256, "one table entry per thread");
    __shared__ float red_f[kWaves];
    __shared__ double red_d[kWaves];
    __shared__ int wsum[kWaves];
    __shared__ double tab[256];
    if (TAIL && threadIdx.x < 256) tab[threadIdx.x] = exp2((double)threadIdx.x / 256.0);
    const double c256 = a.c64 * 256.0;  // exact: a power-of-two multiple
    const int t = blockIdx.x, ch = t % a.S, row = t / a.S;
    const int b = row / a.R, r = row % a.R;
    // The tile's loads go out first; the row maximum and the floor are worked
    // out while they are in flight.
    const T* rowp = (r <= a.k)
        ? static_cast<const T*>(a.target) + ((size_t)b * (a.k + 1) + r) * (size_t)a.V
        : static_cast<const T*>(a.draft) + ((size_t)b * a.k + (r - a.k - 1)) * (size_t)a.V;
    const int lo = ch * a.chunk, hi = min(a.V, lo + a.chunk);
    const int nvec = (hi - lo) / EPV;
    const uint4* base = reinterpret_cast<const uint4*>(rowp + lo);
    uint4 raw[U];
#pragma unroll
    for (int j = 0; j < U; ++j) raw[j] = base[min((int)threadIdx.x + j * kThreads, nvec - 1)];
    float mloc = -INFINITY;
    for (int i = threadIdx.x; i < a.S; i += kThreads)
        mloc = fmaxf(mloc, read_partial(a.partials + (size_t)row * a.S + i).f0);
    const float m = block_max(mloc, red_f);
    if (m == -INFINITY) return;  // nothing to keep; the tail stays 0
    const float x_lo = lowest_in_bins(kCandBins, m, a.bin_scale);
    int n = 0;
    double tail = 0.0;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        float x[EPV];
        Elem<T>::widen(raw[j], x);
        const bool ok = (int)threadIdx.x + j * kThreads < nvec;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const bool c = ok && x[e] >= x_lo;
            n += c ? 1 : 0;
            if (TAIL && ok && !c && x[e] != -INFINITY)
                tail += exp2_256(((double)x[e] - (double)m) * c256, tab);
        }
    }
    if (TAIL) {
        const double tsum = block_sum(tail, red_d);
        if (threadIdx.x == 0 && tsum != 0.0) a.tails[t] = tsum;
    }
    // Exclusive prefix of the candidate counts over the workgroup; the slots.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? wsum[w] : 0;
        total += wsum[w];
    }
    if (total == 0) return;  // the same on every thread
    if (threadIdx.x == 0) a.ccount[t] = (uint32_t)total;
    if (total > a.seg) return;  // overflow: the row's filter reads the row itself
    int pos = before + incl - n;
    float* dst = a.cand + (size_t)t * a.seg;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        float x[EPV];
        Elem<T>::widen(raw[j], x);
        const bool ok = (int)threadIdx.x + j * kThreads < nvec;
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            if (ok && x[e] >= x_lo) dst[pos++] = x[e];
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
    union {
        float cand[kCand];            // general path: one bin's gathered logits
        struct {
            float top[kTop];          // fast path: every logit of the top weight bins
            float sub[kSub];          // fast path: one bin of those, sorted
        } f;
    } buf;
    double bscan[6];
    uint32_t tcnt[kCandMaxChunks];    // candidates per chunk of this row, then their inclusive prefix
    int n_sub;
    unsigned long long red_u[kSelWaves];
    double red_d[kSelWaves];
    float red_f[kSelWaves];
    unsigned long long bcast;
    int red_i;
    int n_gathered;
};

// The first active lane's value.  For values that every lane of the
// workgroup holds alike (read back from LDS after a barrier): the compiler then
// keeps them in scalar registers instead of vector registers that the long
// per-logit loops need.
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline uint32_t uniform(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ inline float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ inline unsigned long long uniform(unsigned long long v) {
    const uint32_t lo = uniform((uint32_t)v), hi = uniform((uint32_t)(v >> 32));
    return ((unsigned long long)hi << 32) | lo;
}
__device__ inline double uniform(double v) {
    return __longlong_as_double((long long)uniform((unsigned long long)__double_as_longlong(v)));
}

__device__ inline unsigned long long wave_inclusive_scan_u64(unsigned long long v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned long long o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    return v;
}

// Append v to buf (capacity cap) at *count when take is set: one LDS atomic per
// wave, each taking lane at the next free slot in lane order (the order within
// buf is not fixed; every reader sorts or sums order-free).  Inactive lanes
// take no part: the leader is the first active lane that takes.
// Returns this lane's slot (-1 when it does not take; >= cap when full).
__device__ inline int wave_append(bool take, float v, float* buf, int cap, int* count) {
    const unsigned long long mask = __ballot(take);
    if (!mask) return -1;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((long long)mask) - 1;
    int base = 0;
    if (lane == leader) base = atomicAdd(count, __popcll(mask));
    base = __shfl(base, leader);
    if (!take) return -1;
    const int i = base + __popcll(mask & ((1ull << lane) - 1));
    if (i < cap) buf[i] = v;
    return i;
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
    *total = uniform(all);
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
    return uniform(r);
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
    return uniform(r);
}

__device__ inline int sel_min_int(int v, SelLds& L) {
    if (threadIdx.x == 0) L.red_i = 0x7fffffff;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) atomicMin(&L.red_i, v);
    __syncthreads();
    const int r = uniform(L.red_i);
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

// Running totals over weight bins [0, nb) of the counts and the fixed-point
// masses (bin units folded in, fp64 in a fixed order): the first bin whose
// running count reaches r (by_count) or whose running mass reaches target, nb
// when none does, with the totals before and through it and over all nb bins.
struct BinScan {
    int bin;
    unsigned long long cnt_ex, cnt_total;
    double mass_ex, mass_in, mass_total;
};

__device__ inline BinScan scan_find(SelLds& L, int nb, bool by_count, unsigned long long r,
                                    double target) {
    // One wave walks the bins 64 at a time (lane l: bin 64 j + l), carrying the
    // running totals; the other waves wait.
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        unsigned long long carry_c = 0;
        double carry_m = 0.0;
        int hit = -1;
        for (int j = 0; j < nb; j += 64) {
            const int b = j + lane;
            const unsigned long long c = b < nb ? L.cnt[b] : 0ull;
            const double mq = b < nb ? (double)L.mass.q[b] * unit_of(b) : 0.0;
            const unsigned long long cin = carry_c + wave_inclusive_scan_u64(c);
            const double min_ = carry_m + wave_inclusive_scan(mq);
            if (hit < 0) {
                const unsigned long long found =
                    __ballot(b < nb && (by_count ? cin >= r : min_ >= target));
                if (found) {
                    hit = j + __ffsll((long long)found) - 1;
                    if (b == hit) {
                        L.bscan[0] = (double)(cin - c);
                        L.bscan[1] = min_ - mq;
                        L.bscan[2] = min_;
                    }
                }
            }
            carry_c = __shfl(cin, 63);
            carry_m = __shfl(min_, 63);
        }
        if (lane == 0) {
            L.red_i = hit < 0 ? nb : hit;
            L.bscan[3] = (double)carry_c;  // totals over the nb bins
            L.bscan[4] = carry_m;
        }
    }
    __syncthreads();
    BinScan out;
    out.bin = uniform(L.red_i);
    out.cnt_total = (unsigned long long)uniform(L.bscan[3]);
    out.mass_total = uniform(L.bscan[4]);
    const bool hit = out.bin < nb;
    out.cnt_ex = hit ? (unsigned long long)uniform(L.bscan[0]) : out.cnt_total;
    out.mass_ex = hit ? uniform(L.bscan[1]) : out.mass_total;
    out.mass_in = hit ? uniform(L.bscan[2]) : out.mass_total;
    __syncthreads();
    return out;
}

// Descending bitonic sort of cand[0, n), padded with -inf up to the next power
// of two (which must fit in the buffer).
__device__ inline void sort_desc(float* cand, int n) {
    if (n <= 64) {
        // One wave, in registers: bitonic network over lanes by shuffles
        // (lane pairs i < j = i ^ stride keep the larger value at i in
        // descending blocks, at j in ascending ones).
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            float v = lane < n ? cand[lane] : -INFINITY;
#pragma unroll
            for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    const float o = __shfl_xor(v, stride);
                    const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
                    v = keep_max ? fmaxf(v, o) : fminf(v, o);
                }
            if (lane < n) cand[lane] = v;
        }
        __syncthreads();
        return;
    }
    if (n <= 512) {
        // Rank sort: entry t goes to the number of entries above it, or equal
        // to it at a smaller index (n broadcast LDS reads per thread, no
        // network of barriers).
        const int t = threadIdx.x;
        float v = 0.f;
        int rank = 0;
        if (t < n) {
            v = cand[t];
            for (int j = 0; j < n; ++j) {
                const float u = cand[j];
                rank += (u > v || (u == v && j < t)) ? 1 : 0;
            }
        }
        __syncthreads();
        if (t < n) cand[rank] = v;
        __syncthreads();
        return;
    }
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
__device__ __attribute__((always_inline)) SelectOut select_in_bin(const T* row, const FilterArgs& a, float m, int bin,
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
    while (n > (uint32_t)kSortCap && done < KB) {
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
    if (n > (uint32_t)kSortCap) {  // one key left: every candidate has the same value
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
            if (i < kSortCap) L.buf.cand[i] = x;
        }
    });
    __syncthreads();
    const int ng = min(L.n_gathered, kSortCap);
    __syncthreads();
    sort_desc(L.buf.cand, ng);
    if (rank_mode) {
        out.tau = L.buf.cand[max(min((int)r, ng), 1) - 1];
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
        if (lo + i < ng) own += qweight(L.buf.cand[lo + i], m, a.c64, bin, acc);
    unsigned long long total;
    unsigned long long run = mass_above + sel_exclusive_scan(own, L, &total);
    int hit = 0x7fffffff;
    unsigned long long run_hit = 0;
    for (int i = 0; i < per; ++i) {
        const int j = lo + i;
        if (j < ng) {
            run += qweight(L.buf.cand[j], m, a.c64, bin, acc);
            const bool group_end = (j == ng - 1) || (L.buf.cand[j + 1] != L.buf.cand[j]);
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
        out.tau = L.buf.cand[max(ng - 1, 0)];
        out.margin = 0.0;
        __syncthreads();
        return out;
    }
    out.tau = L.buf.cand[h];
    const unsigned long long end = L.bcast;
    unsigned long long eq = 0;
    for (int j = threadIdx.x; j < ng; j += kSelThreads) eq += L.buf.cand[j] == out.tau;
    eq = sel_sum_u64(eq, L);
    const unsigned long long start = end - eq * qweight(out.tau, m, a.c64, bin, acc);
    out.margin = fmin(base + (double)end * unit - target, target - (base + (double)start * unit));
    return out;
}

// ---------------------------------------------------------------------------
// Fast path: the top of the row.
// ---------------------------------------------------------------------------

// Every candidate of the row (from the gather kernel): chunk c's in slots
// [c seg, c seg + its count) of `cand`; candidate g (in chunk order) lies in
// the first chunk whose inclusive count prefix L.tcnt exceeds g.  Four loads
// per thread in flight.
template <class F>
__device__ inline void for_each_candidate(const float* cand, int S, int seg, const SelLds& L,
                                          F&& f) {
    const int total = (int)L.tcnt[S - 1];
    for (int g0 = 0; g0 < total; g0 += 4 * kSelThreads) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = g0 + j * kSelThreads + (int)threadIdx.x;
            v[j] = -INFINITY;
            if (g < total) {
                int lo = 0, hi = S - 1;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if ((int)L.tcnt[mid] > g) hi = mid;
                    else lo = mid + 1;
                }
                v[j] = cand[lo * seg + g - (lo ? (int)L.tcnt[lo - 1] : 0)];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) f(v[j]);  // -inf for the slots past the end
    }
}

// Copy the logits of weight bin `bin` that are >= floor_v from the gathered
// top of the row into sub[] and sort them (descending).  False when the bin is
// too large for sub[].
template <typename T, bool VEC>
__device__ inline bool gather_bin(SelLds& L, const T* x, bool complete, int ntop, float m,
                                  const FilterArgs& a, int bin, float floor_v,
                                  const float* cand) {
    const bool fits = L.cnt[bin] <= (uint32_t)kSub;
    __syncthreads();  // every wave has read the count before anyone may rewrite it
    if (!uniform((int)fits)) return false;
    if (threadIdx.x == 0) L.n_sub = 0;
    __syncthreads();
    if (complete) {  // every logit of the bin is in top[]
        for (int i0 = 0; i0 < ntop; i0 += kSelThreads) {
            const int i = i0 + threadIdx.x;
            const float v = i < ntop ? L.buf.f.top[i] : -INFINITY;
            wave_append(i < ntop && bin_of(v, m, a.bin_scale) == bin && v >= floor_v, v,
                        L.buf.f.sub, kSub, &L.n_sub);
        }
    } else {  // top[] overflowed: one pass over the candidates or the row for the bin's logits
        const float x_lo = lowest_in_bins(bin + 1, m, a.bin_scale);
        const float x_hi = lowest_in_bins(bin, m, a.bin_scale);
        const float lo = fmaxf(x_lo, floor_v);
        auto take = [&](float v) { wave_append(v >= lo && v < x_hi, v, L.buf.f.sub, kSub, &L.n_sub); };
        if (cand && bin < kCandBins) for_each_candidate(cand, a.S, a.seg, L, take);
        else for_each_logit<T, VEC, 4>(x, a.V, take);
    }
    __syncthreads();
    sort_desc(L.buf.f.sub, uniform(L.n_sub));
    return true;
}

struct Walk {
    bool found;
    float tau;
    double margin, mass;  // mass: base + the mass of sub's entries >= tau
};

// Top-p inside one sorted bin: the first group end (last entry of a run of
// equal values) of sub[0, ns) whose running mass base + ... reaches target,
// with fp64 weights (fixed point, order-free sums).
__device__ inline Walk walk_sub(SelLds& L, int ns, float m, const FilterArgs& a, int bin,
                                double base, double target) {
    const double unit = unit_of(bin);
    const float* v = L.buf.f.sub;
    if (ns <= 64) {  // one wave: its scan replaces the workgroup's barriers
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            const bool in = lane < ns;
            const float x = in ? v[lane] : -INFINITY;
            const float next = lane + 1 < ns ? v[lane + 1] : -INFINITY;
            const unsigned long long q = in ? qweight(x, m, a.c64, bin, true) : 0ull;
            const unsigned long long run = wave_inclusive_scan_u64(q);
            const bool group_end = in && (lane == ns - 1 || next != x);
            const unsigned long long hits =
                __ballot(group_end && base + (double)run * unit >= target);
            double found = 0.0, tau = -INFINITY, mass = 0.0, margin = 0.0;
            if (hits) {
                const int h = __ffsll((long long)hits) - 1;
                const float th = __shfl(x, h);
                const unsigned long long end = __shfl(run, h);
                const unsigned long long eq = (unsigned long long)__popcll(__ballot(in && x == th));
                const unsigned long long start = end - eq * qweight(th, m, a.c64, bin, true);
                found = 1.0;
                tau = th;
                mass = base + (double)end * unit;
                margin = fmin(mass - target, target - (base + (double)start * unit));
            }
            if (lane == 0) {
                L.bscan[0] = found;
                L.bscan[1] = tau;
                L.bscan[2] = mass;
                L.bscan[3] = margin;
            }
        }
        __syncthreads();
        Walk w;
        w.found = uniform(L.bscan[0]) != 0.0;
        w.tau = (float)uniform(L.bscan[1]);
        w.mass = uniform(L.bscan[2]);
        w.margin = uniform(L.bscan[3]);
        __syncthreads();
        return w;
    }
    const int per = (ns + kSelThreads - 1) / kSelThreads;
    const int lo = threadIdx.x * per;
    unsigned long long own = 0;
    for (int i = 0; i < per; ++i)
        if (lo + i < ns) own += qweight(v[lo + i], m, a.c64, bin, true);
    unsigned long long total;
    unsigned long long run = sel_exclusive_scan(own, L, &total);
    int hit = 0x7fffffff;
    unsigned long long run_hit = 0;
    for (int i = 0; i < per; ++i) {
        const int j = lo + i;
        if (j < ns) {
            run += qweight(v[j], m, a.c64, bin, true);
            const bool group_end = (j == ns - 1) || (v[j + 1] != v[j]);
            if (group_end && base + (double)run * unit >= target && j < hit) {
                hit = j;
                run_hit = run;
            }
        }
    }
    const int h = sel_min_int(hit, L);
    if (hit == h && h < ns) L.bcast = run_hit;
    __syncthreads();
    Walk w;
    w.found = h < ns;
    w.tau = w.found ? uniform(v[h]) : -INFINITY;
    w.margin = 0.0;
    w.mass = 0.0;
    if (w.found) {
        const unsigned long long end = uniform(L.bcast);
        unsigned long long eq = 0;
        for (int j = threadIdx.x; j < ns; j += kSelThreads) eq += v[j] == w.tau;
        eq = sel_sum_u64(eq, L);
        const unsigned long long start = end - eq * qweight(w.tau, m, a.c64, bin, true);
        w.mass = base + (double)end * unit;
        w.margin = fmin(w.mass - target, target - (base + (double)start * unit));
    }
    __syncthreads();
    return w;
}

// Gather every logit of the top weight bins -- 8 octaves below the maximum,
// then 16, 32, ... until the boundaries of the filters that are on lie inside
// -- with per-bin counts and fp64 masses, and read the thresholds and the kept
// mass off that set: top-k from the sorted boundary bin, top-p by a walk over
// its boundary bin (against the top-k set's mass, or against the row's mass
// from the streaming statistics when top-k is off, where a decision closer
// than kRowMassErr is left to the general path).  Returns false, having
// decided nothing, when the set outgrows LDS or a decision is left open.
template <typename T, bool VEC>
__device__ __attribute__((always_inline)) bool fast_filter(const T* x, const FilterArgs& a, float m, double s_row, float tau_m,
                            const float* cand, double rest_cand, float* tau_out,
                            double* s_out, SelLds& L) {
    const bool topk = a.top_k > 0 && a.top_k < a.V;
    const bool topp = a.top_p < 1.0;
    for (int i = threadIdx.x; i < kBins; i += kSelThreads) {
        L.cnt[i] = 0;
        L.mass.q[i] = 0;
    }
    if (threadIdx.x == 0) L.n_gathered = 0;
    __syncthreads();
    // Top-p alone usually reaches further down than 8 octaves: start at 16.
    int lim_prev = 0, lim = (topp && !topk) ? 2 * kFirstLim : kFirstLim;
    bool complete = true;  // top[] holds every logit of the bins below lim
    BinScan sc;
    int n_have = 0;  // entries of top[] already counted (read after a barrier, never during a pass)
    for (;;) {
        const int n0 = n_have;
        // bins [lim_prev, lim) are the logits in [x_lo, x_hi)
        const float x_lo = lowest_in_bins(lim, m, a.bin_scale);
        const float x_hi = lowest_in_bins(lim_prev, m, a.bin_scale);
        auto put = [&](bool take, float v) {
            const int i = wave_append(take, v, L.buf.f.top, kTop, &L.n_gathered);
            if (i >= kTop) {  // no room: count and weigh it here
                const int bn = bin_of(v, m, a.bin_scale);
                atomicAdd(&L.cnt[bn], 1u);
                atomicAdd(&L.mass.q[bn], qweight(v, m, a.c64, bn, true));
            }
        };
        if (cand && lim <= kCandBins) {
            // every logit of bins < kCandBins is among the row's candidates
            for_each_candidate(cand, a.S, a.seg, L, [&](float v) { put(v >= x_lo && v < x_hi, v); });
        } else {
            for_each_logit<T, VEC, 4>(x, a.V, [&](float v) { put(v >= x_lo && v < x_hi, v); });
        }
        __syncthreads();
        const int ngat = uniform(L.n_gathered);
        const int n1 = min(ngat, kTop);
        n_have = n1;
        complete = complete && ngat <= kTop;
        __syncthreads();
        // Counts and fp64 masses of the newly gathered logits, from LDS.
        for (int i = n0 + threadIdx.x; i < n1; i += kSelThreads) {
            const float v = L.buf.f.top[i];
            const int bn = bin_of(v, m, a.bin_scale);
            atomicAdd(&L.cnt[bn], 1u);
            atomicAdd(&L.mass.q[bn], qweight(v, m, a.c64, bn, true));
        }
        __syncthreads();
        sc = topk ? scan_find(L, lim, true, (unsigned long long)a.top_k, 0.0)
                  : scan_find(L, lim, false, 0ull, a.top_p * s_row * (1.0 + 2.0 * kRowMassErr));
        if (sc.bin < lim || lim == kBins) break;
        lim_prev = lim;
        lim = min(2 * lim, kBins);
    }
    const bool whole_row = lim == kBins;  // then the gathered masses are the row's
    const int ntop = min(uniform(L.n_gathered), kTop);

    float tau_k = -INFINITY, tau_p = -INFINITY;
    double s_k = 0.0, s_p = 0.0;
    int bk = lim, nk = 0;
    if (topk) {
        bk = sc.bin;
        const int r = (int)(a.top_k - sc.cnt_ex);
        if (!gather_bin<T, VEC>(L, x, complete, ntop, m, a, bk, -INFINITY, cand)) return false;
        const int ns = uniform(L.n_sub);
        tau_k = uniform(L.buf.f.sub[max(min(r, ns), 1) - 1]);
        unsigned long long c = 0, q = 0;
        if (ns <= 64) {  // one wave
            if (threadIdx.x < 64) {
                const float v = (int)threadIdx.x < ns ? L.buf.f.sub[threadIdx.x] : -INFINITY;
                const bool keep = (int)threadIdx.x < ns && v >= tau_k;
                const unsigned long long kept = __ballot(keep);
                const unsigned long long qs =
                    wave_inclusive_scan_u64(keep ? qweight(v, m, a.c64, bk, true) : 0ull);
                if (threadIdx.x == 63) {
                    L.red_u[0] = (unsigned long long)__popcll(kept);
                    L.red_u[1] = qs;
                }
            }
            __syncthreads();
            c = uniform(L.red_u[0]);
            q = uniform(L.red_u[1]);
            __syncthreads();
            nk = (int)c;
            s_k = sc.mass_ex + (double)q * unit_of(bk);
        } else {
            for (int i = threadIdx.x; i < ns; i += kSelThreads)
                if (L.buf.f.sub[i] >= tau_k) {
                    ++c;
                    q += qweight(L.buf.f.sub[i], m, a.c64, bk, true);
                }
            nk = (int)sel_sum_u64(c, L);
            s_k = sc.mass_ex + (double)sel_sum_u64(q, L) * unit_of(bk);
        }
    }
    if (topp) {
        // With the gather kernel's candidates (and top-k off), the first
        // gather reaches exactly kCandBins bins down and the mass of the rest
        // of the row comes with them, from fp64 weights: the row's mass is
        // then known as well as from a whole-row gather.
        const bool with_tail = !topk && cand && lim == kCandBins;
        const double mass1 = topk        ? s_k
                             : whole_row ? sc.mass_total
                             : with_tail ? sc.mass_total + rest_cand
                                         : s_row;
        const bool exact = topk || whole_row || with_tail;
        const double target = a.top_p * mass1;
        // Bins before bk lie wholly in the top-k set; bin bk's part >= tau_k
        // holds the rest of its mass, which reaches the target.
        const BinScan sp = scan_find(L, topk ? bk : lim, false, 0ull, target);
        const int bp = sp.bin;
        if (!topk && bp == lim) return false;
        int ns;
        if (topk && bp == bk) {
            ns = nk;  // sub holds bin bk sorted: its first nk entries are >= tau_k
        } else {
            if (!gather_bin<T, VEC>(L, x, complete, ntop, m, a, bp, -INFINITY, cand)) return false;
            ns = uniform(L.n_sub);
        }
        Walk w = walk_sub(L, ns, m, a, bp, sp.mass_ex, target);
        if (!w.found) return false;
        // Too close to call against the statistics' mass: the row's mass
        // again, as the gathered bins' fp64 mass plus the rest of the row,
        // first with the fast weights (within ~2e-7 of that rest), then, if
        // still too close, with fp64 weights (then the decision is final).
        if (!exact && w.margin <= kRowMassErr * mass1) {
            const float x_lo = lowest_in_bins(lim, m, a.bin_scale);
            int in_sub = bp;  // the bin held (sorted) in sub[]
            for (int tier = 0; tier < 2; ++tier) {
                const bool acc64 = tier == 1;
                double acc = 0.0;
                // x < x_lo lies at least lim / 16 >= 8 octaves down.
                if (acc64)
                    for_each_logit<T, VEC, 4>(x, a.V, [&](float v) {
                        if (v < x_lo) acc += tail_weight(v, m, a.c64, true);
                    });
                else
                    for_each_logit<T, VEC, 4>(x, a.V, [&](float v) {
                        if (v < x_lo) acc += tail_weight(v, m, a.c64, false);
                    });
                const double rest = sel_sum_f64(acc, L);
                const double mass1b = sc.mass_total + rest;
                const double target_b = a.top_p * mass1b;
                const BinScan sq = scan_find(L, lim, false, 0ull, target_b);
                if (sq.bin == lim) return false;
                if (sq.bin != in_sub) {
                    if (!gather_bin<T, VEC>(L, x, complete, ntop, m, a, sq.bin, -INFINITY, cand))
                        return false;
                    ns = uniform(L.n_sub);
                    in_sub = sq.bin;
                }
                w = walk_sub(L, ns, m, a, sq.bin, sq.mass_ex, target_b);
                if (!w.found) return false;
                if (acc64 || w.margin > 1e-6 * rest + 1e-11 * mass1b) break;
            }
        }
        tau_p = w.tau;
        s_p = w.mass;
    }
    const float tau = fmaxf(tau_m, fmaxf(tau_k, tau_p));
    double s;
    if (topp && tau == tau_p) {
        s = s_p;
    } else if (topk && tau == tau_k) {
        s = s_k;
    } else {
        // min-p above the others: every kept logit lies in the gathered bins
        // (at or before the bin of a threshold below tau).
        const int bt = bin_of(tau, m, a.bin_scale);
        const BinScan st = scan_find(L, bt, true, ~0ull, 0.0);
        if (!gather_bin<T, VEC>(L, x, complete, ntop, m, a, bt, tau, cand)) return false;
        unsigned long long q = 0;
        const int nb_sub = uniform(L.n_sub);
        for (int i = threadIdx.x; i < nb_sub; i += kSelThreads)
            q += qweight(L.buf.f.sub[i], m, a.c64, bt, true);
        s = st.mass_total + (double)sel_sum_u64(q, L) * unit_of(bt);
    }
    *tau_out = tau;
    *s_out = s;
    return true;
}

// General path: top-k and top-p from a histogram of the whole row (counts; for
// top-p, masses with the fast weights, repeated with fp64 weights when the
// fast ones land within kCertify of a group edge) and the boundary bin
// gathered, narrowed by key digits where it is larger than LDS.  Returns tau.
template <typename T, bool VEC>
__device__ __attribute__((always_inline)) float general_thresholds(const T* x, const FilterArgs& a, float m, float tau_m,
                                    SelLds& L) {
    float tau_k = -INFINITY, tau_p = -INFINITY;
    __syncthreads();  // the fast path's last reads of the bins are done
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
    return fmaxf(tau_m, fmaxf(tau_k, tau_p));
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kSelThreads, 8) void filter_kernel(FilterArgs a) {
    __shared__ SelLds L;
    const int row = blockIdx.x, b = row / a.R, r = row % a.R;
    const T* x = filter_row<T>(a, b, r);
    // The gather kernel's candidates of this row (per-chunk counts staged in
    // LDS), usable when every chunk's fit its segment, and the mass of the
    // rest of the row (fixed order).
    float* cand = a.cand ? a.cand + (size_t)row * a.S * a.seg : nullptr;
    int over = 0;
    if (cand)
        for (int ch = threadIdx.x; ch < a.S; ch += kSelThreads) {
            const uint32_t c = a.ccount[(size_t)row * a.S + ch];
            L.tcnt[ch] = c;
            L.mass.cum[ch] = a.tails[(size_t)row * a.S + ch];  // free until the selection
            over |= c > (uint32_t)a.seg;
        }
    over = __syncthreads_or(over);
    if (cand) {  // the counts to an inclusive prefix over the chunks (one wave, S <= 256)
        if (threadIdx.x < 64) {
            const int base = threadIdx.x * 4;
            uint32_t c[4], sum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = base + i < a.S ? L.tcnt[base + i] : 0u;
                sum += c[i];
            }
            uint32_t run = (uint32_t)wave_inclusive_scan_u64(sum) - sum;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                run += c[i];
                if (base + i < a.S) L.tcnt[base + i] = run;
            }
        }
        __syncthreads();
    }
    const float* usable = (cand && !over) ? cand : nullptr;
    double rest_cand = 0.0;
    if (cand)
        for (int ch = 0; ch < a.S; ++ch) rest_cand += L.mass.cum[ch];

    float mloc = -INFINITY;
    for (int ch = threadIdx.x; ch < a.S; ch += kSelThreads)
        mloc = fmaxf(mloc, read_partial(a.partials + (size_t)row * a.S + ch).f0);
    const float m = sel_max(mloc, L);

    float tau = -INFINITY;
    double s = 0.0;
    if (m != -INFINITY) {
        // min-p: the smallest float >= m + T ln(min_p) (x >= it exactly when
        // x >= the real threshold).
        const float tau_m =
            a.min_p > 0.0 ? __double2float_ru((double)m + a.temperature * log(a.min_p)) : -INFINITY;
        const bool topk = a.top_k > 0 && a.top_k < a.V;
        const bool topp = a.top_p < 1.0;
        bool decided = false;
        if (topk || topp) {
            // The row's mass from the statistics partials (fp64, fixed order).
            double sp = 0.0;
            for (int ch = threadIdx.x; ch < a.S; ch += kSelThreads) {
                const PartialRead q = read_partial(a.partials + (size_t)row * a.S + ch);
                if (q.f0 != -INFINITY) sp += q.d * exp2_f64(((double)q.f0 - (double)m) * a.c64);
            }
            const double s_row = sel_sum_f64(sp, L);
            decided = fast_filter<T, VEC>(x, a, m, s_row, tau_m, usable, rest_cand, &tau, &s, L);
        }
        if (!decided) {
            tau = general_thresholds<T, VEC>(x, a, m, tau_m, L);
            double acc = 0.0;
            for_each_logit<T, VEC>(x, a.V, [&](float v) {
                if (v >= tau) acc += weight_of(v, m, a.c64, false);
            });
            s = sel_sum_f64(acc, L);
        }
    }
    if (threadIdx.x == 0) {
        RowFilter f;
        f.tau = tau;
        f.m = m;
        f.s = s;
        a.rowf[row] = f;
    }
    if (cand) {  // leave the workspace zero: the candidates written, the counts, the tails
        __syncthreads();
        const int nslots = a.S * a.seg;
        for (int i = threadIdx.x; i < nslots; i += kSelThreads) {
            const int ch = i / a.seg;
            const uint32_t c = L.tcnt[ch] - (ch ? L.tcnt[ch - 1] : 0u);
            if (c <= (uint32_t)a.seg && (uint32_t)(i & (a.seg - 1)) < c) cand[i] = 0.f;
        }
        for (int ch = threadIdx.x; ch < a.S; ch += kSelThreads) {
            a.tails[(size_t)row * a.S + ch] = 0.0;
            a.ccount[(size_t)row * a.S + ch] = 0u;
        }
    }
}

template <typename T, bool VEC>
static hipError_t launch_filter(const FilterArgs& a, hipStream_t st, const KernelEvents& ev) {
    // The events (when set) take the kernel's own start and end timestamps.
    hipExtLaunchKernelGGL(filter_kernel<T, VEC>, dim3((unsigned)(a.B * a.R)), dim3(kSelThreads),
                          0, st, ev.begin, ev.end, 0, a);
    return hipGetLastError();
}

template <typename T, bool TAIL>
static hipError_t launch_cand(const CandArgs& c, int U, unsigned n_tiles, hipStream_t st) {
    switch (U) {
        case 8: cand_kernel<T, 8, TAIL><<<n_tiles, kThreads, 0, st>>>(c); break;
        case 4: cand_kernel<T, 4, TAIL><<<n_tiles, kThreads, 0, st>>>(c); break;
        case 2: cand_kernel<T, 2, TAIL><<<n_tiles, kThreads, 0, st>>>(c); break;
        default: cand_kernel<T, 1, TAIL><<<n_tiles, kThreads, 0, st>>>(c); break;
    }
    return hipGetLastError();
}

hipError_t run_filter(const StochasticCall& call, const FilterCall& f, const Geometry& g,
                      hipStream_t st, const KernelEvents& ev) {
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
    a.bin_scale = filter_bin_scale(call.temperature);
    a.temperature = (double)call.temperature;
    a.top_k = f.top_k;
    a.top_p = (double)f.top_p;
    a.min_p = (double)f.min_p;
    a.partials = reinterpret_cast<const Partial16*>(ws + g.off_partials);
    a.rowf = reinterpret_cast<RowFilter*>(ws + g.off_rowf);
    // Candidates when the workspace has room (mode 3 layout), the rows are
    // 16-byte aligned and top-k or top-p is on (min-p alone needs one pass over
    // each row for its kept mass either way).
    const bool topk_on = f.top_k > 0 && f.top_k < call.V, topp_on = f.top_p < 1.0f;
    const bool cand = g.cand_seg > 0 && call.vec && (topk_on || topp_on);
    a.cand = cand ? reinterpret_cast<float*>(ws + g.off_cand) : nullptr;
    a.ccount = cand ? reinterpret_cast<uint32_t*>(ws + g.off_ccount) : nullptr;
    a.tails = cand ? reinterpret_cast<double*>(ws + g.off_tails) : nullptr;
    a.seg = cand ? g.cand_seg : 0;
    if (cand) {
        CandArgs c;
        c.target = call.target;
        c.draft = call.draft;
        c.k = call.k;
        c.V = call.V;
        c.R = g.R;
        c.S = g.S;
        c.chunk = g.chunk;
        c.c64 = a.c64;
        c.bin_scale = a.bin_scale;
        c.partials = a.partials;
        c.cand = a.cand;
        c.ccount = a.ccount;
        c.tails = a.tails;
        c.seg = a.seg;
        const unsigned n_tiles = (unsigned)((long long)call.B * g.R * g.S);
        // The tail masses serve top-p without top-k only (its first gather
        // reaches exactly kCandBins bins down).
        const bool tail = topp_on && !topk_on;
        const hipError_t e =
            call.dtype == 1
                ? (tail ? launch_cand<bf16_t, true>(c, g.U, n_tiles, st)
                        : launch_cand<bf16_t, false>(c, g.U, n_tiles, st))
                : (tail ? launch_cand<float, true>(c, g.U, n_tiles, st)
                        : launch_cand<float, false>(c, g.U, n_tiles, st));
        if (e != hipSuccess) return e;
    }
    if (call.dtype == 1)
        return call.vec ? launch_filter<bf16_t, true>(a, st, ev)
                        : launch_filter<bf16_t, false>(a, st, ev);
    return call.vec ? launch_filter<float, true>(a, st, ev) : launch_filter<float, false>(a, st, ev);
}

}  // namespace sv
