// sv_common.hpp -- shared device helpers, launch geometry and workspace layout of
// the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <math.h>
#include <stdint.h>

#ifndef SV_COHERENT_TICKETS
#define SV_COHERENT_TICKETS 1
#endif
// Tile shape: the largest per-thread vector count (at most SV_MAX_U, or
// SV_MAX_U_ARGMAX for the greedy and tree argmax stream) whose tile count
// reaches SV_MIN_TILES (SV_MIN_TILES_ARGMAX).  The argmax tile keeps no
// statistics, so 16 vectors per thread (64 KB tiles, three workgroups per
// compute unit) hold as many bytes in flight as 8 with six, from half as many
// workgroups.  Fewer, larger tiles also shorten small calls: a tile's fixed
// costs (its reductions and publication, and the merge of one more partial)
// outweigh the parallelism of more tiles well before the chip is full.
#ifndef SV_MAX_U
#define SV_MAX_U 8
#endif
#ifndef SV_MAX_U_ARGMAX
#define SV_MAX_U_ARGMAX 16
#endif
#ifndef SV_MIN_TILES
#define SV_MIN_TILES 512
#endif
#ifndef SV_MIN_TILES_ARGMAX
#define SV_MIN_TILES_ARGMAX 128
#endif
// Distance in uint32 words between two requests' arrival counters: each counter
// gets its own cache line, so atomics on different requests do not queue on one
// line.
#ifndef SV_SAMPLER_WGS
#define SV_SAMPLER_WGS 1024
#endif
#ifndef SV_TICKET_STRIDE
#define SV_TICKET_STRIDE 64
#endif

namespace sv {

constexpr int kThreads = 256;           // one workgroup = 4 wave64s
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxK = 64;               // longest linear draft
constexpr int kTreeLdsPathEntries = 4096;  // path tables up to this many entries go to LDS
constexpr int kTicketStride = SV_TICKET_STRIDE;

// Arrival counter of request b.
__host__ __device__ inline uint32_t* ticket_of(uint32_t* base, int b) {
    return base + (size_t)b * kTicketStride;
}

// ---------------------------------------------------------------------------
// Launch geometry and workspace layout.  A pure function of the call's shape
// (never of pointer values), so sizing and launching always agree.
// ---------------------------------------------------------------------------
struct Geometry {
    int R;           // logits rows streamed per request
    int S;           // chunks per row in the streaming kernel
    int chunk;       // elements per chunk (multiple of 2048)
    int U;           // 16-byte vectors per thread per chunk: 1, 2, 4 or 8 (16: argmax)
    int S2;          // stop-row chunks per request (stochastic sampler)
    int chunk2;      // elements per stop-row chunk
    int cand_cap;    // filter candidate slots per row (mode 3), else 0: S segments of cand_seg
    int cand_seg;    // slots per streaming chunk (a power of two)
    size_t off_tickets, off_partials, off_segs, off_rowf, off_ccount, off_tails, off_cand;
    size_t off_masses;   // per request: S2 stop-row chunk masses (one word each)
    size_t bytes;
};

// Sampling filters: weight bins of 1/16 octave below a row's maximum m,
// bin = floor((m - x) * 16 log2(e) / T), the last bin taking everything 128
// octaves down.  Monotone in x (a larger x never gets a larger bin), so every
// bin is an interval of logits, and a smaller m never gives a larger bin.
constexpr int kFilterBins = 2048;
constexpr int kFilterBinsPerOctave = 16;
// The filtered call's candidate gather keeps every logit of a row whose bin is
// below kCandBins (16 octaves), in up to kCandCap slots per row.
constexpr int kCandBins = 256;
constexpr int kCandCap = 16384;
constexpr int kCandMaxChunks = 256;  // rows of more streaming chunks keep no candidates

// Stop-row chunks per request at most (one workgroup-wide scan over their
// masses): with 16 * 4 tokens per thread, vocabularies up to 2^22.
constexpr int kMaxChunks2 = 256;
constexpr int kSamplerOneRound = 256;  // sampler workgroups that fit one per compute unit

// Stochastic tree walk split over several workgroups per request: their
// exchange area in the workspace (mode 4), per request.
constexpr size_t kTreeSyncBytes = 3328;

// Bins per unit of logit, 16 log2(e) / T, rounded to fp32 once: one value for
// every kernel that bins.
inline float filter_bin_scale(float temperature) {
    return (float)(1.4426950408889634074 / (double)temperature * kFilterBinsPerOctave);
}

__host__ __device__ inline int filter_bin_of(float x, float m, float bin_scale) {
    const float t = fmaxf((m - x) * bin_scale, 0.f);
    return t < (float)(kFilterBins - 1) ? (int)t : kFilterBins - 1;
}

// log2(e) / temperature, the factor that turns a logit difference into a
// base-2 exponent.  The fp32 pair (hi, lo) carries it to ~2^-48 relative, so an
// exponent computed as fma(d, hi, d * lo) is rounded once (0.5 ulp); c64 feeds
// the fp64 paths.
struct Scale {
    float hi, lo;
    double c64;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// mode: 0 stochastic, 1 greedy, 2 tree, 3 stochastic with filter candidates
// (mode 0's layout plus a candidate buffer at the end), 5 (internal) mode 0's
// layout with the filtered call's sampler chunks, 4 stochastic tree walk
// (its exchange area only); rows_per_request: k+1 or N+1.
inline bool make_geometry(int mode, int B, int rows_per_request, int V, int elem_bytes,
                          Geometry* g) {
    if (B < 1 || rows_per_request < 1 || V < 1 || (elem_bytes != 2 && elem_bytes != 4))
        return false;
    const int epv = 16 / elem_bytes;  // elements per 16-byte vector
    if (mode == 4) {  // stochastic tree walk: only the exchange area
        if (B < 1 || rows_per_request < 1 || V < 1 || (elem_bytes != 2 && elem_bytes != 4))
            return false;
        *g = Geometry{};
        g->bytes = kTreeSyncBytes * (size_t)B;
        return true;
    }
    // Mode 5 (internal): the stochastic layout for a filtered call whose
    // workspace has no room for the candidates.  Modes 3 and 5 size the
    // sampler alike, so both give a filtered call the same bits.
    bool cand = mode == 3;
    const bool filtered = mode == 3 || mode == 5;
    if (filtered) mode = 0;
    g->R = (mode == 0) ? 2 * rows_per_request - 1 : rows_per_request;
    const long long rows = (long long)B * g->R;
    // Largest per-thread vector count whose tile count reaches the floor;
    // small problems fall back to smaller tiles.
    int U = (mode == 1 || mode == 2) ? SV_MAX_U_ARGMAX : SV_MAX_U;
    for (; U > 1; U >>= 1) {
        long long ce = (long long)kThreads * U * epv;
        long long tiles = rows * ((V + ce - 1) / ce);
        if (tiles >= ((mode == 1 || mode == 2) ? SV_MIN_TILES_ARGMAX : SV_MIN_TILES)) break;
    }
    g->U = U;
    g->chunk = kThreads * U * epv;
    g->S = (V + g->chunk - 1) / g->chunk;
    // Sampler: 8, 16, 32 or 64 consecutive tokens per thread.  8 while the
    // call's sampler workgroups fit one per compute unit (each then runs its
    // chain alone, and a shorter chunk shortens the chain); otherwise the
    // smallest of 16, 32 and 64 that keeps the sampler to about one round of
    // resident workgroups (there the weighing is bound by the chip's ALU
    // throughput and more workgroups only add decisions).  The filtered call's
    // sampler takes at least 16 (its stored 64-token segments are summed by at
    // most 4 threads).
    auto items = [&](int tpt) {
        return (long long)B * ((V + (long long)kThreads * tpt - 1) / ((long long)kThreads * tpt));
    };
    int tpt = 8;
    if (filtered || items(8) > kSamplerOneRound) {
        tpt = 16;
        while (tpt < 64 && (items(tpt) > SV_SAMPLER_WGS || items(tpt) / B > kMaxChunks2)) tpt <<= 1;
    }
    g->chunk2 = kThreads * tpt;
    g->S2 = (mode == 0) ? (V + g->chunk2 - 1) / g->chunk2 : 0;

    size_t off = 0;
    g->off_tickets = off;  // per-request counters, one cache line each
    off = align_up(off + sizeof(uint32_t) * kTicketStride * (size_t)B, 256);
    g->off_partials = off;
    off = align_up(off + 16 * (size_t)rows * (size_t)g->S, 256);
    g->off_segs = off;
    // Stop-row segment masses: per request 256 runs of ceil(n / 256) slots for
    // its n = S2 * chunk2 / 64 segments of 64 tokens.
    const long long nseg = (long long)g->S2 * (g->chunk2 / 64);
    off = align_up(off + sizeof(double) * (size_t)B * (size_t)((nseg + kThreads - 1) / kThreads) *
                             kThreads, 256);
    g->off_rowf = off;  // per-row sampling filter of the filtered call (stochastic only)
    off = align_up(off + (mode == 0 ? 16 * (size_t)rows : 0), 256);
    g->off_masses = off;   // stop-row chunk masses, two rounds (stochastic only)
    off = align_up(off + (mode == 0 ? 16 * (size_t)B * (size_t)g->S2 : 0), 256);
    // Candidates: per row up to kCandCap slots (fewer for a short vocabulary),
    // split into one power-of-two segment per streaming chunk.
    cand = cand && g->S <= kCandMaxChunks;
    const long long vpad = ((long long)V + 63) / 64 * 64;
    const long long per_row = vpad < kCandCap ? vpad : kCandCap;
    int seg = 1;
    while ((long long)seg * 2 * g->S <= per_row) seg *= 2;
    g->cand_seg = cand ? seg : 0;
    g->cand_cap = cand ? seg * g->S : 0;
    g->off_ccount = off;  // candidates found per chunk
    off = align_up(off + (cand ? sizeof(uint32_t) * (size_t)rows * (size_t)g->S : 0), 256);
    g->off_tails = off;   // mass of the other logits per chunk
    off = align_up(off + (cand ? sizeof(double) * (size_t)rows * (size_t)g->S : 0), 256);
    g->off_cand = off;    // candidate logits, cand_cap per row
    off = align_up(off + sizeof(float) * (size_t)rows * (size_t)g->cand_cap, 256);
    g->bytes = off;
    return true;
}

// ---------------------------------------------------------------------------
// Element access.  bf16 logits are carried as raw uint16 bit patterns; widening
// to fp32 is a 16-bit shift (exact).
// ---------------------------------------------------------------------------
struct bf16_t { uint16_t bits; };

template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int kPerVec = 4;
    __device__ static inline float load(const float* p, size_t i) { return p[i]; }
    __device__ static inline void widen(const uint4& v, float* out) {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    }
};

template <> struct Elem<bf16_t> {
    static constexpr int kPerVec = 8;
    __device__ static inline float load(const bf16_t* p, size_t i) {
        return __uint_as_float((uint32_t)p[i].bits << 16);
    }
    __device__ static inline void widen(const uint4& v, float* out) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            out[2 * q] = __uint_as_float(w[q] << 16);
            out[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
    }
};

__device__ inline uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// hi is c rounded toward zero and, when c is a float itself, one step lower, so
// lo = c - hi is strictly positive: then d = -inf gives -inf (never inf - inf).
inline Scale make_scale(float temperature) {
    Scale k;
    k.c64 = 1.4426950408889634074 / (double)temperature;
    float hi = (float)k.c64;
    if ((double)hi >= k.c64) hi = nextafterf(hi, 0.f);
    k.hi = hi;
    k.lo = (float)(k.c64 - (double)hi);
    return k;
}

// Base-2 exponent of a logit difference d = x - m, rounded once.
__device__ inline float scaled(float d, const Scale& k) { return fmaf(d, k.hi, d * k.lo); }

// 2^t in fp64, inline (no call, no stack): t = n + f with n = rint(t) and
// f in [-1/2, 1/2] (exact), 2^f = e^y with y = f ln 2, |y| <= 0.35, from the
// Taylor series of e^y to degree 13 (truncation below 0.35^14 / 14! < 4e-18
// relative) in Horner form; then the exponent n.  Within a few ulp of double;
// below 2^-1074 it underflows to 0, above 2^1023 it overflows to inf.
__device__ inline double exp2_fp64(double t) {
    t = fmin(fmax(t, -1100.0), 1100.0);  // keeps n in int range; the ends round to 0 and inf
    const double n = rint(t);
    const double y = (t - n) * 0.69314718055994530942;
    double p = 1.0 / 6227020800.0;  // 1/13!
    p = fma(p, y, 1.0 / 479001600.0);
    p = fma(p, y, 1.0 / 39916800.0);
    p = fma(p, y, 1.0 / 3628800.0);
    p = fma(p, y, 1.0 / 362880.0);
    p = fma(p, y, 1.0 / 40320.0);
    p = fma(p, y, 1.0 / 5040.0);
    p = fma(p, y, 1.0 / 720.0);
    p = fma(p, y, 1.0 / 120.0);
    p = fma(p, y, 1.0 / 24.0);
    p = fma(p, y, 1.0 / 6.0);
    p = fma(p, y, 0.5);
    p = fma(p, y, 1.0);
    p = fma(p, y, 1.0);
    return ldexp(p, (int)n);
}

// 2^((x - m) * c) in fp64 (accurate to a few ulp of double); 0 for x = -inf.
__device__ inline double exp2_accurate(float x, float m, const Scale& k) {
    if (x == -INFINITY) return 0.0;
    return exp2_fp64(((double)x - (double)m) * k.c64);
}

// 2^(t / 256) in fp64 for t <= 0 (-inf excluded): 2^n 2^(j/256) 2^(f/256)
// with k = floor(t) = 256 n + j, f = t - k in [0, 1) (exact); 2^(j/256) from
// `tab` (256 entries, each the library's fp64 exponential), 2^(f/256) by its
// Taylor polynomial to degree 4 (truncation below (ln2 / 256)^5 / 120 < 2e-15
// relative).  Within a few fp64 ulp; below 2^-1074 it underflows to 0.
__device__ inline double exp2_256(double t, const double* tab) {
    const double kd = floor(fmax(t, -300000.0));  // keeps k in int range; 2^(-300000/256) is 0
    const int k = (int)kd;
    const double f = fmax(t, -300000.0) - kd;
    constexpr double u = 0.69314718055994530942 / 256.0;
    double p = u * u * u * u / 24.0;
    p = fma(p, f, u * u * u / 6.0);
    p = fma(p, f, u * u / 2.0);
    p = fma(p, f, u);
    p = fma(p, f, 1.0);
    return ldexp(tab[k & 255] * p, k >> 8);
}

// The table exp2_256 reads: tab[j] = 2^(j / 256), j < 256, each the library's
// fp64 exponential; written by the first 256 threads, read after a barrier.
__device__ inline void fill_exp_table(double* tab) {
    for (int j = threadIdx.x; j < 256; j += blockDim.x) tab[j] = exp2((double)j / 256.0);
}

// 2^((x - m) c) in fp64 for x <= m from the table `tab` (exp2_256), with
// c256 = 256 c; 0 for x = -inf.  A few fp64 ulp, like exp2_accurate, with four
// polynomial constants instead of its thirteen: in a loop the compiler keeps
// those in registers, and fewer of them leave room for more waves.
__device__ inline double exp2_table(float x, float m, double c256, const double* tab) {
    if (x == -INFINITY) return 0.0;
    return exp2_256(((double)x - (double)m) * c256, tab);
}

// Argmax pairs: larger value wins, the lower index wins a tie.
__device__ inline void merge_argmax(float& v, int& i, float v2, int i2) {
    bool take = (v2 > v) || (v2 == v && i2 < i);
    v = take ? v2 : v;
    i = take ? i2 : i;
}

// ---------------------------------------------------------------------------
// Cross-lane steps on DPP (lane permutations applied by the VALU operand
// network, no LDS round trip).  A wave64 is four rows of 16 lanes.
// ---------------------------------------------------------------------------
namespace dpp {
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7 - i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <- lane 15 - i within each row
constexpr int kRowShr = 0x110;        // + n: lane i <- lane i - n in the row (else 0)
constexpr int kRowShl = 0x100;        // + n: lane i <- lane i + n in the row (else 0)
constexpr int kRowBcast15 = 0x142;    // row r + 1 <- lane 15 of row r
constexpr int kRowBcast31 = 0x143;    // rows 2, 3 <- lane 31
}  // namespace dpp

// Lanes of disabled rows, and lanes whose source is outside their row, get 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline float dpp_f32(float v) {
    return __int_as_float(dpp_i32<CTRL, ROW_MASK>(__float_as_int(v)));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline double dpp_f64(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)dpp_i32<CTRL, ROW_MASK>((int)(unsigned)b);
    const unsigned hi = (unsigned)dpp_i32<CTRL, ROW_MASK>((int)(unsigned)(b >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ inline double readlane_f64(double v, int lane) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, lane);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ inline float readlane_f32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Fixed-order reductions (same result on every run); every lane gets the
// result.  Within a row the butterfly leaves identical bits in all 16 lanes;
// the four row results are then combined in row order.
__device__ inline float wave_max(float v) {
    v = fmaxf(v, dpp_f32<dpp::kQuadSwap1>(v));
    v = fmaxf(v, dpp_f32<dpp::kQuadSwap2>(v));
    v = fmaxf(v, dpp_f32<dpp::kRowHalfMirror>(v));
    v = fmaxf(v, dpp_f32<dpp::kRowMirror>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ inline void wave_reduce_argmax(float& v, int& i) {
#define SV_ARGMAX_STEP(CTRL)                                                   \
    {                                                                          \
        const float v2 = dpp_f32<CTRL>(v);                                     \
        const int i2 = dpp_i32<CTRL>(i);                                       \
        merge_argmax(v, i, v2, i2);                                            \
    }
    SV_ARGMAX_STEP(dpp::kQuadSwap1)
    SV_ARGMAX_STEP(dpp::kQuadSwap2)
    SV_ARGMAX_STEP(dpp::kRowHalfMirror)
    SV_ARGMAX_STEP(dpp::kRowMirror)
#undef SV_ARGMAX_STEP
    float bv = readlane_f32(v, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r)
        merge_argmax(bv, bi, readlane_f32(v, 16 * r), __builtin_amdgcn_readlane(i, 16 * r));
    v = bv;
    i = bi;
}

__device__ inline double wave_reduce_sum(double x) {
    x += dpp_f64<dpp::kQuadSwap1>(x);
    x += dpp_f64<dpp::kQuadSwap2>(x);
    x += dpp_f64<dpp::kRowHalfMirror>(x);
    x += dpp_f64<dpp::kRowMirror>(x);
    return (readlane_f64(x, 0) + readlane_f64(x, 16)) + (readlane_f64(x, 32) + readlane_f64(x, 48));
}

// Inclusive prefix sum over the 64 lanes in lane order: a scan inside each row
// of 16, then the row totals carried forward by row broadcasts.
__device__ inline double wave_inclusive_scan(double x) {
    x += dpp_f64<dpp::kRowShr + 1>(x);
    x += dpp_f64<dpp::kRowShr + 2>(x);
    x += dpp_f64<dpp::kRowShr + 4>(x);
    x += dpp_f64<dpp::kRowShr + 8>(x);
    x += dpp_f64<dpp::kRowBcast15, 0xa>(x);
    x += dpp_f64<dpp::kRowBcast31, 0xc>(x);
    return x;
}

// Workgroup max / sum; `sh` is LDS scratch of kWaves entries.  Every thread
// gets the result.
__device__ inline float block_max(float v, float* sh) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = fmaxf(r, sh[w]);
    __syncthreads();
    return r;
}

__device__ inline double block_sum(double v, double* sh) {
    v = wave_reduce_sum(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = sh[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r += sh[w];
    __syncthreads();
    return r;
}

// Inclusive prefix sum over the workgroup in thread order (deterministic).
// `wave_tot` is LDS scratch of kWaves doubles.  Returns the inclusive prefix;
// *total receives the workgroup total.
__device__ inline double block_inclusive_scan(double x, double* wave_tot, double* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    x = wave_inclusive_scan(x);
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    double before = 0.0, all = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        double t = wave_tot[w];
        if (w < wave) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x;
}

// Values that one workgroup writes and another reads within the same launch
// (partials, masses, stop state) travel through the device-coherent level:
// agent-scope relaxed atomic accesses (sc1 on gfx950), which neither stay dirty
// in one XCD's L2 nor hit stale lines in another's.
template <typename T>
__device__ inline void store_coherent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ inline T load_coherent(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this thread's global stores have completed.
__device__ inline void wait_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Take an arrival ticket on `counter` after thread 0 has written this
// workgroup's contribution (only thread 0 writes what other workgroups read).
// Returns true in every thread of the last of `expected` arrivals; those
// threads then see every other arrival's writes.  The last arrival resets the
// counter to zero (atomically, where the other arrivals incremented it).
__device__ inline bool arrive_last(uint32_t* counter, uint32_t expected, int* lds_flag) {
    if (threadIdx.x == 0) {
#if SV_COHERENT_TICKETS
        // Thread 0's coherent stores complete before the ticket is taken.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#else
        // Release thread 0's writes at device scope, then take the ticket.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#endif
        uint32_t prev = atomicAdd(counter, 1u);
        int last = (prev == expected - 1);
        if (last) atomicExch(counter, 0u);
        *lds_flag = last;
    }
    __syncthreads();
    bool last = *lds_flag != 0;
#if !SV_COHERENT_TICKETS
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // see every arrival's writes
#endif
    return last;
}

}  // namespace sv
