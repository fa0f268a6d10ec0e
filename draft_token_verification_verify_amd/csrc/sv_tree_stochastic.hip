// sv_tree_stochastic.hip -- stochastic verification of a draft tree, and the
// gather of the accepted rows (KV relocation).
//
// Tree rule (page "05 - TensorRT-LLM speculative decoding and auto-deploy",
// "Target-model verification: tree attention and batched parallelism": the
// target scores every tree node in one pass and "rejection sampling" decides
// what is kept; the paths table of "Eagle-2 multi-level tree drafting").  The
// page gives no rule for several candidate children; the one used is the
// linear rule applied to the children of each accepted node in turn
// (multi-candidate speculative sampling, SpecInfer, Miao et al., ASPLOS 2024):
// at node n with target distribution p (row n) and draft distribution q (the
// draft row that n's children were drawn from), children are tested in
// ascending node order -- accept child x when p(x) >= q(x) or u q(x) < p(x) --
// and every rejection replaces p by max(0, p - q) renormalised before the next
// child is tried.  An accepted child becomes the next n; when none is
// accepted, one token is drawn from the last residual (or from row n itself
// if nothing was rejected there) by inverse CDF.  A single-chain tree is the
// linear call.
//
// One workgroup of 1024 threads per request walks its tree.  The parent of
// every node comes from the paths table (the first row that names a node
// fixes its parent).  Each visited node costs one pass over its target and
// draft rows for their softmax statistics, one pass per rejected child for the
// residual's mass, and the final draw one pass for the weights' running total
// by tiles plus one tile for the token.  Every sum runs in a fixed order, so
// results do not change between runs.
#include <algorithm>
#include <atomic>
#include <cstddef>

#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int kTsThreads = 1024;
constexpr int kTsWaves = kTsThreads / 64;
constexpr int kMaxTreeNodes = 1024;            // N + 1
constexpr int kMaxRejections = kMaxTreeNodes;  // a node has at most N children
constexpr int kTsPer = 8;                      // logits per thread per tile (16 would spill registers)
constexpr int kTsTile = kTsThreads * kTsPer;   // logits per tile
constexpr int kTsTiles = 64;                   // tiles per row: V <= 524288
constexpr int kTsMaxSplit = 8;                 // workgroups per request, at most
constexpr int kTsSpinLimit = 1 << 20;          // polls of one exchange word before giving up (default)

// Exchange area of one request whose walk is split over G workgroups (in the
// workspace; zero before the call and after it).  Workgroup g takes the
// row tiles k with k % G == g; every workgroup runs the same walk, so they
// all make the same exchanges in the same order.  Every exchanged value is
// published as 64-bit words that each carry, in their upper half, the round
// that wrote them (round + 1, so never the cleared 0): a reader polls the
// words it needs until their tag is the round's, with no fence between data
// and a flag (a device-scope acquire fence would invalidate the L2 and with
// it the row tiles every workgroup keeps there).  Round r's words sit in slot
// r & 1; a workgroup publishes round r + 1 only after reading all of round r,
// so round r + 2 never overwrites words still to be read.
struct TsSync {
    uint32_t exit;      // workgroups done; the last one clears the area
    uint32_t failed;    // an exchange gave up waiting
    uint32_t ticket;    // request 0's area only: arrival tickets of the whole call
    uint32_t done;      // request 0's area only: workgroups of the call finished
    // per workgroup, six words: target max, target mass (two words), draft
    // max, draft mass (two words); a max is an fp32, so one word carries it
    unsigned long long stat[2][kTsMaxSplit * 6];
    unsigned long long tile[2][kTsTiles][2];         // weight-pass tile sums, by the tiles' owners
    unsigned long long token[2];                     // the final draw's token, by its tile's owner
};
static_assert(sizeof(TsSync) <= kTreeSyncBytes, "exchange area");

struct TreeStochArgs {
    const void* target;
    const void* draft;
    const int32_t* node_tokens;  // [B, N+1]
    const int32_t* paths;        // [B, P, L]
    const float* uniforms;       // [B, N+1]
    int B, N, P, L, V;
    Scale sc;
    int32_t* out_tokens;      // [B, L]
    int32_t* num_accepted;    // [B]
    int32_t* accepted_nodes;  // [B, L] or null
    int G;                    // workgroups per request
    char* sync;               // [B] exchange areas of kTreeSyncBytes (G > 1)
    int spin_limit;           // polls of one exchange word before giving up
};

// This workgroup's place in its request's group.
struct TsGroup {
    int G, g;
    TsSync* sy;
    int round;
    int spin_limit;  // polls of one word before giving up
};

// Publishing and reading tagged words.  A double is two words (low and high
// halves of its bits), each tagged.
__device__ inline uint32_t ts_tag(const TsGroup& grp) { return (uint32_t)grp.round + 1u; }

__device__ inline void ts_put(unsigned long long* w, double v, uint32_t tag) {
    const unsigned long long bits = (unsigned long long)__double_as_longlong(v);
    store_coherent(&w[0], ((unsigned long long)tag << 32) | (bits & 0xffffffffull));
    store_coherent(&w[1], ((unsigned long long)tag << 32) | (bits >> 32));
}

// Whether a poll gives up: past the group's spin limit (the request is then
// marked failed), or once another workgroup of the group has given up (checked
// every 32 polls).  After a first give-up the group's members take different
// paths and later tags never match: without the second test every later wait
// would run to the full limit.
__device__ inline bool ts_give_up(int spins, const TsGroup& grp) {
    if (spins > grp.spin_limit) {
        store_coherent(&grp.sy->failed, 1u);
        return true;
    }
    return (spins & 31) == 31 && load_coherent(&grp.sy->failed) != 0u;
}

// Poll one tagged word until it carries `tag` (bounded by ts_give_up; the word
// is then taken as it is).
__device__ inline uint32_t ts_wait_word(const unsigned long long* w, uint32_t tag,
                                        const TsGroup& grp) {
    unsigned long long v = load_coherent(w);
    for (int spins = 0; (uint32_t)(v >> 32) != tag; ++spins) {
        if (ts_give_up(spins, grp)) break;
        __builtin_amdgcn_s_sleep(2);
        v = load_coherent(w);
    }
    return (uint32_t)v;
}

// A double's two words, polled together (both loads in flight at once, each
// reloaded until it carries `tag`; bounded like ts_wait_word).
__device__ inline void ts_put_float(unsigned long long* w, float v, uint32_t tag) {
    store_coherent(w, ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v));
}

__device__ inline double ts_get(const unsigned long long* w, uint32_t tag, const TsGroup& grp) {
    unsigned long long lo = load_coherent(&w[0]);
    unsigned long long hi = load_coherent(&w[1]);
    for (int spins = 0; (uint32_t)(lo >> 32) != tag || (uint32_t)(hi >> 32) != tag; ++spins) {
        if (ts_give_up(spins, grp)) break;
        __builtin_amdgcn_s_sleep(2);
        if ((uint32_t)(lo >> 32) != tag) lo = load_coherent(&w[0]);
        if ((uint32_t)(hi >> 32) != tag) hi = load_coherent(&w[1]);
    }
    return __longlong_as_double((long long)(((hi & 0xffffffffull) << 32) | (lo & 0xffffffffull)));
}

struct TsLds {
    int first[kMaxTreeNodes];   // first occurrence (row * L + t) of each node in paths
    int parent[kMaxTreeNodes];
    double inv_z[kMaxRejections];  // reciprocal residual masses at the current node
    double tile_sum[kTsTiles];
    double wsum[kTsTiles][kTsWaves];  // per-wave sums of each tile of a weight pass
    uint32_t xw[kTsMaxSplit * 6];     // the group's row statistics, as exchanged (payloads)
    double xterm[2 * kTsMaxSplit];    // their masses at the common maximum
    // Per child of the current node, loaded once per node: the target and
    // draft logits at its token, its uniform and its token.
    float child_t[kMaxTreeNodes];
    float child_d[kMaxTreeNodes];
    float child_u[kMaxTreeNodes];
    int child_x[kMaxTreeNodes];
    float mrg_m[kTsWaves][2];  // per-wave maxima of both rows (statistics merge)
    double mrg_s[kTsWaves][2];  // per-wave rescaled sums of both rows
    double scan_w[kTsWaves];    // per-wave totals (draw scan)
    int pick_w[kTsWaves][2];    // per-wave first hit and last positive token (draw)
    double exp_tab[256];  // 2^(j / 256): the fp64 token weights
    unsigned long long kids[kMaxTreeNodes / 64];  // the current node's children: bit c of word c / 64
    int red_i;
    int pick_tile;
    double pick_base;
};

// 2^((x - m) c) in fp64 for x <= m (finite), from the table `tab` of
// exp2_256, with c256 = 256 c.
__device__ inline double ts_exp2(float x, float m, double c256, const double* tab) {
    return exp2_256(((double)x - (double)m) * c256, tab);
}

// Weight 2^((x - m) c) of a logit in fp64: within 2^-8 of the row maximum
// (most of the mass) the fp64 exponential, exp2_256 on the table `tab` with
// c256 = 256 c; the fp32 one below.
__device__ inline double ts_weight(float x, float m, const Scale& sc, double c256,
                                   const double* tab) {
    if (x == -INFINITY) return 0.0;
    const float a = scaled(x - m, sc);
    if (a > -8.f) return ts_exp2(x, m, c256, tab);
    return (double)fast_exp2(a);
}

// The row is read in tiles of kTsThreads * 8 logits; thread t takes the 8
// consecutive logits at tile * 8192 + 8 t (all of its 16-byte loads issued
// together when the row is aligned).  Tile-major, thread-minor order is
// ascending vocabulary order.
template <typename T, bool VEC>
__device__ inline void ts_load(const T* row, int V, int tile, float* x) {
    const int j0 = tile * kTsTile + (int)threadIdx.x * kTsPer;
    if constexpr (VEC) {
        constexpr int EPV = Elem<T>::kPerVec;
        if (j0 + kTsPer <= V) {
            uint4 raw[kTsPer / EPV];
#pragma unroll
            for (int v = 0; v < kTsPer / EPV; ++v) raw[v] = load16(row + j0 + v * EPV);
#pragma unroll
            for (int v = 0; v < kTsPer / EPV; ++v) Elem<T>::widen(raw[v], x + v * EPV);
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < kTsPer; ++e) x[e] = (j0 + e < V) ? Elem<T>::load(row, j0 + e) : -INFINITY;
}

// One tile's 16-byte vectors of this thread, loaded ahead of their use (the
// next tile's loads are in flight while the current one is summed).  A tile
// that is not whole, or a row that is not 16-byte aligned, is read when used.
template <typename T, bool VEC>
struct TileBuf {
    static constexpr int kVecs = VEC ? kTsPer / Elem<T>::kPerVec : 1;
    uint4 raw[kVecs];
    bool whole = false;
    __device__ inline void fetch(const T* row, int V, int tile) {
        if constexpr (VEC) {
            constexpr int EPV = Elem<T>::kPerVec;
            const int j0 = tile * kTsTile + (int)threadIdx.x * kTsPer;
            whole = j0 + kTsPer <= V;
            if (whole)
#pragma unroll
                for (int v = 0; v < kVecs; ++v) raw[v] = load16(row + j0 + v * EPV);
        }
    }
    __device__ inline void get(const T* row, int V, int tile, float* x) const {
        if constexpr (VEC) {
            constexpr int EPV = Elem<T>::kPerVec;
            if (whole) {
#pragma unroll
                for (int v = 0; v < kVecs; ++v) Elem<T>::widen(raw[v], x + v * EPV);
                return;
            }
        }
        ts_load<T, false>(row, V, tile, x);
    }
};

// Softmax statistics of a row: maximum m and s = sum of 2^((x - m) c), in one
// pass: each thread sums against its running maximum, rescaling its sum (fp64
// exponential) when the maximum grows; threads are then merged in fixed order.
struct RowStats {
    float m;
    double s;
};

struct RunStats {
    float m = -INFINITY;
    double s = 0.0;
    // The 8 logits of one tile: the running maximum first (one rescale at
    // most), then their terms against it.
    __device__ inline void add_tile(const float* x, const Scale& sc, double c256, const double* tab) {
        float tm = m;
#pragma unroll
        for (int e = 0; e < kTsPer; ++e) tm = fmaxf(tm, x[e]);
        if (tm > m) {
            if (m != -INFINITY) s *= ts_exp2(m, tm, c256, tab);
            m = tm;
        }
        const float ms = (m == -INFINITY) ? 0.f : m;
#pragma unroll
        for (int e = 0; e < kTsPer; ++e) s += (double)fast_exp2(scaled(x[e] - ms, sc));
    }
};

// The workgroup's statistics of the target row and, when `both`, of the draft
// row: the maxima in one reduction, then the sums rescaled to them in a
// second (waves combined in wave order).  Each reduction has LDS slots of its
// own that no other code touches, so one barrier apiece suffices: a thread
// reads the maxima before it reaches the second barrier, and the sums before
// the first barrier of the next merge.
__device__ inline void ts_merge(const RunStats& rt, const RunStats& rd, bool both, const Scale& sc,
                                TsLds& L, RowStats* st, RowStats* sd) {
    const int wave = threadIdx.x >> 6;
    const float wt = wave_max(rt.m);
    const float wd = both ? wave_max(rd.m) : -INFINITY;
    if ((threadIdx.x & 63) == 0) {
        L.mrg_m[wave][0] = wt;
        L.mrg_m[wave][1] = wd;
    }
    __syncthreads();
    float mt = L.mrg_m[0][0], md = L.mrg_m[0][1];
#pragma unroll
    for (int w = 1; w < kTsWaves; ++w) {
        mt = fmaxf(mt, L.mrg_m[w][0]);
        md = fmaxf(md, L.mrg_m[w][1]);
    }
    const double c256 = sc.c64 * 256.0;
    const double ft = (rt.m == -INFINITY || mt == -INFINITY) ? 0.0 : ts_exp2(rt.m, mt, c256, L.exp_tab);
    const double vt = wave_reduce_sum(rt.m == -INFINITY ? 0.0 : rt.s * ft);
    double vd = 0.0;
    if (both) {
        const double fd = (rd.m == -INFINITY || md == -INFINITY) ? 0.0 : ts_exp2(rd.m, md, c256, L.exp_tab);
        vd = wave_reduce_sum(rd.m == -INFINITY ? 0.0 : rd.s * fd);
    }
    if ((threadIdx.x & 63) == 0) {
        L.mrg_s[wave][0] = vt;
        L.mrg_s[wave][1] = vd;
    }
    __syncthreads();
    double s_t = L.mrg_s[0][0], s_d = L.mrg_s[0][1];
#pragma unroll
    for (int w = 1; w < kTsWaves; ++w) {
        s_t += L.mrg_s[w][0];
        s_d += L.mrg_s[w][1];
    }
    st->m = mt;
    st->s = s_t;
    if (both) {
        sd->m = md;
        sd->s = s_d;
    }
}

// Statistics of the target row and, when `both`, of the draft row, in one
// pass (over this workgroup's tiles; with G > 1 the workgroups' statistics are
// then merged in workgroup order).
template <typename T, bool VEC>
__device__ void ts_row_stats(const T* trow, const T* drow, bool both, int V, const Scale& sc,
                             TsLds& L, RowStats* st, RowStats* sd, TsGroup& grp) {
    const int tiles = (V + kTsTile - 1) / kTsTile;
    RunStats rt, rd;
    TileBuf<T, VEC> bt, bd;
    if (grp.g < tiles) {
        bt.fetch(trow, V, grp.g);
        if (both) bd.fetch(drow, V, grp.g);
    }
    for (int k = grp.g; k < tiles; k += grp.G) {
        TileBuf<T, VEC> nt, nd;
        if (k + grp.G < tiles) {
            nt.fetch(trow, V, k + grp.G);
            if (both) nd.fetch(drow, V, k + grp.G);
        }
        float xt[kTsPer], xd[kTsPer];
        bt.get(trow, V, k, xt);
        rt.add_tile(xt, sc, sc.c64 * 256.0, L.exp_tab);
        if (both) {
            bd.get(drow, V, k, xd);
            rd.add_tile(xd, sc, sc.c64 * 256.0, L.exp_tab);
        }
        bt = nt;
        bd = nd;
    }
    ts_merge(rt, rd, both, sc, L, st, sd);
    if (grp.G > 1) {
        unsigned long long* slot = grp.sy->stat[grp.round & 1];
        const uint32_t tag = ts_tag(grp);
        if (threadIdx.x == 0) {
            unsigned long long* mine = slot + grp.g * 6;
            ts_put_float(&mine[0], st->m, tag);
            ts_put(&mine[1], st->s, tag);
            ts_put_float(&mine[3], both ? sd->m : 0.f, tag);
            ts_put(&mine[4], both ? sd->s : 0.0, tag);
        }
        if ((int)threadIdx.x < grp.G * 6) L.xw[threadIdx.x] = ts_wait_word(&slot[threadIdx.x], tag, grp);
        __syncthreads();
        // Workgroup w's max and mass of one side, from the exchanged payloads.
        auto xmax = [&](int w, int side) { return __uint_as_float(L.xw[w * 6 + 3 * side]); };
        auto xmass = [&](int w, int side) {
            const int i = w * 6 + 3 * side + 1;
            return __longlong_as_double(
                (long long)(((unsigned long long)L.xw[i + 1] << 32) | L.xw[i]));
        };
        // Each workgroup's mass rescaled to the common maximum: one thread per
        // (side, workgroup), then summed in workgroup order by every thread.
        float M[2];
        for (int side = 0; side < 2; ++side) {
            M[side] = -INFINITY;
            for (int w = 0; w < grp.G; ++w) M[side] = fmaxf(M[side], xmax(w, side));
        }
        if ((int)threadIdx.x < 2 * grp.G) {
            const int side = threadIdx.x / grp.G, w = threadIdx.x % grp.G;
            const float mw = xmax(w, side);
            L.xterm[threadIdx.x] = (mw == -INFINITY || M[side] == -INFINITY)
                                       ? 0.0
                                       : xmass(w, side) *
                                             ts_exp2(mw, M[side], sc.c64 * 256.0, L.exp_tab);
        }
        __syncthreads();
        for (int side = 0; side < (both ? 2 : 1); ++side) {
            double S = 0.0;
            for (int w = 0; w < grp.G; ++w) S += L.xterm[side * grp.G + w];
            RowStats& out = side == 0 ? *st : *sd;
            out.m = M[side];
            out.s = S;
        }
        __syncthreads();  // xw and xterm are read before the next exchange refills them
        ++grp.round;
    }
}

// The current distribution at token x: p after nrej rejections,
// p_i = max(0, p_{i-1} - q) / z_i (p_{i-1} kept where z_i == 0), and q.
// Divisions by the row masses and the residual masses are multiplications by
// their reciprocals (within an ulp of the quotient).
struct Dist {
    float mt, md;
    double inv_st, inv_sd;  // 1 / row mass (0 for a row without mass)
    Scale sc;
    int nrej;
    const double* inv_z;    // 1 / residual mass after each rejection (0: mass was 0)
    __device__ inline void set(float m_t, double s_t, float m_d, double s_d) {
        mt = m_t;
        md = m_d;
        inv_st = (m_t == -INFINITY || !(s_t > 0.0)) ? 0.0 : 1.0 / s_t;
        inv_sd = (m_d == -INFINITY || !(s_d > 0.0)) ? 0.0 : 1.0 / s_d;
    }
    double c256;            // 256 c (exact: c times a power of two)
    const double* tab;      // 2^(j / 256), j < 256
    __device__ inline double p0(float xt) const { return ts_weight(xt, mt, sc, c256, tab) * inv_st; }
    __device__ inline double q(float xd) const { return ts_weight(xd, md, sc, c256, tab) * inv_sd; }
    // p after the first `upto` rejections, given p0 and q at a token.
    __device__ inline double chain(double p, double qv, int upto) const {
        for (int i = 0; i < upto; ++i) {
            const double iz = inv_z[i];
            if (iz > 0.0) p = fmax(p - qv, 0.0) * iz;
        }
        return p;
    }
};

// Sum over the row of w(v) = max(0, p_nrej(v) - q(v)) (residual) or p_nrej(v),
// tile by tile, each tile's sum stored in L.tile_sum (fixed order); returns
// the total.
template <typename T, bool VEC>
__device__ double ts_weight_pass(const T* trow, const T* drow, int V, const Dist& D, bool residual,
                                 TsLds& L, TsGroup& grp) {
    const int tiles = (V + kTsTile - 1) / kTsTile;
    TileBuf<T, VEC> bt, bd;
    if (grp.g < tiles) {
        bt.fetch(trow, V, grp.g);
        if (residual) bd.fetch(drow, V, grp.g);
    }
    for (int k = grp.g; k < tiles; k += grp.G) {
        TileBuf<T, VEC> nt, nd;
        if (k + grp.G < tiles) {
            nt.fetch(trow, V, k + grp.G);
            if (residual) nd.fetch(drow, V, k + grp.G);
        }
        float xt[kTsPer], xd[kTsPer];
        bt.get(trow, V, k, xt);
        if (residual) bd.get(drow, V, k, xd);
        double own = 0.0;
#pragma unroll
        for (int e = 0; e < kTsPer; ++e) {
            const double qv = residual ? D.q(xd[e]) : 0.0;
            const double p = D.chain(D.p0(xt[e]), qv, D.nrej);
            own += residual ? fmax(p - qv, 0.0) : p;
        }
        // The wave's sum now, the waves' sums after the loop (the same order
        // as a workgroup sum per tile, without its barriers).
        own = wave_reduce_sum(own);
        if ((threadIdx.x & 63) == 0) L.wsum[k][threadIdx.x >> 6] = own;
        bt = nt;
        bd = nd;
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < tiles && t % grp.G == grp.g) {
        double r = L.wsum[t][0];
#pragma unroll
        for (int w = 1; w < kTsWaves; ++w) r += L.wsum[t][w];
        L.tile_sum[t] = r;
    }
    __syncthreads();
    if (grp.G > 1) {  // every tile's sum, from its owner
        unsigned long long(*slot)[2] = grp.sy->tile[grp.round & 1];
        const uint32_t tag = ts_tag(grp);
        if (t == 0)
            for (int k = grp.g; k < tiles; k += grp.G) ts_put(slot[k], L.tile_sum[k], tag);
        __syncthreads();  // own sums read from LDS before they are overwritten below
        if (t < tiles && t % grp.G != grp.g) L.tile_sum[t] = ts_get(slot[t], tag, grp);
        __syncthreads();
        ++grp.round;
    }
    double total = 0.0;
    for (int k = 0; k < tiles; ++k) total += L.tile_sum[k];
    return total;
}

// Inverse CDF over the weights of the last ts_weight_pass: the smallest token
// whose running weight exceeds u * Z (Z = that pass's total), else the last
// token with positive weight.
template <typename T, bool VEC>
__device__ int ts_draw_in_tile(const T* trow, const T* drow, int V, const Dist& D, bool residual,
                               double target, int k, TsLds& L);

template <typename T, bool VEC>
__device__ int ts_draw(const T* trow, const T* drow, int V, const Dist& D, bool residual, double Z,
                       double u, TsLds& L, TsGroup& grp) {
    const int tiles = (V + kTsTile - 1) / kTsTile;
    const double target = u * Z;
    if (threadIdx.x == 0) {
        double run = 0.0;
        int pick = -1, last = -1;
        double pick_base = 0.0, last_base = 0.0;
        for (int k = 0; k < tiles; ++k) {
            const double w = L.tile_sum[k];
            if (w > 0.0) {
                last = k;
                last_base = run;
                if (pick < 0 && run + w > target) {
                    pick = k;
                    pick_base = run;
                }
            }
            run += w;
        }
        if (pick < 0) {
            pick = max(last, 0);
            pick_base = last_base;
        }
        L.pick_tile = pick;
        L.pick_base = pick_base;
    }
    __syncthreads();
    const int k = L.pick_tile;
    if (grp.G > 1) {  // the tile's owner finds the token; the others wait for it
        unsigned long long* slot = &grp.sy->token[grp.round & 1];
        const uint32_t tag = ts_tag(grp);
        int tk = 0;
        if (k % grp.G == grp.g) {
            tk = ts_draw_in_tile<T, VEC>(trow, drow, V, D, residual, target, k, L);
            if (threadIdx.x == 0)
                store_coherent(slot, ((unsigned long long)tag << 32) | (uint32_t)tk);
        } else {
            if (threadIdx.x == 0) L.red_i = (int)ts_wait_word(slot, tag, grp);
            __syncthreads();
            tk = L.red_i;
            __syncthreads();
        }
        ++grp.round;
        return tk;
    }
    return ts_draw_in_tile<T, VEC>(trow, drow, V, D, residual, target, k, L);
}

// The token inside tile k: the running weight from the tiles before it plus
// this tile's weights in order, first above the target.
template <typename T, bool VEC>
__device__ int ts_draw_in_tile(const T* trow, const T* drow, int V, const Dist& D, bool residual,
                               double target, int k, TsLds& L) {
    const double base = L.pick_base;
    float xt[kTsPer], xd[kTsPer];
    ts_load<T, VEC>(trow, V, k, xt);
    if (residual) ts_load<T, VEC>(drow, V, k, xd);
    auto weight = [&](int e) {
        const double qv = residual ? D.q(xd[e]) : 0.0;
        const double p = D.chain(D.p0(xt[e]), qv, D.nrej);
        return residual ? fmax(p - qv, 0.0) : p;
    };
    double w[kTsPer], own = 0.0;
#pragma unroll
    for (int e = 0; e < kTsPer; ++e) {
        w[e] = weight(e);
        own += w[e];
    }
    // Exclusive prefix of the threads' sums in thread order (slots of its own,
    // written once per walk: one barrier).
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const double inc = wave_inclusive_scan(own);
    if (lane == 63) L.scan_w[wave] = inc;
    __syncthreads();
    double before = 0.0;
#pragma unroll
    for (int w = 0; w < kTsWaves; ++w)
        if (w < wave) before += L.scan_w[w];
    double run = base + (before + (inc - own));
    const int j0 = k * kTsTile + (int)threadIdx.x * kTsPer;
    int hit = 0x7fffffff, lastpos = -1;
#pragma unroll
    for (int e = 0; e < kTsPer; ++e) {  // the same weights, in the same order
        if (w[e] > 0.0) {
            lastpos = j0 + e;
            if (run + w[e] > target && hit == 0x7fffffff) hit = j0 + e;
        }
        run += w[e];
    }
    // The first hit and the last positive token over the workgroup, in one
    // reduction (slots of their own, written once per walk: one barrier).
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        hit = min(hit, __shfl_xor(hit, d));
        lastpos = max(lastpos, __shfl_xor(lastpos, d));
    }
    if (lane == 0) {
        L.pick_w[wave][0] = hit;
        L.pick_w[wave][1] = lastpos;
    }
    __syncthreads();
    int tok = L.pick_w[0][0], last = L.pick_w[0][1];
#pragma unroll
    for (int w = 1; w < kTsWaves; ++w) {
        tok = min(tok, L.pick_w[w][0]);
        last = max(last, L.pick_w[w][1]);
    }
    if (tok == 0x7fffffff) tok = max(last, 0);  // rounding left every running weight at or below u * Z
    return tok;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kTsThreads) void tree_stochastic_kernel(TreeStochArgs a) {
    __shared__ TsLds L;
    const int N = a.N, V = a.V, Lp = a.L;
    // A split walk's groups are formed by arrival, not by workgroup id: the
    // t-th workgroup to start takes request t / G as its member t % G.  Only
    // the group holding the latest tickets can then be incomplete, so at most
    // G - 1 workgroups of a call ever wait for one not yet placed, whatever
    // else shares the device (two split walks on two streams included).
    TsSync* const area0 = reinterpret_cast<TsSync*>(a.sync);
    int ticket = blockIdx.x;
    if (a.G > 1) {
        if (threadIdx.x == 0) L.red_i = (int)atomicAdd(&area0->ticket, 1u);
        __syncthreads();
        ticket = L.red_i;
        __syncthreads();  // red_i is reused by the draw
        // A workspace that was not zero before the call (a broken
        // precondition) could hand out tickets past the grid: stay in bounds.
        if ((unsigned)ticket >= (unsigned)(a.B * a.G)) ticket = blockIdx.x;
    }
    const int b = ticket / a.G;
    TsGroup grp;
    grp.G = a.G;
    grp.g = ticket % a.G;
    grp.sy = a.G > 1 ? reinterpret_cast<TsSync*>(a.sync + (size_t)b * kTreeSyncBytes) : nullptr;
    grp.round = 0;
    grp.spin_limit = a.spin_limit;
    const bool lead = grp.g == 0;  // writes the outputs
    const int32_t* tok = a.node_tokens + (size_t)b * (N + 1);
    const float* u = a.uniforms + (size_t)b * (N + 1);
    const float u_draw = u[N];  // the final draw's uniform
    const int32_t* paths = a.paths + (size_t)b * a.P * Lp;

    static_assert(kTsThreads >= 256, "one table entry per thread");
    if (threadIdx.x < 256) L.exp_tab[threadIdx.x] = exp2((double)threadIdx.x / 256.0);
    // Parents: the first occurrence (row-major) of a node in a usable row.
    for (int n = threadIdx.x; n <= N; n += kTsThreads) {
        L.first[n] = 0x7fffffff;
        L.parent[n] = -1;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < a.P; r += kTsThreads) {
        const int32_t* row = paths + (size_t)r * Lp;
        if (row[0] < 0 || row[0] > N) continue;
        for (int t = 1; t < Lp; ++t) {
            const int32_t c = row[t];
            if (c < 0 || c > N) break;
            if (c != 0) atomicMin(&L.first[c], r * Lp + t);
        }
    }
    __syncthreads();
    for (int c = 1 + (int)threadIdx.x; c <= N; c += kTsThreads) {
        const int f = L.first[c];
        if (f != 0x7fffffff) L.parent[c] = paths[f - 1];  // the entry before it in its row
    }
    __syncthreads();

    int32_t* out = a.out_tokens + (size_t)b * Lp;
    int32_t* nodes = a.accepted_nodes ? a.accepted_nodes + (size_t)b * Lp : nullptr;
    if (lead)
        for (int t = threadIdx.x; t < Lp; t += kTsThreads) {
            out[t] = -1;
            if (nodes) nodes[t] = -1;
        }

    int n = 0, depth = 0;
    for (;;) {
        const T* trow = static_cast<const T*>(a.target) + ((size_t)b * (N + 1) + n) * (size_t)V;
        const T* drow = static_cast<const T*>(a.draft) + ((size_t)b * (N + 1) + n) * (size_t)V;
        // n's children (tested only while depth + 1 < L) as a bit mask over
        // node ids, one ballot per wave; each child's token, uniform and two
        // logits are loaded here, while the statistics pass runs.
        static_assert(kTsThreads == kMaxTreeNodes, "one thread per node id");
        {
            const int c = threadIdx.x;
            const bool kid = c >= 1 && c <= N && L.parent[c] == n;
            const unsigned long long m = __ballot(kid);
            if ((threadIdx.x & 63) == 0) L.kids[threadIdx.x >> 6] = m;
            if (kid && depth + 1 < Lp) {
                const int32_t x = tok[c];
                const bool ok = x >= 0 && x < V;
                L.child_x[c] = x;
                L.child_u[c] = u[c - 1];
                L.child_t[c] = ok ? Elem<T>::load(trow, x) : 0.f;
                L.child_d[c] = ok ? Elem<T>::load(drow, x) : 0.f;
            }
        }
        __syncthreads();
        const int kid_words = (N >> 6) + 1;  // words covering ids 0..N
        bool has = false;
        for (int w = 0; w < kid_words; ++w) has |= L.kids[w] != 0ull;
        const bool test = has && depth + 1 < Lp;
        Dist D;
        D.sc = a.sc;
        D.nrej = 0;
        D.inv_z = L.inv_z;
        D.c256 = a.sc.c64 * 256.0;
        D.tab = L.exp_tab;
        RowStats st, sd;
        ts_row_stats<T, VEC>(trow, drow, test, V, a.sc, L, &st, &sd, grp);
        D.set(st.m, st.s, test ? sd.m : -INFINITY, test ? sd.s : 0.0);
        int next = -1;
        double Zlast = 0.0;
        if (test) {
            // The children in ascending id order, from the mask (the same
            // for every thread).
            int w = 0;
            unsigned long long m = L.kids[0];
            for (;;) {
                while (m == 0ull && ++w < kid_words) m = L.kids[w];
                if (m == 0ull) break;
                const int c = (w << 6) + __builtin_ctzll(m);
                m &= m - 1ull;
                const int32_t x = L.child_x[c];
                bool accepted = false;
                if (x >= 0 && x < V) {
                    const double qv = D.q(L.child_d[c]);
                    const double pv = D.chain(D.p0(L.child_t[c]), qv, D.nrej);
                    accepted = (pv >= qv) || ((double)L.child_u[c] * qv < pv);
                }
                if (accepted) {
                    next = c;
                    break;
                }
                // Rejected: the residual's mass, then the next sibling against it.
                Zlast = ts_weight_pass<T, VEC>(trow, drow, V, D, true, L, grp);
                if (threadIdx.x == 0) L.inv_z[D.nrej] = Zlast > 0.0 ? 1.0 / Zlast : 0.0;
                __syncthreads();
                ++D.nrej;
            }
        }
        if (next < 0) {
            // Final draw: the last residual max(0, p - q) as it stands (its mass
            // Zlast; p itself where that mass is 0), else row n's p.
            const bool residual = D.nrej > 0 && Zlast > 0.0;
            Dist F = D;
            if (residual) F.nrej = D.nrej - 1;  // w = max(0, p_{nrej-1} - q)
            // (For a residual, the last rejection's pass left exactly these
            // weights' tile sums in L.tile_sum.)
            const double Z = residual ? Zlast
                                      : ts_weight_pass<T, VEC>(trow, drow, V, F, false, L, grp);
            const int token = ts_draw<T, VEC>(trow, drow, V, F, residual, Z, (double)u_draw, L, grp);
            if (threadIdx.x == 0 && lead) {
                out[depth] = token;
                a.num_accepted[b] = depth;
            }
            if (grp.G > 1) {  // the last workgroup out clears the exchange area
                __syncthreads();
                if (threadIdx.x == 0) {
                    __threadfence();
                    if (atomicAdd(&grp.sy->exit, 1u) == (uint32_t)grp.G - 1u) {
                        __threadfence();
                        if (load_coherent(&grp.sy->failed)) a.num_accepted[b] = -2;
                        uint32_t* w = reinterpret_cast<uint32_t*>(grp.sy);
                        constexpr size_t kTicket = offsetof(TsSync, ticket) / 4;
                        constexpr size_t kDone = offsetof(TsSync, done) / 4;
                        for (size_t i = 0; i < sizeof(TsSync) / 4; ++i)
                            if (i != kTicket && i != kDone) store_coherent(&w[i], 0u);
                    }
                    // The call's last workgroup (every ticket taken by then)
                    // clears the call's counters.
                    if (atomicAdd(&area0->done, 1u) == (uint32_t)(a.B * grp.G) - 1u) {
                        store_coherent(&area0->ticket, 0u);
                        store_coherent(&area0->done, 0u);
                    }
                }
            }
            return;
        }
        if (threadIdx.x == 0 && lead) {
            out[depth] = tok[next];
            if (nodes) nodes[depth] = next;
        }
        ++depth;
        n = next;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Accepted-row gather: dst[b, j] = src[b, accepted_nodes[b, j]] for
// j < num_accepted[b] (page "TensorRT-LLM source teardown (10)", KV rewind,
// step 4: the accepted draft rows moved to their logical, contiguous places).
// One workgroup per (request, slot); 16-byte copies when rows allow.
// ---------------------------------------------------------------------------
struct GatherArgs {
    const char* src;
    char* dst;
    size_t row_bytes;
    const int32_t* nodes;
    const int32_t* num_accepted;
    int B, N1, L;
    bool vec;
};

__global__ __launch_bounds__(256) void gather_rows_kernel(GatherArgs g) {
    const int b = blockIdx.x / g.L, j = blockIdx.x % g.L;
    const int na = g.num_accepted[b];
    if (j >= na || j < 0) return;
    const int n = g.nodes[(size_t)b * g.L + j];
    if (n < 0 || n >= g.N1) return;  // not a node of the source: leave the slot
    const char* s = g.src + ((size_t)b * g.N1 + n) * g.row_bytes;
    char* d = g.dst + ((size_t)b * g.L + j) * g.row_bytes;
    if (g.vec) {
        const size_t nv = g.row_bytes / 16;
        const uint4* s4 = reinterpret_cast<const uint4*>(s);
        uint4* d4 = reinterpret_cast<uint4*>(d);
        for (size_t i = threadIdx.x; i < nv; i += 256) d4[i] = s4[i];
    } else {
        for (size_t i = threadIdx.x; i < g.row_bytes; i += 256) d[i] = s[i];
    }
}

// Workgroups of the walk kernel that fit on the device at once (cached per
// device): a split walk needs every workgroup resident, as its exchanges wait
// on each other.
template <typename T, bool VEC>
static int ts_resident_capacity() {
    static int cached[64][4];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    const int slot = (sizeof(T) == 2 ? 2 : 0) + (VEC ? 1 : 0);
    if (cached[dev][slot] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(tree_stochastic_kernel<T, VEC>), kTsThreads,
                0) != hipSuccess)
            return 0;
        cached[dev][slot] = std::max(cus * per_cu, 1);
    }
    return cached[dev][slot];
}

// Workgroups per request for B requests over V tokens: at most one per row
// tile and kTsMaxSplit, and B * G must all be resident at once; 1 when no
// split fits.
template <typename T, bool VEC>
static int ts_split(int B, int V) {
    const int tiles = (V + kTsTile - 1) / kTsTile;
    const int cap = ts_resident_capacity<T, VEC>();
    const int G = cap > 0 ? std::min(std::min(kTsMaxSplit, tiles), cap / B) : 1;
    return G < 2 ? 1 : G;
}

int tree_stochastic_split(int B, int V, int dtype) {
    return dtype == 1 ? ts_split<bf16_t, true>(B, V) : ts_split<float, true>(B, V);
}

template <typename T, bool VEC>
static hipError_t launch_tree(TreeStochArgs a, const TreeStochCall& c, hipStream_t st,
                              const KernelEvents& ev) {
    // Split each request's walk over G workgroups when the workspace holds the
    // exchange areas (ts_split).
    int G = 1;
    if (c.workspace && c.workspace_bytes >= kTreeSyncBytes * (size_t)c.B) G = ts_split<T, VEC>(c.B, c.V);
    a.G = G;
    a.sync = G > 1 ? static_cast<char*>(c.workspace) : nullptr;
    if (G > 1) {
        // A plain launch: the grid is at most the device's resident capacity,
        // so on a device running nothing else every workgroup is resident at
        // once.  (hipLaunchCooperativeKernel gives the same guarantee but
        // costs about 18 us more per call.)  Beside other work, groups formed
        // by arrival (in the kernel) leave at most G - 1 workgroups waiting
        // for one not yet placed; every wait is bounded in any case.
        hipExtLaunchKernelGGL(tree_stochastic_kernel<T, VEC>, dim3((unsigned)(c.B * G)),
                              dim3(kTsThreads), 0, st, ev.begin, ev.end, 0, a);
        return hipGetLastError();
    }
    // The events (when set) take the kernel's own start and end timestamps.
    hipExtLaunchKernelGGL(tree_stochastic_kernel<T, VEC>, dim3((unsigned)c.B), dim3(kTsThreads), 0,
                          st, ev.begin, ev.end, 0, a);
    return hipGetLastError();
}

// Polls of one exchange word before a split walk's workgroup gives up; tests
// lower it to force the give-up path from the host.
static std::atomic<int> g_spin_limit{kTsSpinLimit};

int tree_stochastic_spin_limit(int polls) {
    return g_spin_limit.exchange(polls < 0 ? kTsSpinLimit : polls);
}

hipError_t run_tree_stochastic(const TreeStochCall& c, hipStream_t st, const KernelEvents& ev) {
    TreeStochArgs a;
    a.spin_limit = g_spin_limit.load();
    a.target = c.target;
    a.draft = c.draft;
    a.node_tokens = c.node_tokens;
    a.paths = c.paths;
    a.uniforms = c.uniforms;
    a.B = c.B;
    a.N = c.N;
    a.P = c.P;
    a.L = c.L;
    a.V = c.V;
    a.sc = make_scale(c.temperature);
    a.out_tokens = c.out_tokens;
    a.num_accepted = c.num_accepted;
    a.accepted_nodes = c.accepted_nodes;
    a.G = 1;
    a.sync = nullptr;
    if (c.dtype == 1)
        return c.vec ? launch_tree<bf16_t, true>(a, c, st, ev) : launch_tree<bf16_t, false>(a, c, st, ev);
    return c.vec ? launch_tree<float, true>(a, c, st, ev) : launch_tree<float, false>(a, c, st, ev);
}

hipError_t run_gather_rows(const GatherCall& c, hipStream_t st) {
    GatherArgs g;
    g.src = static_cast<const char*>(c.src);
    g.dst = static_cast<char*>(c.dst);
    g.row_bytes = c.row_bytes;
    g.nodes = c.accepted_nodes;
    g.num_accepted = c.num_accepted;
    g.B = c.B;
    g.N1 = c.N1;
    g.L = c.L;
    g.vec = (c.row_bytes % 16 == 0) && (reinterpret_cast<uintptr_t>(c.src) % 16 == 0) &&
            (reinterpret_cast<uintptr_t>(c.dst) % 16 == 0);
    gather_rows_kernel<<<dim3((unsigned)((long long)c.B * c.L)), dim3(256), 0, st>>>(g);
    return hipGetLastError();
}

}  // namespace sv
