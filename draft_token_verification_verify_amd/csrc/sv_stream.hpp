// sv_stream.hpp -- the tile loop shared by the streaming kernels (softmax
// statistics and argmax).
//
// A tile is one chunk of one logits row: 256 threads x U 16-byte vectors, one
// workgroup per tile, tiles numbered request-major t = (b * R + r) * S + ch.
// Each workgroup issues all of its loads at once, reduces the tile and writes
// one 16-byte partial; nothing else.  The per-request merge of the partials
// happens in the next kernel of the call, after the kernel boundary has made
// every partial visible (no atomics or fences on the streaming path).
#pragma once

#include "sv_common.hpp"

namespace sv {

// Partial of one tile: meaning depends on the op (see the ops).
struct Partial16 {
    float f0;
    float f1;
    double d;
};
static_assert(sizeof(Partial16) == 16, "Partial16 layout");

// f1 of a published statistics partial (a cleared workspace reads 0).
constexpr float kPartialWritten = 1.0f;

// A partial as read back by a consumer: two 8-byte agent-coherent loads.
struct PartialRead {
    float f0;
    bool ok;
    double d;
};
__device__ inline PartialRead read_partial(const Partial16* p) {
    const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
    const unsigned long long h1 = load_coherent(q);
    const unsigned long long h2 = load_coherent(q + 1);
    PartialRead r;
    r.f0 = __uint_as_float((unsigned)h1);
    r.d = __longlong_as_double((long long)h2);
    r.ok = __uint_as_float((unsigned)(h1 >> 32)) == kPartialWritten && h2 != 0ull;
    return r;
}

// Sampling filter of one logits row, as the filtered stochastic call passes it
// from its selection kernel to the sampler: the row keeps the tokens whose
// logit is >= tau (every token when tau = -inf), m is the row maximum and s the
// kept mass, the sum of 2^((x - m) * c) over the kept tokens.
struct RowFilter {
    float tau;
    float m;
    double s;
};
static_assert(sizeof(RowFilter) == 16, "RowFilter layout");

// Tile t, rows 16-byte aligned (V a whole number of vectors).
//   Op::row(b, r) -> const T* row start
//   Op::skip(b, r) -> true for a row that is not read (its partial is
//     Op::publish_skipped's)
//   Op::tile(b, r, lo, hi, raw, nvec, &f0, &f1, &d): reduce the tile held in
//     raw[U] (this thread's vectors; slots >= nvec are padding); thread 0 then
//     calls Op::publish(&partials[t], f0, f1, d).
// A 16-byte load that asks the caches not to keep the line (for rows read once).
__device__ inline uint4 load16_nontemporal(const uint4* p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u w = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(w.x, w.y, w.z, w.w);
}

// NT: non-temporal loads, for rows that nothing in the call reads again while
// they could still be cached.
template <typename T, int U, bool NT = false, class Op>
__device__ __forceinline__ void stream_tile_vec(const Op& op, int t) {
    constexpr int EPV = Elem<T>::kPerVec;
    const int ch = t % op.S, rr = t / op.S;
    const int r = rr % op.R, b = rr / op.R;
    if (op.skip(b, r)) {  // row outside the request's window: nothing to read
        if (threadIdx.x == 0) op.publish_skipped(op.partials + t);
        return;
    }
    const int lo = ch * op.chunk, hi = min(op.V, lo + op.chunk);
    const int nvec = (hi - lo) / EPV;
    const uint4* base = reinterpret_cast<const uint4*>(op.row(b, r) + lo);
    // All U loads issue back to back: slots past the chunk's end reload its last
    // vector (in bounds) and are masked by the op.
    uint4 raw[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const uint4* p = base + min((int)threadIdx.x + j * kThreads, nvec - 1);
        raw[j] = NT ? load16_nontemporal(p) : *p;
    }
    float f0, f1;
    double d;
    op.tile(b, r, lo, hi, raw, nvec, &f0, &f1, &d);
    if (threadIdx.x == 0) op.publish(op.partials + t, f0, f1, d);
}

// Same for rows that are not 16-byte aligned: scalar loads.
template <typename T, class Op>
__device__ __forceinline__ void stream_tile_scalar(const Op& op, int t) {
    const int ch = t % op.S, rr = t / op.S;
    const int r = rr % op.R, b = rr / op.R;
    if (op.skip(b, r)) {
        if (threadIdx.x == 0) op.publish_skipped(op.partials + t);
        return;
    }
    const int lo = ch * op.chunk, hi = min(op.V, lo + op.chunk);
    float f0, f1;
    double d;
    op.tile_scalar(b, r, lo, hi, &f0, &f1, &d);
    if (threadIdx.x == 0) op.publish(op.partials + t, f0, f1, d);
}

// Zero a request's partials once every reader has read them, so that the
// workspace is all zero again when the call completes (a later call of another
// shape may place its arrival counters there).
__device__ inline void clear_partials(Partial16* p, int n) {
    for (int i = threadIdx.x; i < n; i += kThreads)
        *reinterpret_cast<uint4*>(p + i) = make_uint4(0, 0, 0, 0);
}

}  // namespace sv
