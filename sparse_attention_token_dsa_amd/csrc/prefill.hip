// Fused causal-prefill indexer: q . K contraction on bf16 MFMA, ReLU, the
// w-weighted head sum and the causal mask in the epilogue, a streaming per-row
// threshold and the row's exact top-k, in one kernel (PaperTrace, "2.2.2
// MISA, LISA and ResMiSA", section 2.2: score, causal mask and top-k fused
// into one pass, no n^2 score matrix written back).
//
// Layout: a workgroup of 8 waves owns 16 query rows of one sequence, 8
// consecutive ones near the start of the chunk and 8 near its end (so that
// the causal work is about the same for every workgroup), two rows per wave
// (their heads and weights held in registers as MFMA A fragments; each B
// fragment read from LDS feeds both rows, which keeps the LDS read traffic at
// about half of what the MFMAs can absorb), and sweeps the legal keys
// [0, max t] in tiles of 64 keys.  Each tile (16 KiB of bf16
// keys) is staged once in LDS for all 16 rows by direct global-to-LDS loads,
// in blocks of 4 keys padded by 16 bytes: the lanes that read one B-fragment
// chunk (keys 4c + gi, c = 0..15) hit distinct bank groups, and every chunk's
// address is one per-lane base plus an immediate offset.  Column c of MFMA
// group gi is key 4c + gi, so that after the head sum every lane holds the
// scores of 4 consecutive keys.  Four stages are used in pairs: one wait and
// one barrier per two tiles, and the next pair's loads have two tiles of
// compute to arrive.
//
// Epilogue: with ReLU(z) = (z + |z|) / 2,
//     I = sum_j w_j ReLU(z_j) = g . k + sum_j (w_j / 2) |z_j|,   g = sum_j (w_j / 2) q_j,
// the linear part being the one shared keys let the heads merge into
// (PaperTrace, "2.2.2 MISA, LISA and ResMiSA", section 3.1).  The per-head
// part is then one fused multiply-add per (head, key), |z| being a free
// operand modifier, instead of a max and a multiply-add.  g . k is one more
// MFMA tile per 16 keys for all 16 rows of the workgroup (g split into bf16
// hi + lo, so g . k keeps about 16 bits more than bf16): the pair's 8 groups
// are computed by 8 of the waves and pass through LDS to the row's wave when
// the pair's scores are settled.
//
// Streaming threshold: each row keeps an LDS histogram of the scores it has
// kept, over the bins below (monotone in the score).  tau is the highest bin
// such that at least k kept scores lie in bins >= tau; a new score below bin
// tau has k larger ones ahead of it and can never enter the row's top-k, so
// it is dropped with one compare.  The rest (about k (1 + ln(n / k)) per row
// for n keys in random order) are appended as (position, score) pairs to the
// row's survivor list in the workspace; the scores themselves never leave the
// chip.  The count of bin tau is mirrored in a register, so tau is re-derived
// from the histogram only when it can move.  A list has room for a bounded
// number of entries (the host gives max(6 k, 8192) per row when a row has
// more legal keys): a list that fills is compacted in place to the entries in
// bins >= tau, or, when one bin is too crowded for that, to exactly the row's
// current top-k (see pf_compact).
//
// Finish: after the sweep each wave selects its rows' exact top-k from their
// survivors: the histogram gives the bin holding the k-th score; one pass over
// the list emits the scores above it (staged in LDS, written out 64 at a time)
// and collects the ones in it, as 64-bit keys ord(score) << 32 | ~position
// (ties -> lower position), into LDS; a radix select on those keys settles the
// rest.  A bin too crowded for the LDS buffer has its next 10-bit digit counted
// in the same pass, so one more pass over the list settles it or shrinks it to
// LDS size.
#include <type_traits>

#include "sa_frag.h"

namespace sa {

constexpr int kPfWaves = 8;
constexpr int kPfQpw = 2;               // query rows per wave
constexpr int kPfRows = kPfWaves * kPfQpw;
constexpr int kPfTile = 64;
constexpr int kPfBlk = 65;              // uint4 per 4-key block: 1 KiB + 16 B pad
constexpr int kPfStage = 16 * kPfBlk;   // uint4 per stage (16 blocks, 16.25 KiB)
constexpr int kPfBins = 1024;           // histogram size (bins 947 .. 1023 stay empty)
constexpr int kPfDigit = 10;            // radix digit of the finish over LDS candidates
constexpr int kPfWide = 10;             // digit counted in the level-0 pass for crowded bins
constexpr int kPfCand = 1024;           // LDS candidate keys of a wave (its rows in turn)
constexpr int kPfSweep = 8;             // uint4 per lane per block of the level-0 pass
static_assert(2 * kPfCand * 8 <= kPfStage * 16, "two waves' candidate buffers fit one stage");
static_assert((1 << kPfDigit) == kPfBins, "digit histograms reuse the row histogram");
static_assert((1 << kPfWide) * 4 <= kPfCand * 8, "the wide digit histogram fits cb");
static_assert(kPfRows == 16 && kPfWaves == 8, "16 rows: one g tile; 2 blocks per wave fill a stage");
static_assert(kPfQpw == 2, "the 4 lane groups hold 2 rows x 2 tiles of a pair");

// Score bins, monotone in the score:
//   0           x <= -2^32
//   1 .. 64     negative x, one octave each: |x| in [2^(32-b), 2^(33-b))
//   65          -2^-32 < x < 2^-23 (zero and the smallest magnitudes)
//   66 .. 945   positive x in [2^-23, 2^32), 1/16 octave each
//   946         x >= 2^32
constexpr int kPfNegOct = 64;
constexpr int kPfMid = 65;
constexpr int kPfPos0 = 66;
constexpr int kPfPosShift = 19;  // float bits >> 19: exponent and 4 mantissa bits
constexpr int kPfTop = kPfPos0 + 55 * 16;
constexpr int kPfPosE = 104;  // biased exponent of 2^-23
constexpr int kPfNegE = 95;   // biased exponent of 2^-32
static_assert(kPfTop < kPfBins, "bins fit the histogram");

__device__ __forceinline__ int pf_bin(float x) {
    const uint32_t u = __float_as_uint(x);
    const int e = (int)((u >> 23) & 255u);
    const int pos = min(kPfPos0 + (int)(u >> kPfPosShift) - (kPfPosE << 4), kPfTop);
    const int neg = max(kPfNegOct - (e - kPfNegE), 0);
    return (u >> 31) ? (e >= kPfNegE ? neg : kPfMid) : (e >= kPfPosE ? pos : kPfMid);
}

// Smallest order key ord(x) of bin b, 1 <= b <= kPfTop.
__device__ __forceinline__ uint32_t pf_lo_ord(int b) {
    return b <= kPfMid ? 0x80000000u - ((uint32_t)(kPfNegE + 1 + kPfNegOct - b) << 23)
                       : 0x80000000u | ((uint32_t)(b - kPfPos0 + (kPfPosE << 4)) << kPfPosShift);
}

// Bin b as the score interval [lo, hi).
__device__ __forceinline__ float pf_lo(int b) { return b <= 0 ? -INFINITY : ord_to_f32(pf_lo_ord(b)); }
__device__ __forceinline__ float pf_hi(int b) {
    return b >= kPfTop ? INFINITY : ord_to_f32(pf_lo_ord(b + 1));
}

// Key bits a bin fixes: 63 .. top (top = 64: none).
__device__ __forceinline__ int pf_top(int b) {
    return (b >= kPfPos0 && b < kPfTop) ? 32 + kPfPosShift : ((b >= 1 && b <= kPfNegOct) ? 55 : 64);
}

// Number of set bits of m below this lane (no 64-bit lane mask kept live).
__device__ __forceinline__ int below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ unsigned long long pf_key(float sc, int idx) {
    return ((unsigned long long)ord_key(sc) << 32) | (unsigned long long)(~(uint32_t)idx);
}

// LDS add with no return value.  As an asm statement it carries no memory
// operand, so the compiler places no wait for in-flight global-to-LDS tile
// loads before it; LDS operations of one wave complete in issue order, so the
// wave's own later reads of the histogram see it.
__device__ __forceinline__ void lds_add_u32(uint32_t* p, uint32_t v) {
    asm volatile("ds_add_u32 %0, %1" : : "v"((uint32_t)(uintptr_t)p), "v"(v) : "memory");
}


// Scheduling of one pipelined block: M MFMAs, V VALU instructions spread
// evenly between them and, with RELOAD, one LDS read after each k-step's
// NHT MFMAs.
template <int I, int M, int V, int NHT, bool RELOAD>
__device__ __forceinline__ void pf_interleave() {
    if constexpr (I < M) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        constexpr int nv = V * (I + 1) / M - V * I / M;
        if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
        if constexpr (RELOAD && I % NHT == NHT - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        pf_interleave<I + 1, M, V, NHT, RELOAD>();
    }
}

// The same for an E4M3 block: M MFMAs (one per head tile, all 128 dims), V
// VALU instructions spread between them and, with RELOAD, the two LDS reads
// of the next group's key operand right after the first MFMA.
template <int I, int M, int V, bool RELOAD>
__device__ __forceinline__ void pf_interleave8() {
    if constexpr (I < M) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (RELOAD && I == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        constexpr int nv = V * (I + 1) / M - V * I / M;
        if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
        pf_interleave8<I + 1, M, V, RELOAD>();
    }
}

// One pass of a wave over a survivor list sl[0, cnt) of (position, score
// bits) pairs: fn(position, score, valid) for every lane and element, 2
// elements per 16-byte load, 4 loads in flight.  Lists have room for an even
// number of entries, so the clamped 16-byte reads stay inside.  Only crowded
// threshold bins re-read the list.
template <class F>
__device__ __forceinline__ void list_sweep(const uint2* sl, int cnt, F&& fn) {
    const int lane = lane_id();
    const uint4* s4 = reinterpret_cast<const uint4*>(sl);
    const int last = (cnt - 1) >> 1;
#pragma unroll 1
    for (int ub = 0; ub < cnt; ub += 512) {
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = s4[min((ub >> 1) + j * 64 + lane, last)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = ub + 2 * (j * 64 + lane);
            fn((int)v[j].x, __uint_as_float(v[j].y), u < cnt);
            fn((int)v[j].z, __uint_as_float(v[j].w), u + 1 < cnt);
        }
    }
}

// Wave-level: the bin d of an NB-bin histogram that holds the need-th
// largest element (bins scanned from the top); gt = elements above d,
// eq = elements in d.  Wave-uniform results.
template <int NB>
__device__ __forceinline__ void wave_threshold(const uint32_t* h, int need, int& d, int& gt, int& eq) {
    constexpr int kPer = NB / 64;
    const int lane = lane_id();
    int local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) local += (int)h[NB - 1 - (lane * kPer + j)];
    int cum = wave_incl_scan(local) - local;
    int fd = -1, fg = 0, fe = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int bin = NB - 1 - (lane * kPer + j);
        const int hv = (int)h[bin];
        if (cum < need && need <= cum + hv) {
            fd = bin;
            fg = cum;
            fe = hv;
        }
        cum += hv;
    }
    const unsigned long long m = __ballot(fd >= 0);
    const int src = m ? __ffsll((long long)m) - 1 : 0;
    d = __builtin_amdgcn_readlane(fd, src);
    gt = __builtin_amdgcn_readlane(fg, src);
    eq = __builtin_amdgcn_readlane(fe, src);
}

// Exact top-`need` of one row by one wave (see the file header): h holds the
// histogram of the row's cnt survivors sl[0, cnt), which include every legal
// score at or above the final threshold; cb is kPfCand keys of LDS.  Output
// order is unspecified.
//
// Digit levels narrow the threshold bin down on the key ord(score) << 32 |
// ~position: the keys still in play are those in [lo, hi) whose bits above
// pshift equal pval.
__device__ __forceinline__ void pf_finish(uint32_t* h, unsigned long long* cb, const uint2* sl,
                                          int cnt, int need, int32_t* oidx, float* osc) {
    const int lane = lane_id();
    const unsigned long long lt = (1ull << lane) - 1ull;
    int d0, gt0, eq0;
    wave_threshold<kPfBins>(h, need, d0, gt0, eq0);
    const float lo = pf_lo(d0), hi = pf_hi(d0);
    bool take_all = gt0 + eq0 == need;
    const bool fits = !take_all && eq0 <= kPfCand;
    const bool wide = !take_all && !fits;
    int top = pf_top(d0);
    uint32_t* hw = reinterpret_cast<uint32_t*>(cb);
    if (wide)
        for (int x = lane; x < (1 << kPfWide); x += 64) hw[x] = 0u;
    const int wshift = top - kPfWide;

    int out = 0, nc = 0;
    auto put = [&](bool emit, int s, float sc) {
        const unsigned long long me = __ballot(emit);
        if (emit) {
            const int slot = out + __popcll(me & lt);
            if (slot < need) {
                oidx[slot] = s;
                if (osc) osc[slot] = sc;
            }
        }
        out += __popcll(me);
    };
    // Level 0, one pass over the list.  The survivors to emit or to collect
    // (at or above lo; above hi only when bin d0 is crowded) are staged as
    // (position, score bits) pairs in a ring in the row histogram (free once
    // d0 is known); whole 64-entry blocks of it are then sent, all lanes busy,
    // to the output (above hi, or all when taking all) or to cb.  A crowded
    // bin's keys are counted into the wide digit histogram where they are met.
    uint2* ring = reinterpret_cast<uint2*>(h);
    constexpr int kRing = kPfBins / 2;
    int staged = 0, done = 0;
    auto drain = [&](bool all) {
        while (staged - done >= 64 || (all && staged > done)) {
            const int j = done + lane;
            const bool ok = j < staged;
            const uint2 e = ring[j & (kRing - 1)];
            const float sc = __uint_as_float(e.y);
            const bool up = ok && (take_all || sc >= hi);
            put(up, (int)e.x, sc);
            const bool app = ok && fits && !up;
            const unsigned long long ma = __ballot(app);
            if (app) cb[nc + __popcll(ma & lt)] = pf_key(sc, (int)e.x);
            nc += __popcll(ma);
            done += min(64, staged - done);
        }
    };
    // The pass, instantiated for a crowded bin d0 (WIDE) and for the rest.
    auto level0 = [&](auto wide_tag) __attribute__((always_inline)) {
        constexpr bool WIDE = decltype(wide_tag)::value;
        const uint4* s4 = reinterpret_cast<const uint4*>(sl);
        const int last = (cnt - 1) >> 1;
        constexpr int kStep = 128 * kPfSweep;
        uint4 cur[kPfSweep], nxt[kPfSweep];
#pragma unroll
        for (int j = 0; j < kPfSweep; ++j) cur[j] = s4[min(j * 64 + lane, last)];
        for (int ub = 0; ub < cnt; ub += kStep) {
            // The next block is in flight while this one is sorted out
            // (clamped: past the end it re-reads the last entries).
#pragma unroll
            for (int j = 0; j < kPfSweep; ++j)
                nxt[j] = s4[min(((ub + kStep) >> 1) + j * 64 + lane, last)];
#pragma unroll
            for (int j = 0; j < kPfSweep; ++j) {
                const int u = ub + 2 * (j * 64 + lane);
                const uint2 e2[2] = {make_uint2(cur[j].x, cur[j].y), make_uint2(cur[j].z, cur[j].w)};
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const bool in = u + i < cnt;
                    const float sc = __uint_as_float(e2[i].y);
                    if (WIDE && in && sc >= lo && sc < hi)
                        lds_add_u32(&hw[(uint32_t)(pf_key(sc, (int)e2[i].x) >> wshift) &
                                        ((1u << kPfWide) - 1)],
                                    1u);
                    const bool keep = in & (sc >= (WIDE ? hi : lo));
                    const unsigned long long m = __ballot(keep);
                    if (keep) ring[(staged + __popcll(m & lt)) & (kRing - 1)] = e2[i];
                    staged += __popcll(m);
                    // At most 63 + 2 x 64 entries pending: the ring holds 512.
                    if (i == 1) drain(false);
                }
            }
#pragma unroll
            for (int j = 0; j < kPfSweep; ++j) cur[j] = nxt[j];
        }
    };
    if (wide)
        level0(std::true_type{});
    else
        level0(std::false_type{});
    drain(true);
    if (take_all) return;

    int need_rem = need - gt0;
    const bool fixed = top < 64;
    unsigned long long pval = fixed ? (unsigned long long)(pf_lo_ord(d0) >> (top - 32)) : 0ull;
    int pshift = top;
    bool inlds = fits;  // candidates in cb, else re-read the list
    int nsrc = fits ? nc : cnt;
    bool first = wide;  // the wide digit's histogram is already in cb
    while (top > 0) {
        const int width = first ? kPfWide : (top < kPfDigit ? top : kPfDigit);
        const int shift = top - width;
        const unsigned long long mask = (1ull << width) - 1ull;
        auto live = [&](unsigned long long key, float sc) {
            return sc >= lo && sc < hi && (pshift == 64 || (key >> pshift) == pval);
        };
        int d, gt, eq;
        if (first) {
            wave_threshold<(1 << kPfWide)>(hw, need_rem, d, gt, eq);
        } else {
            for (int x = lane; x < kPfBins; x += 64) h[x] = 0u;
            if (inlds) {
                for (int u = lane; u < nsrc; u += 64)
                    lds_add_u32(&h[(uint32_t)((cb[u] >> shift) & mask)], 1u);
            } else {
                list_sweep(sl, cnt, [&](int s, float sc, bool in) {
                    const unsigned long long key = pf_key(sc, s);
                    if (in && live(key, sc)) lds_add_u32(&h[(uint32_t)((key >> shift) & mask)], 1u);
                });
            }
            wave_threshold<kPfBins>(h, need_rem, d, gt, eq);
        }
        take_all = gt + eq == need_rem;
        const bool fits_next = !take_all && eq <= kPfCand;
        int nn = 0;
        // Compaction in place: a kept key moves to a slot at or below the one
        // it was read from, after the read (one wave, LDS in order).
        auto visit = [&](unsigned long long key, bool ok) {
            const uint32_t dig = (uint32_t)((key >> shift) & mask);
            put(ok && (dig > (uint32_t)d || (take_all && dig == (uint32_t)d)),
                (int)(~(uint32_t)key), ord_to_f32((uint32_t)(key >> 32)));
            const bool app = ok && fits_next && dig == (uint32_t)d;
            const unsigned long long ma = __ballot(app);
            if (app) cb[nn + __popcll(ma & lt)] = key;
            nn += __popcll(ma);
        };
        if (inlds) {
            for (int ub = 0; ub < nsrc; ub += 64) {
                const int u = ub + lane;
                const bool ok = u < nsrc;
                visit(ok ? cb[u] : 0ull, ok);
            }
        } else {
            list_sweep(sl, cnt, [&](int s, float sc, bool in) {
                const unsigned long long key = pf_key(sc, s);
                visit(key, in && live(key, sc));
            });
        }
        need_rem -= gt;
        if (take_all) return;
        pval = pshift == 64 ? (unsigned long long)d : ((pval << width) | (unsigned long long)d);
        pshift = shift;
        top = shift;
        inlds = fits_next;
        nsrc = fits_next ? nn : cnt;
        first = false;
    }
}

// Threshold state of one row: list entries, entries in bins >= tau, tau, the
// count of bin tau, and the score a new key must reach.
struct PfRow {
    int cnt, ge, tau, htau;
    float tau_f;
};

// Compaction of a full survivor list (the row holds at least k + kPfRoom
// entries, at least k of them in bins >= tau).  It runs rarely, at the top
// of a pair of tiles, as passes over the list in position order; the last
// keeps, in place, the entries whose order key ord(score) is above xo, or
// equal to xo with position <= pmax, and rebuilds the row histogram:
//  - normally xo is just below bin tau: the entries in bins >= tau stay (at
//    least k, so the row's top-k does);
//  - if that leaves too little room (a crowded bin, e.g. equal scores),
//    exactly the row's current top-k stays: earlier passes bisect the order
//    keys of bin tau for its k-th score s (count of entries at or above a
//    probe), then find pmax, the position of the last entry equal to s that
//    is still in the top-k (ties go to the lower position, and the list is
//    in position order).  The threshold then moves just above s: a later key
//    with score s loses the tie to an earlier one.
// All passes share one loop over the list.
constexpr int kPfRoom = 3 * 2 * kPfTile;
__device__ __forceinline__ PfRow pf_compact(uint2* L, uint32_t* hr, PfRow st, int k,
                                            long long cap) {
    const int lane = lane_id();
    const int n = st.cnt;
    const bool exact = st.ge + kPfRoom > cap;
    // bisection bounds on the order key: at least k entries at or above lo,
    // fewer than k at or above hi (tau is the highest such bin)
    uint32_t lo = st.tau == 0 ? 0u : pf_lo_ord(st.tau);
    uint32_t hi = st.tau >= kPfTop ? 0xffffffffu : pf_lo_ord(st.tau + 1);
    // passes: 0 count at or above the probe, 1 count above s, 2 find pmax,
    // 3 compact
    int kind = exact ? (hi - lo > 1u ? 0 : 1) : 3;
    uint32_t xo = exact ? lo : pf_lo_ord(st.tau) - 1u;
    int pmax = -1, m = 0;
#pragma unroll 1
    for (;;) {
        const uint32_t probe = kind == 0 ? lo + (hi - lo) / 2u : hi;
        if (kind == 3)
            for (int b = lane; b < kPfBins; b += 64) hr[b] = 0u;
        int c = 0, out = 0;
        // 256 entries per step, all four loads issued before any is used
#pragma unroll 1
        for (int ub = 0; ub < n; ub += 256) {
            uint2 ev[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) ev[j] = L[min(ub + 64 * j + lane, n - 1)];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint2 e = ev[j];
                const int u = ub + 64 * j + lane;
                const uint32_t o = ord_key(__uint_as_float(e.y));
                const bool in = u < n;
                if (kind <= 1) {
                    c += __popcll(__ballot(in && o >= probe));
                } else if (kind == 2) {
                    const bool eqs = in && o == xo;
                    const unsigned long long me = __ballot(eqs);
                    const int ne = __popcll(me);
                    if (m > 0 && ne >= m) {
                        const unsigned long long ml = __ballot(eqs && below(me) == m - 1);
                        pmax = __builtin_amdgcn_readlane((int)e.x, __ffsll((long long)ml) - 1);
                    }
                    m -= ne;
                } else {
                    // the step's entries are read before any is written; every
                    // write lands at or below the slot it came from
                    const bool kept = in && (o > xo || (o == xo && (int)e.x <= pmax));
                    const unsigned long long mk = __ballot(kept);
                    if (kept) {
                        L[out + below(mk)] = e;
                        lds_add_u32(&hr[pf_bin(__uint_as_float(e.y))], 1u);
                    }
                    out += __popcll(mk);
                }
            }
        }
        if (kind == 0) {
            if (c >= k) lo = probe; else hi = probe;
            if (hi - lo <= 1u) kind = 1;
        } else if (kind == 1) {
            xo = lo;       // the order key of the k-th score
            m = k - c;     // entries equal to it that are in the top-k
            kind = 2;
        } else if (kind == 2) {
            kind = 3;
        } else {
            st.cnt = out;
            break;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the compacted list is stored
    if (exact) {
        // exactly k entries, all at or above s: tau is the bin of s
        const float sk = ord_to_f32(xo);
        st.ge = st.cnt;
        st.tau = pf_bin(sk);
        st.htau = __builtin_amdgcn_readfirstlane((int)hr[st.tau]);
        st.tau_f = fmaxf(pf_lo(st.tau), ord_to_f32(xo + 1u));
    }
    return st;
}

// PACK2 (bf16 keys, at most 8 heads, NHT = 1): the wave's two rows share one
// 16-row head tile, row 0's heads on tile rows 0-3 and 8-11, row 1's on 4-7
// and 12-15, so one MFMA per k-step scores both rows and the head sum of a
// lane group's row is one lane-group swap away (lane groups g and g ^ 2 hold
// the same row, and lane group g keeps the row g & 1, as the unpacked form).
template <int NHT, bool F8, bool PACK2>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_kernel(PrefillArgs a) {
    static_assert(!PACK2 || (NHT == 1 && !F8), "packed rows: one bf16 head tile");
    // The stages are four distinct LDS objects: the compiler then tracks the
    // direct-to-LDS loads per object and places no wait of its own for the
    // pair in flight before reads of the other pair.
    __shared__ uint4 kt0[kPfStage], kt1[kPfStage], kt2[kPfStage], kt3[kPfStage];
    __shared__ uint32_t hist[kPfRows][kPfBins];
    // A fragments of the rows' g (hi, lo: tile row = workgroup row) and the
    // g . k values of the last two pairs (pair parity, tile, row, 4 keys).
    __shared__ uint4 gfrag[2][4][64];
    __shared__ float4 gk[2][2][kPfRows][kPfTile / 4];

    // Rows in groups of 8: workgroup x takes group x (waves 0-3) and group
    // G-1-x (waves 4-7), a short and a long causal row range.  Waves w and
    // w + 4 share a SIMD, so once the short rows are done the long ones have
    // its MFMA pipe to themselves, and every workgroup carries about the same
    // work.
    const int seq = blockIdx.y;
    const int G = (a.T + 7) >> 3;
    const int gA = blockIdx.x, gB = G - 1 - blockIdx.x;  // gA <= gB
    const int tid = threadIdx.x;
    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Position of the sequence's first row: the common offset, or for a
    // ragged batch its own length less T.
    const int offset =
        a.seq_lens ? min(max(a.seq_lens[seq], a.T), a.L) - a.T : a.offset;
    const int tmax = offset + min(gB * 8 + 7, a.T - 1);
    const int ntiles = tmax / kPfTile + 1;

    // Per-row state of this wave's two rows (workgroup rows 2 wid + qq).
    // With F8 the A fragments are the rows' E4M3 query codes, and the
    // weights carry the query scales.
    std::conditional_t<F8, QFrag8<NHT>, QFrag<NHT>> f[kPfQpw];
    int tq[kPfQpw], tau[kPfQpw], cnt[kPfQpw], cnt_ge[kPfQpw], htau[kPfQpw];
    float tau_f[kPfQpw];
    bool act[kPfQpw];
    long long rowq[kPfQpw];
    uint2* sl[kPfQpw];
    uint32_t* h[kPfQpw];
#pragma unroll
    for (int qq = 0; qq < kPfQpw; ++qq) {
        const int r = wid * kPfQpw + qq;
        const int i = (r < 8 ? gA : gB) * 8 + (r & 7);
        act[qq] = i < a.T && (r < 8 || gB != gA);
        rowq[qq] = (long long)seq * a.T + min(i, a.T - 1);
        tq[qq] = act[qq] ? offset + i : -1;
        tau[qq] = 0;
        tau_f[qq] = -INFINITY;
        cnt[qq] = 0;
        cnt_ge[qq] = 0;
        htau[qq] = 0;
        sl[qq] = a.surv + rowq[qq] * a.cap;
        h[qq] = hist[r];
        for (int x = lane; x < kPfBins; x += 64) h[qq][x] = 0u;
        const float* wrow = a.w + rowq[qq] * a.H;
        // F8: the wave quantizes the row's heads into its own slice of the
        // key stages (free until the first fill) and the scales into gk.
        uint4* qc = (wid >> 1 == 0 ? kt0 : wid >> 1 == 1 ? kt1 : wid >> 1 == 2 ? kt2 : kt3) +
                    (wid & 1) * 512;
        float* qs = reinterpret_cast<float*>(&gk[0][0][0][0]) + kPfRows * kD + wid * 64;
        if constexpr (F8) {
            quantize_q8_wave(a.q + rowq[qq] * a.H * kD, a.H, qc, qs);
            load_qfrag_fp8<NHT>(f[qq], qc, qs, wrow, a.H, g, c);
        } else if constexpr (!PACK2) {
            load_qfrag<NHT>(f[qq], a.q + rowq[qq] * a.H * kD, wrow, a.H, nullptr, 0, g, c);
        }
        if constexpr (!PACK2)
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    f[qq].wv[ht][e] = act[qq] ? 0.5f * f[qq].wv[ht][e] : 0.f;
        // g = sum_j (w_j / 2) q_j of the row, two dims per lane, heads in
        // order, staged in gk (free until the sweep starts); lanes 0..15 then
        // pack the row's A-fragment entries: lane t holds dims
        // (kk*4 + grp)*8 .. +8 with kk = t / 4, grp = t % 4, for tile row r.
        // (F8: g of the decoded query codes, with the weights w_j b_j.)
        const float wl =
            act[qq] && lane < a.H ? 0.5f * (F8 ? wrow[lane] * qs[lane] : wrow[lane]) : 0.f;
        const uint16_t* qr = a.q + rowq[qq] * a.H * kD;
        float g0 = 0.f, g1 = 0.f;
        for (int j = 0; j < a.H; ++j) {
            const float wj = __shfl(wl, j);
            float x0, x1;
            if constexpr (F8) {
                // dims 2 lane, 2 lane + 1: chunk lane / 8, word (lane % 8) / 2
                const uint32_t wd =
                    reinterpret_cast<const uint32_t*>(qc + qslot(j, lane >> 3))[(lane & 7) >> 1];
                const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8(wd, false);
                const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8(wd, true);
                x0 = (lane & 1) ? hi2[0] : lo2[0];
                x1 = (lane & 1) ? hi2[1] : lo2[1];
            } else {
                const uint32_t two = *reinterpret_cast<const uint32_t*>(qr + j * kD + 2 * lane);
                x0 = bf16_bits_to_f32(two & 0xffffu);
                x1 = bf16_bits_to_f32(two >> 16);
            }
            g0 = fmaf(wj, x0, g0);
            g1 = fmaf(wj, x1, g1);
        }
        float* gt = reinterpret_cast<float*>(&gk[0][0][0][0]) + r * kD;
        gt[2 * lane] = g0;
        gt[2 * lane + 1] = g1;
        if (lane < 16) {
            const int kk = lane >> 2, grp = lane & 3;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v0 = gt[(kk * 4 + grp) * 8 + 2 * e];
                const float v1 = gt[(kk * 4 + grp) * 8 + 2 * e + 1];
                const uint32_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
                hi[e] = h0 | (h1 << 16);
                lo[e] = f32_to_bf16_bits(v0 - bf16_bits_to_f32(h0)) |
                        (f32_to_bf16_bits(v1 - bf16_bits_to_f32(h1)) << 16);
            }
            gfrag[0][kk][16 * grp + r] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            gfrag[1][kk][16 * grp + r] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
    }
    if constexpr (PACK2) {
        // Tile row c: row (c >> 2) & 1, head (c & 3) + 4 (c >> 3); output row
        // 4g + e of lane group g: row g & 1, head e + 4 (g >> 1).
        const int ra = (c >> 2) & 1, ja = (c & 3) + 4 * (c >> 3);
        const bool va = ja < a.H;
        const uint16_t* qa =
            a.q + ((ra ? rowq[1] : rowq[0]) * a.H + (va ? ja : 0)) * kD + g * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            f[0].a[0][kk] = va ? ldg16(qa + kk * 32) : make_uint4(0u, 0u, 0u, 0u);
        const int rw = g & 1;
        const float* ww = a.w + (rw ? rowq[1] : rowq[0]) * a.H;
        const bool aw = rw ? act[1] : act[0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jw = e + 4 * (g >> 1);
            f[0].wv[0][e] = aw && jw < a.H ? 0.5f * ww[jw] : 0.f;
        }
    }
    __syncthreads();  // fragments visible; the staging area is free again
    const int tw = max(tq[0], tq[kPfQpw - 1]);  // last legal key of this wave

    const uint16_t* kseq = a.keys + (long long)seq * a.L * kD;
    // Stage fill: each load instruction of a wave writes one 4-key block (64
    // lanes x 16 bytes at consecutive addresses); wave w fills blocks w and
    // w + 8: lane l brings chunk l%16 of key 4*block + l/16.  Tiles past the
    // last are clamped re-reads.  The fills are buffer loads over the tile's
    // 16 KiB (base key k0): unlike the global form, they leave the compiler's
    // LDS wait counts exact, so the B-fragment reads of the sweep are waited
    // for one by one.
    // F8: a tile is 64 keys x 128 codes (8 KiB, one 1 KiB load per wave:
    // key 8 wid + l / 8, LDS slot l % 8 holding the key's global 16-byte
    // chunk (l % 8) ^ ((key / 4) % 8), so that the 8 lanes of a B-fragment
    // read hit 8 different bank groups), then the tile's 64 scales (256 B,
    // wave 0) at uint4 512 of the stage.
    const uint8_t* cseq = F8 ? a.codes + (long long)seq * a.L * kD : nullptr;
    const float* sseq = F8 ? a.kscale + (long long)seq * a.L : nullptr;
    auto issue = [&](uint4* stage, int tile) __attribute__((always_inline)) {
        const int k0 = min(tile * kPfTile, tmax);
        if constexpr (F8) {
            const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(cseq + (long long)k0 * kD), 0, kPfTile * kD, 0x00020000);
            const int kt = 8 * wid + (lane >> 3);
            const int s = min(tile * kPfTile + kt, tmax);
            const int m = (lane & 7) ^ ((kt >> 2) & 7);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rc, (__attribute__((address_space(3))) void*)(stage + wid * 64), 16,
                (uint32_t)((s - k0) * kD + m * 16), 0, 0, 0);
            if (wid == 0) {
                const __amdgpu_buffer_rsrc_t rs8 = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float*>(sseq + k0), 0, kPfTile * 4, 0x00020000);
                const int s2 = min(tile * kPfTile + lane, tmax);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs8, (__attribute__((address_space(3))) void*)(stage + 512), 4,
                    (uint32_t)((s2 - k0) * 4), 0, 0, 0);
            }
            return;
        }
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(kseq + (long long)k0 * kD), 0, kPfTile * kD * 2, 0x00020000);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int blk = wid + kPfWaves * jb;
            const int key = 4 * blk + (lane >> 4);
            const int s = min(tile * kPfTile + key, tmax);  // k0 <= s < k0 + 64
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(stage + blk * kPfBlk), 16,
                (uint32_t)((s - k0) * kD * 2 + (lane & 15) * 16), 0, 0, 0);
        }
    };
    // B fragment of step kk for key 4c + gi: block c, row gi, chunk kk*4 + g.
    const int bbase = c * kPfBlk + g;
    // F8 B operand of key 4c + gi: its chunks 2g and 2g + 1 (dims 32g ..
    // 32g+31), at slots (4c + gi) * 8 + (chunk ^ (c % 8)).
    const int b8lo = c * 32 + ((2 * g) ^ (c & 7)), b8hi = c * 32 + ((2 * g + 1) ^ (c & 7));
    auto load_b8 = [&](const uint4* ktile, int gi) __attribute__((always_inline)) {
        const uint4 lo = ktile[b8lo + gi * 8], hi = ktile[b8hi + gi * 8];
        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // F8: scales of keys 4c .. 4c+3 of the pair's two tiles.
    float ksr[2][4];

    // Scores of tile j of a pair: lane (g, c) keeps, for the row and tile of
    // its lane group (row g & 1, tile g >> 1), the per-head part of the
    // scores of keys 4c .. 4c+3 in st.
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
    // The pair's 16 blocks (group G = 4 j + gi of its two tiles, row qq) run
    // as a software pipeline: block n issues its MFMAs into acc[qq] while
    // the epilogue of block n - 1 (the other accumulator set) is interleaved
    // between them, so that the wave keeps the MFMA pipe fed by itself.  The
    // B fragments of group G + 1 are re-read into the registers of group G
    // right after the second row's last use of each k-step; only the pair's
    // first read waits in full.  The second tile's stage always holds a
    // (possibly clamped) fill, so reading it ahead is harmless.
    uint4 bf[4];
    f32x4 acc[kPfQpw][NHT];
    auto load_b = [&](const uint4* ktile, int gi) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bf[kk] = ktile[bbase + gi * 16 + kk * 4];
    };
    auto epilogue = [&](int qq, int j, int gi) __attribute__((always_inline)) {
        float sc = 0.f;
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int e = 0; e < 4; ++e) sc = fmaf(f[qq].wv[ht][e], fabsf(acc[qq][ht][e]), sc);
        sc = sum_lane_groups(sc);
        if constexpr (F8) sc *= ksr[j][gi];
        st[gi] = g == 2 * j + qq ? sc : st[gi];
    };
    // Block (G, qq); RELOAD: re-read group G + 1 (at ntile, group ngi) behind
    // the MFMAs; PREV: run the epilogue of the block before, (pj, pgi, 1 - qq).
    auto block = [&](auto reload_c, auto prev_c, int qq, const uint4* ntile, int ngi, int pj,
                     int pgi) __attribute__((always_inline)) {
        constexpr bool kReload = decltype(reload_c)::value;
        constexpr bool kPrev = decltype(prev_c)::value;
        // Each block is scheduled on its own.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!F8) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht)
                    acc[qq][ht] = mfma16x16x32(f[qq].a[ht][kk], bf[kk],
                                               kk ? acc[qq][ht] : f32x4{0.f, 0.f, 0.f, 0.f});
                if (kReload) bf[kk] = ntile[bbase + ngi * 16 + kk * 4];
            }
            if (kPrev) epilogue(1 - qq, pj, pgi);
            pf_interleave<0, 4 * NHT, (kPrev ? 4 * NHT + 7 : 0), NHT, kReload>();
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // E4M3 blocks: B operands alternate between two register sets per group,
    // so the next group's operand loads during the current group's first
    // block (the other set's last reader is the block before).
    i32x8 bfr[2];
    auto block8 = [&](auto reload_c, auto prev_c, auto cur_c, int qq, const uint4* ntile, int ngi,
                      int pj, int pgi) __attribute__((always_inline)) {
        constexpr bool kReload = decltype(reload_c)::value;
        constexpr bool kPrev = decltype(prev_c)::value;
        constexpr int kCur = decltype(cur_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (F8) {
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) acc[qq][ht] = mfma16x16x128_fp8(f[qq].a[ht], bfr[kCur]);
            if (kReload) bfr[1 - kCur] = load_b8(ntile, ngi);
            if (kPrev) epilogue(1 - qq, pj, pgi);
            pf_interleave8<0, NHT, (kPrev ? 4 * NHT + 8 : 0), kReload>();
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto pair_scores8 = [&](const uint4* ka, const uint4* kb, bool two) __attribute__((always_inline)) {
        const std::true_type y;
        const std::false_type n;
        const std::integral_constant<int, 0> b0;
        const std::integral_constant<int, 1> b1;
        const float4 sa4 = reinterpret_cast<const float4*>(ka + 512)[c];
        const float4 sb4 = reinterpret_cast<const float4*>(kb + 512)[c];
        ksr[0][0] = sa4.x; ksr[0][1] = sa4.y; ksr[0][2] = sa4.z; ksr[0][3] = sa4.w;
        ksr[1][0] = sb4.x; ksr[1][1] = sb4.y; ksr[1][2] = sb4.z; ksr[1][3] = sb4.w;
        bfr[0] = load_b8(ka, 0);
        block8(y, n, b0, 0, ka, 1, 0, 0);
        block8(n, y, b0, 1, ka, 0, 0, 0);
        block8(y, y, b1, 0, ka, 2, 0, 0);
        block8(n, y, b1, 1, ka, 0, 0, 1);
        block8(y, y, b0, 0, ka, 3, 0, 1);
        block8(n, y, b0, 1, ka, 0, 0, 2);
        block8(y, y, b1, 0, kb, 0, 0, 2);
        block8(n, y, b1, 1, kb, 0, 0, 3);
        if (two) {
            block8(y, y, b0, 0, kb, 1, 0, 3);
            block8(n, y, b0, 1, kb, 0, 1, 0);
            block8(y, y, b1, 0, kb, 2, 1, 0);
            block8(n, y, b1, 1, kb, 0, 1, 1);
            block8(y, y, b0, 0, kb, 3, 1, 1);
            block8(n, y, b0, 1, kb, 0, 1, 2);
            block8(n, y, b1, 0, kb, 0, 1, 2);
            block8(n, y, b1, 1, kb, 0, 1, 3);
            epilogue(1, 1, 3);
        } else {
            epilogue(1, 0, 3);
        }
    };
    auto pair_scores = [&](const uint4* ka, const uint4* kb, bool two) __attribute__((always_inline)) {
        const std::true_type y;
        const std::false_type n;
        load_b(ka, 0);
        block(n, n, 0, ka, 0, 0, 0);
        block(y, y, 1, ka, 1, 0, 0);
        block(n, y, 0, ka, 0, 0, 0);
        block(y, y, 1, ka, 2, 0, 1);
        block(n, y, 0, ka, 0, 0, 1);
        block(y, y, 1, ka, 3, 0, 2);
        block(n, y, 0, ka, 0, 0, 2);
        block(y, y, 1, kb, 0, 0, 3);
        if (two) {
            block(n, y, 0, kb, 0, 0, 3);
            block(y, y, 1, kb, 1, 1, 0);
            block(n, y, 0, kb, 0, 1, 0);
            block(y, y, 1, kb, 2, 1, 1);
            block(n, y, 0, kb, 0, 1, 1);
            block(y, y, 1, kb, 3, 1, 2);
            block(n, y, 0, kb, 0, 1, 2);
            block(n, y, 1, kb, 0, 1, 3);
            epilogue(1, 1, 3);
        } else {
            epilogue(1, 0, 3);
        }
    };

    // PACK2: one block per 16-key group for both rows; blocks alternate
    // between the two accumulator sets, each re-reads the next group's B
    // fragments behind its MFMAs and runs the epilogue of the group before.
    auto epilogue2 = [&](int set, int j, int gi) __attribute__((always_inline)) {
        float sc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sc = fmaf(f[0].wv[0][e], fabsf(acc[set][0][e]), sc);
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc), __float_as_uint(sc),
                                                        false, false);
        sc = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        st[gi] = (g >> 1) == j ? sc : st[gi];
    };
    auto block2 = [&](auto reload_c, auto prev_c, int set, const uint4* ntile, int ngi, int pj,
                      int pgi) __attribute__((always_inline)) {
        constexpr bool kReload = decltype(reload_c)::value;
        constexpr bool kPrev = decltype(prev_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PACK2) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                acc[set][0] = mfma16x16x32(f[0].a[0][kk], bf[kk],
                                           kk ? acc[set][0] : f32x4{0.f, 0.f, 0.f, 0.f});
                if (kReload) bf[kk] = ntile[bbase + ngi * 16 + kk * 4];
            }
            if (kPrev) epilogue2(1 - set, pj, pgi);
            pf_interleave<0, 4, (kPrev ? 8 : 0), 1, kReload>();
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto pair_scores2 = [&](const uint4* ka, const uint4* kb, bool two) __attribute__((always_inline)) {
        const std::true_type y;
        const std::false_type n;
        load_b(ka, 0);
        block2(y, n, 0, ka, 1, 0, 0);
        block2(y, y, 1, ka, 2, 0, 0);
        block2(y, y, 0, ka, 3, 0, 1);
        block2(y, y, 1, kb, 0, 0, 2);
        if (two) {
            block2(y, y, 0, kb, 1, 0, 3);
            block2(y, y, 1, kb, 2, 1, 0);
            block2(y, y, 0, kb, 3, 1, 1);
            block2(n, y, 1, kb, 0, 1, 2);
            epilogue2(1, 1, 3);
        } else {
            epilogue2(1, 0, 3);
        }
    };

    // Raise tau of row r while the bins at and above tau + 1 still hold k
    // kept scores (the histogram adds of this wave are in LDS order before
    // these reads).
    auto raise = [&](int r) {
        uint32_t* hr = r ? h[1] : h[0];
        int t = r ? tau[1] : tau[0];
        int ge = r ? cnt_ge[1] : cnt_ge[0];
        int ht;
        for (;;) {
            const int bb = t + lane;
            const int hv = bb < kPfBins ? (int)hr[bb] : 0;
            const int excl = wave_incl_scan(hv) - hv;
            const bool ok = bb < kPfBins && ge - excl >= a.k;
            const int lstar = __popcll(__ballot(ok)) - 1;
            t += lstar;
            ge -= __builtin_amdgcn_readlane(excl, lstar);
            if (lstar < 63 || t >= kPfBins - 1) {
                ht = __builtin_amdgcn_readlane(hv, lstar);
                break;
            }
        }
        // Wave-uniform: keep them in scalar registers.
        t = __builtin_amdgcn_readfirstlane(t);
        ge = __builtin_amdgcn_readfirstlane(ge);
        ht = __builtin_amdgcn_readfirstlane(ht);
        const float tf = pf_lo(t);
        if (r) {
            tau[1] = t;
            cnt_ge[1] = ge;
            htau[1] = ht;
            tau_f[1] = tf;
        } else {
            tau[0] = t;
            cnt_ge[0] = ge;
            htau[0] = ht;
            tau_f[0] = tf;
        }
    };

    // A pair's scores are settled at the top of the next pair, right after its
    // stage wait: each lane completes its 4 scores with the pair's g . k,
    // tests them against its row's threshold, appends the survivors to the
    // row's list (positions from a row-local prefix count over the lanes of
    // the row) and to its histogram, and tau moves when it can.
    constexpr unsigned long long kRow0 = 0x0000FFFF0000FFFFull;  // lane groups 0 and 2
    int pend_base = -1, pend_buf = 0;
    auto settle = [&]() __attribute__((always_inline)) {
        if (pend_base < 0) return;
        const int qs = g & 1;
        const int key0 = pend_base + (g >> 1) * kPfTile + 4 * c;
        // g . k of the pair is complete: every wave passed the pair's end
        // barrier after its LDS stores (slots of tiles past the workgroup's
        // last key are never written and only meet masked keys).
        const float4 gv = gk[pend_buf][g >> 1][wid * kPfQpw + qs][c];
        st[0] += gv.x;
        st[1] += gv.y;
        st[2] += gv.z;
        st[3] += gv.w;
        const int tqs = qs ? tq[1] : tq[0];
        const float thr = qs ? tau_f[1] : tau_f[0];
        const int taus = qs ? tau[1] : tau[0];
        bool sv[4];
        int bn[4];
        int n = 0, nt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sv[e] = key0 + e <= tqs && st[e] >= thr;
            bn[e] = pf_bin(st[e]);
            n += sv[e];
            nt += sv[e] && bn[e] == taus;
        }
        const unsigned long long b0 = __ballot(n & 1), b1 = __ballot(n & 2), b2 = __ballot(n & 4);
        const unsigned long long mrow = qs ? ~kRow0 : kRow0;
        int p = (qs ? cnt[1] : cnt[0]) + below(b0 & mrow) + 2 * below(b1 & mrow) +
                4 * below(b2 & mrow);
        uint2* dst = qs ? sl[1] : sl[0];
        uint32_t* hq = qs ? h[1] : h[0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (sv[e]) {
                dst[p] = make_uint2((uint32_t)(key0 + e), __float_as_uint(st[e]));
                lds_add_u32(&hq[bn[e]], 1u);
            }
            p += sv[e];
        }
        const unsigned long long t0 = __ballot(nt & 1), t1 = __ballot(nt & 2), t2 = __ballot(nt & 4);
#pragma unroll
        for (int r = 0; r < kPfQpw; ++r) {
            const unsigned long long m = r ? ~kRow0 : kRow0;
            const int tot = __popcll(b0 & m) + 2 * __popcll(b1 & m) + 4 * __popcll(b2 & m);
            const int tt = __popcll(t0 & m) + 2 * __popcll(t1 & m) + 4 * __popcll(t2 & m);
            cnt[r] += tot;
            cnt_ge[r] += tot;
            htau[r] += tt;
            if (cnt_ge[r] - htau[r] >= a.k) raise(r);
        }
        pend_base = -1;
    };

    // g . k for one group of the pair per wave (group wave % 4 of tile
    // wave / 4): 4 k-steps x (hi, lo) into one accumulator.  D row 4g+e is
    // workgroup row 4g+e, column c is key 4c + gi of the tile.
    auto gk_unit = [&](const uint4* ka, const uint4* kb, int tile, int buf)
                       __attribute__((always_inline)) {
        const int j = wid >> 2, gi = wid & 3;
        if ((tile + j) * kPfTile > tmax) return;
        const uint4* ktile = j ? kb : ka;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // One k-step's fragments at a time (12 registers, not 48).
            asm volatile("" ::: "memory");
            uint4 bq;
            if constexpr (F8) {
                // dims (kk*4 + g)*8 .. +8 of key 4c + gi: half (kk*4 + g) % 2 of
                // its 16-byte chunk (kk*4 + g) / 2, widened exactly to bf16
                const int ch = (kk * 4 + g) >> 1;
                const uint2 v = reinterpret_cast<const uint2*>(
                    ktile + (4 * c + gi) * 8 + (ch ^ (c & 7)))[(kk * 4 + g) & 1];
                bq = widen8(v.x, v.y);
            } else {
                bq = ktile[bbase + gi * 16 + kk * 4];
            }
            d = mfma16x16x32(gfrag[0][kk][lane], bq, d);
            d = mfma16x16x32(gfrag[1][kk][lane], bq, d);
        }
        if constexpr (F8) {
            const float ks = reinterpret_cast<const float*>(ktile + 512)[4 * c + gi];
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] *= ks;
        }
        float* dst = reinterpret_cast<float*>(&gk[buf][j][0][0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(4 * g + e) * kPfTile + 4 * c + gi] = d[e];
    };

    // One barrier per pair: after it, the pair's data is visible to all and
    // every wave is done with the other pair's stages, which are refilled
    // for the pair after next.
    auto pair = [&](const uint4* ka, const uint4* kb, uint4* na, uint4* nb, int tile)
                    __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        // Settle and the g . k unit read LDS locations the compiler cannot
        // tell apart from the stage fills, so they run before the fills are
        // issued (nothing in flight, no wait); the fills still have the
        // pair's two tiles of compute to land.
        settle();
        const int buf = (tile >> 1) & 1;
        gk_unit(ka, kb, tile, buf);
        issue(na, tile + 2);
        issue(nb, tile + 3);
        const int kbase = tile * kPfTile;
        if (kbase <= tw) {
            if constexpr (F8)
                pair_scores8(ka, kb, kbase + kPfTile <= tw);
            else if constexpr (PACK2)
                pair_scores2(ka, kb, kbase + kPfTile <= tw);
            else
                pair_scores(ka, kb, kbase + kPfTile <= tw);
            pend_base = kbase;  // keys past a row's last legal one are never kept
            pend_buf = buf;
        }
    };

    issue(kt0, 0);
    issue(kt1, 1);
    // Bounded survivor lists: a row whose legal keys outnumber its list slots
    // (a.cap) has its list compacted, out of line, when fewer than kPfRoom
    // slots are left (three settles' worth: the check runs once per two
    // pairs, and the last settle follows the loop).
    auto maybe_compact = [&](int r) __attribute__((always_inline)) {
        const bool aq = r ? act[1] : act[0];
        const int tqr = r ? tq[1] : tq[0];
        PfRow st{r ? cnt[1] : cnt[0], r ? cnt_ge[1] : cnt_ge[0], r ? tau[1] : tau[0],
                 r ? htau[1] : htau[0], r ? tau_f[1] : tau_f[0]};
        if (__builtin_expect(!aq || tqr < a.cap || st.cnt + kPfRoom <= a.cap, 1)) return;
        st = pf_compact(r ? sl[1] : sl[0], r ? h[1] : h[0], st, a.k, a.cap);
        if (r) {
            cnt[1] = st.cnt; cnt_ge[1] = st.ge; tau[1] = st.tau; htau[1] = st.htau; tau_f[1] = st.tau_f;
        } else {
            cnt[0] = st.cnt; cnt_ge[0] = st.ge; tau[0] = st.tau; htau[0] = st.htau; tau_f[0] = st.tau_f;
        }
    };
    for (int tile = 0; tile < ntiles; tile += 4) {
#pragma unroll 1
        for (int r = 0; r < kPfQpw; ++r) maybe_compact(r);
        pair(kt0, kt1, kt2, kt3, tile);
        if (tile + 2 >= ntiles) break;
        pair(kt2, kt3, kt0, kt1, tile + 2);
    }
    // The last pair's g . k stores of all waves complete before it is settled.
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    settle();

    // The key stages are free once every wave is past its last tile and the
    // last (clamped) fills have landed: they hold the candidate buffers, one
    // per wave (two per stage), used by the wave's rows in turn.  Each wave
    // finishes its own rows from the survivor lists it wrote.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll 1
    for (int qq = 0; qq < kPfQpw; ++qq) {
        // One copy of the finish for both rows (selects, not array indexing,
        // keep the per-row values in registers).
        const bool aq = qq ? act[1] : act[0];
        if (!aq) continue;
        const int tqq = qq ? tq[1] : tq[0];
        const long long rq = qq ? rowq[1] : rowq[0];
        const int need = min(a.k, tqq + 1);
        int32_t* oidx = a.out_idx + rq * a.out_stride;
        float* osc = a.out_score ? a.out_score + rq * a.out_stride : nullptr;
        for (int u = need + lane; u < a.k; u += 64) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        const int sq = wid >> 1;
        uint4* stage = sq == 0 ? kt0 : (sq == 1 ? kt1 : (sq == 2 ? kt2 : kt3));
        unsigned long long* cb = reinterpret_cast<unsigned long long*>(stage) + (wid & 1) * kPfCand;
        pf_finish(qq ? h[1] : h[0], cb, qq ? sl[1] : sl[0], qq ? cnt[1] : cnt[0], need, oidx, osc);
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int rows, hipStream_t s) {
    // Even capacity (16-byte list reads); a list shorter than the longest row
    // must leave room for the k kept entries and three settles.
    if (a.cap % 2 != 0) return hipErrorInvalidValue;
    if (a.cap < (long long)a.offset + a.T && a.cap < (long long)a.k + 3 * 2 * kPfTile)
        return hipErrorInvalidValue;
    const int batch = rows / a.T;
    const dim3 grid((unsigned)(((a.T + 7) / 8 + 1) / 2), (unsigned)batch);
    const int nht = (a.H + 15) / 16;
    const dim3 block(64 * kPfWaves);
    if (a.codes) {
        if (!a.kscale) return hipErrorInvalidValue;
        prof_begin(K_PREFILL_FP8, s);
        switch (nht) {
            case 1: sa_launch(prefill_kernel<1, true, false>, grid, block, 0, s, a); break;
            case 2: sa_launch(prefill_kernel<2, true, false>, grid, block, 0, s, a); break;
            case 3: sa_launch(prefill_kernel<3, true, false>, grid, block, 0, s, a); break;
            default: sa_launch(prefill_kernel<4, true, false>, grid, block, 0, s, a); break;
        }
        prof_end(K_PREFILL_FP8, s);
        return hipGetLastError();
    }
    prof_begin(K_PREFILL, s);
    // At most 8 heads (MISA's routed heads, LISA's head rows): two rows per tile.
    if (a.H <= 8) {
        sa_launch(prefill_kernel<1, false, true>, grid, block, 0, s, a);
    } else {
        switch (nht) {
            case 1: sa_launch(prefill_kernel<1, false, false>, grid, block, 0, s, a); break;
            case 2: sa_launch(prefill_kernel<2, false, false>, grid, block, 0, s, a); break;
            case 3: sa_launch(prefill_kernel<3, false, false>, grid, block, 0, s, a); break;
            default: sa_launch(prefill_kernel<4, false, false>, grid, block, 0, s, a); break;
        }
    }
    prof_end(K_PREFILL, s);
    return hipGetLastError();
}

}  // namespace sa
