// Fused causal-prefill indexer: q . K contraction on bf16 MFMA, ReLU, the
// w-weighted head sum and the causal mask in the epilogue, a streaming per-row
// threshold and the row's exact top-k, in one kernel (PaperTrace, "2.2.2
// MISA, LISA and ResMiSA", section 2.2: score, causal mask and top-k fused
// into one pass, no n^2 score matrix written back).
//
// Layout: a workgroup of 16 waves owns 16 consecutive query rows of one
// sequence, one row per wave (the row's heads held as MFMA A fragments in
// registers; 1024 threads keep each wave within 128 registers, so every SIMD
// runs 4 waves and their epilogue VALU work interleaves with the others'
// MFMAs), and sweeps the legal keys [0, max t] in tiles of 64 keys.  Each
// tile (16 KiB of bf16 keys) is staged once in LDS for all 16 rows by direct
// global-to-LDS loads, with a 16-byte XOR swizzle so the B-fragment reads are
// free of bank conflicts.  Column c of MFMA group gi is key 4c + gi, so that
// after the head sum every lane holds the scores of consecutive keys.  Four
// stages are used in pairs: one wait and one barrier per two tiles, and the
// next pair's loads have two tiles of compute to arrive.
//
// Streaming threshold: each row keeps an LDS histogram of the scores it has
// kept, over the bins below (monotone in the score).  tau is the highest bin
// such that at least k kept scores lie in bins >= tau; a new score below bin
// tau has k larger ones ahead of it and can never enter the row's top-k, so
// it is dropped with one compare.  The rest (about k (1 + ln(n / k)) per row
// for n keys in random order) are appended as (position, score) pairs to the
// row's survivor list in the workspace; the scores themselves never leave the
// chip.  The count of bin tau is mirrored in a register, so tau is re-derived
// from the histogram only when it can move.
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

constexpr int kPfWaves = 16;
constexpr int kPfRows = kPfWaves;       // one query row per wave
constexpr int kPfTile = 64;
constexpr int kPfStage = kPfTile * 16;  // uint4 per stage (16 KiB)
constexpr int kPfBins = 1024;           // histogram size (bins 947 .. 1023 stay empty)
constexpr int kPfDigit = 10;            // radix digit of the finish over LDS candidates
constexpr int kPfWide = 10;             // digit counted in the level-0 pass for crowded bins
constexpr int kPfCand = 512;            // LDS candidate keys per row: four rows per stage
constexpr int kPfSweep = 4;             // uint4 per lane per block of the level-0 pass
static_assert(4 * kPfCand * 8 == kPfStage * 16, "four rows' candidate buffers fill one stage");
static_assert((1 << kPfDigit) == kPfBins, "digit histograms reuse the row histogram");
static_assert((1 << kPfWide) * 4 == kPfCand * 8, "the wide digit histogram fills cb");
static_assert(kPfStage == 64 * kPfWaves, "one 16-byte load per thread fills a stage");

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
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    int cum = incl - local;
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
    d = __shfl(fd, src);
    gt = __shfl(fg, src);
    eq = __shfl(fe, src);
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

template <int NHT>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_kernel(PrefillArgs a) {
    // The stages are four distinct LDS objects: the compiler then tracks the
    // direct-to-LDS loads per object and places no wait of its own for the
    // pair in flight before reads of the other pair.
    __shared__ uint4 kt0[kPfStage], kt1[kPfStage], kt2[kPfStage], kt3[kPfStage];
    __shared__ uint32_t hist[kPfRows][kPfBins];
    __shared__ float4 wts[kPfRows][kMaxH / 4];  // each row's w (zero past H)

    const int seq = blockIdx.y;
    const int i0 = blockIdx.x * kPfRows;
    const int tid = threadIdx.x;
    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const unsigned long long lt = (1ull << lane) - 1ull;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tmax = a.offset + min(i0 + kPfRows, a.T) - 1;
    const int ntiles = tmax / kPfTile + 1;

    // This wave's row.
    const int i = i0 + wid;
    const bool act = i < a.T;
    const long long rowq = (long long)seq * a.T + min(i, a.T - 1);
    const int tq = act ? a.offset + i : -1;  // last legal key (-1: no row)
    uint2* const sl = a.surv + rowq * a.cap;
    uint32_t* const h = hist[wid];
    for (int x = lane; x < kPfBins; x += 64) h[x] = 0u;
    QFrag<NHT> f;  // A fragments only: the epilogue reads w from LDS, which
                   // keeps the wave within 128 registers
    load_qfrag<NHT>(f, a.q + rowq * a.H * kD, a.w + rowq * a.H, a.H, nullptr, 0, g, c);
    reinterpret_cast<float*>(wts[wid])[lane] = act && lane < a.H ? a.w[rowq * a.H + lane] : 0.f;
    int tau = 0, cnt = 0, cnt_ge = 0, htau = 0;
    float tau_f = -INFINITY;

    const uint16_t* kseq = a.keys + (long long)seq * a.L * kD;
    // Stage fill: each wave's load instruction writes 1 KiB of LDS (64 lanes x
    // 16 bytes at consecutive addresses) = 4 key rows, block = wave.  Lane l
    // lands at key 4*wave + l/16, slot l%16 of the row, and fetches the chunk
    // that belongs in that slot under the swizzle slot ^ (key/4 % 16), i.e.
    // slot ^ wave.  Tiles past the last are clamped re-reads.
    auto issue = [&](uint4* stage, int tile) __attribute__((always_inline)) {
        const int key = 4 * wid + (lane >> 4);
        const int s = min(tile * kPfTile + key, tmax);
        const int chunk = (lane & 15) ^ wid;
        __builtin_amdgcn_global_load_lds(kseq + (long long)s * kD + chunk * 8, stage + wid * 64,
                                         16, 0, 0);
    };

    // Scores of tile j of a pair.  After the head sum every lane holds the
    // score of key 4c + gi of group gi; lane group g keeps those of tile
    // g >> 1, keys 4c + 2 (g & 1) and 4c + 2 (g & 1) + 1, in st.
    float st[2] = {0.f, 0.f};
    auto tile_scores = [&](const uint4* ktile, int j) __attribute__((always_inline)) {
#pragma unroll
        for (int gi = 0; gi < kPfTile / 16; ++gi) {
            uint4 kb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kb[kk] = ktile[(4 * c + gi) * 16 + ((kk * 4 + g) ^ c)];
            f32x4 acc[NHT];
            group_dots<NHT, 4>(f, kb, acc);
            // Compiler-only barrier: w is read again from LDS for each group
            // instead of being kept live in 16 registers across the tiles.
            asm volatile("" ::: "memory");
            float sc = 0.f;
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                // Heads 16 ht + 4 g + e of accumulator element e (one 16-byte
                // LDS read, shared by the 16 lanes of the group).
                const float4 w4 = wts[wid][4 * ht + g];
                sc = fmaf(w4.x, fmaxf(acc[ht][0], 0.f), sc);
                sc = fmaf(w4.y, fmaxf(acc[ht][1], 0.f), sc);
                sc = fmaf(w4.z, fmaxf(acc[ht][2], 0.f), sc);
                sc = fmaf(w4.w, fmaxf(acc[ht][3], 0.f), sc);
            }
            sc = sum_lane_groups(sc);
            st[gi & 1] = g == 2 * j + (gi >> 1) ? sc : st[gi & 1];
        }
    };

    // Raise tau while the bins at and above tau + 1 still hold k kept scores
    // (this wave's histogram adds are in LDS order before these reads).
    auto raise = [&]() {
        int t = tau, ge = cnt_ge, ht;
        for (;;) {
            const int bb = t + lane;
            const int hv = bb < kPfBins ? (int)h[bb] : 0;
            int incl = hv;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (lane >= off) incl += y;
            }
            const int excl = incl - hv;
            const bool ok = bb < kPfBins && ge - excl >= a.k;
            const int lstar = __popcll(__ballot(ok)) - 1;
            t += lstar;
            ge -= __shfl(excl, lstar);
            if (lstar < 63 || t >= kPfBins - 1) {
                ht = __shfl(hv, lstar);
                break;
            }
        }
        // Wave-uniform: keep them in scalar registers.
        tau = __builtin_amdgcn_readfirstlane(t);
        cnt_ge = __builtin_amdgcn_readfirstlane(ge);
        htau = __builtin_amdgcn_readfirstlane(ht);
        tau_f = pf_lo(tau);
    };

    // A pair's scores are settled at the top of the next pair, right after its
    // stage wait: each lane tests its 2 scores against the row's threshold,
    // appends the survivors to the row's list (positions from a prefix count
    // over the wave) and to its histogram, and tau moves when it can.  The
    // list stores then have two tiles of compute to complete before the next
    // wait (which counts them too) comes round.
    int pend_base = -1;
    auto settle = [&]() __attribute__((always_inline)) {
        if (pend_base < 0) return;
        const int key0 = pend_base + (g >> 1) * kPfTile + 4 * c + 2 * (g & 1);
        bool sv[2];
        int bn[2];
        int n = 0, nt = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            sv[e] = key0 + e <= tq && st[e] >= tau_f;
            bn[e] = pf_bin(st[e]);
            n += sv[e];
            nt += sv[e] && bn[e] == tau;
        }
        const unsigned long long b0 = __ballot(n & 1), b1 = __ballot(n & 2);
        int p = cnt + __popcll(b0 & lt) + 2 * __popcll(b1 & lt);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (sv[e]) {
                sl[p] = make_uint2((uint32_t)(key0 + e), __float_as_uint(st[e]));
                lds_add_u32(&h[bn[e]], 1u);
            }
            p += sv[e];
        }
        const unsigned long long t0 = __ballot(nt & 1), t1 = __ballot(nt & 2);
        const int tot = __popcll(b0) + 2 * __popcll(b1);
        cnt += tot;
        cnt_ge += tot;
        htau += __popcll(t0) + 2 * __popcll(t1);
        if (cnt_ge - htau >= a.k) raise();
        pend_base = -1;
    };

    // One barrier per pair: after it, the pair's data is visible to all and
    // every wave is done with the other pair's stages, which are refilled
    // right away.
    auto pair = [&](const uint4* ka, const uint4* kb, uint4* na, uint4* nb, int tile)
                    __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        issue(na, tile + 2);
        issue(nb, tile + 3);
        settle();
        const int kbase = tile * kPfTile;
        if (kbase <= tq) {
            tile_scores(ka, 0);
            if (kbase + kPfTile <= tq) tile_scores(kb, 1);
            pend_base = kbase;  // keys past the row's last legal one are never kept
        }
    };

    issue(kt0, 0);
    issue(kt1, 1);
    for (int tile = 0; tile < ntiles; tile += 4) {
        pair(kt0, kt1, kt2, kt3, tile);
        if (tile + 2 >= ntiles) break;
        pair(kt2, kt3, kt0, kt1, tile + 2);
    }
    settle();

    // The key stages are free once every wave is past its last tile and the
    // last (clamped) fills have landed: they hold the candidate buffers, four
    // rows per stage.  Each wave finishes its own row from the survivor list
    // it wrote.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!act) return;
    const int need = min(a.k, tq + 1);
    int32_t* oidx = a.out_idx + rowq * a.out_stride;
    float* osc = a.out_score ? a.out_score + rowq * a.out_stride : nullptr;
    for (int u = need + lane; u < a.k; u += 64) {
        oidx[u] = -1;
        if (osc) osc[u] = -INFINITY;
    }
    const int sq = wid >> 2;
    uint4* stage = sq == 0 ? kt0 : (sq == 1 ? kt1 : (sq == 2 ? kt2 : kt3));
    unsigned long long* cb = reinterpret_cast<unsigned long long*>(stage) + (wid & 3) * kPfCand;
    pf_finish(h, cb, sl, cnt, need, oidx, osc);
}

hipError_t launch_prefill(const PrefillArgs& a, int rows, hipStream_t s) {
    if (a.cap % 2 != 0 || a.cap < (long long)a.offset + a.T) return hipErrorInvalidValue;
    const int batch = rows / a.T;
    const dim3 grid((unsigned)((a.T + kPfRows - 1) / kPfRows), (unsigned)batch);
    const int nht = (a.H + 15) / 16;
    prof_begin(K_PREFILL, s);
    switch (nht) {
        case 1: prefill_kernel<1><<<grid, dim3(64 * kPfWaves), 0, s>>>(a); break;
        case 2: prefill_kernel<2><<<grid, dim3(64 * kPfWaves), 0, s>>>(a); break;
        case 3: prefill_kernel<3><<<grid, dim3(64 * kPfWaves), 0, s>>>(a); break;
        default: prefill_kernel<4><<<grid, dim3(64 * kPfWaves), 0, s>>>(a); break;
    }
    prof_end(K_PREFILL, s);
    return hipGetLastError();
}

}  // namespace sa
