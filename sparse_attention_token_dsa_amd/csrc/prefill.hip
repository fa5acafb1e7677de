// Fused causal-prefill indexer: q . K contraction on bf16 MFMA, ReLU, the
// w-weighted head sum and the causal mask in the epilogue, and the row's exact
// top-k, in one kernel (PaperTrace, "2.2.2 MISA, LISA and ResMiSA", section
// 2.2: score, causal mask and top-k fused into one pass).
//
// Layout: a workgroup of 4 waves owns 8 consecutive query rows of one
// sequence (two rows per wave, their heads held as MFMA A fragments in
// registers: each B fragment read from LDS feeds both rows) and sweeps the
// legal keys [0, max t] in tiles of 64 keys.  Each tile (16 KiB of bf16 keys)
// is staged once in LDS for all 8 rows by direct global-to-LDS loads, with a
// 16-byte XOR swizzle so the B-fragment reads are free of bank conflicts.
// Column c of MFMA group gi is key 4c + gi, so that after the head sum every
// lane holds the scores of 4 consecutive keys.  Four stages are used in pairs: one wait and one barrier per two tiles, and
// the next pair's loads have two tiles of compute to arrive.
//
// Per tile and row the sweep does no selection work: each legal score is
// added to the row's LDS histogram (bins of 1/8 octave over [2^-32, 2^32);
// zero, negative and smaller scores share bin 0, which is not counted but
// derived at the end, larger ones the last bin) and stored to the row's
// score line in the workspace (4 bytes per legal key, written once and read
// once; one 16-byte non-temporal store per lane per pair of tiles).
//
// Finish: after the sweep each wave selects its rows' exact top-k: the
// histogram gives the bin holding the k-th score; one pass over the row emits
// the scores above it (staged in LDS, written out 64 at a time) and collects
// the ones in it, as 64-bit keys ord(score) << 32 | ~position (ties -> lower
// position), into LDS; a radix select on those keys (9-bit digits) settles
// the rest.  Only when the bin holds more keys than the LDS buffer does a
// digit level re-read the row.
#include <type_traits>

#include "sa_frag.h"

namespace sa {

constexpr int kPfWaves = 4;
constexpr int kPfQpw = 2;  // query rows per wave
constexpr int kPfRows = kPfWaves * kPfQpw;
constexpr int kPfTile = 64;
constexpr int kPfStage = kPfTile * 16;  // uint4 per stage (16 KiB)
constexpr int kPfBins = 512;
constexpr int kPfDigit = 9;  // radix digit of the finish: 2^9 = kPfBins
// A bin is ord(score) >> 20: sign, exponent and 3 mantissa bits.
constexpr int kPfBinShift = 20;
// ord(2^-32) >> 20: prefix of the first inner bin.
constexpr int kPfBase = (int)((0x80000000u | (95u << 23)) >> kPfBinShift);
// Key bits fixed by an inner bin: 63 .. 32 + kPfBinShift.
constexpr int kPfKeyTop = 32 + kPfBinShift;
constexpr int kPfCand = 1024;  // LDS candidate keys per row: two rows per stage
constexpr int kPfSweep = 4;    // float4 per lane per block of the level-0 pass (double-buffered)
static_assert(2 * kPfCand * 8 == kPfStage * 16, "two rows' candidate buffers fill one stage");
static_assert((1 << kPfDigit) == kPfBins, "digit histograms reuse the row histogram");
static_assert(kPfQpw == 2 && kPfTile == 64, "the 4 lane groups store 2 rows x 2 tiles of a pair");

__device__ __forceinline__ int pf_bin(float sc) {
    const int v = (int)(ord_key(sc) >> kPfBinShift) - kPfBase;
    return v < 0 ? 0 : (v > kPfBins - 1 ? kPfBins - 1 : v);
}

// Smallest score in bin b, 1 <= b < kPfBins.
__device__ __forceinline__ float pf_edge(int b) {
    return ord_to_f32((uint32_t)(b + kPfBase) << kPfBinShift);
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

// One pass of a wave over a row's cnt scores: fn(position, score, valid) for
// every lane and element, 4 consecutive scores per lane, 4 loads in flight.
// Rows are padded to a multiple of 4 floats, so the clamped float4 reads stay
// inside the row.  Only rows whose threshold bin is crowded re-read the row.
template <class F>
__device__ __forceinline__ void row_sweep(const float* sr, int cnt, F&& fn) {
    const int lane = lane_id();
    const float4* sr4 = reinterpret_cast<const float4*>(sr);
    const int last4 = (cnt - 1) >> 2;
#pragma unroll 1
    for (int ub = 0; ub < cnt; ub += 1024) {
        float4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = sr4[min((ub >> 2) + j * 64 + lane, last4)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = ub + 4 * (j * 64 + lane);
            fn(u, v[j].x, u < cnt);
            fn(u + 1, v[j].y, u + 1 < cnt);
            fn(u + 2, v[j].z, u + 2 < cnt);
            fn(u + 3, v[j].w, u + 3 < cnt);
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
// histogram of the row's cnt legal scores sr[0, cnt) (bin 0 not counted); cb
// is kPfCand keys of LDS.  Output order is unspecified.
//
// Digit levels narrow the threshold bin down on the key ord(score) << 32 |
// ~position: the keys still in play are those in [lo, hi) whose bits above
// pshift equal pval.  When the bin holds more keys than cb, the level-0 pass
// also counts their next kPfWide-bit digit, in cb used as a histogram, so
// that one more pass settles the bin or shrinks it to LDS size.
constexpr int kPfWide = 11;
static_assert((1 << kPfWide) * 4 == kPfCand * 8, "the wide digit histogram fills cb");

__device__ __forceinline__ void pf_finish(uint32_t* h, unsigned long long* cb, const float* sr,
                                          int cnt, int need, int32_t* oidx, float* osc) {
    const int lane = lane_id();
    const unsigned long long lt = (1ull << lane) - 1ull;
    {
        // The sweep does not count bin 0: it holds the rest of the row.
        int part = 0;
        for (int x = lane; x < kPfBins; x += 64) part += x ? (int)h[x] : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        if (lane == 0) h[0] = (uint32_t)(cnt - part);
    }
    int d0, gt0, eq0;
    wave_threshold<kPfBins>(h, need, d0, gt0, eq0);
    // Bin d0 as a score interval [lo, hi).
    const float lo = d0 == 0 ? -INFINITY : pf_edge(d0);
    const float hi = d0 == kPfBins - 1 ? INFINITY : pf_edge(d0 + 1);
    bool take_all = gt0 + eq0 == need;
    const bool fits = !take_all && eq0 <= kPfCand;
    const bool wide = !take_all && !fits;
    // An inner bin fixes the key bits above kPfKeyTop; the clamped end bins
    // fix nothing.
    const bool clamped = d0 == 0 || d0 == kPfBins - 1;
    int top = clamped ? 64 : kPfKeyTop;
    uint32_t* hw = reinterpret_cast<uint32_t*>(cb);
    if (wide)
        for (int x = lane; x < (1 << kPfWide); x += 64) hw[x] = 0u;

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
    // Level 0, one pass over the row.  The scores to emit or to collect
    // (at or above lo: bin d0 and above, about k + eq0 of them; above hi
    // only when bin d0 is too crowded for cb) are staged as (position, score
    // bits) pairs in a ring in the row histogram (free once d0 is known);
    // whole 64-entry blocks of it are then sent, all lanes busy, to the
    // output (above hi, or all when taking all) or to cb.  A crowded bin's
    // keys are counted into the wide digit histogram where they are met.
    const int wshift = top - kPfWide;
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
        const float4* sr4 = reinterpret_cast<const float4*>(sr);
        const int last4 = (cnt - 1) >> 2;
        constexpr int kStep = 256 * kPfSweep;
        float4 cur[kPfSweep], nxt[kPfSweep];
#pragma unroll
        for (int j = 0; j < kPfSweep; ++j) cur[j] = sr4[min(j * 64 + lane, last4)];
        for (int ub = 0; ub < cnt; ub += kStep) {
            // The next block is in flight while this one is sorted out
            // (clamped: past the end it re-reads the last float4).
#pragma unroll
            for (int j = 0; j < kPfSweep; ++j)
                nxt[j] = sr4[min(((ub + kStep) >> 2) + j * 64 + lane, last4)];
#pragma unroll
            for (int j = 0; j < kPfSweep; ++j) {
                const int u = ub + 4 * (j * 64 + lane);
                const float e4[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool in = u + i < cnt;
                    if (WIDE && in && e4[i] >= lo && e4[i] < hi)
                        lds_add_u32(&hw[(uint32_t)(pf_key(e4[i], u + i) >> wshift) & ((1u << kPfWide) - 1)], 1u);
                    const bool keep = in & (e4[i] >= (WIDE ? hi : lo));
                    const unsigned long long m = __ballot(keep);
                    if (keep)
                        ring[(staged + __popcll(m & lt)) & (kRing - 1)] =
                            make_uint2((uint32_t)(u + i), __float_as_uint(e4[i]));
                    staged += __popcll(m);
                    // At most 63 + 2 x 64 entries pending: the ring holds 256.
                    if (i & 1) drain(false);
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
    {
        drain(true);
    }
    if (take_all) return;

    int need_rem = need - gt0;
    unsigned long long pval = clamped ? 0ull : (unsigned long long)(d0 + kPfBase);
    int pshift = top;
    bool inlds = fits;  // candidates in cb, else re-read the row
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
                row_sweep(sr, cnt, [&](int u, float sc, bool in) {
                    const unsigned long long key = pf_key(sc, u);
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
            row_sweep(sr, cnt, [&](int u, float sc, bool in) {
                const unsigned long long key = pf_key(sc, u);
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

    const int seq = blockIdx.y;
    const int i0 = blockIdx.x * kPfRows;
    const int tid = threadIdx.x;
    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tmax = a.offset + min(i0 + kPfRows, a.T) - 1;
    const int ntiles = tmax / kPfTile + 1;

    // Per-row state of this wave's two rows.
    QFrag<NHT> f[kPfQpw];
    int tq[kPfQpw];
    bool act[kPfQpw];
    long long rowq[kPfQpw];
    float* srow[kPfQpw];
    uint32_t* h[kPfQpw];
#pragma unroll
    for (int qq = 0; qq < kPfQpw; ++qq) {
        const int i = i0 + wid * kPfQpw + qq;
        act[qq] = i < a.T;
        rowq[qq] = (long long)seq * a.T + min(i, a.T - 1);
        tq[qq] = act[qq] ? a.offset + i : -1;
        srow[qq] = a.scores + rowq[qq] * a.stride;
        h[qq] = hist[wid * kPfQpw + qq];
        for (int x = lane; x < kPfBins; x += 64) h[qq][x] = 0u;
        load_qfrag<NHT>(f[qq], a.q + rowq[qq] * a.H * kD, a.w + rowq[qq] * a.H, a.H, nullptr, 0,
                        g, c);
        if (!act[qq]) {
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
                for (int e = 0; e < 4; ++e) f[qq].wv[ht][e] = 0.f;
        }
    }
    const int tw = max(tq[0], tq[kPfQpw - 1]);  // last legal key of this wave

    const uint16_t* kseq = a.keys + (long long)seq * a.L * kD;
    // Stage fill: a wave's load instruction writes 1 KiB of LDS (64 lanes x
    // 16 bytes at consecutive addresses) = 4 key rows, block blk = 4j + wave.
    // Lane l lands at key 4*blk + l/16, slot l%16 of the row, and fetches the
    // chunk that belongs in that slot under the swizzle slot ^ (key/4 % 16),
    // i.e. slot ^ blk.  Tiles past the last are clamped re-reads.
    constexpr int kPfLoads = kPfStage / (64 * kPfWaves);
    auto issue = [&](uint4* stage, int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kPfLoads; ++j) {
            const int blk = kPfWaves * j + wid;
            const int key = 4 * blk + (lane >> 4);
            const int s = min(tile * kPfTile + key, tmax);
            const int chunk = (lane & 15) ^ blk;
            __builtin_amdgcn_global_load_lds(kseq + (long long)s * kD + chunk * 8,
                                             stage + blk * 64, 16, 0, 0);
        }
    };

    // Scores of tile j of a pair: lane (g, c) keeps, for the row and tile of
    // its lane group (row g & 1, tile g >> 1), the scores of keys 4c .. 4c+3
    // (st, stored at the next pair), and adds the score of key 4c + g of each
    // row to that row's histogram.
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
    auto tile_scores = [&](const uint4* ktile, int kbase, int j) __attribute__((always_inline)) {
        float hv[kPfQpw];
#pragma unroll
        for (int qq = 0; qq < kPfQpw; ++qq) hv[qq] = 0.f;
#pragma unroll
        for (int gi = 0; gi < kPfTile / 16; ++gi) {
            uint4 kb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kb[kk] = ktile[(4 * c + gi) * 16 + ((kk * 4 + g) ^ c)];
#pragma unroll
            for (int qq = 0; qq < kPfQpw; ++qq) {
                // One row at a time keeps 16 accumulator registers live; the
                // other wave on the SIMD fills the MFMA pipe meanwhile.
                f32x4 acc[NHT];
                group_dots<NHT, 4>(f[qq], kb, acc);
                float sc = 0.f;
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sc = fmaf(f[qq].wv[ht][e], fmaxf(acc[ht][e], 0.f), sc);
                sc = sum_lane_groups(sc);
                hv[qq] = g == gi ? sc : hv[qq];
                st[gi] = g == 2 * j + qq ? sc : st[gi];
            }
        }
        const int s = kbase + 4 * c + g;
#pragma unroll
        for (int qq = 0; qq < kPfQpw; ++qq) {
            // Positive scores only: bin = (float bits >> 20) - 760 there.
            const int v = (int)(__float_as_uint(hv[qq]) >> kPfBinShift) - (kPfBase - 2048);
            if (s <= tq[qq] && hv[qq] > 0.f && v > 0) lds_add_u32(&h[qq][min(v, kPfBins - 1)], 1u);
        }
    };

    // A pair's scores are stored at the top of the next pair, right after its
    // stage wait, so the stores have two tiles of compute to complete before
    // the next wait (which counts them too) comes round.  Keys past the row's
    // last legal one inside its last tile are stored too (the line has room
    // up to the next multiple of 64) and never read.
    int pend_base = -1;
    auto put = [&]() __attribute__((always_inline)) {
        if (pend_base < 0) return;
        const int qs = g & 1;
        const int kb0 = pend_base + (g >> 1) * kPfTile;
        if (kb0 <= (qs ? tq[1] : tq[0]))
            __builtin_nontemporal_store(st, reinterpret_cast<f32x4*>((qs ? srow[1] : srow[0]) + kb0 + 4 * c));
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
        put();
        const int kbase = tile * kPfTile;
        if (kbase <= tw) {
            tile_scores(ka, kbase, 0);
            if (kbase + kPfTile <= tw) tile_scores(kb, kbase + kPfTile, 1);
            pend_base = kbase;  // keys past tw are never stored
        }
    };

    issue(kt0, 0);
    issue(kt1, 1);
    for (int tile = 0; tile < ntiles; tile += 4) {
        pair(kt0, kt1, kt2, kt3, tile);
        if (tile + 2 >= ntiles) break;
        pair(kt2, kt3, kt0, kt1, tile + 2);
    }
    put();

    // The key stages are free once every wave is past its last tile and the
    // last (clamped) fills have landed: they hold the candidate buffers, two
    // rows per stage.  Each wave finishes its own rows from the score lines
    // it wrote.
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
        uint4* stage = wid == 0 ? kt0 : (wid == 1 ? kt1 : (wid == 2 ? kt2 : kt3));
        unsigned long long* cb = reinterpret_cast<unsigned long long*>(stage) + qq * kPfCand;
        pf_finish(qq ? h[1] : h[0], cb, qq ? srow[1] : srow[0], tqq + 1, need, oidx, osc);
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int rows, hipStream_t s) {
    if (a.stride % 64 != 0 || a.stride < (long long)a.offset + a.T) return hipErrorInvalidValue;
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
