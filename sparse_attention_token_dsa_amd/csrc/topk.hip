// Per-row exact top-k by radix select (PaperTrace, "2.2.2 MISA, LISA and
// ResMiSA", section 2.2: score, causal mask and top-k belong together; the
// top-k is a cost of its own that does not shrink with the head count).
//
// Every candidate becomes the 64-bit key  ord(score) << 32 | ~index : larger
// scores win and, among equal scores, the lower index wins.  Keys are
// distinct, so the selection is exact.  Each level sorts the keys still in
// play into bins by a map that never decreases along the key order: a
// histogram, a scan from the top that finds the bin holding the k-th key,
// and one pass that emits every key above it and keeps the keys in it for
// the next level.  The filter and the select's general path take fixed
// digits of the key from the top (12/10/10 bits of the score, then 12/10/10
// of the index, only reached on exact score ties); the select's register
// path fits its bins to the range of the keys in play.
//
// Two kernels:
//  * topk_filter_kernel -- long dense score rows (decode scans).  The first
//    digit's histogram was built by the score kernel; many workgroups per row
//    each find the first-digit threshold and sweep a slice of the row,
//    emitting sure winners and appending threshold-digit keys to a per-row
//    candidate array in the workspace.
//  * topk_select_kernel -- one 1024-thread workgroup per row for everything
//    else: candidate arrays left by the filter, short dense rows (block
//    scores) and (score, index) lists (rescored pools, prefill survivors).
//    Sources of at most 8192 keys are held in registers, with bins fitted
//    to the range of the keys in play (below); for larger ones, candidates
//    of later digits are compacted into LDS when they fit, and if not, the
//    source is rescanned with a prefix filter.
#include "sa_select.h"

namespace sa {

constexpr int kTopkThreads = 1024;
constexpr int kFilterThreads = 512;
// Dense elements per filter workgroup: 16 per thread.  Larger chunks mean
// fewer workgroups re-reading the row histogram (8192: 8.1 us for the 8 x 128K
// decode rows against 10.8 us at 4096).
constexpr int kFilterChunk = 8192;
constexpr int kLdsCand = 4096;           // keys per LDS candidate buffer
// Rows per CU from which the select runs 512 threads per row (16 keys per
// thread, half-size LDS buffers, 4 waves per SIMD at 128 VGPRs: two rows per
// CU at once) instead of 1024 (one row per CU, shorter per row).
constexpr int kManyRows = 2;
constexpr int kBatch = 8;                // keys per thread in flight in a pass over a source

__device__ __forceinline__ unsigned long long make_key(float sc, int idx) {
    return ((unsigned long long)ord_key(sc) << 32) | (unsigned long long)(~(uint32_t)idx);
}
__device__ __forceinline__ int key_idx(unsigned long long k) { return (int)(~(uint32_t)k); }
__device__ __forceinline__ float key_score(unsigned long long k) {
    return ord_to_f32((uint32_t)(k >> 32));
}

__constant__ int kShift[6] = {52, 42, 32, 20, 10, 0};
__constant__ int kWidth[6] = {12, 10, 10, 12, 10, 10};

__device__ __forceinline__ int dense_len(const TopkArgs& a, int row) {
    const int t = row_pos(row, a.T, a.offset, a.seq_lens, a.len_cap);
    const int n = t / a.len_div + 1;
    return n < a.len_cap ? n : a.len_cap;
}

// ------------------------------------------------------------ filter

// The scan left, per row, the histogram of the scores' first digit.  Each
// workgroup finds the digit d holding the row's k-th score from it, sweeps
// kFilterChunk scores (float4 loads, the row stride is a multiple of 64),
// stages its winners (digit > d, or = d when those fit exactly) and its
// candidates (digit = d) in LDS, reserves its output ranges with one atomic
// each and copies them out.  The first workgroup of the row also records d,
// the count above it and the count on it for the finishing kernel.
__global__ __launch_bounds__(kFilterThreads) void topk_filter_kernel(TopkArgs a,
                                                                     unsigned long long* cand) {
    // Winners (from the front) and candidates (from the back) staged as keys
    // in one buffer: each score is at most one of them.  64 KiB, so the
    // filter fits beside a key scan's workgroup on the same CU.
    __shared__ unsigned long long s_buf[kFilterChunk];
    __shared__ int s_ne, s_nc, s_base[2];
    __shared__ int s_wave[kFilterThreads / 64];
    __shared__ Thresh th;
    const int row = blockIdx.y;
    const int tid = threadIdx.x;
    const int n = dense_len(a, row);
    const int lo = blockIdx.x * kFilterChunk;
    if (lo >= n) return;
    const int hi = min(lo + kFilterChunk, n);
    // The slice's scores are loaded first: they do not depend on the
    // threshold, so their latency overlaps the histogram's.
    const float* src = a.dense + (long long)row * a.dense_stride;
    constexpr int kPer = kFilterChunk / kFilterThreads;  // scores per thread
    static_assert(kPer % 4 == 0 && kPer <= 32, "float4 loads; one bit per score in a mask");
    float vs[kPer];
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
        const int u0 = lo + (tid + i * kFilterThreads) * 4;
        float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (u0 < hi) v4 = *reinterpret_cast<const float4*>(src + u0);
        vs[4 * i] = v4.x;
        vs[4 * i + 1] = v4.y;
        vs[4 * i + 2] = v4.z;
        vs[4 * i + 3] = v4.w;
    }
    uint32_t* hist = reinterpret_cast<uint32_t*>(s_buf);  // 16 KiB, reused below
    const uint32_t* grow = a.state + (long long)row * kRowState;
    for (int x = tid; x < kHist0Bins; x += kFilterThreads) hist[x] = grow[x];
    lds_barrier();
    const int need = min(a.k, n);
    find_threshold<kFilterThreads>(hist, kHist0Bins, need, s_wave, &th);
    int* ctl = reinterpret_cast<int*>(a.state + (long long)row * kRowState + kHist0Bins);
    const uint32_t d = (uint32_t)th.dstar;
    const bool take_all = th.gt + th.eq == need;
    if (blockIdx.x == 0 && tid == 0) {
        ctl[CTL_NEED] = need;
        ctl[CTL_DIGIT] = th.dstar;
        ctl[CTL_GT] = th.gt;
        ctl[CTL_EQ] = th.eq;
    }
    if (tid == 0) {
        s_ne = 0;
        s_nc = 0;
    }
    lds_barrier();
    // Each thread classifies its kPer scores (float4 loads, all issued first),
    // then one wave-level prefix sum of its (emit, candidate) counts and one
    // LDS atomic per wave and kind give it its staging slots.
    uint32_t emask = 0u, cmask = 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int u = lo + (tid + (j >> 2) * kFilterThreads) * 4 + (j & 3);
        const bool in = u < hi;
        const uint32_t dig = ord_key(vs[j]) >> (32 - kHist0Bits);
        if (in && (dig > d || (take_all && dig == d))) emask |= 1u << j;
        if (in && !take_all && dig == d) cmask |= 1u << j;
    }
    const int lane = lane_id();
    const int mine = __popc(emask) | (__popc(cmask) << 16);
    const int incl = wave_incl_scan(mine);
    int wbase = 0;
    if (lane == 63) {
        const int te = incl & 0xffff, tc = incl >> 16;
        const int be = te ? atomicAdd(&s_ne, te) : 0;
        const int bc = tc ? atomicAdd(&s_nc, tc) : 0;
        wbase = be | (bc << 16);
    }
    wbase = __builtin_amdgcn_readlane(wbase, 63);
    const int excl = incl - mine;
    int se = (wbase & 0xffff) + (excl & 0xffff);
    int sc2 = (wbase >> 16) + (excl >> 16);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int u = lo + (tid + (j >> 2) * kFilterThreads) * 4 + (j & 3);
        if (emask & (1u << j)) s_buf[se++] = make_key(vs[j], u);
        if (cmask & (1u << j)) s_buf[kFilterChunk - 1 - sc2++] = make_key(vs[j], u);
    }
    lds_barrier();
    if (tid == 0) {
        s_base[0] = s_ne ? atomicAdd(&ctl[CTL_EMITTED], s_ne) : 0;
        s_base[1] = s_nc ? atomicAdd(&ctl[CTL_CANDS], s_nc) : 0;
    }
    lds_barrier();
    int32_t* oidx = a.out_idx + (long long)row * a.out_stride;
    float* osc = a.out_score ? a.out_score + (long long)row * a.out_stride : nullptr;
    for (int x = tid; x < s_ne; x += kFilterThreads) {
        const int slot = s_base[0] + x;
        if (slot < need) {
            const unsigned long long key = s_buf[x];
            oidx[slot] = key_idx(key);
            if (osc) osc[slot] = key_score(key);
        }
    }
    unsigned long long* crow = cand + (long long)row * a.cand_cap;
    for (int x = tid; x < s_nc; x += kFilterThreads) {
        const long long cs = (long long)s_base[1] + x;
        if (cs < a.cand_cap) crow[cs] = s_buf[kFilterChunk - 1 - x];
    }
}

// ------------------------------------------------------------ select

enum SrcKind { SRC_DENSE = 0, SRC_LIST = 1, SRC_KEYS = 2 };

template <int NT, int LC>
struct SelShared {
    alignas(16) uint32_t hist[kHist0Bins];
    unsigned long long lbuf[2][LC];
    int wave[NT / 64];
    uint32_t wr[4 * (NT / 64)];  // per-wave ranges, by field then wave
    Thresh th;
    int out, cand;
};

__device__ __forceinline__ unsigned long long src_key(int kind, const float* dsrc,
                                                      const float* lsc, const int32_t* lid,
                                                      const unsigned long long* ksrc, int u,
                                                      bool& valid) {
    if (kind == SRC_DENSE) return make_key(dsrc[u], u);
    if (kind == SRC_KEYS) return ksrc[u];
    const int id = lid[u];
    valid = valid && id >= 0;
    return make_key(lsc[u], id);
}

// Sources of at most kSelMax keys (rescored lists, block score
// rows, the filter's candidates): every key is loaded once into registers,
// all loads in flight together, and the selection runs on the registers.
// Each level sorts the keys still in play into at most kSelBins bins by a
// map that never decreases along the key order, finds the bin that holds the
// need-th largest key, emits the keys above it and keeps the keys in it.  The
// map comes from the range of the keys in play: while their scores differ,
// equal slices of the [min, max] score interval (a fixed radix digit of the
// ordered bits follows the float exponent and puts most scores of a narrow
// band into one bin); once a slicing level keeps more than half its keys, or
// the interval is not a usable float range, radix digits of the ordered score
// bits above the smallest; once the scores are all equal, radix digits of the
// index part.  When at most kRankMax keys remain, each is placed by its exact
// rank among them (a cost that grows with the square of their number).
constexpr int kSelMax = 8192;  // keys of a row the register-resident path holds
constexpr int kRankMax = 256;
constexpr int kSelBins = 1024;

// Wave 0 finds the bin of a kSelBins-bin histogram (16-byte aligned; bins
// above the map's range hold zero) that holds the need-th largest key,
// scanning from the top, into *out.  Each lane takes 16 adjacent bins in
// four 16-byte reads, all in flight together.  One barrier, after which
// every thread reads *out.
__device__ __forceinline__ void wave0_threshold(const uint32_t* hist, int need, Thresh* out) {
    static_assert(kSelBins == 64 * 16, "16 bins per lane of wave 0");
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int base = kSelBins - 16 - 16 * lane;  // lane 0 takes the top bins
        const uint4* hp = reinterpret_cast<const uint4*>(hist + base);
        uint32_t v[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 x = hp[c];
            v[4 * c] = x.x;
            v[4 * c + 1] = x.y;
            v[4 * c + 2] = x.z;
            v[4 * c + 3] = x.w;
        }
        int local = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) local += (int)v[j];
        int cum = wave_incl_scan(local) - local;
#pragma unroll
        for (int j = 15; j >= 0; --j) {
            const int h = (int)v[j];
            if (cum < need && need <= cum + h) {
                out->dstar = base + j;
                out->gt = cum;
                out->eq = h;
            }
            cum += h;
        }
    }
    lds_barrier();
}

// Largest value over the wave, in every lane (identity 0).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    const auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Each wave publishes the range of its keys in play (score order bits and
// index part, as maxima of the value and of its complement) and their count;
// read_range takes them after the next barrier.
template <int NT, int NK, class SS>
__device__ __forceinline__ void publish_range(const unsigned long long* kr, uint32_t alive,
                                              SS& S) {
    uint32_t omax = 0u, oinv = 0u, lmax = 0u, linv = 0u;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NK; ++j)
        if ((alive >> j) & 1u) {
            const uint32_t o = (uint32_t)(kr[j] >> 32), l = (uint32_t)kr[j];
            omax = o > omax ? o : omax;
            oinv = ~o > oinv ? ~o : oinv;
            lmax = l > lmax ? l : lmax;
            linv = ~l > linv ? ~l : linv;
            ++cnt;
        }
    omax = wave_max_u32(omax);
    oinv = wave_max_u32(oinv);
    lmax = wave_max_u32(lmax);
    linv = wave_max_u32(linv);
    cnt = __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
    if (lane_id() == 0) {
        constexpr int NW = NT / 64;
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
        S.wr[w] = omax;
        S.wr[NW + w] = oinv;
        S.wr[2 * NW + w] = lmax;
        S.wr[3 * NW + w] = linv;
        S.wave[w] = cnt;
    }
}

// Block-wide range of the keys in play, as wave-uniform values: lane l reads
// word l of the 4 x NW per-wave ranges (field l / NW, wave l % NW; one 4-byte
// read per lane rather than every thread reading them all), and each run of
// NW lanes takes its maximum with DPP row shifts.
template <int NW, class SS>
__device__ __forceinline__ void read_range(const SS& S, uint32_t& omax, uint32_t& oinv,
                                           uint32_t& lmax, uint32_t& linv) {
    static_assert(NW == 16 || NW == 8, "runs of 16 or 8 lanes per field");
    const auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    uint32_t x = lane_id() < 4 * NW ? S.wr[lane_id()] : 0u;
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));
    x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));
    if constexpr (NW == 16)
        x = mx(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));
    omax = (uint32_t)__builtin_amdgcn_readlane((int)x, NW - 1);
    oinv = (uint32_t)__builtin_amdgcn_readlane((int)x, 2 * NW - 1);
    lmax = (uint32_t)__builtin_amdgcn_readlane((int)x, 3 * NW - 1);
    linv = (uint32_t)__builtin_amdgcn_readlane((int)x, 4 * NW - 1);
}

template <int NT, class SS>
__device__ __forceinline__ void select_in_registers(const TopkArgs& a, int kind,
                                                    const float* dsrc, const float* lsc,
                                                    const int32_t* lid,
                                                    const unsigned long long* ksrc, int nsrc,
                                                    int32_t* oidx, float* osc, SS& S,
                                                    const unsigned long long* pre = nullptr,
                                                    const int* pctl = nullptr) {
    constexpr int NK = kSelMax / NT;  // keys per thread
    const int tid = threadIdx.x, lane = lane_id();
    const int row = blockIdx.x;
    unsigned long long kr[NK];
    uint32_t alive = 0u;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int u = tid + j * NT;
        bool valid = u < nsrc;
        if (pre)
            kr[j] = valid ? pre[j] : 0ull;  // loaded by the caller
        else
            kr[j] = valid ? src_key(kind, dsrc, lsc, lid, ksrc, u, valid) : 0ull;
        if (valid) alive |= 1u << j;
    }
    int need = 0, need_rem = 0;
    if (kind == SRC_KEYS) {
        // continue after the filter: its winners are written, its
        // candidates are the keys on the row's first-digit threshold
        const int* ctl = pctl ? pctl
                              : reinterpret_cast<const int*>(a.state + (long long)row * kRowState +
                                                             kHist0Bins);
        need = ctl[CTL_NEED];
        const int gt = ctl[CTL_GT];
        for (int u = need + tid; u < a.k; u += NT) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        if (gt + ctl[CTL_EQ] == need) return;  // the filter emitted everything
        need_rem = need - gt;
        if (tid == 0) S.out = gt;
    } else if (tid == 0) {
        S.out = 0;
    }
    publish_range<NT, NK>(kr, alive, S);
    // the first level's bins (two kSelBins halves of S.hist alternate)
    for (int x = tid; x < kSelBins; x += NT) S.hist[x] = 0u;
    lds_barrier();
    int nalive = lane < NT / 64 ? S.wave[lane] : 0;
    nalive = __builtin_amdgcn_readlane(wave_incl_scan(nalive), 63);
    if (kind != SRC_KEYS) {
        need = min(a.k, nalive);
        for (int u = need + tid; u < a.k; u += NT) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        if (need <= 0) return;
        need_rem = need;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    uint32_t* hcur = S.hist;
    uint32_t* hnext = S.hist + kSelBins;
    bool slice_ok = true;
    for (;;) {
        uint32_t omax, oinv, lmax, linv;
        read_range<NT / 64>(S, omax, oinv, lmax, linv);
        const uint32_t omin = ~oinv, lmin = ~linv;
        // this level's map (uniform over the block)
        int mode;  // 0: score slices, 1: score-bit radix, 2: index-bit radix
        float fmin = 0.f, inv = 0.f;
        uint32_t base = 0u;
        int shift = 0, nbins = kSelBins;
        if (omax != omin) {
            fmin = ord_to_f32(omin);
            const float range = ord_to_f32(omax) - fmin;
            const uint32_t rb = __float_as_uint(range);
            // finite ends, and a range that is finite and not tiny (so that
            // kSelBins / range is finite)
            mode = (slice_ok && omin >= 0x00800000u && omax < 0xff800000u &&
                    rb >= 0x0da24260u /* 1e-30f */ && rb < 0x7f800000u)
                       ? 0
                       : 1;
            if (mode == 0) {
                inv = (float)kSelBins / range;
            } else {
                base = omin;
                const uint32_t span = omax - omin;
                const int bits = 32 - __clz(span);
                shift = bits > 10 ? bits - 10 : 0;
                nbins = (int)(span >> shift) + 1;
            }
        } else {
            mode = 2;
            base = lmin;
            const uint32_t span = lmax - lmin;
            const int bits = span ? 32 - __clz(span) : 0;
            shift = bits > 10 ? bits - 10 : 0;
            nbins = (int)(span >> shift) + 1;
        }
        // (recomputed where used rather than held in registers)
        auto digit = [&](int j) {
            if (mode == 0) {
                // monotone: a rounded difference, a rounded product, truncation
                const int d = (int)((key_score(kr[j]) - fmin) * inv);
                return (uint32_t)min(max(d, 0), kSelBins - 1);
            }
            const uint32_t v = mode == 1 ? (uint32_t)(kr[j] >> 32) : (uint32_t)kr[j];
            return (v - base) >> shift;
        };
#pragma unroll
        for (int j = 0; j < NK; ++j)
            if ((alive >> j) & 1u) atomicAdd(&hcur[digit(j)], 1u);
        lds_barrier();
        wave0_threshold(hcur, need_rem, &S.th);
        const uint32_t d = (uint32_t)S.th.dstar;
        const int gt = S.th.gt;
        const int eq = S.th.eq;
        // (one bin: every key in play is the same key, any of them will do)
        const bool take_all = gt + eq == need_rem || nbins == 1;
        // winners of this level: one LDS atomic per wave for all its keys
        // (the ballots are taken twice rather than held)
        auto emits = [&](int j) {
            const uint32_t g = digit(j);
            return ((alive >> j) & 1u) && (g > d || (take_all && g == d));
        };
        int wtot = 0;
#pragma unroll
        for (int j = 0; j < NK; ++j) wtot += __popcll(__ballot(emits(j)));
        int obase = 0;
        if (wtot) {
            if (lane == 0) obase = atomicAdd(&S.out, wtot);
            obase = __builtin_amdgcn_readlane(obase, 0);
        }
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const bool e = emits(j);
            const unsigned long long m = __ballot(e);
            if (e) {
                const int slot = obase + __popcll(m & below);
                if (slot < need) {
                    oidx[slot] = key_idx(kr[j]);
                    if (osc) osc[slot] = key_score(kr[j]);
                }
            }
            obase += __popcll(m);
        }
        // keys on the threshold bin stay in play
#pragma unroll
        for (int j = 0; j < NK; ++j)
            if (digit(j) != d) alive &= ~(1u << j);
        need_rem -= gt;
        if (take_all) return;
        if (eq <= kRankMax) {
            // Few keys left: compact them into LDS and place each by its
            // rank among them (keys are distinct).
            if (tid == 0) S.cand = 0;
            lds_barrier();
            int ctot = 0;
#pragma unroll
            for (int j = 0; j < NK; ++j) ctot += __popcll(__ballot((alive >> j) & 1u));
            int cbase = 0;
            if (ctot) {
                if (lane == 0) cbase = atomicAdd(&S.cand, ctot);
                cbase = __builtin_amdgcn_readlane(cbase, 0);
            }
#pragma unroll
            for (int j = 0; j < NK; ++j) {
                const bool al = (alive >> j) & 1u;
                const unsigned long long cm = __ballot(al);
                if (al) S.lbuf[0][cbase + __popcll(cm & below)] = kr[j];
                cbase += __popcll(cm);
            }
            lds_barrier();
            const int done = need - need_rem;  // winners already written
            for (int c = tid; c < eq; c += NT) {
                const unsigned long long key = S.lbuf[0][c];
                int rank = 0;
                int o = 0;
                for (; o + 4 <= eq; o += 4) {
                    unsigned long long v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = S.lbuf[0][o + e];
#pragma unroll
                    for (int e = 0; e < 4; ++e) rank += v[e] > key;
                }
                for (; o < eq; ++o) rank += S.lbuf[0][o] > key;
                if (rank < need_rem) {
                    oidx[done + rank] = key_idx(key);
                    if (osc) osc[done + rank] = key_score(key);
                }
            }
            return;
        }
        // a slicing level that kept most of its keys: radix digits from here
        if (mode == 0 && 2 * eq > nalive) slice_ok = false;
        nalive = eq;
        // the next level's bins, free since the level before this one
        for (int x = tid; x < kSelBins; x += NT) hnext[x] = 0u;
        uint32_t* t = hcur;
        hcur = hnext;
        hnext = t;
        publish_range<NT, NK>(kr, alive, S);
        lds_barrier();
    }
}

// mode: SRC_DENSE / SRC_LIST: full selection from level 0.
//       SRC_KEYS: continue after topk_filter_kernel (its candidates + row state).
template <int NT, int LC>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4)))
void topk_select_kernel(TopkArgs a, int kind,
                                                                   const unsigned long long* cand) {
    constexpr int NK = kSelMax / NT;
    __shared__ SelShared<NT, LC> S;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    int32_t* oidx = a.out_idx + (long long)row * a.out_stride;
    float* osc = a.out_score ? a.out_score + (long long)row * a.out_stride : nullptr;

    const float* dsrc = nullptr;
    const float* lsc = nullptr;
    const int32_t* lid = nullptr;
    const unsigned long long* ksrc = nullptr;
    int nsrc0;
    if (kind == SRC_LIST) {
        nsrc0 = a.list_count ? a.list_count[row] : a.list_cap;
        nsrc0 = max(0, min(nsrc0, a.list_cap));
        lsc = a.list_score + (long long)row * a.list_stride;
        lid = a.list_idx + (long long)row * a.list_stride;
    } else {
        const int n = dense_len(a, row);
        dsrc = a.dense + (long long)row * a.dense_stride;
        nsrc0 = n;
    }

    int start_level = 0, need = 0, need_rem = 0;
    unsigned long long pfx = 0ull;
    int pfx_shift = 64;  // 64: no prefix filter yet
    if (kind == SRC_KEYS) {
        const int* ctl = reinterpret_cast<const int*>(a.state + (long long)row * kRowState +
                                                      kHist0Bins);
        ksrc = cand + (long long)row * a.cand_cap;
        // the row's counters in one read
        const int4 c0 = reinterpret_cast<const int4*>(ctl)[0];
        const int4 c1 = reinterpret_cast<const int4*>(ctl)[1];
        const int cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const int ncand = cv[CTL_CANDS];
        // The register path's keys are loaded together with the count, not
        // after it (the candidate array holds cand_cap keys per row, so the
        // loads stay in bounds); those past the count are dropped.
        unsigned long long pre[NK];
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int u = tid + j * NT;
            pre[j] = u < a.cand_cap ? ksrc[u] : 0ull;
        }
        nsrc0 = (int)min((long long)ncand, a.cand_cap);
        if (nsrc0 <= NK * NT) {
            select_in_registers<NT>(a, kind, dsrc, lsc, lid, ksrc, nsrc0, oidx, osc, S, pre, cv);
            return;
        }
    }
    if (nsrc0 <= NK * NT) {
        select_in_registers<NT>(a, kind, dsrc, lsc, lid, ksrc, nsrc0, oidx, osc, S);
        return;
    }
    if (kind == SRC_KEYS) {
        const int* ctl = reinterpret_cast<const int*>(a.state + (long long)row * kRowState +
                                                      kHist0Bins);
        need = ctl[CTL_NEED];
        const int gt = ctl[CTL_GT];
        for (int u = need + tid; u < a.k; u += NT) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        if (gt + ctl[CTL_EQ] == need) return;  // the filter emitted everything
        need_rem = need - gt;
        pfx = (unsigned long long)ctl[CTL_DIGIT];
        pfx_shift = kShift[0];
        start_level = 1;
        ksrc = cand + (long long)row * a.cand_cap;
        nsrc0 = (int)min((long long)ctl[CTL_CANDS], a.cand_cap);
        if (tid == 0) S.out = gt;
        lds_barrier();
    } else {
        for (int x = tid; x < kHist0Bins; x += NT) S.hist[x] = 0u;
        lds_barrier();
        for (int ub = 0; ub < nsrc0; ub += NT * kBatch) {
            unsigned long long kb[kBatch];
            bool vb[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int u = ub + j * NT + tid;
                vb[j] = u < nsrc0;
                kb[j] = vb[j] ? src_key(kind, dsrc, lsc, lid, nullptr, u, vb[j]) : 0ull;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (vb[j]) atomicAdd(&S.hist[(uint32_t)(kb[j] >> kShift[0])], 1u);
        }
        lds_barrier();
        int local = 0;
        for (int j = 0; j < kHist0Bins / NT; ++j)
            local += (int)S.hist[tid * (kHist0Bins / NT) + j];
        int nvalid;
        block_excl_scan<NT>(local, S.wave, &nvalid);
        need = min(a.k, nvalid);
        for (int u = need + tid; u < a.k; u += NT) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        if (need <= 0) return;
        need_rem = need;
        if (tid == 0) S.out = 0;
        lds_barrier();
    }

    // Current source: the global source (with prefix filter) or an LDS buffer.
    int cur_lds = -1;     // -1: global source; 0/1: S.lbuf[cur_lds]
    int nsrc = nsrc0;
    for (int level = start_level; level < 6; ++level) {
        const int shift = kShift[level];
        const int nbins = 1 << kWidth[level];
        const unsigned long long mask = (unsigned long long)(nbins - 1);
        const bool hist_ready = (level == 0);  // level-0 histogram built above
        if (!hist_ready) {
            for (int x = tid; x < nbins; x += NT) S.hist[x] = 0u;
            lds_barrier();
            // kBatch keys per thread loaded before any is used, so a pass over
            // a global source costs a few memory round trips, not one per key
            for (int ub = 0; ub < nsrc; ub += NT * kBatch) {
                unsigned long long kb[kBatch];
                bool vb[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    const int u = ub + j * NT + tid;
                    vb[j] = u < nsrc;
                    kb[j] = 0ull;
                    if (vb[j]) {
                        if (cur_lds >= 0) {
                            kb[j] = S.lbuf[cur_lds][u];
                        } else {
                            kb[j] = src_key(kind, dsrc, lsc, lid, ksrc, u, vb[j]);
                            vb[j] = vb[j] && (pfx_shift == 64 || (kb[j] >> pfx_shift) == pfx);
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < kBatch; ++j)
                    if (vb[j]) atomicAdd(&S.hist[(uint32_t)((kb[j] >> shift) & mask)], 1u);
            }
            lds_barrier();
        }
        find_threshold<NT>(S.hist, nbins, need_rem, S.wave, &S.th);
        const uint32_t d = (uint32_t)S.th.dstar;
        const int gt = S.th.gt;
        const bool take_all = gt + S.th.eq == need_rem;
        const bool next_fits = !take_all && S.th.eq <= LC;
        const int dst = cur_lds == 0 ? 1 : 0;
        if (tid == 0) S.cand = 0;
        lds_barrier();
        for (int ub = 0; ub < nsrc; ub += NT * kBatch) {
            unsigned long long kb[kBatch];
            bool vb[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int u = ub + j * NT + tid;
                vb[j] = u < nsrc;
                kb[j] = 0ull;
                if (vb[j]) {
                    if (cur_lds >= 0) {
                        kb[j] = S.lbuf[cur_lds][u];
                    } else {
                        kb[j] = src_key(kind, dsrc, lsc, lid, ksrc, u, vb[j]);
                        vb[j] = vb[j] && (pfx_shift == 64 || (kb[j] >> pfx_shift) == pfx);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const unsigned long long key = kb[j];
                const uint32_t dig = (uint32_t)((key >> shift) & mask);
                const bool emit = vb[j] && (dig > d || (take_all && dig == d));
                const bool app = vb[j] && next_fits && dig == d;
                const int slot = wave_append(emit, &S.out);
                if (emit && slot < need) {
                    oidx[slot] = key_idx(key);
                    if (osc) osc[slot] = key_score(key);
                }
                const int cslot = wave_append(app, &S.cand);
                if (app && cslot < LC) S.lbuf[dst][cslot] = key;
            }
        }
        lds_barrier();
        need_rem -= gt;
        if (take_all) break;
        pfx = (pfx_shift == 64) ? (unsigned long long)d : ((pfx << kWidth[level]) | d);
        pfx_shift = shift;
        if (next_fits) {
            cur_lds = dst;
            nsrc = min(S.cand, LC);
        } else {
            cur_lds = -1;
            nsrc = nsrc0;
        }
        lds_barrier();
    }
}

// ------------------------------------------------------ one wave per row

// Many rows with short sources (prefill rows' block scores, short lists):
// one wave selects one row, KPL keys per lane, with no barrier and no LDS.
// The need-th largest key T is found bit by bit from the top: T | bit stays
// when at least need keys are >= it (a count of ballots per step); the keys
// are distinct, so exactly need keys are >= T and those are emitted.  Four
// rows per 256-thread workgroup.
template <int KPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(TopkArgs a, int kind, int rows) {
    const int lane = lane_id();
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    const float* dsrc = nullptr;
    const float* lsc = nullptr;
    const int32_t* lid = nullptr;
    int nsrc;
    if (kind == SRC_LIST) {
        nsrc = a.list_count ? a.list_count[row] : a.list_cap;
        nsrc = max(0, min(nsrc, a.list_cap));
        lsc = a.list_score + (long long)row * a.list_stride;
        lid = a.list_idx + (long long)row * a.list_stride;
    } else {
        nsrc = dense_len(a, row);
        dsrc = a.dense + (long long)row * a.dense_stride;
    }
    unsigned long long kr[KPL];
    uint32_t alive = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int u = lane + 64 * j;
        bool valid = u < nsrc;
        kr[j] = valid ? src_key(kind, dsrc, lsc, lid, nullptr, u, valid) : 0ull;
        if (valid) alive |= 1u << j;
    }
    int nvalid = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) nvalid += __popcll(__ballot((alive >> j) & 1u));
    const int need = min(a.k, nvalid);
    int32_t* oidx = a.out_idx + (long long)row * a.out_stride;
    float* osc = a.out_score ? a.out_score + (long long)row * a.out_stride : nullptr;
    for (int u = need + lane; u < a.k; u += 64) {
        oidx[u] = -1;
        if (osc) osc[u] = -INFINITY;
    }
    if (need <= 0) return;
    // The bits above the highest one where the largest and the smallest key
    // differ are common to every key; the search starts below them and ends
    // as soon as exactly need keys are at or above the candidate.
    unsigned long long kmax = 0ull, kmin = ~0ull;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
        if ((alive >> j) & 1u) {
            kmax = kr[j] > kmax ? kr[j] : kmax;
            kmin = kr[j] < kmin ? kr[j] : kmin;
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long xm = __shfl_xor(kmax, o), xn = __shfl_xor(kmin, o);
        kmax = xm > kmax ? xm : kmax;
        kmin = xn < kmin ? xn : kmin;
    }
    const unsigned long long diff = kmax ^ kmin;
    const int top = diff ? 63 - __clzll(diff) : -1;
    unsigned long long T = top >= 63 ? 0ull : kmax & ~((2ull << top) - 1ull);
    if (top < 0) T = kmax;  // a single key
    for (int bit = top; bit >= 0; --bit) {
        const unsigned long long cand = T | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) cnt += __popcll(__ballot(((alive >> j) & 1u) && kr[j] >= cand));
        if (cnt >= need) T = cand;
        if (cnt == need) break;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const bool e = ((alive >> j) & 1u) && kr[j] >= T;
        const unsigned long long m = __ballot(e);
        if (e) {
            const int slot = base + __popcll(m & below);
            oidx[slot] = key_idx(kr[j]);
            if (osc) osc[slot] = key_score(kr[j]);
        }
        base += __popcll(m);
    }
}

hipError_t launch_topk_dense_filtered(const TopkArgs& a, int rows, int maxn,
                                      unsigned long long* cand, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    prof_begin(K_TOPK_FILTER, s);
    sa_launch(topk_filter_kernel, dim3((maxn + kFilterChunk - 1) / kFilterChunk, rows),
                         dim3(kFilterThreads), 0, s, a, cand);
    prof_end(K_TOPK_FILTER, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_begin(K_TOPK, s);
    if (rows >= kManyRows * cu_count())
        sa_launch(topk_select_kernel<kTopkThreads / 2, kLdsCand / 2>, dim3(rows),
                  dim3(kTopkThreads / 2), 0, s, a, SRC_KEYS, cand);
    else
        sa_launch(topk_select_kernel<kTopkThreads, kLdsCand>, dim3(rows), dim3(kTopkThreads), 0,
                  s, a, SRC_KEYS, cand);
    prof_end(K_TOPK, s);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, int rows, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int kind = a.dense ? SRC_DENSE : SRC_LIST;
    prof_begin(K_TOPK, s);
    const int maxsrc = a.dense ? a.len_cap : a.list_cap;
    if (rows >= kManyRows * cu_count() && maxsrc <= 64 * 16) {
        // short sources of many rows: a wave per row
        const dim3 grid((unsigned)((rows + 3) / 4));
        if (maxsrc <= 64 * 4)
            sa_launch(topk_wave_kernel<4>, grid, dim3(256), 0, s, a, kind, rows);
        else if (maxsrc <= 64 * 8)
            sa_launch(topk_wave_kernel<8>, grid, dim3(256), 0, s, a, kind, rows);
        else
            sa_launch(topk_wave_kernel<16>, grid, dim3(256), 0, s, a, kind, rows);
    } else if (rows >= kManyRows * cu_count())
        sa_launch(topk_select_kernel<kTopkThreads / 2, kLdsCand / 2>, dim3(rows),
                  dim3(kTopkThreads / 2), 0, s, a, kind, nullptr);
    else
        sa_launch(topk_select_kernel<kTopkThreads, kLdsCand>, dim3(rows), dim3(kTopkThreads), 0,
                  s, a, kind, nullptr);
    prof_end(K_TOPK, s);
    return hipGetLastError();
}

}  // namespace sa
