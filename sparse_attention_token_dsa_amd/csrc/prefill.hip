// Fused causal-prefill indexer: q . K contraction on bf16 MFMA, ReLU, the
// w-weighted head sum and the causal mask in the epilogue, and the row's exact
// top-k, in one kernel (PaperTrace, "2.2.2 MISA, LISA and ResMiSA", section
// 2.2: score, causal mask and top-k fused into one pass).
//
// Layout: a workgroup of 4 waves owns 8 consecutive query rows of one
// sequence (two rows per wave, their heads held as MFMA A fragments in
// registers: each B fragment read from LDS feeds both rows) and sweeps the
// legal keys [0, max t] in tiles of 64 keys.  Each tile (16 KiB of bf16 keys)
// is staged once in LDS for all 8 rows by direct global-to-LDS loads, two
// stages deep (the next tile is in flight while one is computed), with a
// 16-byte XOR swizzle so the B-fragment reads are free of bank conflicts.
//
// Per tile and row the sweep does no selection work: each legal score is
// added to the row's LDS histogram (bins of 1/16 octave over [2^-32, 2^32);
// zero, negative and smaller scores share bin 0, larger ones the last bin)
// and stored, one coalesced 256-byte store per row, to the row's score line
// in the workspace (4 bytes per legal key, written once and read once).
//
// Finish: after the sweep each wave selects its rows' exact top-k: the
// histogram gives the bin holding the k-th score; one pass over the row emits
// the scores above it and collects the ones in it, as 64-bit keys
// ord(score) << 32 | ~position (ties -> lower position), into LDS; a radix
// select on those keys (10-bit digits) settles the rest.  Only when the bin
// holds more keys than the LDS buffer does a digit level re-read the row.
#include "sa_frag.h"

namespace sa {

constexpr int kPfWaves = 4;
constexpr int kPfQpw = 2;  // query rows per wave
constexpr int kPfRows = kPfWaves * kPfQpw;
constexpr int kPfTile = 64;
constexpr int kPfBins = 1024;
// A bin is ord(score) >> 19: sign, exponent and 4 mantissa bits.
constexpr int kPfBinShift = 19;
// ord(2^-32) >> 19: prefix of the first inner bin.
constexpr int kPfBase = (int)((0x80000000u | (95u << 23)) >> kPfBinShift);
// Key bits fixed by an inner bin: 63 .. 32 + kPfBinShift.
constexpr int kPfKeyTop = 32 + kPfBinShift;
constexpr int kPfCand = 512;  // LDS candidate keys per row
constexpr int kPfSweep = 8;   // float4 loads in flight per lane in a row pass
static_assert(kPfRows / 2 * kPfCand * 8 == kPfTile * 16 * 16,
              "half of the rows' candidate buffers fill one stage");

__device__ __forceinline__ int pf_bin(float sc) {
    const int v = (int)(ord_key(sc) >> kPfBinShift) - kPfBase;
    return v < 0 ? 0 : (v > kPfBins - 1 ? kPfBins - 1 : v);
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
// every lane and element, 4 consecutive scores per lane and kPfSweep loads in
// flight.  Rows are padded to a multiple of 4 floats, so the clamped float4
// reads stay inside the row.
template <class F>
__device__ __forceinline__ void row_sweep(const float* sr, int cnt, F&& fn) {
    const int lane = lane_id();
    const float4* sr4 = reinterpret_cast<const float4*>(sr);
    const int last4 = (cnt - 1) >> 2;
    for (int ub = 0; ub < cnt; ub += 256 * kPfSweep) {
        float4 v[kPfSweep];
#pragma unroll
        for (int j = 0; j < kPfSweep; ++j) v[j] = sr4[min((ub >> 2) + j * 64 + lane, last4)];
#pragma unroll
        for (int j = 0; j < kPfSweep; ++j) {
            const int u = ub + 4 * (j * 64 + lane);
            fn(u, v[j].x, u < cnt);
            fn(u + 1, v[j].y, u + 1 < cnt);
            fn(u + 2, v[j].z, u + 2 < cnt);
            fn(u + 3, v[j].w, u + 3 < cnt);
        }
    }
}

// Wave-level: the bin d of a 1024-bin histogram that holds the need-th
// largest element (bins scanned from the top); gt = elements above d,
// eq = elements in d.  Wave-uniform results.
__device__ __forceinline__ void wave_threshold(const uint32_t* h, int need, int& d, int& gt, int& eq) {
    const int lane = lane_id();
    int local = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) local += (int)h[kPfBins - 1 - (lane * 16 + j)];
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    int cum = incl - local;
    int fd = -1, fg = 0, fe = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int bin = kPfBins - 1 - (lane * 16 + j);
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
// histogram of the row's cnt legal scores sr[0, cnt); cb is kPfCand keys of
// LDS.  Output order is unspecified.
__device__ __forceinline__ void pf_finish(uint32_t* h, unsigned long long* cb, const float* sr,
                                          int cnt, int need, int32_t* oidx, float* osc) {
    const int lane = lane_id();
    const unsigned long long lt = (1ull << lane) - 1ull;
    int d0, gt0, eq0;
    wave_threshold(h, need, d0, gt0, eq0);
    bool take_all = gt0 + eq0 == need;
    const bool fits = !take_all && eq0 <= kPfCand;
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
    row_sweep(sr, cnt, [&](int u, float sc, bool in) {
        const int bin = pf_bin(sc);
        put(in && (bin > d0 || (take_all && bin == d0)), u, sc);
        const bool app = in && fits && bin == d0;
        const unsigned long long ma = __ballot(app);
        if (app) cb[nc + __popcll(ma & lt)] = pf_key(sc, u);
        nc += __popcll(ma);
    });
    if (take_all) return;

    int need_rem = need - gt0;
    // An inner bin fixes the key bits above kPfKeyTop; the clamped end bins
    // fix nothing.
    const bool clamped = d0 == 0 || d0 == kPfBins - 1;
    int top = clamped ? 64 : kPfKeyTop;
    unsigned long long pval = clamped ? 0ull : (unsigned long long)(d0 + kPfBase);
    int pshift = top;
    bool inlds = fits;  // candidates in cb, else re-read the row
    int nsrc = fits ? nc : cnt;
    while (top > 0) {
        const int width = top < 10 ? top : 10;
        const int shift = top - width;
        const unsigned long long mask = (1ull << width) - 1ull;
        auto live = [&](unsigned long long key, float sc) {
            return pf_bin(sc) == d0 && (pshift == 64 || (key >> pshift) == pval);
        };
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
        int d, gt, eq;
        wave_threshold(h, need_rem, d, gt, eq);
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
    }
}

template <int NHT>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_kernel(PrefillArgs a) {
    // Two stages as two distinct LDS objects: the compiler then tracks the
    // direct-to-LDS loads per stage and places no wait of its own for the
    // stage in flight before reads of the other.
    __shared__ uint4 kt0[kPfTile * 16], kt1[kPfTile * 16];
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
    // 16 bytes at consecutive addresses) = 4 key rows.  Lane l lands at key
    // 4*(4j + wave) + l/16, slot l%16 of the row, and fetches the chunk that
    // belongs in that slot under the swizzle (slot ^ (key & 15)).  Tiles past
    // the last are clamped re-reads, so every stage issues exactly kPfLoads
    // loads per thread.
    constexpr int kPfLoads = kPfTile * 16 / (64 * kPfWaves);
    auto issue = [&](uint4* stage, int tile) {
#pragma unroll
        for (int j = 0; j < kPfLoads; ++j) {
            const int blk = kPfWaves * j + wid;
            const int key = 4 * blk + (lane >> 4);
            const int s = min(tile * kPfTile + key, tmax);
            const int chunk = (lane & 15) ^ (key & 15);
            __builtin_amdgcn_global_load_lds(kseq + (long long)s * kD + chunk * 8,
                                             stage + blk * 64, 16, 0, 0);
        }
    };

    // A tile's scores are stored at the top of the next tile, right after its
    // stage wait, so the stores have a whole tile of compute to complete
    // before the next wait (which counts them too) comes round.
    float pend[kPfQpw];
    int pend_base = -1;
    auto put = [&]() {
        if (pend_base < 0) return;
        const int s = pend_base + lane;
#pragma unroll
        for (int qq = 0; qq < kPfQpw; ++qq)
            if (s <= tq[qq]) srow[qq][s] = pend[qq];
        pend_base = -1;
    };

    // One barrier per tile: after it, this tile's data is visible to all and
    // every wave is done with the other stage, which is refilled right away
    // (its next tile then has this tile's compute time to arrive).
    auto consume = [&](const uint4* ktile, uint4* other, int tile) {
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        issue(other, tile + 1);
        put();
        const int kbase = tile * kPfTile;
        if (kbase <= tw) {
            // Scores of the tile, parked so that lane l holds key kbase + l of
            // each row: the 4 MFMA groups run branch-free.
            float mine[kPfQpw];
#pragma unroll
            for (int qq = 0; qq < kPfQpw; ++qq) mine[qq] = 0.f;
#pragma unroll
            for (int gi = 0; gi < kPfTile / 16; ++gi) {
                const int kl = gi * 16 + c;
                uint4 kb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    kb[kk] = ktile[kl * 16 + ((kk * 4 + g) ^ (kl & 15))];
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
                        for (int e = 0; e < 4; ++e)
                            sc = fmaf(f[qq].wv[ht][e], fmaxf(acc[ht][e], 0.f), sc);
                    sc = sum_lane_groups(sc);
                    mine[qq] = g == gi ? sc : mine[qq];
                }
            }
            const int s = kbase + lane;
#pragma unroll
            for (int qq = 0; qq < kPfQpw; ++qq) {
                if (s <= tq[qq]) lds_add_u32(&h[qq][pf_bin(mine[qq])], 1u);
                pend[qq] = mine[qq];
            }
            pend_base = kbase;
        }
    };

    issue(kt0, 0);
    for (int tile = 0; tile < ntiles; tile += 2) {
        consume(kt0, kt1, tile);
        if (tile + 1 >= ntiles) break;
        consume(kt1, kt0, tile + 1);
    }
    put();

    // The key tiles are free once every wave is past its last tile and the
    // last (clamped) stage fill has landed: they hold the candidate buffers,
    // rows 0-3 in kt0 and rows 4-7 in kt1.  Each wave finishes its own rows
    // from the score lines it wrote.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < kPfQpw; ++qq) {
        if (!act[qq]) continue;
        const int need = min(a.k, tq[qq] + 1);
        int32_t* oidx = a.out_idx + rowq[qq] * a.out_stride;
        float* osc = a.out_score ? a.out_score + rowq[qq] * a.out_stride : nullptr;
        for (int u = need + lane; u < a.k; u += 64) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        const int r = wid * kPfQpw + qq;
        unsigned long long* cb = reinterpret_cast<unsigned long long*>(r < kPfRows / 2 ? kt0 : kt1) +
                                 (r % (kPfRows / 2)) * kPfCand;
        pf_finish(h[qq], cb, srow[qq], tq[qq] + 1, need, oidx, osc);
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
