// Per-row exact top-k by radix select (PaperTrace, "2.2.2 MISA, LISA and
// ResMiSA", section 2.2: score, causal mask and top-k belong together; the
// top-k is a cost of its own that does not shrink with the head count).
//
// Every candidate becomes the 64-bit key  ord(score) << 32 | ~index : larger
// scores win and, among equal scores, the lower index wins.  Keys are
// distinct, so the selection is exact.  Keys are consumed from the top in
// digits of 12/10/10 bits (score) then 12/10/10 bits (index, only reached on
// exact score ties).  Per digit: a histogram, a scan from the top that finds
// the digit value holding the k-th key, and one pass that emits every key
// above it and keeps the keys on it for the next digit.
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
//    Candidates of later digits are compacted into LDS when they fit; if not,
//    the source is rescanned with a prefix filter.
#include "sa_common.h"

namespace sa {

constexpr int kTopkThreads = 1024;
constexpr int kFilterThreads = 256;
constexpr int kFilterChunk = 4096;       // dense elements per filter workgroup
constexpr int kLdsCand = 4096;           // keys per LDS candidate buffer

__device__ __forceinline__ unsigned long long make_key(float sc, int idx) {
    return ((unsigned long long)ord_key(sc) << 32) | (unsigned long long)(~(uint32_t)idx);
}
__device__ __forceinline__ int key_idx(unsigned long long k) { return (int)(~(uint32_t)k); }
__device__ __forceinline__ float key_score(unsigned long long k) {
    return ord_to_f32((uint32_t)(k >> 32));
}

__constant__ int kShift[6] = {52, 42, 32, 20, 10, 0};
__constant__ int kWidth[6] = {12, 10, 10, 12, 10, 10};

// Block-wide exclusive scan of one int per thread; *total gets the sum.
// Every thread of the block must call it (it contains barriers).
template <int NT>
__device__ int block_excl_scan(int v, int* s_wave, int* total) {
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wid] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int sw = s_wave[w];
        if (w < wid) base += sw;
        tot += sw;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

struct Thresh {
    int dstar, gt, eq;
};

// Digit value holding the need-th largest key, scanning bins from the top.
// Returns it in *out (written to shared memory by one thread, then synced).
template <int NT>
__device__ void find_threshold(const uint32_t* hist, int nbins, int need, int* s_wave,
                               Thresh* out) {
    const int per = nbins / NT;
    const int tid = threadIdx.x;
    int local = 0;
    for (int j = 0; j < per; ++j) local += (int)hist[nbins - 1 - (tid * per + j)];
    int total;
    int cum = block_excl_scan<NT>(local, s_wave, &total);
    for (int j = 0; j < per; ++j) {
        const int bin = nbins - 1 - (tid * per + j);
        const int h = (int)hist[bin];
        if (cum < need && need <= cum + h) {
            out->dstar = bin;
            out->gt = cum;
            out->eq = h;
        }
        cum += h;
    }
    __syncthreads();
}

__device__ __forceinline__ int dense_len(int row, int T, int offset, int len_div, int len_cap) {
    const int b = row / T;
    const int t = offset + (row - b * T);
    const int n = t / len_div + 1;
    return n < len_cap ? n : len_cap;
}

// ------------------------------------------------------------ filter

// Global counters per row: [0] = emitted so far, [1] = candidates appended.
// Each workgroup counts its emits and candidates first, reserves its output
// ranges with one atomic each, then writes: two passes over its slice (the
// second hits L2) instead of a global atomic round trip per wave iteration.
__global__ __launch_bounds__(kFilterThreads) void topk_filter_kernel(TopkArgs a,
                                                                     int* counters,
                                                                     unsigned long long* cand) {
    __shared__ uint32_t hist[kHist0Bins];
    __shared__ int s_wave[kFilterThreads / 64];
    __shared__ Thresh th;
    __shared__ int s_base[2];
    const int row = blockIdx.y;
    const int tid = threadIdx.x;
    const int n = dense_len(row, a.T, a.offset, a.len_div, a.len_cap);
    const int lo = blockIdx.x * kFilterChunk;
    if (lo >= n) return;
    const int hi = min(lo + kFilterChunk, n);
    const uint32_t* h0 = a.hist0 + (long long)row * kHist0Bins;
    for (int x = tid; x < kHist0Bins; x += kFilterThreads) hist[x] = h0[x];
    __syncthreads();
    const int need = min(a.k, n);
    find_threshold<kFilterThreads>(hist, kHist0Bins, need, s_wave, &th);
    const uint32_t d = (uint32_t)th.dstar;
    const bool take_all = th.gt + th.eq == need;
    const float* src = a.dense + (long long)row * a.dense_stride;

    int ne = 0, nc = 0;
    for (int u = lo + tid; u < hi; u += kFilterThreads) {
        const uint32_t dig = ord_key(src[u]) >> (32 - kHist0Bits);
        ne += (dig > d || (take_all && dig == d)) ? 1 : 0;
        nc += (!take_all && dig == d) ? 1 : 0;
    }
    int E, C;
    int pe = block_excl_scan<kFilterThreads>(ne, s_wave, &E);
    int pc = block_excl_scan<kFilterThreads>(nc, s_wave, &C);
    int* cnt = counters + 2 * row;
    if (tid == 0) {
        s_base[0] = E ? atomicAdd(&cnt[0], E) : 0;
        s_base[1] = C ? atomicAdd(&cnt[1], C) : 0;
    }
    __syncthreads();
    if (ne + nc == 0) return;
    pe += s_base[0];
    pc += s_base[1];
    int32_t* oidx = a.out_idx + (long long)row * a.out_stride;
    float* osc = a.out_score ? a.out_score + (long long)row * a.out_stride : nullptr;
    unsigned long long* crow = cand + (long long)row * a.cand_cap;
    for (int u = lo + tid; u < hi; u += kFilterThreads) {
        const float sc = src[u];
        const uint32_t dig = ord_key(sc) >> (32 - kHist0Bits);
        if (dig > d || (take_all && dig == d)) {
            if (pe < need) {
                oidx[pe] = u;
                if (osc) osc[pe] = sc;
            }
            ++pe;
        } else if (dig == d) {
            if (pc < a.cand_cap) crow[pc] = make_key(sc, u);
            ++pc;
        }
    }
}

// ------------------------------------------------------------ select

enum SrcKind { SRC_DENSE = 0, SRC_LIST = 1, SRC_KEYS = 2 };

struct SelShared {
    uint32_t hist[kHist0Bins];
    unsigned long long lbuf[2][kLdsCand];
    int wave[kTopkThreads / 64];
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

// mode: SRC_DENSE / SRC_LIST: full selection from level 0.
//       SRC_KEYS: continue after topk_filter_kernel (candidates + hist0).
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(TopkArgs a, int kind,
                                                                   const int* counters,
                                                                   const unsigned long long* cand) {
    __shared__ SelShared S;
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
        const int n = dense_len(row, a.T, a.offset, a.len_div, a.len_cap);
        dsrc = a.dense + (long long)row * a.dense_stride;
        nsrc0 = n;
    }

    int start_level = 0, need = 0, need_rem = 0;
    unsigned long long pfx = 0ull;
    int pfx_shift = 64;  // 64: no prefix filter yet
    if (kind == SRC_KEYS) {
        const uint32_t* h0 = a.hist0 + (long long)row * kHist0Bins;
        for (int x = tid; x < kHist0Bins; x += kTopkThreads) S.hist[x] = h0[x];
        __syncthreads();
        need = min(a.k, nsrc0);
        find_threshold<kTopkThreads>(S.hist, kHist0Bins, need, S.wave, &S.th);
        for (int u = need + tid; u < a.k; u += kTopkThreads) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        if (S.th.gt + S.th.eq == need) return;  // the filter emitted everything
        need_rem = need - S.th.gt;
        pfx = (unsigned long long)S.th.dstar;
        pfx_shift = kShift[0];
        start_level = 1;
        ksrc = cand + (long long)row * a.cand_cap;
        nsrc0 = (int)min((long long)counters[2 * row + 1], a.cand_cap);
        if (tid == 0) S.out = S.th.gt;
        __syncthreads();
    } else {
        for (int x = tid; x < kHist0Bins; x += kTopkThreads) S.hist[x] = 0u;
        __syncthreads();
        for (int u = tid; u < nsrc0; u += kTopkThreads) {
            bool valid = true;
            const unsigned long long key = src_key(kind, dsrc, lsc, lid, nullptr, u, valid);
            if (valid) atomicAdd(&S.hist[(uint32_t)(key >> kShift[0])], 1u);
        }
        __syncthreads();
        int local = 0;
        for (int j = 0; j < kHist0Bins / kTopkThreads; ++j)
            local += (int)S.hist[tid * (kHist0Bins / kTopkThreads) + j];
        int nvalid;
        block_excl_scan<kTopkThreads>(local, S.wave, &nvalid);
        need = min(a.k, nvalid);
        for (int u = need + tid; u < a.k; u += kTopkThreads) {
            oidx[u] = -1;
            if (osc) osc[u] = -INFINITY;
        }
        if (need <= 0) return;
        need_rem = need;
        if (tid == 0) S.out = 0;
        __syncthreads();
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
            for (int x = tid; x < nbins; x += kTopkThreads) S.hist[x] = 0u;
            __syncthreads();
            for (int u = tid; u < nsrc; u += kTopkThreads) {
                bool valid = true;
                unsigned long long key;
                if (cur_lds >= 0) {
                    key = S.lbuf[cur_lds][u];
                } else {
                    key = src_key(kind, dsrc, lsc, lid, ksrc, u, valid);
                    valid = valid && (pfx_shift == 64 || (key >> pfx_shift) == pfx);
                }
                if (valid) atomicAdd(&S.hist[(uint32_t)((key >> shift) & mask)], 1u);
            }
            __syncthreads();
        }
        find_threshold<kTopkThreads>(S.hist, nbins, need_rem, S.wave, &S.th);
        const uint32_t d = (uint32_t)S.th.dstar;
        const int gt = S.th.gt;
        const bool take_all = gt + S.th.eq == need_rem;
        const bool next_fits = !take_all && S.th.eq <= kLdsCand;
        const int dst = cur_lds == 0 ? 1 : 0;
        if (tid == 0) S.cand = 0;
        __syncthreads();
        for (int ub = 0; ub < nsrc; ub += kTopkThreads) {
            const int u = ub + tid;
            bool valid = u < nsrc;
            unsigned long long key = 0ull;
            if (valid) {
                if (cur_lds >= 0) {
                    key = S.lbuf[cur_lds][u];
                } else {
                    key = src_key(kind, dsrc, lsc, lid, ksrc, u, valid);
                    valid = valid && (pfx_shift == 64 || (key >> pfx_shift) == pfx);
                }
            }
            const uint32_t dig = (uint32_t)((key >> shift) & mask);
            const bool emit = valid && (dig > d || (take_all && dig == d));
            const bool app = valid && next_fits && dig == d;
            const int slot = wave_append(emit, &S.out);
            if (emit && slot < need) {
                oidx[slot] = key_idx(key);
                if (osc) osc[slot] = key_score(key);
            }
            const int cslot = wave_append(app, &S.cand);
            if (app && cslot < kLdsCand) S.lbuf[dst][cslot] = key;
        }
        __syncthreads();
        need_rem -= gt;
        if (take_all) break;
        pfx = (pfx_shift == 64) ? (unsigned long long)d : ((pfx << kWidth[level]) | d);
        pfx_shift = shift;
        if (next_fits) {
            cur_lds = dst;
            nsrc = min(S.cand, kLdsCand);
        } else {
            cur_lds = -1;
            nsrc = nsrc0;
        }
        __syncthreads();
    }
}

hipError_t launch_topk_dense_filtered(const TopkArgs& a, int rows, int maxn, int* counters,
                                      unsigned long long* cand, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    prof_begin(K_TOPK_FILTER, s);
    topk_filter_kernel<<<dim3((maxn + kFilterChunk - 1) / kFilterChunk, rows),
                         dim3(kFilterThreads), 0, s>>>(a, counters, cand);
    prof_end(K_TOPK_FILTER, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prof_begin(K_TOPK, s);
    topk_select_kernel<<<dim3(rows), dim3(kTopkThreads), 0, s>>>(a, SRC_KEYS, counters, cand);
    prof_end(K_TOPK, s);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, int rows, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int kind = a.dense ? SRC_DENSE : SRC_LIST;
    prof_begin(K_TOPK, s);
    topk_select_kernel<<<dim3(rows), dim3(kTopkThreads), 0, s>>>(a, kind, nullptr, nullptr);
    prof_end(K_TOPK, s);
    return hipGetLastError();
}

}  // namespace sa
