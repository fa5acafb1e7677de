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
#include "sa_select.h"

namespace sa {

constexpr int kTopkThreads = 1024;
constexpr int kFilterThreads = 512;
// Dense elements per filter workgroup: 16 per thread.  Larger chunks mean
// fewer workgroups re-reading the row histogram (8192: 8.1 us for the 8 x 128K
// decode rows against 10.8 us at 4096).
constexpr int kFilterChunk = 8192;
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
    __shared__ int s_idx[kFilterChunk];
    __shared__ float s_sc[kFilterChunk];
    __shared__ unsigned long long s_cand[kFilterChunk];
    __shared__ int s_ne, s_nc, s_base[2];
    __shared__ int s_wave[kFilterThreads / 64];
    __shared__ Thresh th;
    const int row = blockIdx.y;
    const int tid = threadIdx.x;
    const int n = dense_len(a, row);
    const int lo = blockIdx.x * kFilterChunk;
    if (lo >= n) return;
    const int hi = min(lo + kFilterChunk, n);
    uint32_t* hist = reinterpret_cast<uint32_t*>(s_cand);  // 16 KiB, reused below
    const uint32_t* grow = a.state + (long long)row * kRowState;
    for (int x = tid; x < kHist0Bins; x += kFilterThreads) hist[x] = grow[x];
    __syncthreads();
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
    __syncthreads();
    // Each thread classifies its kPer scores (float4 loads, all issued first),
    // then one wave-level prefix sum of its (emit, candidate) counts and one
    // LDS atomic per wave and kind give it its staging slots.
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
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    int wbase = 0;
    if (lane == 63) {
        const int te = incl & 0xffff, tc = incl >> 16;
        const int be = te ? atomicAdd(&s_ne, te) : 0;
        const int bc = tc ? atomicAdd(&s_nc, tc) : 0;
        wbase = be | (bc << 16);
    }
    wbase = __shfl(wbase, 63);
    const int excl = incl - mine;
    int se = (wbase & 0xffff) + (excl & 0xffff);
    int sc2 = (wbase >> 16) + (excl >> 16);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int u = lo + (tid + (j >> 2) * kFilterThreads) * 4 + (j & 3);
        if (emask & (1u << j)) {
            s_idx[se] = u;
            s_sc[se] = vs[j];
            ++se;
        }
        if (cmask & (1u << j)) s_cand[sc2++] = make_key(vs[j], u);
    }
    __syncthreads();
    if (tid == 0) {
        s_base[0] = s_ne ? atomicAdd(&ctl[CTL_EMITTED], s_ne) : 0;
        s_base[1] = s_nc ? atomicAdd(&ctl[CTL_CANDS], s_nc) : 0;
    }
    __syncthreads();
    int32_t* oidx = a.out_idx + (long long)row * a.out_stride;
    float* osc = a.out_score ? a.out_score + (long long)row * a.out_stride : nullptr;
    for (int x = tid; x < s_ne; x += kFilterThreads) {
        const int slot = s_base[0] + x;
        if (slot < need) {
            oidx[slot] = s_idx[x];
            if (osc) osc[slot] = s_sc[x];
        }
    }
    unsigned long long* crow = cand + (long long)row * a.cand_cap;
    for (int x = tid; x < s_nc; x += kFilterThreads) {
        const long long cs = (long long)s_base[1] + x;
        if (cs < a.cand_cap) crow[cs] = s_cand[x];
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
//       SRC_KEYS: continue after topk_filter_kernel (its candidates + row state).
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(TopkArgs a, int kind,
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
        need = ctl[CTL_NEED];
        const int gt = ctl[CTL_GT];
        for (int u = need + tid; u < a.k; u += kTopkThreads) {
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
    sa_launch(topk_select_kernel, dim3(rows), dim3(kTopkThreads), 0, s, a, SRC_KEYS, cand);
    prof_end(K_TOPK, s);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, int rows, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int kind = a.dense ? SRC_DENSE : SRC_LIST;
    prof_begin(K_TOPK, s);
    sa_launch(topk_select_kernel, dim3(rows), dim3(kTopkThreads), 0, s, a, kind, nullptr);
    prof_end(K_TOPK, s);
    return hipGetLastError();
}

}  // namespace sa
