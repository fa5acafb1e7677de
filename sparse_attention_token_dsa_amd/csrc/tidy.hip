// Index tidy-up after the token top-k (PaperTrace, "2.2.2 MISA, LISA and
// ResMiSA", section 2.2: the gather of the selected tokens coalesces better
// when the indices are put in physical page / offset order; the tidy-up keeps
// the set free of duplicates and its valid length, and its time counts as
// selector time.  Section 2.3 asks the profiler for the number of distinct
// pages and of contiguous runs per row).
//
// One workgroup per query row: each selected position s (>= 0) becomes its
// physical slot table[b][s / page] * page + s % page (or s itself without a
// table), duplicates are dropped, and the row's unique slots are written in
// ascending order, -1 padded, with three counts: unique slots, distinct pages,
// maximal runs of consecutive slots.  Two forms:
//  - bitmap (slot bound known and <= 2^18): one bit per slot in LDS, set
//    with LDS atomics, then each thread walks its words with a popcount
//    prefix sum for its output position;
//  - sort (any slot range, k <= 4096): bitonic sort of the slots in LDS.
#include "sa_common.h"

namespace sa {

namespace {

constexpr int kTidyThreads = 256;

// Physical slot of selected position s of sequence b, or -1 (empty, past the
// table, an unmapped page, or at/after the slot bound).
__device__ __forceinline__ int tidy_slot(const TidyArgs& a, const int32_t* tab, int s) {
    if (s < 0) return -1;
    int v = s;
    if (tab) {
        const int pg = s / a.page;
        if (pg >= a.pages_per_seq) return -1;
        const int phys = tab[pg];
        if (phys < 0) return -1;
        v = phys * a.page + (s - pg * a.page);
    }
    if (a.max_slots > 0 && v >= a.max_slots) return -1;
    return v;
}

// Block-wide sums of two per-thread counts (part: kTidyThreads ints of LDS).
__device__ __forceinline__ void tidy_write_stats(const TidyArgs& a, int row, int total, int np,
                                                 int ns, int* part) {
    const int tid = threadIdx.x;
    __syncthreads();
    part[tid] = np;
    __syncthreads();
    for (int off = kTidyThreads / 2; off > 0; off >>= 1) {
        if (tid < off) part[tid] += part[tid + off];
        __syncthreads();
    }
    const int pages = part[0];
    __syncthreads();
    part[tid] = ns;
    __syncthreads();
    for (int off = kTidyThreads / 2; off > 0; off >>= 1) {
        if (tid < off) part[tid] += part[tid + off];
        __syncthreads();
    }
    if (tid == 0) {
        int32_t* st = a.out_stats + (long long)row * 3;
        st[0] = total;
        st[1] = pages;
        st[2] = part[0];
    }
}

__global__ __launch_bounds__(kTidyThreads) void tidy_bitmap_kernel(TidyArgs a) {
    extern __shared__ uint32_t bits[];  // ceil(max_slots / 32) words
    __shared__ int part[kTidyThreads];
    __shared__ int lastv[kTidyThreads];
    const int row = blockIdx.x;
    const int b = row / a.T;
    const int tid = threadIdx.x;
    const int nw = (a.max_slots + 31) >> 5;
    for (int x = tid; x < nw; x += kTidyThreads) bits[x] = 0u;
    __syncthreads();
    const int32_t* in = a.idx + (long long)row * a.k;
    const int32_t* tab = a.table ? a.table + (long long)b * a.pages_per_seq : nullptr;
    for (int x = tid; x < a.k; x += kTidyThreads) {
        const int v = tidy_slot(a, tab, in[x]);
        if (v >= 0) atomicOr(&bits[v >> 5], 1u << (v & 31));
    }
    __syncthreads();
    const int wpt = (nw + kTidyThreads - 1) / kTidyThreads;
    const int w0 = min(tid * wpt, nw), w1 = min(w0 + wpt, nw);
    int cnt = 0, last = -1;
    for (int x = w0; x < w1; ++x) {
        const uint32_t m = bits[x];
        cnt += __popc(m);
        if (m) last = x * 32 + 31 - __clz(m);
    }
    part[tid] = cnt;
    lastv[tid] = last;
    __syncthreads();
    for (int off = 1; off < kTidyThreads; off <<= 1) {  // inclusive sum and max scans
        const int add = tid >= off ? part[tid - off] : 0;
        const int mx = tid >= off ? lastv[tid - off] : -1;
        __syncthreads();
        part[tid] += add;
        lastv[tid] = max(lastv[tid], mx);
        __syncthreads();
    }
    int pos = part[tid] - cnt;
    const int total = part[kTidyThreads - 1];
    int prev = tid > 0 ? lastv[tid - 1] : -1;  // the largest slot before my words
    int np = 0, ns = 0;
    int32_t* out = a.out_slots + (long long)row * a.k;
    for (int x = w0; x < w1; ++x) {
        uint32_t m = bits[x];
        while (m) {
            const int v = x * 32 + __ffs(m) - 1;
            m &= m - 1u;
            out[pos++] = v;
            if (prev < 0 || prev / a.page != v / a.page) ++np;
            if (prev < 0 || prev + 1 != v) ++ns;
            prev = v;
        }
    }
    for (int x = total + tid; x < a.k; x += kTidyThreads) out[x] = -1;
    if (a.out_stats) tidy_write_stats(a, row, total, np, ns, part);
}

__global__ __launch_bounds__(kTidyThreads) void tidy_kernel(TidyArgs a) {
    const int row = blockIdx.x;
    const int b = row / a.T;
    const int tid = threadIdx.x;
    const int n2 = a.n2;  // power of two, >= k and >= kTidyThreads
    __shared__ uint32_t key[kTidyMax];
    __shared__ int part[kTidyThreads];
    const int32_t* in = a.idx + (long long)row * a.k;
    const int32_t* tab = a.table ? a.table + (long long)b * a.pages_per_seq : nullptr;
    for (int x = tid; x < n2; x += kTidyThreads) {
        uint32_t v = 0xffffffffu;  // empty / invalid: sorts last
        if (x < a.k) {
            const int s = tidy_slot(a, tab, in[x]);
            if (s >= 0) v = (uint32_t)s;
        }
        key[x] = v;
    }
    __syncthreads();
    // bitonic sort, ascending
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int x = tid; x < (n2 >> 1); x += kTidyThreads) {
                const int i = (x / stride) * 2 * stride + (x % stride);
                const int j = i + stride;
                const bool up = (i & size) == 0;
                const uint32_t ki = key[i], kj = key[j];
                if ((ki > kj) == up) {
                    key[i] = kj;
                    key[j] = ki;
                }
            }
            __syncthreads();
        }
    }
    // Each thread owns n2 / kTidyThreads consecutive sorted entries: count
    // its first-of-a-value entries (unique slots), page starts and run
    // starts, then an exclusive scan of the unique counts gives its output
    // position.
    const int per = n2 / kTidyThreads;
    const int x0 = tid * per;
    int nu = 0, np = 0, ns = 0;
    for (int x = x0; x < x0 + per; ++x) {
        const uint32_t v = key[x];
        if (v == 0xffffffffu) break;
        const uint32_t prev = x > 0 ? key[x - 1] : 0xffffffffu;
        if (x > 0 && prev == v) continue;
        ++nu;
        if (x == 0 || prev / (uint32_t)a.page != v / (uint32_t)a.page) ++np;
        if (x == 0 || prev + 1u != v) ++ns;
    }
    part[tid] = nu;
    __syncthreads();
    for (int off = 1; off < kTidyThreads; off <<= 1) {  // inclusive scan
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int pos = part[tid] - nu;
    const int total = part[kTidyThreads - 1];
    int32_t* out = a.out_slots + (long long)row * a.k;
    for (int x = x0; x < x0 + per; ++x) {
        const uint32_t v = key[x];
        if (v == 0xffffffffu) break;
        if (x > 0 && key[x - 1] == v) continue;
        out[pos++] = (int32_t)v;
    }
    for (int x = total + tid; x < a.k; x += kTidyThreads) out[x] = -1;
    if (a.out_stats) tidy_write_stats(a, row, total, np, ns, part);
}

}  // namespace

hipError_t launch_tidy(const TidyArgs& a, int rows, hipStream_t s) {
    prof_begin(K_TIDY, s);
    if (a.max_slots > 0 && a.max_slots <= kTidyBitmapMax)
        sa_launch(tidy_bitmap_kernel, dim3((unsigned)rows), dim3(kTidyThreads),
                  (uint32_t)((a.max_slots + 31) >> 5) * 4u, s, a);
    else
        sa_launch(tidy_kernel, dim3((unsigned)rows), dim3(kTidyThreads), 0, s, a);
    prof_end(K_TIDY, s);
    return hipGetLastError();
}

}  // namespace sa
