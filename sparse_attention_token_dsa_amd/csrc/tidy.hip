// Index tidy-up after the token top-k (PaperTrace, "2.2.2 MISA, LISA and
// ResMiSA", section 2.2: the gather of the selected tokens coalesces better
// when the indices are put in physical page / offset order; the tidy-up keeps
// the set free of duplicates and its valid length, and its time counts as
// selector time.  Section 2.3 asks the profiler for the number of distinct
// pages and of contiguous runs per row).
//
// One workgroup per query row: each selected position s (>= 0) becomes its
// physical slot table[b][s / page] * page + s % page (or s itself without a
// table), the slots are sorted in LDS (bitonic, ascending), duplicates are
// dropped, and the row's unique slots are written in order, -1 padded, with
// three counts: unique slots, distinct pages, maximal runs of consecutive
// slots.
#include "sa_common.h"

namespace sa {

namespace {

constexpr int kTidyThreads = 256;

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
            const int s = in[x];
            if (s >= 0) {
                if (!tab) {
                    v = (uint32_t)s;
                } else {
                    const int pg = s / a.page;
                    if (pg < a.pages_per_seq) {
                        const int phys = tab[pg];
                        if (phys >= 0) v = (uint32_t)phys * (uint32_t)a.page + (uint32_t)(s - pg * a.page);
                    }
                }
            }
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
    if (a.out_stats) {
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
}

}  // namespace

hipError_t launch_tidy(const TidyArgs& a, int rows, hipStream_t s) {
    prof_begin(K_TIDY, s);
    tidy_kernel<<<dim3((unsigned)rows), dim3(kTidyThreads), 0, s>>>(a);
    prof_end(K_TIDY, s);
    return hipGetLastError();
}

}  // namespace sa
