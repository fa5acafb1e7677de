// Block-level helpers of the radix select, shared by the score kernels
// (which find the first-digit threshold once per row) and the top-k kernels.
// Internal header.
#pragma once

#include "sa_common.h"

namespace sa {

// Block-wide exclusive scan of one int per thread; *total gets the sum.
// Every thread of the block must call it (it contains barriers).
template <int NT>
__device__ int block_excl_scan(int v, int* s_wave, int* total) {
    const int lane = lane_id(), wid = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) s_wave[wid] = x;
    lds_barrier();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int sw = s_wave[w];
        if (w < wid) base += sw;
        tot += sw;
    }
    lds_barrier();
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
    lds_barrier();
}

}  // namespace sa
