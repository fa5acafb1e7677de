// Fused causal-prefill indexer: q . K contraction on bf16 MFMA, ReLU, the
// w-weighted head sum and the causal mask in the epilogue, and a streaming
// per-row threshold, so the n^2 score matrix never reaches HBM (PaperTrace,
// "2.2.2 MISA, LISA and ResMiSA", section 2.2: fuse score, causal mask and
// top-k and avoid writing n^2 scores back).
//
// Layout: a workgroup of 8 waves owns 8 consecutive query rows of one
// sequence (one row per wave, its 64 heads held as MFMA A fragments in
// registers) and sweeps the legal keys [0, max t] in tiles of 64 keys.  Each
// tile (16 KiB of bf16 keys) is staged once in LDS for all 8 rows, double
// buffered, with a 16-byte XOR swizzle so the B-fragment reads are free of
// bank conflicts.
//
// Streaming threshold: each wave keeps an LDS histogram of the scores it has
// kept, in bins of 1/16 octave over [2^-64, 2^64) (everything below, zero and
// negative scores in bin 0, everything above in the last bin).  tau is the
// highest bin such that at least k kept scores lie in bins >= tau; a new score
// in a bin below tau has k larger scores ahead of it and can never enter the
// row's top-k, so it is dropped.  Scores in bins >= tau are appended with
// their positions to the row's survivor list in the workspace; an exact
// top-k over the survivors finishes the row.
#include "sa_frag.h"

namespace sa {

constexpr int kPfWaves = 8;
constexpr int kPfTile = 64;
constexpr int kPfBins = 2048;
// ord(2^-64) >> 19: first key of bin 0 for positive scores.
constexpr int kPfBinBase = (int)((0x80000000u | (63u << 23)) >> 19);

__device__ __forceinline__ int pf_bin(float sc) {
    const int v = (int)(ord_key(sc) >> 19) - kPfBinBase;
    return v < 0 ? 0 : (v > kPfBins - 1 ? kPfBins - 1 : v);
}

template <int NHT>
__global__ __launch_bounds__(512) void prefill_kernel(PrefillArgs a) {
    __shared__ uint4 ktile[2][kPfTile * 16];
    __shared__ uint32_t hist[kPfWaves][kPfBins];

    const int seq = blockIdx.y;
    const int i0 = blockIdx.x * kPfWaves;
    const int tid = threadIdx.x;
    const int lane = lane_id(), wid = tid >> 6, g = lane >> 4, c = lane & 15;
    const int i = i0 + wid;
    const bool active = i < a.T;
    const long long row = (long long)seq * a.T + i;
    const int t = a.offset + i;
    const int tmax = a.offset + min(i0 + kPfWaves, a.T) - 1;
    const int ntiles = tmax / kPfTile + 1;

    for (int x = lane; x < kPfBins; x += 64) hist[wid][x] = 0u;

    QFrag<NHT> f;
    if (active) {
        load_qfrag<NHT>(f, a.q + row * a.H * kD, a.w + row * a.H, a.H, nullptr, 0, g, c);
    } else {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.a[ht][kk] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int e = 0; e < 4; ++e) f.wv[ht][e] = 0.f;
        }
    }

    const uint16_t* kseq = a.keys + (long long)seq * a.L * kD;
    // Staging: thread -> (key = tid/16 + 32j, 16-byte chunk c16 = tid % 16).
    const int c16 = tid & 15, kr = tid >> 4;
    uint4 st[2];
    auto gload = [&](int tile) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = min(tile * kPfTile + kr + 32 * j, tmax);
            st[j] = ldg16(kseq + (long long)s * kD + c16 * 8);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int key = kr + 32 * j;
            ktile[buf][key * 16 + (c16 ^ (key & 15))] = st[j];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    float* ssc = a.surv_score + row * a.cap;
    int32_t* sid = a.surv_idx + row * a.cap;
    uint32_t* h = hist[wid];
    int tau = 0, cnt = 0, cnt_ge = 0;

    for (int tile = 0; tile < ntiles; ++tile) {
        const int buf = tile & 1;
        const bool more = tile + 1 < ntiles;
        if (more) gload(tile + 1);
        const int kbase = tile * kPfTile;
        if (active && kbase <= t) {
#pragma unroll
            for (int gi = 0; gi < kPfTile / 16; ++gi) {
                const int kl = gi * 16 + c;
                uint4 kb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kb[kk] = ktile[buf][kl * 16 + ((kk * 4 + g) ^ (kl & 15))];
                const float sc = group_score<NHT, 4>(f, kb);
                const int s = kbase + kl;
                const bool valid = g == 0 && s <= t;
                const int bin = pf_bin(sc);
                const bool surv = valid && bin >= tau;
                const unsigned long long m = __ballot(surv);
                if (m) {
                    const int rank = __popcll(m & ((1ull << lane) - 1ull));
                    if (surv) {
                        ssc[cnt + rank] = sc;
                        sid[cnt + rank] = s;
                        atomicAdd(&h[bin], 1u);
                    }
                    const int pc = __popcll(m);
                    cnt += pc;
                    cnt_ge += pc;
                    if (cnt_ge - (int)a.k >= 0) {
                        // Raise tau while the bins at and above tau+1 still hold k scores.
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): see own adds
                        for (;;) {
                            const int bb = tau + lane;
                            const int hv = bb < kPfBins ? (int)h[bb] : 0;
                            int incl = hv;
#pragma unroll
                            for (int off = 1; off < 64; off <<= 1) {
                                const int y = __shfl_up(incl, off);
                                if (lane >= off) incl += y;
                            }
                            const int excl = incl - hv;
                            const bool ok = bb < kPfBins && cnt_ge - excl >= a.k;
                            const unsigned long long okm = __ballot(ok);
                            const int lstar = 63 - __clzll((long long)okm);
                            const int drop = __shfl(excl, lstar);
                            tau += lstar;
                            cnt_ge -= drop;
                            if (lstar < 63 || tau >= kPfBins - 1) break;
                        }
                    }
                }
            }
        }
        if (more) lstore(buf ^ 1);
        __syncthreads();
    }
    if (active && lane == 0) a.surv_count[row] = cnt;
}

hipError_t launch_prefill(const PrefillArgs& a, int rows, hipStream_t s) {
    const int batch = rows / a.T;
    const dim3 grid((unsigned)((a.T + kPfWaves - 1) / kPfWaves), (unsigned)batch);
    const int nht = (a.H + 15) / 16;
    prof_begin(K_PREFILL, s);
    switch (nht) {
        case 1: prefill_kernel<1><<<grid, dim3(512), 0, s>>>(a); break;
        case 2: prefill_kernel<2><<<grid, dim3(512), 0, s>>>(a); break;
        case 3: prefill_kernel<3><<<grid, dim3(512), 0, s>>>(a); break;
        default: prefill_kernel<4><<<grid, dim3(512), 0, s>>>(a); break;
    }
    prof_end(K_PREFILL, s);
    return hipGetLastError();
}

}  // namespace sa
