// Score kernels of the gfx950 indexer: the streaming key scan (DSA decode,
// MISA routed scan, HISA block scan), the gathered rescoring (MISA-dagger
// pool, HISA fine stage), the MISA router, and the causal tail pooling.
//
// Every kernel computes I = sum_j w_j * ReLU(q_j . k) (PaperTrace, "2.2.2
// MISA, LISA and ResMiSA", section 1) with the q . k contraction on the bf16
// MFMA unit: one query's heads form the M dimension (16 per tile), 16 keys
// form N, and the 128 key dims are the contraction, split in 4 steps of 32.
// The ReLU, the w-weighted head sum and the causal bound are applied to the
// accumulator registers; only one fp32 score per key leaves the kernel.
#include "sa_frag.h"

namespace sa {

// ------------------------------------------------------------ scan

// One workgroup = 4 waves scans keys [cs, ce) of one query row (ce - cs <=
// kScanMaxChunk).  Each wave takes G*16 consecutive keys per step and the
// workgroup advances 4*G*16 keys per step; NBUF register buffers rotate, so
// the key loads of the next NBUF - 1 steps are in flight while one step is
// computed.  Scores are staged in LDS and written out coalesced at the end,
// so the loop issues no global stores.
//
// With a row state (HIST), the scores' first radix digit is histogrammed in
// LDS and added to the row's global histogram for the top-k filter, which
// runs after this kernel and so sees every workgroup's counts.
template <int KS>
constexpr int scan_waves() { return 4; }

template <int NHT, int KSTEPS, int G, int NBUF, int NSTEP, bool HIST, bool ROUTED>
__global__ __launch_bounds__(64 * scan_waves<KSTEPS>()) void scan_kernel(ScanArgs a) {
    constexpr int NW = scan_waves<KSTEPS>();
    constexpr int NT = 64 * NW;
    constexpr int KROW = KSTEPS * 32;
    constexpr int WKEYS = G * 16;
    constexpr int STEP = NW * WKEYS;
    const int row = blockIdx.y;
    const int b = row / a.T;
    const int t = row_pos(row, a.T, a.offset, a.seq_lens, a.len_cap);
    int n = t / a.len_div + 1;
    if (n > a.len_cap) n = a.len_cap;
    const int cs = blockIdx.x * a.chunk;
    if (cs >= n) return;
    const int ce = min(cs + a.chunk, n);

    __shared__ uint32_t lhist[HIST ? kHist0Bins : 1];
    __shared__ float sbuf[kScanMaxChunk];
    if (HIST) {
        for (int x = threadIdx.x; x < kHist0Bins; x += NT) lhist[x] = 0u;
        __syncthreads();
    }

    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t* heads = ROUTED ? a.heads + (long long)row * a.hsel : nullptr;
    QFrag<NHT> f;
    load_qfrag<NHT, ROUTED>(f, a.q + (long long)row * a.H * kD, a.w + (long long)row * a.H, a.H,
                            heads, a.hsel, g, c);

    const uint16_t* kseq = a.keys + (long long)b * a.seq_stride;
    const uint16_t* tailp =
        (KSTEPS == 8 && a.tail && a.tail_flag[row]) ? a.tail + (long long)row * 256 : nullptr;

    auto kptr = [&](int s) -> const uint16_t* {
        if (KSTEPS == 8 && tailp && s == n - 1) return tailp;
        return kseq + (long long)s * KROW;
    };
    // Keys (KSTEPS = 4): coalesced loads, 4 whole 256-byte rows per load
    // instruction (lane l: key l/16 of the quad, 16-byte chunk l%16), then a
    // per-wave LDS transpose into the MFMA B layout (lane (g, c) needs key c,
    // chunk kk*4+g).  Loading the B layout directly would touch 16 rows per
    // instruction with 64 bytes each, which costs about a third of the HBM
    // rate.  The transpose tile is XOR-swizzled (chunk ^ key) so both the
    // row writes and the column reads are free of bank conflicts.
    __shared__ uint4 tbuf[KSTEPS == 4 ? NW : 1][KSTEPS == 4 ? 256 : 1];
    // Loads past the end re-read the last key, so they can be unconditional:
    // the wait before each compute then covers exactly the older buffer.
    auto loadG = [&](uint4 (&buf)[G][KSTEPS], int base) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            if (KSTEPS == 4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = min(base + gi * 16 + 4 * j + (lane >> 4), ce - 1);
                    buf[gi][j] = ldg16_stream(kseq + (long long)s * kD + (lane & 15) * 8);
                }
            } else {
                const int s = min(base + gi * 16 + c, ce - 1);
                load_key<KSTEPS>(buf[gi], kptr(s), g);
            }
        }
    };
    auto computeG = [&](const uint4 (&buf)[G][KSTEPS], int base) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const int s = base + gi * 16 + c;
            float sc;
            if (KSTEPS == 4) {
                uint4* tp = tbuf[wid];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = 4 * j + (lane >> 4);
                    tp[key * 16 + ((lane & 15) ^ key)] = buf[gi][j];
                }
                uint4 kb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kb[kk] = tp[c * 16 + ((kk * 4 + g) ^ c)];
                sc = group_score<NHT, 4>(f, kb);
            } else {
                sc = group_score<NHT, KSTEPS>(f, buf[gi]);
            }
            if (g == 0 && s < ce) {
                sbuf[s - cs] = sc;
                if (HIST) atomicAdd(&lhist[ord_key(sc) >> (32 - kHist0Bits)], 1u);
            }
        }
    };

    // Loads are unconditional: past the end they re-read the last key, so
    // every load keeps its place in the pipeline and the compiler's waits
    // stay exact.  With NSTEP > 0 (full chunks) the loop is unrolled
    // completely and every step is computed (past the end nothing is
    // stored); otherwise steps past the end (at most NBUF - 1) are skipped.
    const int base = cs + wid * WKEYS;
    uint4 buf[NBUF][G][KSTEPS];
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) loadG(buf[u], base + u * STEP);
    if constexpr (NSTEP > 0) {
#pragma unroll
        for (int it = 0; it < NSTEP; ++it) {
            if (it + NBUF - 1 < NSTEP)
                loadG(buf[(it + NBUF - 1) % NBUF], base + (it + NBUF - 1) * STEP);
            computeG(buf[it % NBUF], base + it * STEP);
        }
    } else {
        const int nsteps = (ce - cs + STEP - 1) / STEP;
#pragma unroll 4
        for (int it0 = 0; it0 < nsteps; it0 += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                loadG(buf[(u + NBUF - 1) % NBUF], base + (it0 + u + NBUF - 1) * STEP);
                if (it0 + u < nsteps) computeG(buf[u], base + (it0 + u) * STEP);
            }
        }
    }
    __syncthreads();
    float* srow = a.scores + (long long)row * a.score_stride;
    for (int x = threadIdx.x; x < ce - cs; x += NT) srow[cs + x] = sbuf[x];
    if (HIST) {
        uint32_t* grow = a.state + (long long)row * kRowState;
        for (int x = threadIdx.x; x < kHist0Bins; x += NT) {
            const uint32_t v = lhist[x];
            if (v) atomicAdd(&grow[x], v);
        }
    }
}

// ----------------------------------------------------------- gather

// Rescore a per-row candidate list with all heads.  List mode: candidate u
// is token list[u]; block mode: candidate u is token list[u / bsz] * bsz +
// u % bsz.  Candidates past the causal bound, past L or with a negative id
// get score -inf and index -1.  A workgroup takes kGatherChunk candidates;
// each wave resolves its kGatherGroups x 16 candidate ids, issues every key
// load (16 KiB in flight per wave), then runs the MFMA groups.
template <int NHT, bool BLOCKS, bool F8>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
    constexpr int NG = kGatherGroups;
    const int row = blockIdx.y;
    const int b = row / a.T;
    const int t = a.offset + (row - b * a.T);
    const int cs = blockIdx.x * kGatherChunk;
    if (cs >= a.ncand) return;
    const int ce = min(cs + kGatherChunk, a.ncand);
    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t* lrow = a.list + (long long)row * a.list_len;
    int sid[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int u = cs + (gi * 4 + wid) * 16 + c;
        int s = -1;
        if (u < ce) {
            if (BLOCKS) {
                const int q = u / a.bsz;
                const int blk = lrow[q];
                s = blk >= 0 ? blk * a.bsz + (u - q * a.bsz) : -1;
            } else {
                s = lrow[u];
            }
        }
        sid[gi] = (s >= 0 && s <= t && s < a.L) ? s : -1;
    }
    QFrag<NHT> f;
    load_qfrag<NHT>(f, a.q + (long long)row * a.H * kD, a.w + (long long)row * a.H, a.H,
                    nullptr, 0, g, c);
    uint4 kb[NG][4];
    float ks[NG];
    if (F8) {
        // FP8 cache: the same dims as load_key (k-step kk, lane group g:
        // dims 32kk + 8g .. +8), widened exactly; the key's scale multiplies
        // the head sum.
        const uint8_t* cseq = a.codes + (long long)b * a.seq_stride;
        const float* sseq = a.kscale + (long long)b * (a.seq_stride / kD);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const long long s = sid[gi] >= 0 ? sid[gi] : 0;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint2 v = *reinterpret_cast<const uint2*>(cseq + s * kD + 32 * kk + 8 * g);
                kb[gi][kk] = widen8(v.x, v.y);
            }
            ks[gi] = sseq[s];
        }
    } else {
        const uint16_t* kseq = a.keys + (long long)b * a.seq_stride;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            load_key<4>(kb[gi], kseq + (long long)(sid[gi] >= 0 ? sid[gi] : 0) * kD, g);
            ks[gi] = 1.f;
        }
    }
    float* osc = a.out_score + (long long)row * a.ncand;
    int32_t* oid = a.out_idx + (long long)row * a.ncand;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int u = cs + (gi * 4 + wid) * 16 + c;
        float sc = group_score<NHT, 4>(f, kb[gi]);
        if (F8) sc *= ks[gi];
        if (g == 0 && u < ce) {
            osc[u] = sid[gi] >= 0 ? sc : -INFINITY;
            oid[u] = sid[gi];
        }
    }
}

// ----------------------------------------------------------- router

// MISA router for one query row (summary page "MISA", method steps 2-3):
// E_j = |w_j| * mean_m ReLU(q_j . pooled_m) over the blocks that intersect
// [0, t], then the h largest E (ties -> lower head), written ascending.
template <int NHT>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
    const int row = blockIdx.x;
    const int b = row / a.T;
    const int t = a.offset + (row - b * a.T);
    const int Mt = min(t / a.B + 1, a.nblk);
    const int lane = lane_id(), wid = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    QFrag<NHT> f;
    load_qfrag<NHT>(f, a.q + (long long)row * a.H * kD, a.w + (long long)row * a.H, a.H,
                    nullptr, 0, g, c);
    const uint16_t* kseq = a.reps + (long long)b * a.seq_stride;
    const uint16_t* tailp = (a.tail && a.tail_flag[row]) ? a.tail + (long long)row * 256 : nullptr;

    float sum[NHT][4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[ht][i] = 0.f;

    for (int base = wid * 16; base < Mt; base += 64) {
        const int m = base + c;
        const bool valid = m < Mt;
        const int ml = valid ? m : Mt - 1;
        const uint16_t* kp = (tailp && ml == Mt - 1) ? tailp : kseq + (long long)ml * 256;
        uint4 kb[8];
        load_key<8>(kb, kp, g);
        f32x4 acc[NHT];
        group_dots<NHT, 8>(f, kb, acc);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[ht][i] += valid ? fmaxf(acc[ht][i], 0.f) : 0.f;
    }
    __shared__ float part[4][kMaxH];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = sum[ht][i];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            if (c == 0) part[wid][ht * 16 + 4 * g + i] = v;
        }
    __syncthreads();
    if (wid == 0) {
        __shared__ float sE[kMaxH];
        const int j = lane;
        float E = -1.f;  // absent heads rank below every real head (E >= 0)
        if (j < a.H) {
            const float S = part[0][j] + part[1][j] + part[2][j] + part[3][j];
            E = fabsf(a.w[(long long)row * a.H + j]) * S / (float)Mt;
            if (a.E_out) a.E_out[(long long)row * a.H + j] = E;
        }
        sE[j] = E;  // same wave writes then reads: LDS keeps the order
        int rank = 0;
#pragma unroll
        for (int j4 = 0; j4 < kMaxH; j4 += 4) {
            const float4 e4 = *reinterpret_cast<const float4*>(&sE[j4]);
            const float es[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) rank += (es[u] > E) || (es[u] == E && j4 + u < j);
        }
        const bool sel = j < a.H && rank < a.h;
        const unsigned long long msk = __ballot(sel);
        const int pos = __popcll(msk & ((1ull << lane) - 1ull));
        if (sel) a.heads_out[(long long)row * a.h + pos] = j;
    }
    // The routed scan that follows adds its histogram into a zeroed row state
    // (one launch fewer on the MISA path).
    if (a.zero_state)
        for (int x = threadIdx.x; x < kRowState; x += 256)
            a.zero_state[(long long)row * kRowState + x] = 0u;
}

// ------------------------------------------------------------- tail

// Causal tail of the block pooling: for a row whose last legal block is cut
// by the causal bound (t is not the block's last key), the representative is
// the mean of keys [m*block, t]; written as a hi/lo bf16 pair like the cached
// representatives.  flag[row] tells the score kernels whether to use it.
__global__ __launch_bounds__(256) void tail_kernel(const uint16_t* keys, const uint8_t* codes,
                                                   const float* scales, long long seq_stride,
                                                   int T, int offset, int L, int block,
                                                   uint16_t* tail, uint8_t* flag) {
    const int row = blockIdx.x;
    const int b = row / T;
    const int t = offset + (row - b * T);
    const int lo = (t / block) * block;
    const int last = min(lo + block, L) - 1;
    const bool partial = last > t;
    if (threadIdx.x == 0) flag[row] = partial ? 1 : 0;
    if (!partial) return;
    const int c16 = threadIdx.x & 15, kl = threadIdx.x >> 4;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    // (FP8 cache: codes seq_stride bytes apart per sequence, scales
    // seq_stride / 128 apart.)
    const uint16_t* kseq = codes ? nullptr : keys + (long long)b * seq_stride;
    const uint8_t* cseq = codes ? codes + (long long)b * seq_stride : nullptr;
    const float* sseq = codes ? scales + (long long)b * (seq_stride / kD) : nullptr;
    for (int s = lo + kl; s <= t; s += 16) {
        float x[8];
        key8_f32(kseq, cseq, sseq, s, c16, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
    __shared__ float red[16][kD];
#pragma unroll
    for (int e = 0; e < 8; ++e) red[kl][c16 * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kD) {
        float S = 0.f;
        for (int r = 0; r < 16; ++r) S += red[r][threadIdx.x];
        const float mean = S / (float)(t - lo + 1);
        const uint32_t hi = f32_to_bf16_bits(mean);
        const uint32_t lo16 = f32_to_bf16_bits(mean - bf16_bits_to_f32(hi));
        tail[(long long)row * 256 + threadIdx.x] = (uint16_t)hi;
        tail[(long long)row * 256 + kD + threadIdx.x] = (uint16_t)lo16;
    }
}

__global__ void fill_u32_kernel(uint32_t* p, long long n, uint32_t v) {
    for (long long x = blockIdx.x * (long long)blockDim.x + threadIdx.x; x < n;
         x += (long long)gridDim.x * blockDim.x)
        p[x] = v;
}

// ---------------------------------------------------------- launchers

hipError_t launch_fill_u32(uint32_t* p, long long n, uint32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    long long blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    prof_begin(K_FILL, s);
    sa_launch(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    prof_end(K_FILL, s);
    return hipGetLastError();
}

// Keys (KSTEPS = 4): one 16-key group per wave and step, 4 register buffers
// (three steps of loads in flight), nontemporal loads, and about one
// workgroup per CU: long contiguous streams per workgroup read fastest (the
// L = 131072, batch-8 scan takes 45.7 us right after a cache flush with 4096
// keys per workgroup, 55.5 us with 1024 keys and 4 groups x 2 buffers).
// Block representatives (KSTEPS = 8, a few thousand per row at most): 2
// groups, one step of 128 per workgroup, so the grid still covers the chip.
template <int KS>
constexpr int scan_groups() { return KS == 4 ? 1 : 2; }
template <int KS>
constexpr int scan_bufs() { return KS == 4 ? 4 : 1; }

template <int NHT, int KS, int NSTEP>
static void scan_dispatch_hist(const ScanArgs& a, dim3 grid, hipStream_t s) {
    constexpr int G = scan_groups<KS>();
    constexpr int NB = scan_bufs<KS>();
    if (a.heads) {
        if (a.state)
            sa_launch(scan_kernel<NHT, KS, G, NB, NSTEP, true, true>, grid, dim3(64 * scan_waves<KS>()), 0, s, a);
        else
            sa_launch(scan_kernel<NHT, KS, G, NB, NSTEP, false, true>, grid, dim3(64 * scan_waves<KS>()), 0, s, a);
    } else {
        if (a.state)
            sa_launch(scan_kernel<NHT, KS, G, NB, NSTEP, true, false>, grid, dim3(64 * scan_waves<KS>()), 0, s, a);
        else
            sa_launch(scan_kernel<NHT, KS, G, NB, NSTEP, false, false>, grid, dim3(64 * scan_waves<KS>()), 0, s, a);
    }
}

// Full chunks of keys take the completely unrolled loop (about 2% faster).
template <int NHT>
static void scan_dispatch_keys(const ScanArgs& a, dim3 grid, hipStream_t s) {
    constexpr int kFull = kScanMaxChunk / (scan_waves<4>() * 16 * scan_groups<4>());
    if (a.chunk == kScanMaxChunk) {
        scan_dispatch_hist<NHT, 4, kFull>(a, grid, s);
    } else {
        scan_dispatch_hist<NHT, 4, 0>(a, grid, s);
    }
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int scan_chunk(int ksteps, long long rows, int maxn) {
    if (ksteps != 4) return scan_waves<8>() * 16 * scan_groups<8>();
    constexpr int step = scan_waves<4>() * 16 * scan_groups<4>();
    const long long wgs = cu_count();
    long long c = (rows * (long long)maxn + wgs - 1) / wgs;
    c = (c + step - 1) / step * step;
    c = c < (long long)step * scan_bufs<4>() ? (long long)step * scan_bufs<4>() : c;
    c = c > kScanMaxChunk ? kScanMaxChunk : c;
    return (int)c;
}

hipError_t launch_scan(const ScanArgs& a, int rows, int nht, int ksteps, bool routed,
                       hipStream_t s) {
    const int maxn = a.len_cap;
    const dim3 grid((unsigned)((maxn + a.chunk - 1) / a.chunk), (unsigned)rows);
    const int kid = ksteps == 8 ? K_BLOCK_SCORE
                  : (routed ? K_SCAN_ROUTED : K_SCAN);
    prof_begin(kid, s);
    if (ksteps == 4) {
        switch (nht) {
            case 1: scan_dispatch_keys<1>(a, grid, s); break;
            case 2: scan_dispatch_keys<2>(a, grid, s); break;
            case 3: scan_dispatch_keys<3>(a, grid, s); break;
            default: scan_dispatch_keys<4>(a, grid, s); break;
        }
    } else {
        switch (nht) {
            case 1: scan_dispatch_hist<1, 8, 1>(a, grid, s); break;
            case 2: scan_dispatch_hist<2, 8, 1>(a, grid, s); break;
            case 3: scan_dispatch_hist<3, 8, 1>(a, grid, s); break;
            default: scan_dispatch_hist<4, 8, 1>(a, grid, s); break;
        }
    }
    prof_end(kid, s);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, int rows, int nht, bool block_mode,
                         hipStream_t s) {
    const dim3 grid((unsigned)((a.ncand + kGatherChunk - 1) / kGatherChunk), (unsigned)rows);
    prof_begin(K_GATHER, s);
#define SA_GATHER(N)                                                            \
    if (a.codes) {                                                              \
        if (block_mode)                                                         \
            sa_launch(gather_kernel<N, true, true>, grid, dim3(256), 0, s, a);  \
        else                                                                    \
            sa_launch(gather_kernel<N, false, true>, grid, dim3(256), 0, s, a); \
    } else if (block_mode) {                                                    \
        sa_launch(gather_kernel<N, true, false>, grid, dim3(256), 0, s, a);     \
    } else {                                                                    \
        sa_launch(gather_kernel<N, false, false>, grid, dim3(256), 0, s, a);    \
    }
    switch (nht) {
        case 1: SA_GATHER(1) break;
        case 2: SA_GATHER(2) break;
        case 3: SA_GATHER(3) break;
        default: SA_GATHER(4) break;
    }
#undef SA_GATHER
    prof_end(K_GATHER, s);
    return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& a, int rows, hipStream_t s) {
    const int nht = (a.H + 15) / 16;
    prof_begin(K_ROUTER, s);
    switch (nht) {
        case 1: sa_launch(router_kernel<1>, dim3(rows), dim3(256), 0, s, a); break;
        case 2: sa_launch(router_kernel<2>, dim3(rows), dim3(256), 0, s, a); break;
        case 3: sa_launch(router_kernel<3>, dim3(rows), dim3(256), 0, s, a); break;
        default: sa_launch(router_kernel<4>, dim3(rows), dim3(256), 0, s, a); break;
    }
    prof_end(K_ROUTER, s);
    return hipGetLastError();
}

hipError_t launch_tail(const uint16_t* keys, long long seq_stride, int T, int offset, int L,
                       int block, int rows, uint16_t* tail, uint8_t* flag, hipStream_t s,
                       const uint8_t* codes, const float* scales) {
    prof_begin(K_TAIL, s);
    sa_launch(tail_kernel, dim3(rows), dim3(256), 0, s, keys, codes, scales, seq_stride, T, offset,
              L, block, tail, flag);
    prof_end(K_TAIL, s);
    return hipGetLastError();
}

}  // namespace sa
