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

// MISA router for one query row (summary page "MISA", method steps 2-3):
// E_j = |w_j| * mean_m ReLU(q_j . pooled_m) over the blocks that intersect
// [0, t], then the h largest E (ties -> lower head).  A workgroup of 4 waves
// computes it: each wave takes two groups of 16 blocks per pass on the MFMA
// (all heads as M; both groups' loads in flight together), the ReLU sums meet
// in LDS, and wave 0 ranks the heads.  On return (after a barrier) s_heads[0..h)
// holds the routed heads in ascending order in every thread's view, and
// s_w[0..H) the head weights; E_out (nullable) gets the row's E.  With s_q
// (LDS, [kMaxH][16] uint4) the row's q is left there too: head j's 16-byte
// chunk x at s_q[j * 16 + x].
struct RouteIn {
    const uint16_t* q;      // the row's [H, 128]
    const float* w;         // the row's [H]
    const uint16_t* reps;   // the row's sequence [nblk, 256] hi/lo
    const uint16_t* tailp;  // mean of a cut last block [256], or null
    int H, Mt, h;
    float* E_out;           // the row's [H], or null
};

// The router's register operands: the row's q fragments (all heads) and the
// first pass of representatives (two groups of 16 blocks per wave).
template <int NHT>
struct RouteRegs {
    QFrag<NHT> f;
    uint4 kb[2][8];
    bool valid[2];
    uint32_t qvalid;  // slots of f, for mask_qfrag in route_finish
};

template <int NHT>
__device__ __forceinline__ void route_load_reps(const RouteIn& r, int base, RouteRegs<NHT>& R,
                                                int g, int c) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int m = base + 64 * u + c;
        R.valid[u] = m < r.Mt;
        const int ml = R.valid[u] ? m : r.Mt - 1;
        const uint16_t* kp = (r.tailp && ml == r.Mt - 1) ? r.tailp : r.reps + (long long)ml * 256;
        load_key<8>(R.kb[u], kp, g);
    }
}

// Issue the router's first loads (q, w and the first pass of blocks), with
// nothing that waits for them; the caller may issue other loads before
// route_finish consumes these.
template <int NHT>
__device__ __forceinline__ void route_issue(const RouteIn& r, RouteRegs<NHT>& R) {
    const int lane = lane_id(), wid = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    R.qvalid = load_qfrag_issue<NHT>(R.f, r.q, r.w, r.H, nullptr, 0, g, c);
    route_load_reps(r, wid * 16, R, g, c);
}

// The workgroup barriers here order LDS only: global loads the caller has in
// flight stay in flight.
template <int NHT>
__device__ __forceinline__ void route_finish(const RouteIn& r, RouteRegs<NHT>& R, int* s_heads,
                                             float* s_w, uint4* s_q = nullptr) {
    const int lane = lane_id(), wid = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
    mask_qfrag<NHT>(R.f, R.qvalid);
    float sum[NHT][4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[ht][i] = 0.f;
    for (int base = wid * 16;;) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 acc[NHT];
            group_dots<NHT, 8>(R.f, R.kb[u], acc);
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sum[ht][i] += R.valid[u] ? fmaxf(acc[ht][i], 0.f) : 0.f;
        }
        base += 128;
        if (base >= r.Mt) break;
        route_load_reps(r, base, R, g, c);
    }
    __shared__ float part[4][kMaxH];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = sum_row16(sum[ht][i]);
            if (c == 0) {
                part[wid][ht * 16 + 4 * g + i] = v;
                if (wid == 0) s_w[ht * 16 + 4 * g + i] = R.f.wv[ht][i];
            }
        }
    if (s_q && wid == 0) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) s_q[(ht * 16 + c) * 16 + kk * 4 + g] = R.f.a[ht][kk];
    }
    lds_barrier();
    if (wid == 0) {
        __shared__ float sE[kMaxH];
        const int j = lane;
        float E = -1.f;  // absent heads rank below every real head (E >= 0)
        if (j < r.H) {
            const float S = part[0][j] + part[1][j] + part[2][j] + part[3][j];
            E = fabsf(s_w[j]) * S / (float)r.Mt;
            if (r.E_out) r.E_out[j] = E;
        }
        sE[j] = E;  // same wave writes then reads: LDS keeps the order
        int rank = 0;
#pragma unroll
        for (int j4 = 0; j4 < kMaxH; j4 += 4) {
            const float4 e4 = *reinterpret_cast<const float4*>(&sE[j4]);
            const float es[4] = {e4.x, e4.y, e4.z, e4.w};
            // branch-free: (larger E) or (equal E and lower head)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                rank += (int)(es[u] > E) + (int)((es[u] == E) & (j4 + u < j));
        }
        const bool sel = j < r.H && rank < r.h;
        const unsigned long long msk = __ballot(sel);
        const int pos = __popcll(msk & ((1ull << lane) - 1ull));
        if (sel) s_heads[pos] = j;
    }
    lds_barrier();
}

template <int NHT>
__device__ __forceinline__ void route_wg(const RouteIn& r, int* s_heads, float* s_w) {
    RouteRegs<NHT> R;
    route_issue<NHT>(r, R);
    route_finish<NHT>(r, R, s_heads, s_w);
}

// The routed heads' q fragments (tile rows = s_heads[0..hsel), padded with
// zero rows) from the copies route_wg left in LDS.
template <int NHT>
__device__ __forceinline__ void routed_qfrag_lds(QFrag<NHT>& f, const uint4* s_q,
                                                 const float* s_w, const int* s_heads, int hsel,
                                                 int g, int c) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const int u = ht * 16 + c;
        const int v = u < hsel ? s_heads[u] : -1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            f.a[ht][kk] = v >= 0 ? s_q[v * 16 + kk * 4 + g] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u2 = ht * 16 + 4 * g + i;
            f.wv[ht][i] = u2 < hsel ? s_w[s_heads[u2]] : 0.f;
        }
    }
}

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

// With POOL (keys, one decode row per sequence reading all of its keys), the
// workgroup also sums the keys it streams into block means: each lane adds
// the 8 dims it loaded of its 4 keys per step; at the end of every small
// block the four lanes holding the same dims are summed (lane-group swaps)
// into a per-wave LDS slot, and after the sweep the four waves' slots are
// added in a fixed order into the small and large block means (hi/lo bf16).
template <int NHT, int KSTEPS, int G, int NBUF, int NSTEP, bool HIST, bool ROUTED,
          bool POOL = false>
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
    // The pooling scan runs two workgroups per CU on half-size chunks (its
    // extra arithmetic needs the second workgroup's waves to hide latency).
    constexpr int kMaxChunk = POOL ? kScanPoolChunk : kScanMaxChunk;
    __shared__ float sbuf[kMaxChunk];

    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    QFrag<NHT> f;
    // POOL: per-wave partial sums of each small block of the chunk
    constexpr int kPoolSlots = kMaxChunk / 128;
    __shared__ float pbuf[POOL ? NW : 1][POOL ? kPoolSlots : 1][POOL ? kD : 1];
    float pacc[POOL ? 8 : 1];
#pragma unroll
    for (int e = 0; e < (POOL ? 8 : 1); ++e) pacc[e] = 0.f;
    const int psteps = POOL ? a.pool_small / STEP : 1;  // workgroup steps per small block
    const int nsteps_all = (ce - cs + STEP - 1) / STEP;

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
    auto computeG = [&](const uint4 (&buf)[G][KSTEPS], int base, int it) {
        if constexpr (POOL) {
            // This lane's dims 8c' .. 8c'+7 (c' = lane & 15) of keys
            // base + 4j + (lane >> 4), two keys at a time: the same dim of
            // keys j and j + 1 packed into one bf16 pair (a byte permute) and
            // summed into the dim's fp32 accumulator by one dot product with
            // (1, 1) -- or 0 for a key past the chunk (a re-read).
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            const int k0 = base + (lane >> 4);
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                const uint32_t mw = (k0 + 4 * j < ce ? 0x3F80u : 0u) |
                                    (k0 + 4 * j + 4 < ce ? 0x3F800000u : 0u);
                const bf16x2_t m = __builtin_bit_cast(bf16x2_t, mw);
                const uint32_t w0[4] = {buf[0][j].x, buf[0][j].y, buf[0][j].z, buf[0][j].w};
                const uint32_t w1[4] = {buf[0][j + 1].x, buf[0][j + 1].y, buf[0][j + 1].z,
                                        buf[0][j + 1].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
                    pacc[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(
                        __builtin_bit_cast(bf16x2_t, lo), m, pacc[2 * e], false);
                    pacc[2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                        __builtin_bit_cast(bf16x2_t, hi), m, pacc[2 * e + 1], false);
                }
            }
            // end of a small block (a power-of-two number of steps) or of the
            // chunk: the four lanes holding the same dims are summed into this
            // wave's slot of the block
            if (it < nsteps_all && ((it & (psteps - 1)) == psteps - 1 || it + 1 == nsteps_all)) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[e] = sum_lane_groups(pacc[e]);
                    pacc[e] = 0.f;
                }
                if (g == 0) {
                    float4* dst = reinterpret_cast<float4*>(&pbuf[wid][it >> a.pool_shift][8 * c]);
                    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
                    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
                }
            }
        }
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
    const int32_t* heads = ROUTED ? a.heads + (long long)row * a.hsel : nullptr;
    // MISA routing inside the scan: every workgroup of the row computes the
    // same heads (same inputs, same arithmetic), so the router costs no launch
    // of its own.  Its loads go first, the first key loads behind them, and
    // its barriers order LDS only, so the keys stay in flight while it runs.
    constexpr bool kRoute = ROUTED && KSTEPS == 4;
    __shared__ int s_rheads[kRoute ? kMaxH : 1];
    __shared__ float s_rw[kRoute ? kMaxH : 1];
    __shared__ uint4 s_rq[kRoute ? kMaxH * 16 : 1];
    RouteIn rin;
    RouteRegs<kRoute ? 4 : 1> rregs;
    const bool route = kRoute && a.route_reps;
    // Loads in this order: the query (or the router's inputs), the first
    // key steps, and only then anything that waits for the query.
    uint32_t qvalid = 0u;
    if constexpr (!ROUTED)
        qvalid = load_qfrag_issue<NHT>(f, a.q + (long long)row * a.H * kD,
                                       a.w + (long long)row * a.H, a.H, nullptr, 0, g, c);
    if constexpr (kRoute) {
        if (route) {
            rin.q = a.q + (long long)row * a.H * kD;
            rin.w = a.w + (long long)row * a.H;
            rin.reps = a.route_reps + (long long)b * a.route_seq_stride;
            rin.tailp = nullptr;
            rin.H = a.H;
            rin.Mt = min(t / a.route_B + 1, a.route_nblk);
            rin.h = a.hsel;
            rin.E_out = nullptr;
            route_issue(rin, rregs);
        }
    }
#pragma unroll
    for (int u = 0; u < NBUF - 1; ++u) loadG(buf[u], base + u * STEP);
    if (HIST) {
        // LDS only: the key loads just issued stay in flight
        for (int x = threadIdx.x; x < kHist0Bins; x += NT) lhist[x] = 0u;
        lds_barrier();
    }
    if constexpr (!ROUTED) mask_qfrag<NHT>(f, qvalid);
    if constexpr (kRoute) {
        if (route) {
            route_finish(rin, rregs, s_rheads, s_rw, s_rq);
            if (blockIdx.x == 0 && a.route_heads_out)
                for (int u = threadIdx.x; u < a.hsel; u += NT)
                    a.route_heads_out[(long long)row * a.hsel + u] = s_rheads[u];
            routed_qfrag_lds<NHT>(f, s_rq, s_rw, s_rheads, a.hsel, g, c);
            heads = nullptr;
        }
    }
    if (ROUTED && heads)
        load_qfrag<NHT, ROUTED>(f, a.q + (long long)row * a.H * kD, a.w + (long long)row * a.H,
                                a.H, heads, a.hsel, g, c);
    if constexpr (NSTEP > 0) {
#pragma unroll
        for (int it = 0; it < NSTEP; ++it) {
            if (it + NBUF - 1 < NSTEP)
                loadG(buf[(it + NBUF - 1) % NBUF], base + (it + NBUF - 1) * STEP);
            computeG(buf[it % NBUF], base + it * STEP, it);
        }
    } else {
        const int nsteps = (ce - cs + STEP - 1) / STEP;
#pragma unroll 4
        for (int it0 = 0; it0 < nsteps; it0 += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                loadG(buf[(u + NBUF - 1) % NBUF], base + (it0 + u + NBUF - 1) * STEP);
                if (it0 + u < nsteps) computeG(buf[u], base + (it0 + u) * STEP, it0 + u);
            }
        }
    }
    __syncthreads();
    float* srow = a.scores + (long long)row * a.score_stride;
    for (int x = threadIdx.x; x < ce - cs; x += NT) srow[cs + x] = sbuf[x];
    if constexpr (POOL) {
        // Block means of this chunk (cs is a multiple of the large block): the
        // four waves' partials in a fixed order, so every call rounds alike.
        const int sb = a.pool_small, lb = a.pool_large;
        const int nsb = (ce - cs + sb - 1) / sb, per = lb / sb;
        const int nsmall = (a.len_cap + sb - 1) / sb, nlarge = (a.len_cap + lb - 1) / lb;
        auto blk_sum = [&](int k, int d) {
            return ((pbuf[0][k][d] + pbuf[1][k][d]) + pbuf[2][k][d]) + pbuf[3][k][d];
        };
        for (int x = threadIdx.x; x < nsb * kD; x += NT) {
            const int k = x >> 7, d = x & (kD - 1);
            const int lo = cs + k * sb;
            const float mean = blk_sum(k, d) / (float)(min(lo + sb, ce) - lo);
            uint16_t* o = a.pool_out_small + ((long long)b * nsmall + lo / sb) * 2 * kD;
            const uint32_t hi = f32_to_bf16_bits(mean);
            o[d] = (uint16_t)hi;
            o[kD + d] = (uint16_t)f32_to_bf16_bits(mean - bf16_bits_to_f32(hi));
        }
        const int nlb = (ce - cs + lb - 1) / lb;
        for (int x = threadIdx.x; x < nlb * kD; x += NT) {
            const int m = x >> 7, d = x & (kD - 1);
            const int lo = cs + m * lb;
            float S = 0.f;
            for (int i = 0; i < per; ++i) {
                const int k = m * per + i;
                if (k < nsb) S += blk_sum(k, d);
            }
            const float mean = S / (float)(min(lo + lb, ce) - lo);
            uint16_t* o = a.pool_out_large + ((long long)b * nlarge + lo / lb) * 2 * kD;
            const uint32_t hi = f32_to_bf16_bits(mean);
            o[d] = (uint16_t)hi;
            o[kD + d] = (uint16_t)f32_to_bf16_bits(mean - bf16_bits_to_f32(hi));
        }
    }
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
// get score -inf and index -1.  A workgroup takes one chunk of kGatherChunk
// candidates of its row, or with SWEEP (many rows) every gridDim.x-th chunk
// of the row with one load of the query fragments; in a chunk each wave
// resolves its kGatherGroups x 16 candidate ids, issues every key load
// (16 KiB in flight per wave), then runs the MFMA groups.  (Prefetching the
// next chunk's ids during the MFMAs costs a wave per SIMD and was slower.)
template <int NHT, bool BLOCKS, bool F8, bool SWEEP>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
    constexpr int NG = kGatherGroups;
    const int row = blockIdx.y;
    const int b = row / a.T;
    const int t = a.offset + (row - b * a.T);
    if (blockIdx.x * kGatherChunk >= a.ncand) return;
    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t* lrow = a.list + (long long)row * a.list_len;
    // candidate ids of the chunk at cs (the first chunk's list loads go out
    // before the query loads: load counters are in order, so a wait for the
    // keys would otherwise be a wait for the query as well)
    int sid[NG];
    auto resolve = [&](int cs, int (&ids)[NG]) {
        const int ce = min(cs + kGatherChunk, a.ncand);
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
            ids[gi] = (s >= 0 && s <= t && s < a.L) ? s : -1;
        }
    };
    int cs = blockIdx.x * kGatherChunk;
    resolve(cs, sid);
    QFrag<NHT> f;
    load_qfrag<NHT>(f, a.q + (long long)row * a.H * kD, a.w + (long long)row * a.H, a.H,
                    nullptr, 0, g, c);
    float* osc = a.out_score + (long long)row * a.ncand;
    int32_t* oid = a.out_idx + (long long)row * a.ncand;
    for (;;) {
        const int ce = min(cs + kGatherChunk, a.ncand);
        uint4 kb[NG][4];
        float ks[NG];
        if (F8) {
            // FP8 cache: the same dims as load_key (k-step kk, lane group g:
            // dims 32kk + 8g .. +8), widened exactly; the key's scale
            // multiplies the head sum.
            const uint8_t* cseq = a.codes + (long long)b * a.seq_stride;
            const float* sseq = a.kscale + (long long)b * (a.seq_stride / kD);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const long long s = sid[gi] >= 0 ? sid[gi] : 0;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint2 v =
                        *reinterpret_cast<const uint2*>(cseq + s * kD + 32 * kk + 8 * g);
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
        const int nxt = cs + gridDim.x * kGatherChunk;
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
        if (!SWEEP || nxt >= a.ncand) break;
        cs = nxt;
        resolve(cs, sid);
    }
}

// ----------------------------------------------------------- router

template <int NHT>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
    const int row = blockIdx.x;
    const int b = row / a.T;
    const int t = a.offset + (row - b * a.T);
    __shared__ int s_heads[kMaxH];
    __shared__ float s_w[kMaxH];
    RouteIn r;
    r.q = a.q + (long long)row * a.H * kD;
    r.w = a.w + (long long)row * a.H;
    r.reps = a.reps + (long long)b * a.seq_stride;
    r.tailp = (a.tail && a.tail_flag[row]) ? a.tail + (long long)row * 256 : nullptr;
    r.H = a.H;
    r.Mt = min(t / a.B + 1, a.nblk);
    r.h = a.h;
    r.E_out = a.E_out ? a.E_out + (long long)row * a.H : nullptr;
    route_wg<NHT>(r, s_heads, s_w);
    for (int u = threadIdx.x; u < a.h; u += 256) a.heads_out[(long long)row * a.h + u] = s_heads[u];
    // The routed heads' q rows and weights, for the fused prefill: 16 lanes
    // per head, 16 bytes each.
    if (a.qp) {
        for (int x = threadIdx.x; x < a.h * 16; x += 256) {
            const int u = x >> 4, part = x & 15;
            const int j = s_heads[u];
            const uint4 v = ldg16(a.q + ((long long)row * a.H + j) * kD + part * 8);
            *reinterpret_cast<uint4*>(a.qp + ((long long)row * a.h + u) * kD + part * 8) = v;
            if (part == 0) a.wp[(long long)row * a.h + u] = a.w[(long long)row * a.H + j];
        }
    }
    // The routed scan that follows adds its histogram into a zeroed row state
    // (one launch fewer on the MISA path).
    if (a.zero_state)
        for (int x = threadIdx.x; x < kRowState; x += 256)
            a.zero_state[(long long)row * kRowState + x] = 0u;
}

// Many rows with few blocks each (prefill rows): one row per wave.  The
// wave loads its row's q fragments and 32 representatives per pass (two
// groups of 16, lane column c = block), sums ReLU(q . rep) over its blocks,
// then ranks the heads itself, as route_finish does for a workgroup; no
// workgroup barrier.  (One row per 256-thread workgroup left three of its
// waves idle at 32 blocks and paid the row's load latency 4096 times.)
template <int NHT>
__global__ __launch_bounds__(256) void router_rows_kernel(RouterArgs a, int rows) {
    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * 4 + wid;
    if (row >= rows) return;  // wave-uniform
    const int b = row / a.T;
    const int t = a.offset + (row - b * a.T);
    const int Mt = min(t / a.B + 1, a.nblk);
    const uint16_t* reps = a.reps + (long long)b * a.seq_stride;
    const uint16_t* tailp =
        (a.tail && a.tail_flag[row]) ? a.tail + (long long)row * 256 : nullptr;
    QFrag<NHT> f;
    const uint32_t qv = load_qfrag_issue<NHT>(f, a.q + (long long)row * a.H * kD,
                                              a.w + (long long)row * a.H, a.H, nullptr, 0, g, c);
    uint4 kb[2][8];
    bool valid[2];
    auto load_reps = [&](int base) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int m = base + 16 * u + c;
            valid[u] = m < Mt;
            const int ml = valid[u] ? m : Mt - 1;
            const uint16_t* kp = (tailp && ml == Mt - 1) ? tailp : reps + (long long)ml * 256;
            load_key<8>(kb[u], kp, g);
        }
    };
    load_reps(0);
    mask_qfrag<NHT>(f, qv);
    float sum[NHT][4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[ht][i] = 0.f;
    for (int base = 0;;) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 acc[NHT];
            group_dots<NHT, 8>(f, kb[u], acc);
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
                for (int i = 0; i < 4; ++i) sum[ht][i] += valid[u] ? fmaxf(acc[ht][i], 0.f) : 0.f;
        }
        base += 32;
        if (base >= Mt) break;
        load_reps(base);
    }
    // E_j = |w_j| * mean over the blocks; absent heads rank below every real
    // head (E >= 0).  Lane j then ranks head j by (E desc, j asc).
    __shared__ float sE[4][kMaxH];
    __shared__ int sH[4][kMaxH];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = sum_row16(sum[ht][i]);
            const int j = ht * 16 + 4 * g + i;
            if (c == 0) sE[wid][j] = j < a.H ? fabsf(f.wv[ht][i]) * v / (float)Mt : -1.f;
        }
    for (int j = NHT * 16 + lane; j < kMaxH; j += 64) sE[wid][j] = -1.f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int j = lane;
    const float E = sE[wid][j];
    if (a.E_out && j < a.H) a.E_out[(long long)row * a.H + j] = E;
    int rank = 0;
#pragma unroll
    for (int j4 = 0; j4 < kMaxH; j4 += 4) {
        const float4 e4 = *reinterpret_cast<const float4*>(&sE[wid][j4]);
        const float es[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
            rank += (int)(es[u] > E) + (int)((es[u] == E) & (j4 + u < j));
    }
    const bool sel = j < a.H && rank < a.h;
    const unsigned long long msk = __ballot(sel);
    const int pos = __popcll(msk & ((1ull << lane) - 1ull));
    if (sel) {
        sH[wid][pos] = j;
        a.heads_out[(long long)row * a.h + pos] = j;
    }
    if (a.qp) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int x = lane; x < a.h * 16; x += 64) {
            const int u = x >> 4, part = x & 15;
            const int jj = sH[wid][u];
            const uint4 v = ldg16(a.q + ((long long)row * a.H + jj) * kD + part * 8);
            *reinterpret_cast<uint4*>(a.qp + ((long long)row * a.h + u) * kD + part * 8) = v;
            if (part == 0) a.wp[(long long)row * a.h + u] = a.w[(long long)row * a.H + jj];
        }
    }
    if (a.zero_state)
        for (int x = lane; x < kRowState; x += 64)
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
    // four keys per thread in flight (a long cut block is up to block - 1 keys)
    for (int s0 = lo + kl; s0 <= t; s0 += 64) {
        float x[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = s0 + 16 * u;
            if (s <= t) {
                key8_f32(kseq, cseq, sseq, s, c16, x[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += x[u][e];
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

template <int NHT>
static void scan_dispatch_pooled(const ScanArgs& a, dim3 grid, hipStream_t s) {
    constexpr int kFull = kScanPoolChunk / (scan_waves<4>() * 16 * scan_groups<4>());
    constexpr int G = scan_groups<4>();
    constexpr int NB = scan_bufs<4>();
    if (a.chunk == kScanPoolChunk)
        sa_launch(scan_kernel<NHT, 4, G, NB, kFull, true, false, true>, grid, dim3(64 * scan_waves<4>()), 0, s, a);
    else
        sa_launch(scan_kernel<NHT, 4, G, NB, 0, true, false, true>, grid, dim3(64 * scan_waves<4>()), 0, s, a);
}

hipError_t launch_scan_pooled(const ScanArgs& a, int rows, int nht, hipStream_t s) {
    const int maxn = a.len_cap;
    const dim3 grid((unsigned)((maxn + a.chunk - 1) / a.chunk), (unsigned)rows);
    prof_begin(K_SCAN_POOL, s);
    switch (nht) {
        case 1: scan_dispatch_pooled<1>(a, grid, s); break;
        case 2: scan_dispatch_pooled<2>(a, grid, s); break;
        case 3: scan_dispatch_pooled<3>(a, grid, s); break;
        default: scan_dispatch_pooled<4>(a, grid, s); break;
    }
    prof_end(K_SCAN_POOL, s);
    return hipGetLastError();
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
    if (ksteps != 4) {
        // Block representatives: one step per workgroup for few rows; a
        // row's whole block range per workgroup once rows alone give 8
        // workgroups per CU (prefill rows: the query fragments are loaded
        // once per row instead of once per 128 blocks).
        constexpr int step8 = scan_waves<8>() * 16 * scan_groups<8>();
        if (rows >= 8LL * cu_count())
            return std::min(kScanMaxChunk, (maxn + step8 - 1) / step8 * step8);
        return step8;
    }
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
    } else if (a.chunk == scan_waves<8>() * 16 * scan_groups<8>()) {
        // one step per workgroup: the loop unrolled to that step
        switch (nht) {
            case 1: scan_dispatch_hist<1, 8, 1>(a, grid, s); break;
            case 2: scan_dispatch_hist<2, 8, 1>(a, grid, s); break;
            case 3: scan_dispatch_hist<3, 8, 1>(a, grid, s); break;
            default: scan_dispatch_hist<4, 8, 1>(a, grid, s); break;
        }
    } else {
        // a row's whole block range: the stepping loop
        switch (nht) {
            case 1: scan_dispatch_hist<1, 8, 0>(a, grid, s); break;
            case 2: scan_dispatch_hist<2, 8, 0>(a, grid, s); break;
            case 3: scan_dispatch_hist<3, 8, 0>(a, grid, s); break;
            default: scan_dispatch_hist<4, 8, 0>(a, grid, s); break;
        }
    }
    prof_end(kid, s);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, int rows, int nht, bool block_mode,
                         hipStream_t s) {
    // Workgroups per row: every chunk its own for few rows; fewer, each
    // sweeping several chunks with one query load, once rows alone give
    // about 8 workgroups per CU.
    const int chunks = (a.ncand + kGatherChunk - 1) / kGatherChunk;
    const int want = (8 * cu_count() + rows - 1) / rows;
    const int per_row = std::max(1, std::min(chunks, want));
    const dim3 grid((unsigned)per_row, (unsigned)rows);
    prof_begin(K_GATHER, s);
#define SA_GATHER4(N, SW)                                                           \
    if (a.codes) {                                                                  \
        if (block_mode)                                                             \
            sa_launch(gather_kernel<N, true, true, SW>, grid, dim3(256), 0, s, a);  \
        else                                                                        \
            sa_launch(gather_kernel<N, false, true, SW>, grid, dim3(256), 0, s, a); \
    } else if (block_mode) {                                                        \
        sa_launch(gather_kernel<N, true, false, SW>, grid, dim3(256), 0, s, a);     \
    } else {                                                                        \
        sa_launch(gather_kernel<N, false, false, SW>, grid, dim3(256), 0, s, a);    \
    }
#define SA_GATHER(N)              \
    if (per_row < chunks) {       \
        SA_GATHER4(N, true)       \
    } else {                      \
        SA_GATHER4(N, false)      \
    }
    switch (nht) {
        case 1: SA_GATHER(1) break;
        case 2: SA_GATHER(2) break;
        case 3: SA_GATHER(3) break;
        default: SA_GATHER(4) break;
    }
#undef SA_GATHER4
#undef SA_GATHER
    prof_end(K_GATHER, s);
    return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& a, int rows, hipStream_t s) {
    const int nht = (a.H + 15) / 16;
    prof_begin(K_ROUTER, s);
    if (rows >= 4 * cu_count()) {
        // many rows (prefill): one row per wave
        const dim3 grid((unsigned)((rows + 3) / 4));
        switch (nht) {
            case 1: sa_launch(router_rows_kernel<1>, grid, dim3(256), 0, s, a, rows); break;
            case 2: sa_launch(router_rows_kernel<2>, grid, dim3(256), 0, s, a, rows); break;
            case 3: sa_launch(router_rows_kernel<3>, grid, dim3(256), 0, s, a, rows); break;
            default: sa_launch(router_rows_kernel<4>, grid, dim3(256), 0, s, a, rows); break;
        }
        prof_end(K_ROUTER, s);
        return hipGetLastError();
    }
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
