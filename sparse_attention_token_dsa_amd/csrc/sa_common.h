// Shared device helpers and host-side launch plumbing of the gfx950 indexer
// library.  Internal header: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // indexer head dim (bf16 elements per key)
constexpr int kMaxH = 64;        // heads supported
constexpr int kHist0Bits = 12;   // first radix digit = top 12 bits of the ordered score
constexpr int kHist0Bins = 1 << kHist0Bits;
constexpr int kScanMaxChunk = 4096;  // keys per scan workgroup (LDS score staging)
constexpr int kScanPoolChunk = 2048; // keys per workgroup of the scan that also pools
constexpr int kGatherGroups = 4;     // 16-candidate groups per gather wave
constexpr int kGatherChunk = 4 * 16 * kGatherGroups;
// Per-row state of the dense top-k, zeroed before each scan: the first-digit
// histogram, then control words.
constexpr int kRowState = kHist0Bins + 8;
enum RowCtl {
    CTL_EMITTED = 0,  // winners written by the filter
    CTL_CANDS = 1,    // threshold-digit candidates appended by the filter
    CTL_DONE = 2,     // scan workgroups finished
    CTL_NEED = 3,     // min(k, n)
    CTL_DIGIT = 4,    // first-digit value holding the k-th score
    CTL_GT = 5,       // scores above that digit
    CTL_EQ = 6        // scores on that digit
};

// ------------------------------------------------------------ scalars

// Order-preserving map float -> uint32: a > b  <=>  ord(a) > ord(b)
// (for non-NaN values; -0 sorts just below +0).
__device__ __forceinline__ uint32_t ord_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_to_f32(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

// Absolute position of query row `row`: offset + i, or with per-sequence
// lengths (ragged batches) len_b - T + i, len_b clamped to [T, cap].
__device__ __forceinline__ int row_pos(int row, int T, int offset, const int32_t* seq_lens,
                                       int cap) {
    const int b = row / T;
    const int i = row - b * T;
    if (!seq_lens) return offset + i;
    const int len = min(max(seq_lens[b], T), cap);
    return len - T + i;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ------------------------------------------------------------- MFMA

// D[16x16] += A[16x32] * B[32x16], bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l & 15) and B column (l & 15), each with the 8
// contraction elements of group (l >> 4); D lane l holds column (l & 15),
// rows 4*(l >> 4) + 0..3.  A and B only need to agree on which contraction
// element sits where, so callers may assign any 16-byte chunk to a group.
__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Two OCP E4M3 codes (bytes 0-1 of w, or 2-3 with HI) widened to two bf16
// values, exactly (every E4M3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, v);
}

// Eight E4M3 codes (two per 16-bit half of x and y) -> 8 bf16 values in dim
// order.
__device__ __forceinline__ uint4 widen8(uint32_t x, uint32_t y) {
    return make_uint4(fp8x2_to_bf16x2<false>(x), fp8x2_to_bf16x2<true>(x),
                      fp8x2_to_bf16x2<false>(y), fp8x2_to_bf16x2<true>(y));
}

// Dims 8p .. 8p+7 of key s of one sequence in fp32: the bf16 key (kseq), or
// with an FP8 cache (cseq != null) the codes times the key's scale sseq[s].
__device__ __forceinline__ void key8_f32(const uint16_t* kseq, const uint8_t* cseq,
                                         const float* sseq, long long s, int p, float (&x)[8]) {
    uint4 v;
    float a = 1.f;
    if (cseq) {
        const uint2 c = *reinterpret_cast<const uint2*>(cseq + s * 128 + p * 8);
        v = widen8(c.x, c.y);
        a = sseq[s];
    } else {
        v = ldg16(kseq + s * 128 + p * 8);
    }
    const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(wds[e] << 16) * a;
        x[2 * e + 1] = __uint_as_float(wds[e] & 0xffff0000u) * a;
    }
}

// 16-byte load of streamed data (keys read once per kernel), marked
// nontemporal: it streams past the caches instead of displacing lines that
// are reused.  On this chip it also raises the cold read rate (about 6.2
// TB/s against 5.6 for plain loads in a read-only kernel).
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroup barrier that orders LDS only: the waits before it cover LDS
// operations, so global loads in flight stay in flight (a plain
// __syncthreads() also waits for every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave on the VALU: row shifts
// 1, 2, 4, 8 inside each 16-lane row (lanes past the row start add 0), then
// lane 15 broadcast into rows 1 and 3 and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Wave-aggregated append: every lane of the wave must call it.  Lanes with
// pred get consecutive slots starting at an atomically reserved base.
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
    unsigned long long m = __ballot(pred);
    int lane = lane_id();
    int rank = __popcll(m & ((1ull << lane) - 1ull));
    int base = 0;
    if (m) {
        int leader = __ffsll((long long)m) - 1;
        if (lane == leader) base = atomicAdd(counter, __popcll(m));
        base = __builtin_amdgcn_readlane(base, leader);
    }
    return base + rank;
}

// ------------------------------------------------------ kernel ids

enum KernelId {
    K_FILL = 0,
    K_SCAN,
    K_SCAN_ROUTED,
    K_BLOCK_SCORE,
    K_TOPK,
    K_TOPK_FILTER,
    K_POOL,
    K_POOL2,
    K_TAIL,
    K_ROUTER,
    K_GATHER,
    K_PREFILL,
    K_QUANT8,
    K_SCAN8,
    K_EXTREMA,
    K_RES_ROUTER,
    K_HEAD_ROWS,
    K_TIDY,
    K_SCAN8Q,
    K_SCAN_POOL,
    K_PREFILL_FP8,
    K_COUNT
};

// Host side: bracket a launch with profiling events when enabled.
// Per-kernel timing (sa_profile_enable).  prof_begin(kid, s) opens a record
// whose events the next sa_launch on this host thread attaches to its own
// dispatch (hipExtLaunchKernelGGL), so they time the kernel and not the
// dispatch gap before it; prof_end closes the record (dropped if no kernel
// was launched in between).
void prof_begin(int kid, hipStream_t s);
void prof_end(int kid, hipStream_t s);
bool prof_pending(hipEvent_t* start, hipEvent_t* stop);  // takes the open record's events
void prof_reset_thread();

// Every kernel launch of the library goes through here.
template <typename... KArgs, typename... Args>
inline void sa_launch(void (*kern)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                      Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (prof_pending(&e0, &e1))
        hipExtLaunchKernelGGL(kern, grid, block, lds, s, e0, e1, 0u, static_cast<KArgs>(args)...);
    else
        kern<<<grid, block, lds, s>>>(static_cast<KArgs>(args)...);
}

// ---------------------------------------------------- launch records

// Score scan over a contiguous legal key range per query row.
struct ScanArgs {
    const uint16_t* q;      // [rows, H, 128]
    const float* w;         // [rows, H]
    const uint16_t* keys;   // key rows of kstep*32 bf16 each
    long long seq_stride;   // elements between sequences in `keys`
    const uint16_t* tail;   // block reps only: per-row partial rep [rows, 256] or null
    const uint8_t* tail_flag;
    const int32_t* heads;   // routed: [rows, hsel]
    int hsel;
    int T, H, offset;
    int len_div, len_cap;   // legal count n = min(t / len_div + 1, len_cap)
    int chunk;              // keys per workgroup (multiple of 128)
    float* scores;          // [rows, score_stride]
    long long score_stride;
    uint32_t* state;        // [rows, kRowState] (zeroed) or null: build the first-digit
                            // histogram and the k-th-score digit for the dense top-k
    int k;                  // top-k size for the state
    // FP8 keys instead of `keys` (decode keys only): E4M3 codes, 128 bytes per
    // key, sequences seq_stride bytes apart, and one fp32 scale per key
    // (sequences seq_stride / 128 apart).
    const uint8_t* codes;
    const float* kscale;
    // Ragged batches: per-sequence lengths [batch] (row positions from
    // row_pos with cap = len_cap), or null.
    const int32_t* seq_lens;
    // FP8 keys only: the query converted to E4M3 as well (per-head scale
    // folded into the weight) and the contraction on the fp8 MFMA.
    int q_fp8;
    // Block means of the streamed keys (decode rows that read every key of
    // their sequence once): [batch, ceil(L / pool_small), 2, 128] and the same
    // for pool_large, hi/lo bf16 like sa_pool_blocks.  pool_small is a power
    // of two >= 128, pool_large a multiple of it; the chunk is a multiple of
    // pool_large.  Null: no pooling.
    uint16_t* pool_out_small;
    uint16_t* pool_out_large;
    int pool_small, pool_large;
    int pool_shift;         // log2(pool_small / 64): workgroup steps per small block
    // Routed key scans (decode rows) that route their row themselves: every
    // workgroup of the row runs the MISA router on the row's pooled blocks
    // (route_reps: [batch, route_nblk, 256] hi/lo, route_seq_stride elements
    // apart; blocks of route_B keys, none cut by the causal bound) before its
    // keys, and the row's first workgroup writes the hsel routed heads,
    // ascending, to route_heads_out [rows, hsel].  Null route_reps: the heads
    // come from `heads`.
    const uint16_t* route_reps;
    long long route_seq_stride;
    int route_B, route_nblk;
    int32_t* route_heads_out;
};

struct GatherArgs {
    const uint16_t* q;
    const float* w;
    const uint16_t* keys;   // [batch, L, 128]
    long long seq_stride;
    const int32_t* list;    // [rows, list_len]
    int list_len;
    int bsz;                // block mode: tokens per listed block
    int ncand;              // candidates per row
    int T, H, L, offset;
    float* out_score;       // [rows, ncand]
    int32_t* out_idx;       // [rows, ncand]
    // FP8 key cache instead of `keys` (codes [batch, L, 128] with the same
    // seq_stride, one fp32 scale per key), or null.
    const uint8_t* codes;
    const float* kscale;
};

struct RouterArgs {
    const uint16_t* q;
    const float* w;
    const uint16_t* reps;   // [batch, nblk, 256] hi/lo
    long long seq_stride;
    const uint16_t* tail;
    const uint8_t* tail_flag;
    int T, H, offset, B, nblk, h;
    int32_t* heads_out;     // [rows, h]
    float* E_out;           // [rows, H] or null
    uint32_t* zero_state;   // [rows, kRowState] cleared for the routed scan that follows, or null
    // Routed head rows for the fused prefill, or null: qp [rows, h, 128] =
    // q of the routed heads (ascending), wp [rows, h] their weights.
    uint16_t* qp;
    float* wp;
};

// LISA / ResMiSA head rows and routing.
struct ResmisaArgs {
    const uint16_t* q;      // [rows, H, 128]
    const float* w;         // [rows, H]
    const uint16_t* ext;    // [batch, nblk, 2, 128]: per-block key max, then min
    const uint16_t* tail;   // [rows, 2, 128] extrema of a cut last block, or null
    const uint8_t* tail_flag;
    int T, H, offset, block, nblk;
    int r;                  // routed residual heads (0: LISA)
    int Hp;                 // output heads per row: 4 + r, or H when r == H
    float* part;            // [rows, nchunk, H]: max_b ReLU(U-) per router workgroup
    int nchunk;             // router workgroups per row (64 blocks each)
    int32_t* heads_out;     // [rows, r] ascending, or null
    uint16_t* qp;           // [rows, Hp, 128] output head rows
    float* wp;              // [rows, Hp] output weights
    uint32_t* zero_state;   // [rows, kRowState] to clear for the decode scan, or null
};

// Index tidy-up: per row, physical slots sorted ascending, unique, -1 padded.
constexpr int kTidyMax = 4096;          // selected indices per row (sorting form)
constexpr int kTidyBitmapMax = 1 << 18;  // slot bound of the bitmap form (32 KiB of LDS)
struct TidyArgs {
    const int32_t* idx;     // [rows, k], -1 = empty
    int k, T;
    int n2;                 // sort width: power of two >= max(k, 256)
    int max_slots;          // slots >= max_slots are dropped (0: no bound)
    const int32_t* table;   // [batch, pages_per_seq] physical page of each logical page, or null
    int pages_per_seq, page;
    int32_t* out_slots;     // [rows, k]
    int32_t* out_stats;     // [rows, 3]: unique slots, distinct pages, contiguous runs; or null
};

struct TopkArgs {
    // dense source: scores[row * dense_stride + s], s < n(row)
    const float* dense;
    long long dense_stride;
    int T, offset, len_div, len_cap;
    // list source: (list_score, list_idx)[row * list_stride + u], u < count(row);
    // entries with idx < 0 are skipped
    const float* list_score;
    const int32_t* list_idx;
    long long list_stride;
    const int32_t* list_count;  // per-row counts or null (then list_cap)
    int list_cap;
    uint32_t* state;            // dense filter path: per-row state left by the scan
    int k;
    int32_t* out_idx;           // [rows, out_stride]
    float* out_score;           // nullable
    long long out_stride;
    long long cand_cap;         // candidate keys per row (filter path)
    const int32_t* seq_lens;    // ragged batches (dense source): as in ScanArgs, or null
};

struct PrefillArgs {
    const uint16_t* q;
    const float* w;
    const uint16_t* keys;
    int T, H, L, offset, k;
    uint2* surv;                // [rows, cap] (position, score bits) survivor lists (workspace)
    long long cap;              // survivor slots per row, even: >= offset + T (every
                                // legal key), or >= k + 384 (compacted when full)
    int32_t* out_idx;           // [rows, out_stride]
    float* out_score;           // nullable
    long long out_stride;
    // Ragged batches: per-sequence key counts [batch] (clamped to [T, L]); the
    // rows of sequence b sit at seq_lens[b] - T + i instead of offset + i.
    const int32_t* seq_lens;
    // FP8 key cache (keys unused): E4M3 codes [batch, L, 128] and one fp32
    // scale per key [batch, L]; the query is quantized to E4M3 in the kernel
    // (per head, the key rule) and the contraction runs on the fp8 MFMA.
    const uint8_t* codes;
    const float* kscale;
};

// Launchers (defined next to their kernels).
hipError_t launch_fill_u32(uint32_t* p, long long n, uint32_t v, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, int rows, int nht, int ksteps, bool routed,
                       hipStream_t s);
// The DSA decode scan (keys, every row's whole history) that also writes the
// block means of the keys it streams (a.pool_out_small / a.pool_out_large).
hipError_t launch_scan_pooled(const ScanArgs& a, int rows, int nht, hipStream_t s);
// Keys per scan workgroup for 4 (keys) or 8 (block reps) k-steps, rows x maxn keys.
int scan_chunk(int ksteps, long long rows, int maxn);
// FP8 key scan (DSA decode rows): scores of codes/kscale keys, chunk from scan8_chunk.
hipError_t launch_scan8(const ScanArgs& a, int rows, int nht, hipStream_t s);
int scan8_chunk(long long rows, int maxn);
int cu_count();  // compute units of the current device (cached per device)
hipError_t launch_gather(const GatherArgs& a, int rows, int nht, bool block_mode,
                         hipStream_t s);
hipError_t launch_router(const RouterArgs& a, int rows, hipStream_t s);
// keys, or codes + scales (FP8 cache) when codes is not null.
hipError_t launch_tail(const uint16_t* keys, long long seq_stride, int T, int offset, int L,
                       int block, int rows, uint16_t* tail, uint8_t* flag, hipStream_t s,
                       const uint8_t* codes = nullptr, const float* scales = nullptr);
hipError_t launch_topk(const TopkArgs& a, int rows, hipStream_t s);
// Dense rows scanned with a row state: multi-workgroup filter + per-row finish.
// cand: [rows, a.cand_cap] keys.
hipError_t launch_topk_dense_filtered(const TopkArgs& a, int rows, int maxn,
                                      unsigned long long* cand, hipStream_t s);
hipError_t launch_pool(const uint16_t* keys, int batch, int L, int block, uint16_t* out,
                       hipStream_t s, const uint8_t* codes = nullptr,
                       const float* scales = nullptr);
hipError_t launch_pool2(const uint16_t* keys, int batch, int L, int small, int large,
                        uint16_t* out_small, uint16_t* out_large, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int rows, hipStream_t s);
// LISA / ResMiSA: block extrema, cut-block extrema, routing, head rows.
hipError_t launch_extrema(const uint16_t* keys, int batch, int L, int block, uint16_t* out,
                          hipStream_t s);
hipError_t launch_extrema_tail(const uint16_t* keys, long long seq_stride, int T, int offset,
                               int L, int block, int rows, uint16_t* tail, uint8_t* flag,
                               hipStream_t s);
hipError_t launch_resmisa_router(const ResmisaArgs& a, int rows, hipStream_t s);
hipError_t launch_head_rows(const ResmisaArgs& a, int rows, hipStream_t s);
hipError_t launch_tidy(const TidyArgs& a, int rows, hipStream_t s);
// Per-key FP8 quantization of n keys of 128 bf16 values.
hipError_t launch_quantize_fp8(const uint16_t* keys, long long n, uint8_t* codes, float* scales,
                               hipStream_t s);

}  // namespace sa
