// Decode scan over an FP8 key cache: the DSA score of every causal key of
// one query row, with the keys held as OCP E4M3 codes (128 bytes per key)
// and one fp32 scale per key (PaperTrace, "2.3 from the formula to the FP8
// cache").  The score is
//   I = a_s * sum_j w_j * ReLU(q_j . decode(c_s)),
// which equals the score of the dequantized key a_s * decode(c_s) because
// the scale is positive and ReLU commutes with it.  Every E4M3 value is a
// bf16 value, so the codes are widened exactly and the contraction runs on
// the bf16 MFMA with the same fp32 accumulation as the bf16 key path.
//
// Per wave and step: 16 keys (2 KiB of codes).  The codes go to LDS as they
// come from HBM, each lane reads back 32 consecutive bytes of one key, and
// widens them to bf16 in registers.  The contraction does not care about the
// order of the key dims, so lane group g takes dims 32g .. 32g+31 of key c
// (k-step kk: dims 32g + 8kk .. +8), and the q fragments are loaded with the
// same permutation.  Loads run 3 steps ahead (4-slot register ring), the
// MFMAs of a step are interleaved with the head sum of the step before, and
// buffer loads past the end of the chunk return zeros, so no address needs
// clamping and every step of the unrolled loop is uniform.
//
// With the query converted to E4M3 as well (the section's "query converted to
// the compute type"): each head vector is quantized by the key-cache rule
// (b = max|q|/448, codes of q/b in fp32, round to nearest even, saturating) by
// the whole workgroup into LDS, b is folded into the fp32 weight, and the
// contraction of 16 keys x 16 heads x all 128 dims is one 16x16x128 fp8 MFMA
// fed by the codes as they sit in LDS: a quarter of the matrix instructions
// of the widened path and no widening.
#include "sa_frag.h"

namespace sa {

namespace {

constexpr int kS8Waves = 8;                 // 512 threads: two waves per SIMD
constexpr int kS8Step = kS8Waves * 16;      // keys per workgroup step
constexpr int kS8Ring = 4;                  // register ring of loaded steps
constexpr int kS8Ahead = kS8Ring - 1;       // steps of loads in flight
// Step i stages step i+1 before it issues the load of step i + kS8Ahead, so
// the load of step i+1 must have been issued in an earlier step.
static_assert(kS8Ring >= 3, "the register ring must hold at least three steps");
static_assert(64 * kS8Waves == kMaxH * 8, "the query quantizer takes 8 threads per head");
constexpr int kBufFlags = 0x00020000;       // raw buffer, 32-bit elements
constexpr int kNontemporal = 2;             // cache policy bit of a streaming load

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// The workgroup (512 threads: 8 per head, 16 dims each) quantizes the query
// row's head vectors into LDS: scale b = max|q| / 448 (1 for a zero vector),
// codes of q / b clamped to +-448 and rounded to nearest even.  Heads at or
// past H get zero codes and scale 1.  q8_load issues the thread's two loads
// (head 0 stands in for absent heads), q8_store quantizes once they landed.
__device__ __forceinline__ void q8_load(const uint16_t* qrow, int H, uint4& v0, uint4& v1) {
    const int h = threadIdx.x >> 3, part = threadIdx.x & 7;
    const uint16_t* p = qrow + (h < H ? h : 0) * kD + part * 16;
    v0 = ldg16(p);
    v1 = ldg16(p + 8);
}
__device__ __forceinline__ void q8_store(const uint4& v0, const uint4& v1, int H, uint4* qcode,
                                         float* qscale) {
    const int h = threadIdx.x >> 3, part = threadIdx.x & 7;
    const uint32_t wds[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float x[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[2 * e] = h < H ? bf16_bits_to_f32(wds[e] & 0xffffu) : 0.f;
        x[2 * e + 1] = h < H ? bf16_bits_to_f32(wds[e] >> 16) : 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[e]));
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 8));
    const float b = m > 0.f ? m / 448.0f : 1.0f;
    uint32_t out[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[4 * u + e] / b, -448.0f), 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
        out[u] = (uint32_t)pk;
    }
    qcode[qslot(h, part)] = make_uint4(out[0], out[1], out[2], out[3]);
    if (part == 0) qscale[h] = b;
}

// q fragments in the permuted dim order: head tile ht, row c = head slot
// ht*16 + c; lane group g of k-step kk holds dims 32g + 8kk .. +8.  A slot is
// head u itself, or with a routed head list (heads, hsel: MISA's routed
// scan) the u-th listed head.  The head ids come first (the routed list in
// one batch of loads), then every q / w load back to back with no wait in
// between; absent slots (past H or hsel) load head 0 and are returned as
// clear bits of the weight mask, for mask_qfrag8 to zero their weights once
// the loads have landed (zero weight is enough: their dot products are
// finite and are multiplied by it).
template <int NHT>
__device__ __forceinline__ uint32_t load_qfrag8(QFrag<NHT>& f, const uint16_t* qrow,
                                                const float* wrow, int H,
                                                const int32_t* heads, int hsel, int g, int c) {
    int ha[NHT], hw[NHT][4];
    bool va[NHT], vw[NHT][4];
    if (heads) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            ha[ht] = head_at<true>(ht * 16 + c, H, heads, hsel, va[ht]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hw[ht][i] = head_at<true>(ht * 16 + 4 * g + i, H, heads, hsel, vw[ht][i]);
        }
    } else {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            ha[ht] = head_at<false>(ht * 16 + c, H, heads, hsel, va[ht]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hw[ht][i] = head_at<false>(ht * 16 + 4 * g + i, H, heads, hsel, vw[ht][i]);
        }
    }
    uint32_t wmask = 0u;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const uint16_t* qp = qrow + ha[ht] * kD + 32 * g;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) f.a[ht][kk] = ldg16(qp + 8 * kk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.wv[ht][i] = wrow[hw[ht][i]];
            if (vw[ht][i]) wmask |= 1u << (4 * ht + i);
        }
    }
    return wmask;
}

template <int NHT>
__device__ __forceinline__ void mask_qfrag8(QFrag<NHT>& f, uint32_t wmask) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (!((wmask >> (4 * ht + i)) & 1u)) f.wv[ht][i] = 0.f;
}

// MFMA i of a step, then nv VALU instructions of the previous step's head sum.
template <int I, int M, int V>
__device__ __forceinline__ void s8_interleave() {
    if constexpr (I < M) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        constexpr int nv = V * (I + 1) / M - V * I / M;
        if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x002, nv, 0);
        s8_interleave<I + 1, M, V>();
    }
}

template <int NHT, bool HIST, bool QF8>
__global__ __launch_bounds__(64 * kS8Waves) void scan8_kernel(ScanArgs a) {
    const int row = blockIdx.y;
    const int b = row / a.T;
    const int t = row_pos(row, a.T, a.offset, a.seq_lens, a.len_cap);
    int n = t / a.len_div + 1;
    if (n > a.len_cap) n = a.len_cap;
    const int cs = blockIdx.x * a.chunk;
    if (cs >= n) return;
    const int ce = min(cs + a.chunk, n);
    const int len = ce - cs;

    __shared__ uint32_t lhist[HIST ? kHist0Bins : 1];
    __shared__ float sbuf[kScanMaxChunk];
    // Per wave, two tiles of 16 keys x 8 chunks of 16 bytes; key r's chunk m
    // sits in slot r*8 + (m ^ (r & 7)), so both the row writes and the
    // per-key reads of 8 consecutive lanes hit 8 different bank groups.
    __shared__ uint4 tile[kS8Waves][2][128];
    __shared__ uint4 qcode[QF8 ? kMaxH * 8 : 1];
    __shared__ float qscale[QF8 ? kMaxH : 1];

    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    QFrag<NHT> f;
    QFrag8<NHT> f8;
    const uint16_t* qrow = a.q + (long long)row * a.H * kD;
    const float* wrow = a.w + (long long)row * a.H;
    // The query's loads are issued first and used only after the key
    // prefetch below is in flight.
    uint4 qv0, qv1;
    uint32_t wmask = 0u;
    if constexpr (QF8)
        q8_load(qrow, a.H, qv0, qv1);
    else
        wmask = load_qfrag8<NHT>(f, qrow, wrow, a.H,
                                 a.heads ? a.heads + (long long)row * a.hsel : nullptr, a.hsel,
                                 g, c);
    float (&wv)[NHT][4] = QF8 ? f8.wv : f.wv;

    const uint8_t* cbase = a.codes + (long long)b * a.seq_stride + (long long)cs * kD;
    const float* sbase = a.kscale + (long long)b * (a.seq_stride / kD) + cs;
    const int wkey = wid * 16;
    // Loads: lane l takes chunk l%8 of key l/8 (and of key 8 + l/8) of the
    // wave's 16, so each load instruction reads 8 whole keys; the scale of
    // key c goes to every lane of column c.
    const int voff0 = (wkey + (lane >> 3)) * kD + (lane & 7) * 16;
    const int voff1 = voff0 + 8 * kD;
    const int voffs = (wkey + c) * 4;
    const int wsl0 = (lane >> 3) * 8 + ((lane & 7) ^ (lane >> 3));
    const int wsl1 = wsl0 + 64;
    const int rsl0 = c * 8 + ((2 * g) ^ (c & 7));
    const int rsl1 = c * 8 + ((2 * g + 1) ^ (c & 7));
    uint4* const tw = &tile[wid][0][0];

    u32x4 lc0[kS8Ring], lc1[kS8Ring];
    uint32_t ls[kS8Ring];
    auto load = [&](int i, int slot) __attribute__((always_inline)) {
        const int k0 = i * kS8Step;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(cbase) + (long long)k0 * kD, (short)0,
            max(len - k0, 0) * kD, kBufFlags);
        lc0[slot] = __builtin_amdgcn_raw_buffer_load_b128(rc, voff0, 0, kNontemporal);
        lc1[slot] = __builtin_amdgcn_raw_buffer_load_b128(rc, voff1, 0, kNontemporal);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(sbase) + k0, (short)0, max(len - k0, 0) * 4, kBufFlags);
        ls[slot] = __builtin_amdgcn_raw_buffer_load_b32(rs, voffs, 0, 0);
    };
    auto stage = [&](int p, int slot) __attribute__((always_inline)) {
        const u32x4 v0 = lc0[slot], v1 = lc1[slot];
        tw[p * 128 + wsl0] = make_uint4(v0.x, v0.y, v0.z, v0.w);
        tw[p * 128 + wsl1] = make_uint4(v1.x, v1.y, v1.z, v1.w);
    };
    uint4 r0, r1;
    auto fetch = [&](int p) __attribute__((always_inline)) {
        r0 = tw[p * 128 + rsl0];
        r1 = tw[p * 128 + rsl1];
    };
    f32x4 acc[2][NHT];
    float scl[2];
    // Head sum of a finished step: sum_j w_j ReLU(dot_j) over the lane's 4
    // rows per head tile, then over the 4 lane groups, times the key scale.
    auto head_sum = [&](int p) __attribute__((always_inline)) -> float {
        float part[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            part[ht] = wv[ht][0] * fmaxf(acc[p][ht][0], 0.f);
#pragma unroll
            for (int e = 1; e < 4; ++e) part[ht] = fmaf(wv[ht][e], fmaxf(acc[p][ht][e], 0.f), part[ht]);
        }
        float sc = part[0];
#pragma unroll
        for (int ht = 1; ht < NHT; ++ht) sc += part[ht];
        return sum_lane_groups(sc) * scl[p];
    };
    // Step i's key scores into the chunk's LDS row (steps outside the chunk,
    // including the step before the first, store nothing).
    auto store = [&](float sc, int i) __attribute__((always_inline)) {
        const int rel = i * kS8Step + wkey + c;
        if (g == 0 && (unsigned)rel < (unsigned)len) {
            sbuf[rel] = sc;
            if (HIST) atomicAdd(&lhist[ord_key(sc) >> (32 - kHist0Bits)], 1u);
        }
    };

    // Prologue: loads of steps 0 .. kS8Ahead-1 (in flight while the
    // histogram is cleared and the query finished), step 0 staged and
    // fetched.
#pragma unroll
    for (int u = 0; u < kS8Ahead; ++u) load(u, u);
    if (HIST)
        for (int x = threadIdx.x; x < kHist0Bins; x += 64 * kS8Waves) lhist[x] = 0u;
    if constexpr (QF8)
        q8_store(qv0, qv1, a.H, qcode, qscale);
    else
        mask_qfrag8<NHT>(f, wmask);
    // LDS only: a full barrier would also wait for the loads just issued
    if (HIST || QF8) lds_barrier();
    if constexpr (QF8) load_qfrag_fp8<NHT>(f8, qcode, qscale, wrow, a.H, g, c);
    stage(0, 0);
    fetch(0);
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) acc[1][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    scl[1] = 0.f;

    const int nsteps = (len + kS8Step - 1) / kS8Step;
#pragma unroll 1
    for (int i0 = 0; i0 < nsteps; i0 += kS8Ring) {
#pragma unroll
        for (int u = 0; u < kS8Ring; ++u) {
            const int i = i0 + u;
            const int p = u & 1;
            scl[p] = __uint_as_float(ls[u]);
            if constexpr (QF8) {
                const i32x8 kb = {(int)r0.x, (int)r0.y, (int)r0.z, (int)r0.w,
                                  (int)r1.x, (int)r1.y, (int)r1.z, (int)r1.w};
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht) acc[p][ht] = mfma16x16x128_fp8(f8.a[ht], kb);
            } else {
                uint4 kb[4];
                kb[0] = widen8(r0.x, r0.y);
                kb[1] = widen8(r0.z, r0.w);
                kb[2] = widen8(r1.x, r1.y);
                kb[3] = widen8(r1.z, r1.w);
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht) acc[p][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int ht = 0; ht < NHT; ++ht)
                        acc[p][ht] = mfma16x16x32(f.a[ht][kk], kb[kk], acc[p][ht]);
            }
            const float sc = head_sum(1 - p);
            stage(1 - p, (u + 1) % kS8Ring);
            fetch(1 - p);
            load(i + kS8Ahead, (u + kS8Ahead) % kS8Ring);
            // (With four MFMAs a step the compiler's own order is as fast.)
            if constexpr (!QF8) s8_interleave<0, 4 * NHT, 8 * NHT + 8>();
            store(sc, i - 1);
        }
    }
    const int last = (nsteps + kS8Ring - 1) / kS8Ring * kS8Ring - 1;
    store(head_sum(1), last);

    lds_barrier();
    float* srow = a.scores + (long long)row * a.score_stride;
    for (int x = threadIdx.x; x < len; x += 64 * kS8Waves) srow[cs + x] = sbuf[x];
    if (HIST) {
        uint32_t* grow = a.state + (long long)row * kRowState;
        for (int x = threadIdx.x; x < kHist0Bins; x += 64 * kS8Waves) {
            const uint32_t v = lhist[x];
            if (v) atomicAdd(&grow[x], v);
        }
    }
}

template <int NHT, bool QF8>
void scan8_dispatch(const ScanArgs& a, dim3 grid, hipStream_t s) {
    if (a.state)
        sa_launch(scan8_kernel<NHT, true, QF8>, grid, dim3(64 * kS8Waves), 0, s, a);
    else
        sa_launch(scan8_kernel<NHT, false, QF8>, grid, dim3(64 * kS8Waves), 0, s, a);
}

template <bool QF8>
void scan8_heads(const ScanArgs& a, dim3 grid, int nht, hipStream_t s) {
    switch (nht) {
        case 1: scan8_dispatch<1, QF8>(a, grid, s); break;
        case 2: scan8_dispatch<2, QF8>(a, grid, s); break;
        case 3: scan8_dispatch<3, QF8>(a, grid, s); break;
        default: scan8_dispatch<4, QF8>(a, grid, s); break;
    }
}

}  // namespace

// Keys per workgroup: about one workgroup per CU, a multiple of a whole
// unrolled loop (kS8Ring steps), at most kScanMaxChunk.
int scan8_chunk(long long rows, int maxn) {
    constexpr int unit = kS8Step * kS8Ring;
    const long long wgs = cu_count();
    long long c = (rows * (long long)maxn + wgs - 1) / wgs;
    c = (c + unit - 1) / unit * unit;
    c = c > kScanMaxChunk ? kScanMaxChunk : c;
    return (int)c;
}

hipError_t launch_scan8(const ScanArgs& a, int rows, int nht, hipStream_t s) {
    const dim3 grid((unsigned)((a.len_cap + a.chunk - 1) / a.chunk), (unsigned)rows);
    const int id = a.q_fp8 ? K_SCAN8Q : K_SCAN8;
    prof_begin(id, s);
    if (a.q_fp8)
        scan8_heads<true>(a, grid, nht, s);
    else
        scan8_heads<false>(a, grid, nht, s);
    prof_end(id, s);
    return hipGetLastError();
}

}  // namespace sa
