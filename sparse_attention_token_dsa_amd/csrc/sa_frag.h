// Query-fragment helpers shared by the MFMA score kernels.  Internal header.
//
// One query's heads form the M dimension of v_mfma_f32_16x16x32_bf16 (16
// heads per tile), 16 keys form N, and the 128 key dims are the contraction,
// split in 4 steps of 32.  The indexer epilogue sum_j w_j * ReLU(z_j) runs on
// the accumulator registers (PaperTrace, "2.2.2 MISA, LISA and ResMiSA",
// section 1).
#pragma once

#include "sa_common.h"

namespace sa {

// ------------------------------------------------------------ fragments

// A fragments of one query: tile ht covers heads ht*16 .. ht*16+15 (row c of
// the tile = lane & 15); contraction group g = lane >> 4 of step kk holds
// dims (kk*4 + g)*8 .. +8.  wv[ht][i] is the weight of output row 4g+i.
template <int NHT>
struct QFrag {
    uint4 a[NHT][4];
    float wv[NHT][4];
};

// Head of tile row u: identity over H, or entry u of a routed head list.
// Returns a loadable head id (0 when absent) and sets `valid`.
template <bool ROUTED>
__device__ __forceinline__ int head_at(int u, int H, const int32_t* heads, int hsel, bool& valid) {
    if (ROUTED) {
        const int v = heads[u < hsel ? u : hsel - 1];
        valid = u < hsel && v >= 0 && v < H;
        return valid ? v : 0;
    }
    valid = u < H;
    return valid ? u : 0;
}

// All head ids first, then every q / w load back to back (no branches).
// Returns the slots' validity (bit ht: q row of tile ht; bit 8 + 4 ht + i:
// weight i of tile ht) for mask_qfrag, which zeroes the absent slots once the
// loads have landed: a caller can issue other loads in between.
template <int NHT, bool ROUTED = false>
__device__ __forceinline__ uint32_t load_qfrag_issue(QFrag<NHT>& f, const uint16_t* qrow,
                                                     const float* wrow, int H,
                                                     const int32_t* heads, int hsel, int g,
                                                     int c) {
    int ha[NHT], hw[NHT][4];
    uint32_t valid = 0u;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        bool va;
        ha[ht] = head_at<ROUTED>(ht * 16 + c, H, heads, hsel, va);
        if (va) valid |= 1u << ht;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bool vw;
            hw[ht][i] = head_at<ROUTED>(ht * 16 + 4 * g + i, H, heads, hsel, vw);
            if (vw) valid |= 1u << (8 + 4 * ht + i);
        }
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) f.a[ht][kk] = ldg16(qrow + ha[ht] * kD + (kk * 4 + g) * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) f.wv[ht][i] = wrow[hw[ht][i]];
    }
    return valid;
}

template <int NHT>
__device__ __forceinline__ void mask_qfrag(QFrag<NHT>& f, uint32_t valid) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        if (!((valid >> ht) & 1u))
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.a[ht][kk] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (!((valid >> (8 + 4 * ht + i)) & 1u)) f.wv[ht][i] = 0.f;
    }
}

// Both steps in one (the fused prefill at 256 VGPRs spills ten times more
// with the two-step form: its register allocation is that tight).
template <int NHT, bool ROUTED = false>
__device__ __forceinline__ void load_qfrag(QFrag<NHT>& f, const uint16_t* qrow,
                                           const float* wrow, int H, const int32_t* heads,
                                           int hsel, int g, int c) {
    int ha[NHT], hw[NHT][4];
    bool va[NHT], vw[NHT][4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        ha[ht] = head_at<ROUTED>(ht * 16 + c, H, heads, hsel, va[ht]);
#pragma unroll
        for (int i = 0; i < 4; ++i) hw[ht][i] = head_at<ROUTED>(ht * 16 + 4 * g + i, H, heads, hsel, vw[ht][i]);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) f.a[ht][kk] = ldg16(qrow + ha[ht] * kD + (kk * 4 + g) * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) f.wv[ht][i] = wrow[hw[ht][i]];
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        if (!va[ht])
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.a[ht][kk] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (!vw[ht][i]) f.wv[ht][i] = 0.f;
    }
}

// Sum of a value over the 16 lanes of its row (lanes 16g .. 16g+15): four
// DPP row rotations (8, 4, 2, 1) on the VALU, no LDS round trips.  Every
// lane of the row ends with the row's sum (the rounding order depends on the
// lane; callers read one fixed lane).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xf, 0xf,
                                                      false));
}
__device__ __forceinline__ float sum_row16(float v) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    v += row_ror<1>(v);
    return v;
}

// Sum of a value over the four 16-lane groups (lanes l, l^16, l^32, l^48),
// returned in every lane: two gfx950 row swaps, no LDS traffic.
__device__ __forceinline__ float sum_lane_groups(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                              false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                               false);
    return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// Raw per-head dot products of one 16-key group: acc[ht][i] = q_{ht*16+4g+i} . k_c.
// KSTEPS = 8 is the hi/lo split representative (q . hi + q . lo).
template <int NHT, int KSTEPS>
__device__ __forceinline__ void group_dots(const QFrag<NHT>& f, const uint4 (&b)[KSTEPS],
                                           f32x4 (&acc)[NHT]) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) acc[ht] = mfma16x16x32(f.a[ht][kk & 3], b[kk], acc[ht]);
}

// Indexer score of key column c, returned in every lane of the column.
template <int NHT, int KSTEPS>
__device__ __forceinline__ float group_score(const QFrag<NHT>& f, const uint4 (&b)[KSTEPS]) {
    f32x4 acc[NHT];
    group_dots<NHT, KSTEPS>(f, b, acc);
    float sc = 0.f;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc = fmaf(f.wv[ht][i], fmaxf(acc[ht][i], 0.f), sc);
    return sum_lane_groups(sc);
}

template <int KSTEPS>
__device__ __forceinline__ void load_key(uint4 (&b)[KSTEPS], const uint16_t* kp, int g) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) b[kk] = ldg16(kp + (kk * 4 + g) * 8);
}

// ------------------------------------------------------ E4M3 operands

typedef int i32x8 __attribute__((ext_vector_type(8)));

// q codes for the fp8 MFMA: per head tile, lane (c, g) holds 32 codes of head
// ht*16 + c, dims 32g .. 32g+31, the same dims as the key operand of lane g.
template <int NHT>
struct QFrag8 {
    i32x8 a[NHT];
    float wv[NHT][4];
};

// Codes of a head vector in LDS: [head][8 chunks of 16 codes], chunk m of
// head h in slot h*8 + (m ^ (h & 7)).
__device__ __forceinline__ int qslot(int h, int m) { return h * 8 + (m ^ (h & 7)); }

// A fragments from the LDS codes, and the weights folded with the scales.
template <int NHT>
__device__ __forceinline__ void load_qfrag_fp8(QFrag8<NHT>& f, const uint4* qcode,
                                               const float* qscale, const float* wrow, int H,
                                               int g, int c) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const int h = ht * 16 + c;
        const uint4 lo = qcode[qslot(h, 2 * g)], hi = qcode[qslot(h, 2 * g + 1)];
        f.a[ht] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hw = ht * 16 + 4 * g + i;
            f.wv[ht][i] = hw < H ? wrow[hw] * qscale[hw] : 0.f;
        }
    }
}

// One wave quantizes a query row's head vectors by the key-cache rule: lane h
// takes head h (all 128 dims), scale b = max|q| / 448 (1 for a zero vector),
// codes of q / b (fp32 division) clamped to +-448 and rounded to nearest even,
// into qcode (qslot layout) and b into qscale.  Heads at or past H get zero
// codes and scale 1.
__device__ __forceinline__ void quantize_q8_wave(const uint16_t* qrow, int H, uint4* qcode,
                                                 float* qscale) {
    const int h = lane_id();
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = h < H ? ldg16(qrow + h * kD + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t wds[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(wds[e] & 0xffffu)),
                               fabsf(bf16_bits_to_f32(wds[e] >> 16))));
    }
    const float b = m > 0.f ? m / 448.0f : 1.0f;
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
        const uint32_t wds[8] = {v[2 * mm].x, v[2 * mm].y, v[2 * mm].z, v[2 * mm].w,
                                 v[2 * mm + 1].x, v[2 * mm + 1].y, v[2 * mm + 1].z,
                                 v[2 * mm + 1].w};
        uint32_t out[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float y[4];
            y[0] = bf16_bits_to_f32(wds[2 * u] & 0xffffu);
            y[1] = bf16_bits_to_f32(wds[2 * u] >> 16);
            y[2] = bf16_bits_to_f32(wds[2 * u + 1] & 0xffffu);
            y[3] = bf16_bits_to_f32(wds[2 * u + 1] >> 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(y[e] / b, -448.0f), 448.0f);
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
            out[u] = (uint32_t)pk;
        }
        qcode[qslot(h, mm)] = make_uint4(out[0], out[1], out[2], out[3]);
    }
    qscale[h] = b;
}

// 16 keys x 16 heads x 128 dims in E4M3, fp32 accumulate (no block scales).
__device__ __forceinline__ f32x4 mfma16x16x128_fp8(const i32x8& a, const i32x8& b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f},
                                                            0, 0, 0, 0, 0, 0);
}

}  // namespace sa
