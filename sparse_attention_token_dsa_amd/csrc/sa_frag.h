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

// All head ids first, then every q / w load back to back (no branches), then
// the zero-masking of absent heads.
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

}  // namespace sa
