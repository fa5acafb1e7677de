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

// Head of tile row u: identity over H, or entry u of a routed head list
// (ids outside [0, H) are treated as absent).
__device__ __forceinline__ int head_at(int u, int H, const int32_t* heads, int hsel) {
    if (heads) {
        const int v = u < hsel ? heads[u] : -1;
        return (v >= 0 && v < H) ? v : -1;
    }
    return u < H ? u : -1;
}

template <int NHT>
__device__ __forceinline__ void load_qfrag(QFrag<NHT>& f, const uint16_t* qrow,
                                           const float* wrow, int H, const int32_t* heads,
                                           int hsel, int g, int c) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const int hr = head_at(ht * 16 + c, H, heads, hsel);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            f.a[ht][kk] = hr >= 0 ? ldg16(qrow + hr * kD + (kk * 4 + g) * 8)
                                  : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hw = head_at(ht * 16 + 4 * g + i, H, heads, hsel);
            f.wv[ht][i] = hw >= 0 ? wrow[hw] : 0.f;
        }
    }
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
    sc += __shfl_xor(sc, 16);
    sc += __shfl_xor(sc, 32);
    return sc;
}

template <int KSTEPS>
__device__ __forceinline__ void load_key(uint4 (&b)[KSTEPS], const uint16_t* kp, int g) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) b[kk] = ldg16(kp + (kk * 4 + g) * 8);
}

}  // namespace sa
