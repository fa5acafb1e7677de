// LISA and ResMiSA (PaperTrace, "2.2.2 MISA, LISA and ResMiSA", sections 3.1
// and 3.2) on top of the DSA score kernels.
//
// With one key shared by all heads, ReLU(x) = x + ReLU(-x) splits the score
// into l = g . k (g = sum_j w_j q_j, the fused query) and per-head
// corrections.  LISA ranks by l; ResMiSA adds the corrections
// w_h ReLU(-(q_h . k)) of r routed heads A.  Both are DSA scores of a few
// synthetic heads, because ReLU(x) - ReLU(-x) = x:
//   l = ReLU(g . k) - ReLU(-g . k),
//   l + sum_{h in A} w_h ReLU(-z_h) = g' . k + sum_{h in A} w_h ReLU(z_h),
//   g' = sum_{h not in A} w_h q_h.
// So this file only builds, per query row, the head rows
//   [g'_hi, g'_lo, -g'_hi, -g'_lo, q_{a_1}, ..., q_{a_r}]   (bf16)
// with weights [1, 1, -1, -1, w_{a_1}, ..., w_{a_r}] (g' split into a bf16
// hi/lo pair keeps it to ~2^-16 relative; with r = H, g' = 0 and the linear
// heads are left out), and the DSA decode scan or the fused prefill scores
// them.  ResMiSA's routing needs, per head, S_h = |w_h| max_b ReLU(U-_{h,b})
// over the blocks of the legal history, where for a block's per-dimension key
// extrema [kmin, kmax]
//   U-_{h,b} = sum_d (max(-q_{h,d}, 0) kmax_d - max(q_{h,d}, 0) kmin_d)
//            = [q-_h | -q+_h] . [kmax_b | kmin_b],
// a 256-long dot product that runs on the bf16 MFMA (q-, -q+ and the extrema
// of bf16 keys are all exact bf16 values).
#include "sa_frag.h"

namespace sa {

namespace {

// --------------------------------------------------------- extrema

// Block b of keys [lo, hi): per-dimension max then min, as bf16 (the extrema
// of bf16 values are bf16 values).  256 threads: thread (kl = tid >> 4,
// c16 = tid & 15) covers dims c16*8 .. +8 of keys lo+kl, lo+kl+16, ...
__device__ __forceinline__ void block_extrema(const uint16_t* kseq, int lo, int hi,
                                              uint16_t* out) {
    const int c16 = threadIdx.x & 15, kl = threadIdx.x >> 4;
    float mx[8], mn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mx[e] = -INFINITY;
        mn[e] = INFINITY;
    }
#pragma unroll 4
    for (int s = lo + kl; s < hi; s += 16) {
        const uint4 v = ldg16_stream(kseq + (long long)s * kD + c16 * 8);
        const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = bf16_bits_to_f32(wds[e] & 0xffffu), b = bf16_bits_to_f32(wds[e] >> 16);
            mx[2 * e] = fmaxf(mx[2 * e], a);
            mn[2 * e] = fminf(mn[2 * e], a);
            mx[2 * e + 1] = fmaxf(mx[2 * e + 1], b);
            mn[2 * e + 1] = fminf(mn[2 * e + 1], b);
        }
    }
    __shared__ float rmx[16][kD], rmn[16][kD];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        rmx[kl][c16 * 8 + e] = mx[e];
        rmn[kl][c16 * 8 + e] = mn[e];
    }
    __syncthreads();
    if (threadIdx.x < kD) {
        float a = rmx[0][threadIdx.x], b = rmn[0][threadIdx.x];
        for (int u = 1; u < 16; ++u) {
            a = fmaxf(a, rmx[u][threadIdx.x]);
            b = fminf(b, rmn[u][threadIdx.x]);
        }
        out[threadIdx.x] = (uint16_t)(__float_as_uint(a) >> 16);
        out[kD + threadIdx.x] = (uint16_t)(__float_as_uint(b) >> 16);
    }
}

__global__ __launch_bounds__(256) void extrema_kernel(const uint16_t* keys, int L, int block,
                                                      int nblk, uint16_t* out) {
    const int b = blockIdx.y, m = blockIdx.x;
    const int lo = m * block, hi = min(lo + block, L);
    block_extrema(keys + (long long)b * L * kD, lo, hi,
                  out + ((long long)b * nblk + m) * 2 * kD);
}

// Rows whose last legal block is cut by the causal bound get the extrema of
// that block's legal keys; flag[row] says which rows have one.
__global__ __launch_bounds__(256) void extrema_tail_kernel(const uint16_t* keys,
                                                           long long seq_stride, int T,
                                                           int offset, int L, int block,
                                                           uint16_t* tail, uint8_t* flag) {
    const int row = blockIdx.x;
    const int b = row / T;
    const int t = offset + (row - b * T);
    const int lo = (t / block) * block;
    const bool partial = t + 1 < min(lo + block, L);
    if (threadIdx.x == 0) flag[row] = partial ? 1 : 0;
    if (!partial) return;
    block_extrema(keys + (long long)b * seq_stride, lo, t + 1, tail + (long long)row * 2 * kD);
}

// ---------------------------------------------------------- router

// Max over the 16 lanes of a DPP row (lanes 16g .. 16g+15), in every lane:
// row rotations by 8, 4, 2, 1.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));
    return v;
}

// Grid (nchunk, rows); 4 waves x 16 blocks.  For every head h and legal
// block m of the workgroup: U = [q-_h | -q+_h] . [kmax_m | kmin_m] on the
// MFMA (8 k-steps of 32), ReLU, max over the blocks; the workgroup's maximum
// per head goes to part[row][chunk][h].  Workgroups past the row's legal
// blocks write nothing: the reader takes only the row's own chunks.
template <int NHT>
__global__ __launch_bounds__(256) void resmisa_router_kernel(ResmisaArgs a) {
    const int row = blockIdx.y;
    const int b = row / a.T;
    const int t = a.offset + (row - b * a.T);
    const int nb = t / a.block + 1;
    const int m0 = blockIdx.x * 64;
    if (m0 >= nb) return;
    const int lane = lane_id(), g = lane >> 4, c = lane & 15;
    const int wid = threadIdx.x >> 6;
    const uint16_t* qrow = a.q + (long long)row * a.H * kD;

    // A fragments: step kk < 4 multiplies kmax dims (kk*4+g)*8 .. +8 with
    // q- (max(-q, 0)); step kk >= 4 multiplies the same dims of kmin with -q+.
    uint4 fa[NHT][8];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const int h = ht * 16 + c;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint4 v = h < a.H ? ldg16(qrow + (long long)h * kD + (kk * 4 + g) * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
            const uint32_t in[4] = {v.x, v.y, v.z, v.w};
            uint32_t neg[4], pos[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t nw = 0u, pw = 0u;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t x = (in[e] >> (16 * half)) & 0xffffu;
                    const bool nonzero = (x & 0x7fffu) != 0u;
                    const bool negative = (x & 0x8000u) != 0u;
                    // q- = -q where q < 0; -q+ = -q where q > 0; else 0
                    const uint32_t qn = (nonzero && negative) ? (x ^ 0x8000u) : 0u;
                    const uint32_t qp = (nonzero && !negative) ? (x | 0x8000u) : 0u;
                    nw |= qn << (16 * half);
                    pw |= qp << (16 * half);
                }
                neg[e] = nw;
                pos[e] = pw;
            }
            fa[ht][kk] = make_uint4(neg[0], neg[1], neg[2], neg[3]);
            fa[ht][kk + 4] = make_uint4(pos[0], pos[1], pos[2], pos[3]);
        }
    }

    const int m = m0 + wid * 16 + c;
    const bool legal = m < nb;
    const int ml = legal ? m : nb - 1;
    const uint16_t* rep = (a.tail && a.tail_flag[row] && ml == nb - 1)
                              ? a.tail + (long long)row * 2 * kD
                              : a.ext + ((long long)b * a.nblk + ml) * 2 * kD;
    uint4 kb[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kb[kk] = ldg16(rep + (kk * 4 + g) * 8);
    f32x4 acc[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) acc[ht] = mfma16x16x32(fa[ht][kk], kb[kk], acc[ht]);

    // acc[ht][i] = U for head ht*16 + 4g + i and block m.  ReLU, drop
    // illegal blocks, max over the 16 blocks (lanes) of the lane group.
    __shared__ float wmax[4][64];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = row16_max(legal ? fmaxf(acc[ht][i], 0.f) : 0.f);
            if (c == 0) wmax[wid][ht * 16 + 4 * g + i] = v;
        }
    __syncthreads();
    if (threadIdx.x < a.H) {
        const int h = threadIdx.x;
        float v = wmax[0][h];
        for (int u = 1; u < 4; ++u) v = fmaxf(v, wmax[u][h]);
        a.part[((long long)row * a.nchunk + blockIdx.x) * a.H + h] = v;
    }
}

// ----------------------------------------------------- head rows

// One workgroup of 128 threads per query row.  The row's q (H x 128 bf16,
// 16 KiB at H = 64) and w go to LDS first, every 16-byte load issued before
// any is used.  Routed heads (r > 0): the r largest S_h = |w_h| max_b
// ReLU(U-) (the max over the router workgroups that cover the row's legal
// blocks), ties to the lower head, listed in ascending order.  Thread x then forms
// g'_x = sum over the other heads (ascending) of w_h q_{h,x} in fp32 and
// writes dim x of every output head row.  With zero_state it also clears the
// row's state for the decode scan (one launch fewer on the decode path).
__global__ __launch_bounds__(128) void head_rows_kernel(ResmisaArgs a) {
    const int row = blockIdx.x;
    const int H = a.H, r = a.r;
    __shared__ uint4 sq4[kMaxH * kD / 8];
    __shared__ float sw[kMaxH], sS[kMaxH];
    __shared__ int inA[kMaxH];
    __shared__ int list[kMaxH];
    const uint16_t* sq = reinterpret_cast<const uint16_t*>(sq4);
    const float* wrow = a.w + (long long)row * H;
    const uint4* q4 = reinterpret_cast<const uint4*>(a.q + (long long)row * H * kD);
    const int n4 = H * kD / 8;
    uint4 tmp[kMaxH * kD / 8 / 128];
#pragma unroll
    for (int i = 0; i < kMaxH * kD / 8 / 128; ++i) {
        const int idx = threadIdx.x + i * 128;
        tmp[i] = idx < n4 ? q4[idx] : make_uint4(0u, 0u, 0u, 0u);
    }
    float wv = 0.f, sv = 0.f;
    if (threadIdx.x < H) {
        wv = wrow[threadIdx.x];
        if (r > 0) {  // part is null for LISA (r = 0)
            const int t = a.offset + row % a.T;
            const int nc = (t / a.block + 1 + 63) / 64;
            const float* pr = a.part + (long long)row * a.nchunk * H + threadIdx.x;
            float m = 0.f;
#pragma unroll 8
            for (int c2 = 0; c2 < nc; ++c2) m = fmaxf(m, pr[(long long)c2 * H]);
            sv = m * fabsf(wv);
        }
    }
#pragma unroll
    for (int i = 0; i < kMaxH * kD / 8 / 128; ++i) sq4[threadIdx.x + i * 128] = tmp[i];
    if (threadIdx.x < kMaxH) {
        sw[threadIdx.x] = wv;
        sS[threadIdx.x] = sv;
    }
    __syncthreads();
    if (threadIdx.x < H) {
        const int h = threadIdx.x;
        int rank = 0;
        for (int j = 0; j < H; ++j) rank += (sS[j] > sS[h] || (sS[j] == sS[h] && j < h)) ? 1 : 0;
        inA[h] = rank < r ? 1 : 0;
    }
    __syncthreads();
    if (threadIdx.x < H) {
        const int h = threadIdx.x;
        if (inA[h]) {
            int pos = 0;
            for (int j = 0; j < h; ++j) pos += inA[j];
            list[pos] = h;
            if (a.heads_out) a.heads_out[(long long)row * r + pos] = h;
        }
    }
    __syncthreads();
    const int x = threadIdx.x;  // one key dim per thread
    const bool linear = r < H;
    const int nlin = linear ? 4 : 0;
    uint16_t* qo = a.qp + (long long)row * a.Hp * kD;
    float* wo = a.wp + (long long)row * a.Hp;
    if (linear) {
        float gx = 0.f;
#pragma unroll 8
        for (int h = 0; h < H; ++h) {
            const float wh = inA[h] ? 0.f : sw[h];  // routed heads leave the linear term
            gx = fmaf(wh, bf16_bits_to_f32(sq[h * kD + x]), gx);
        }
        const uint32_t hi = f32_to_bf16_bits(gx);
        const uint32_t lo = f32_to_bf16_bits(gx - bf16_bits_to_f32(hi));
        qo[0 * kD + x] = (uint16_t)hi;
        qo[1 * kD + x] = (uint16_t)lo;
        qo[2 * kD + x] = (uint16_t)(hi ^ 0x8000u);
        qo[3 * kD + x] = (uint16_t)(lo ^ 0x8000u);
        if (x < 4) wo[x] = x < 2 ? 1.f : -1.f;
    }
#pragma unroll 4
    for (int u = 0; u < r; ++u) {
        const int h = list[u];
        qo[(long long)(nlin + u) * kD + x] = sq[h * kD + x];
        if (x == 0) wo[nlin + u] = sw[h];
    }
    // The decode scan that follows adds its histogram into a zeroed row state.
    if (a.zero_state)
        for (int u = x; u < kRowState; u += 128) a.zero_state[(long long)row * kRowState + u] = 0u;
}

}  // namespace

hipError_t launch_extrema(const uint16_t* keys, int batch, int L, int block, uint16_t* out,
                          hipStream_t s) {
    const int nblk = (L + block - 1) / block;
    prof_begin(K_EXTREMA, s);
    sa_launch(extrema_kernel, dim3((unsigned)nblk, (unsigned)batch), dim3(256), 0, s, keys, L, block,
                                                                              nblk, out);
    prof_end(K_EXTREMA, s);
    return hipGetLastError();
}

hipError_t launch_extrema_tail(const uint16_t* keys, long long seq_stride, int T, int offset,
                               int L, int block, int rows, uint16_t* tail, uint8_t* flag,
                               hipStream_t s) {
    prof_begin(K_EXTREMA, s);
    sa_launch(extrema_tail_kernel, dim3((unsigned)rows), dim3(256), 0, s, keys, seq_stride, T, offset,
                                                                   L, block, tail, flag);
    prof_end(K_EXTREMA, s);
    return hipGetLastError();
}

hipError_t launch_resmisa_router(const ResmisaArgs& a, int rows, hipStream_t s) {
    const dim3 grid((unsigned)a.nchunk, (unsigned)rows);
    const int nht = (a.H + 15) / 16;
    prof_begin(K_RES_ROUTER, s);
    switch (nht) {
        case 1: sa_launch(resmisa_router_kernel<1>, grid, dim3(256), 0, s, a); break;
        case 2: sa_launch(resmisa_router_kernel<2>, grid, dim3(256), 0, s, a); break;
        case 3: sa_launch(resmisa_router_kernel<3>, grid, dim3(256), 0, s, a); break;
        default: sa_launch(resmisa_router_kernel<4>, grid, dim3(256), 0, s, a); break;
    }
    prof_end(K_RES_ROUTER, s);
    return hipGetLastError();
}

hipError_t launch_head_rows(const ResmisaArgs& a, int rows, hipStream_t s) {
    prof_begin(K_HEAD_ROWS, s);
    sa_launch(head_rows_kernel, dim3((unsigned)rows), dim3(128), 0, s, a);
    prof_end(K_HEAD_ROWS, s);
    return hipGetLastError();
}

}  // namespace sa
