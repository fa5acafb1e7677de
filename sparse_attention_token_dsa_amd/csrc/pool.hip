// Key-cache-side kernels.
//
// Block mean-pooling of the indexer keys: MISA's pooled keys (summary page
// "MISA", method step 1, B = 1024) and HISA's block representatives
// (PaperTrace section 2.1 / blog "Route 1: HISA", b = 128).  HBM-bound: every
// key is read once with 16-byte loads; sums are fp32; the mean is stored as a
// hi/lo bf16 pair so the bf16 MFMA score kernels can use it at fp32 accuracy.
//
// FP8 quantization of the keys (PaperTrace section 2.3, the FP8 cache: one
// scale per block, here per key): a = max |k| / 448, codes = E4M3(k / a).
#include "sa_common.h"

namespace sa {

// 16 lanes per key, 8 values per lane (16-byte loads, 8-byte code stores):
// the max-abs reduction over the 16 lanes, the fp32 scale and divisions, then
// the hardware E4M3 conversion (round to nearest even) of values clamped to
// +-448, which is the saturating rounding.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* keys, long long n,
                                                           uint8_t* codes, float* scales) {
    // 16 lanes per key (lane part p: dims 8p .. 8p+7), 16 keys per workgroup.
    const long long s = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4;
    if (s >= n) return;  // whole 16-lane groups leave together
    const int part = threadIdx.x & 15;
    const uint4 v = ldg16_stream(keys + s * kD + part * 8);
    const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_bits_to_f32(wds[e] & 0xffffu);
        x[2 * e + 1] = bf16_bits_to_f32(wds[e] >> 16);
    }
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
    const float a = m > 0.f ? m / 448.0f : 1.0f;
    // x / a is at most 448 up to the rounding of a; the clamp keeps the
    // conversion on the saturating side (beyond 448 it would give NaN).
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[4 * h + e] / a, -448.0f), 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
        out[h] = (uint32_t)pk;
    }
    *reinterpret_cast<uint2*>(codes + s * kD + part * 8) = make_uint2(out[0], out[1]);
    if (part == 0) scales[s] = a;
}

hipError_t launch_quantize_fp8(const uint16_t* keys, long long n, uint8_t* codes, float* scales,
                               hipStream_t s) {
    if (n <= 0) return hipSuccess;
    prof_begin(K_QUANT8, s);
    sa_launch(quantize_fp8_kernel, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, s, keys, n, codes, scales);
    prof_end(K_QUANT8, s);
    return hipGetLastError();
}

// 256 threads: thread (kl = tid >> 4, c16 = tid & 15) sums dims c16*8..+8 of
// keys lo+kl, lo+kl+16, ...; the 16 partial sums per dim are reduced in LDS.
__device__ __forceinline__ void block_sum_partial(const uint16_t* kseq, int lo, int hi,
                                                  float (&acc)[8]) {
    const int c16 = threadIdx.x & 15, kl = threadIdx.x >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int s = lo + kl; s < hi; s += 16) {
        const uint4 v = ldg16_stream(kseq + (long long)s * kD + c16 * 8);
        const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += bf16_bits_to_f32(wds[e] & 0xffffu);
            acc[2 * e + 1] += bf16_bits_to_f32(wds[e] >> 16);
        }
    }
}

__device__ __forceinline__ void write_rep(uint16_t* out, float mean, int dim) {
    const uint32_t hi = f32_to_bf16_bits(mean);
    const uint32_t lo = f32_to_bf16_bits(mean - bf16_bits_to_f32(hi));
    out[dim] = (uint16_t)hi;
    out[kD + dim] = (uint16_t)lo;
}

// Block means of bf16 keys, or of an FP8 cache's dequantized keys (codes
// non-null: code times the key's scale, in fp32).
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* keys, const uint8_t* codes,
                                                   const float* scales, int L, int block,
                                                   int nblk, uint16_t* out) {
    const int b = blockIdx.y, m = blockIdx.x;
    const int lo = m * block, hi = min(lo + block, L);
    const int c16 = threadIdx.x & 15, kl = threadIdx.x >> 4;
    float acc[8];
    if (codes) {
        const uint8_t* cseq = codes + (long long)b * L * kD;
        const float* sseq = scales + (long long)b * L;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int s = lo + kl; s < hi; s += 16) {
            float x[8];
            key8_f32(nullptr, cseq, sseq, s, c16, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += x[e];
        }
    } else {
        block_sum_partial(keys + (long long)b * L * kD, lo, hi, acc);
    }
    __shared__ float red[16][kD];
#pragma unroll
    for (int e = 0; e < 8; ++e) red[kl][c16 * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kD) {
        float S = 0.f;
        for (int r = 0; r < 16; ++r) S += red[r][threadIdx.x];
        write_rep(out + ((long long)b * nblk + m) * 2 * kD, S / (float)(hi - lo), threadIdx.x);
    }
}

// One workgroup per large block: its small blocks are summed one after the
// other (each written as a small representative) and their sums accumulate
// into the large block's mean.
__global__ __launch_bounds__(256) void pool2_kernel(const uint16_t* keys, int L, int small,
                                                    int large, int nsmall, int nlarge,
                                                    uint16_t* out_small, uint16_t* out_large) {
    const int b = blockIdx.y, M = blockIdx.x;
    const int LO = M * large, HI = min(LO + large, L);
    const uint16_t* kseq = keys + (long long)b * L * kD;
    __shared__ float red[16][kD];
    const int c16 = threadIdx.x & 15, kl = threadIdx.x >> 4;
    float total = 0.f;
    for (int lo = LO; lo < HI; lo += small) {
        const int hi = min(lo + small, HI);
        float acc[8];
        block_sum_partial(kseq, lo, hi, acc);
#pragma unroll
        for (int e = 0; e < 8; ++e) red[kl][c16 * 8 + e] = acc[e];
        __syncthreads();
        if (threadIdx.x < kD) {
            float S = 0.f;
            for (int r = 0; r < 16; ++r) S += red[r][threadIdx.x];
            total += S;
            write_rep(out_small + ((long long)b * nsmall + lo / small) * 2 * kD,
                      S / (float)(hi - lo), threadIdx.x);
        }
        __syncthreads();
    }
    if (threadIdx.x < kD)
        write_rep(out_large + ((long long)b * nlarge + M) * 2 * kD, total / (float)(HI - LO),
                  threadIdx.x);
}

hipError_t launch_pool(const uint16_t* keys, int batch, int L, int block, uint16_t* out,
                       hipStream_t s, const uint8_t* codes, const float* scales) {
    const int nblk = (L + block - 1) / block;
    prof_begin(K_POOL, s);
    sa_launch(pool_kernel, dim3(nblk, batch), dim3(256), 0, s, keys, codes, scales, L, block,
              nblk, out);
    prof_end(K_POOL, s);
    return hipGetLastError();
}

hipError_t launch_pool2(const uint16_t* keys, int batch, int L, int small, int large,
                        uint16_t* out_small, uint16_t* out_large, hipStream_t s) {
    const int nsmall = (L + small - 1) / small;
    const int nlarge = (L + large - 1) / large;
    prof_begin(K_POOL2, s);
    sa_launch(pool2_kernel, dim3(nlarge, batch), dim3(256), 0, s, keys, L, small, large, nsmall,
                                                           nlarge, out_small, out_large);
    prof_end(K_POOL2, s);
    return hipGetLastError();
}

}  // namespace sa
