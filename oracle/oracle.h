/*
 * CPU oracle for the DSA lightning-indexer selector (DSA, MISA, HISA).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  It shares no code
 * with the HIP library.  All arithmetic is fp64; see oracle.c for the
 * definitions and the pages each one follows.
 *
 * Row numbering: a "row" is a flat query row id b*T + i of a problem; its
 * absolute position is t = causal_offset + i and its legal keys are s <= t.
 * Every output row holds the selected indices sorted by (score desc, index
 * asc), padded with -1 / -inf up to topk.
 */
#ifndef SA_ORACLE_H
#define SA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

typedef struct {
    const uint16_t* q;  /* [Bt, T, H, d] bf16 bit patterns */
    const float* w;     /* [Bt, T, H] */
    const uint16_t* K;  /* [Bt, L, d] bf16 bit patterns, one shared key head */
    int32_t Bt, T, H, d, L;
    int32_t causal_offset; /* absolute position of row 0 of each sequence */
    /* Optional FP8 key cache in place of K (DSA, MISA, HISA): key s of
     * sequence b is scales[b, s] * e4m3(codes[b, s, :]) (PaperTrace section
     * 2.3).  K may then be NULL. */
    const uint8_t* codes; /* [Bt, L, d] or NULL */
    const float* scales;  /* [Bt, L] */
} oracle_problem;

/* rows: flat row ids to evaluate (NULL = every row, nrows ignored).
 * Outputs are indexed by the position in `rows`.
 * out_rowscore (nullable): [nrows, L] full score row, NaN past t. */
int oracle_dsa(const oracle_problem* p, int topk, const int32_t* rows, int nrows,
               int32_t* out_idx, double* out_score, double* out_rowscore, int nthreads);

/* MISA (kprime == 0) or MISA-dagger (kprime >= topk).
 * override_heads [nrows, h] / override_pool [nrows, kprime] (nullable, -1 entries
 * skipped) replace the oracle's own discrete choice, for staged comparison.
 * out_E [nrows, H], out_heads [nrows, h] (ascending), out_pool [nrows, kprime],
 * out_hatrow [nrows, L] (routed score row, NaN past t): all nullable.
 * out_score is the routed score for kprime == 0, the full score otherwise. */
int oracle_misa(const oracle_problem* p, int topk, int B, int h, int kprime,
                const int32_t* rows, int nrows, const int32_t* override_heads,
                const int32_t* override_pool, int32_t* out_heads, double* out_E,
                int32_t* out_pool, double* out_hatrow, int32_t* out_idx, double* out_score,
                int nthreads);

/* HISA.  override_blocks [nrows, r] (nullable, -1 skipped); coarse_heads
 * [nrows, hsel] (nullable, ascending): block scores over those heads only
 * (the MISA x HISA composition; the fine stage keeps every head); out_blocks
 * [nrows, r] in selection order, -1 padded; out_J [nrows, ceil(L/b)] block
 * scores, NaN for blocks past t.  Rejects r*b < topk. */
int oracle_hisa(const oracle_problem* p, int topk, int b, int r, const int32_t* rows,
                int nrows, const int32_t* override_blocks, const int32_t* coarse_heads,
                int hsel, int32_t* out_blocks, double* out_J, int32_t* out_idx,
                double* out_score, int nthreads);

/* Means of consecutive blocks of `block` keys (last block truncated at L):
 * out [Bt, ceil(L/block), d]. */
int oracle_pool(const uint16_t* K, int Bt, int L, int d, int block, double* out);

/* OCP E4M3: value of a code; nearest code (ties to even, saturating at 448). */
double oracle_fp8_e4m3_decode(uint8_t c);
uint8_t oracle_fp8_e4m3_encode(float x);

/* Per-key FP8 quantization of n_keys bf16 keys of d values: scales [n_keys]
 * (max |k| / 448 in fp32, 1 for all-zero keys), codes [n_keys, d]. */
int oracle_quantize_keys_fp8(const uint16_t* K, long n_keys, int d, uint8_t* codes,
                             float* scales, int nthreads);

/* DSA on FP8 keys (codes [Bt, L, d], scales [Bt, L]); p->K is not used.
 * Scores are sum_j w_j max(q_j . (a_s decode(c_s)), 0) in fp64. */
int oracle_dsa_fp8(const oracle_problem* p, const uint8_t* codes, const float* scales, int topk,
                   const int32_t* rows, int nrows, int32_t* out_idx, double* out_score,
                   double* out_rowscore, int nthreads);

/* DSA on FP8 keys with the query quantized per head by the key rule as well:
 * I = sum_j w_j max((b_j e4m3(qc_j)) . (a_s e4m3(c_s)), 0) in fp64. */
int oracle_dsa_fp8q(const oracle_problem* p, const uint8_t* codes, const float* scales, int topk,
                    const int32_t* rows, int nrows, int32_t* out_idx, double* out_score,
                    double* out_rowscore, int nthreads);

/* LISA ([PT] 3.1): top-k by the linear score l = g . k, g = sum_j w_j q_j. */
int oracle_lisa(const oracle_problem* p, int topk, const int32_t* rows, int nrows,
                int32_t* out_idx, double* out_score, double* out_rowscore, int nthreads);

/* ResMiSA ([PT] 3.2): r residual heads routed by S_h = |w_h| max_b ReLU(U-),
 * extrema over blocks of `block` legal keys; score R = l + sum_{h in A}
 * w_h ReLU(-(q_h . k)).  r = 0 is LISA.  out_heads [nrows, r] ascending,
 * out_S [nrows, H], out_rowscore [nrows, L] (NaN past t); each may be NULL.
 * override_heads [nrows, r] replaces the routing (staged checks). */
int oracle_resmisa(const oracle_problem* p, int topk, int block, int r, const int32_t* rows,
                   int nrows, const int32_t* override_heads, int32_t* out_heads, double* out_S,
                   double* out_rowscore, int32_t* out_idx, double* out_score, int nthreads);

/* U- = sum_d (max(-q_d,0) kmax_d - max(q_d,0) kmin_d) for one head and box. */
double oracle_box_bound(const double* q, const double* kmin, const double* kmax, int d);

#ifdef __cplusplus
}
#endif

#endif
