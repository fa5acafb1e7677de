/*
 * sa_indexer.h -- C ABI of the MI355X (gfx950) DSA lightning-indexer selector.
 *
 * What it computes.  For a query row at absolute position t, every causal
 * prefix token s <= t gets the indexer score
 *
 *     I[t,s] = sum_j w[t,j] * max(q[t,j] . k[s], 0)          (j < H, one shared key head)
 *
 * and the row keeps the token-level top-k (PaperTrace, "2.2.2 MISA, LISA and
 * ResMiSA", section 1 and the two-head example of section 3.1; the
 * Index -> Select -> Attend pipeline of the blog "The new bottleneck of
 * sparse attention").  Two accelerations share the interface:
 *   - MISA (summary page "MISA: Mixture of Indexer Sparse Attention",
 *     method steps 1-6): block-pooled router picks h of the H heads per
 *     query, tokens are scored with those heads only; MISA-dagger keeps a
 *     k' pool and reranks it with all heads.
 *   - HISA (PaperTrace section 2.1; blog "Route 1: HISA"): block
 *     representatives are scored, r blocks are kept, their tokens are
 *     rescored exactly, token top-k.
 * Further entry points: MISA x HISA in series, LISA's linear score and
 * ResMiSA (PaperTrace sections 3.1-3.2), an FP8 (E4M3) key cache for DSA,
 * MISA and HISA with the query in bf16 or in E4M3 (section 2.3), ragged
 * batches with per-sequence lengths, and the index tidy-up after the top-k
 * (section 2.2).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE memory owned by the caller, row-major
 *     and contiguous; nothing is retained after the call returns.
 *   - q    : bf16 bit patterns [batch, T, H, d]
 *     w    : fp32 [batch, T, H]
 *     keys : bf16 bit patterns [batch, L, d]    (one shared key head)
 *   - d must be 128.  1 <= H <= 64.
 *   - Query row i of a sequence sits at absolute position
 *     t = causal_offset + i; its legal keys are 0..t (0 <= causal_offset,
 *     causal_offset + T <= L).  Decode: T = 1, causal_offset = L - 1.
 *   - Outputs out_idx [batch, T, topk] int32 and out_score [batch, T, topk]
 *     fp32 hold, per row, the SET of the min(topk, t+1) selected positions
 *     (order unspecified) and the score each was ranked by; unused slots are
 *     -1 / -inf.  out_score may be NULL.  Among exactly equal scores the lower
 *     position is kept.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream); outputs are valid once the stream has reached the call.
 *   - The library allocates no device memory: each call takes a workspace
 *     `ws` of at least the size its *_ws function reports (any alignment is
 *     accepted; 256 B is recommended).  Workspace contents need no
 *     initialisation and are clobbered.
 *   - Query rows per call: batch * T <= 65535 (rows are a grid dimension of
 *     the scan kernels), except the fused prefill path of indexer_score_topk,
 *     indexer_score_topk_ragged and lisa_score_topk (T >= 16), which takes
 *     batch <= 65535 sequences of any T; SA_EUNSUPPORTED otherwise.
 *   - Inputs must be finite; NaN / inf scores give unspecified selections.
 *   - Return value: SA_OK or a negative SA_E* code; sa_last_error() then
 *     returns a message for the calling thread.  On error nothing has been
 *     launched, except SA_EHIP, which reports a failed launch.
 */
#ifndef SA_INDEXER_H
#define SA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_OK 0
#define SA_EINVAL (-1)       /* bad argument: shape, budget, NULL pointer */
#define SA_EUNSUPPORTED (-2) /* valid but not implemented: d != 128, H > 64 */
#define SA_EWORKSPACE (-3)   /* ws_bytes smaller than the *_ws size */
#define SA_EHIP (-4)         /* HIP launch failure */

typedef struct sa_shape {
    int32_t batch;         /* sequences */
    int32_t T;             /* query rows per sequence */
    int32_t H;             /* indexer heads H_I */
    int32_t d;             /* indexer head dim, must be 128 */
    int32_t L;             /* keys per sequence */
    int32_t causal_offset; /* absolute position of query row 0 */
    int32_t topk;          /* k >= 1 */
} sa_shape;

/* ---------------------------------------------------------------- DSA */

/* Workspace bytes for indexer_score_topk on this shape. */
int indexer_score_topk_ws(const sa_shape* s, size_t* ws_bytes);

/* DSA lightning indexer: score every causal prefix token with all H heads,
 * keep the top-k (PaperTrace section 1; section 2.2 asks for score, causal
 * mask and top-k fused so that no n^2 score matrix is written).
 * Rows with T >= 16 per sequence take the fused prefill kernel (scores never
 * leave the chip; survivors of a running per-row threshold are kept in a
 * bounded per-row list of min(t + 1, max(6 topk, 8192)) entries, compacted in
 * place when it fills, so the workspace is O(rows * topk));
 * smaller T take the decode scan, which writes one O(L) score row per query
 * into the workspace. */
int indexer_score_topk(const uint16_t* q, const float* w, const uint16_t* keys,
                       const sa_shape* s, int32_t* out_idx, float* out_score, void* ws,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------- DSA + block pooling */

/* Workspace bytes for indexer_score_topk_pooled (the same as for
 * indexer_score_topk on this shape). */
int indexer_score_topk_pooled_ws(const sa_shape* s, int32_t small, int32_t large,
                                 size_t* ws_bytes);

/* indexer_score_topk for decode rows that also writes the block means of the
 * keys it streams: the outputs of sa_pool_blocks2(keys, ..., small, large),
 * the cache-side state MISA ("MISA" summary page, method step 1: blocks of B)
 * and HISA (PaperTrace section 2.1: blocks of b) score against, without a
 * second pass over the key cache.
 *   s          T must be 1 and causal_offset L - 1 (each sequence's one query
 *              row reads every key), else SA_EUNSUPPORTED.
 *   small      block of out_small: a power of two >= 128.
 *   large      block of out_large: a multiple of small that divides 2048
 *              (SA_EUNSUPPORTED otherwise).
 *   out_small  [batch, ceil(L/small), 2, d], out_large [batch, ceil(L/large),
 *              2, d]: per block the fp32 mean as hi = bf16(mean), lo =
 *              bf16(mean - hi), as sa_pool_blocks (sums in another order:
 *              equal to its output up to fp32 rounding).
 *   pools_ready  a hipEvent_t recorded on `stream` as soon as the block means
 *              are written (before the top-k kernels of the call), so that
 *              work on other streams can start on them; or NULL.
 * Selection, outputs, ownership and errors otherwise as in
 * indexer_score_topk. */
int indexer_score_topk_pooled(const uint16_t* q, const float* w, const uint16_t* keys,
                              const sa_shape* s, int32_t small, int32_t large,
                              uint16_t* out_small, uint16_t* out_large, int32_t* out_idx,
                              float* out_score, void* ws, size_t ws_bytes, void* pools_ready,
                              void* stream);

/* ------------------------------------------- decode selectors in phases */

/* Phases of indexer_score_topk_pooled_phase and misa_route_phase.
 * SA_PHASE_SCAN streams the keys: the score row and first-digit histogram of
 * every query row go into the workspace (and, for the pooled call, the block
 * means into out_small / out_large).  SA_PHASE_SELECT takes the top-k from
 * what the scan left in the workspace (for MISA-dagger, the k' pool, its
 * rescoring with all heads and the final top-k).  Both bits together are the
 * whole call.  Between the two phases a caller may run other work on the
 * GPU, for example the scans of other selectors, so that the latency-bound
 * selections of several selectors run side by side once every key stream is
 * done (the top-k is a cost of its own next to the key scan, one that does
 * not shrink with the head count: PaperTrace, "2.2.2 MISA, LISA and
 * ResMiSA", section 2.2).  The operations are those of
 * indexer_score_topk_pooled and misa_route. */
#define SA_PHASE_SCAN 1
#define SA_PHASE_SELECT 2

/* indexer_score_topk_pooled in phases.
 *   phases  SA_PHASE_SCAN, SA_PHASE_SELECT or both (SA_EINVAL otherwise).
 * The SA_PHASE_SELECT call must follow the SA_PHASE_SCAN call on the same
 * stream order, with the same arguments and the same workspace, which the
 * caller does not touch in between; nothing checks this.  Each call launches
 * only its phase's kernels; out_idx / out_score are written by the select
 * phase, out_small / out_large by the scan phase.  Arguments, shapes and
 * errors otherwise as in indexer_score_topk_pooled (no pools_ready event:
 * the scan phase's end is the caller's own ordering point). */
int indexer_score_topk_pooled_phase(const uint16_t* q, const float* w, const uint16_t* keys,
                                    const sa_shape* s, int32_t small, int32_t large,
                                    uint16_t* out_small, uint16_t* out_large, int32_t* out_idx,
                                    float* out_score, void* ws, size_t ws_bytes, int32_t phases,
                                    void* stream);

/* ------------------------------------------------ allocation-free DSA */

/* Size of the static device scratch behind indexer_score_topk_noalloc: 32 MiB
 * per GPU, held by the library from the first call on that GPU until the
 * process ends. */
#define SA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* indexer_score_topk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and outputs, with the workspace
 * taken from a static device array of SA_NOALLOC_SCRATCH_BYTES instead of a
 * caller buffer.  The call allocates nothing (no hipMalloc / hipFree); the
 * first call on a device looks up that device's array address once.
 *   - Shapes whose indexer_score_topk_ws size exceeds
 *     SA_NOALLOC_SCRATCH_BYTES are rejected with SA_EWORKSPACE (e.g. 8
 *     decode rows at L = 131072 need about 12.2 MiB and fit; the 4096-row
 *     chunked prefill at L = 32768 needs 1 GiB and does not).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     the same GPU (concurrent streams, or host threads, without ordering
 *     between them) race and give undefined results.  Calls ordered on one
 *     stream are safe; the array keeps the last call's contents, and each
 *     call clears what it needs zeroed itself.
 * Arguments, ownership and errors otherwise as in indexer_score_topk. */
int indexer_score_topk_noalloc(const uint16_t* q, const float* w, const uint16_t* keys,
                               const sa_shape* s, int32_t* out_idx, float* out_score,
                               void* stream);

/* ----------------------------------------------------------- tidy-up */

/* Index tidy-up after any selector (PaperTrace "2.2.2 MISA, LISA and
 * ResMiSA", section 2.2: put the selected tokens in physical page / offset
 * order for a coalesced gather, keep the set free of duplicates and its valid
 * length; section 2.3: count the distinct pages and contiguous runs).
 *   idx          device int32 [rows, k] selected positions per row, -1 empty
 *                (any order, duplicates allowed); rows = batch * T, row r
 *                belongs to sequence r / T.
 *   block_table  device int32 [batch, pages_per_seq]: physical page of each
 *                logical page of the sequence, or NULL (slot = position).
 *                Positions past the table, or on a page mapped to a negative
 *                entry, are dropped.  Slots must fit in int32.
 *   page_size    tokens per page (>= 1): slot = table[b][s / page_size] *
 *                page_size + s % page_size.
 *   max_slots    number of physical slots (slots >= max_slots are dropped),
 *                or 0 if unbounded.  With 0 < max_slots <= 2^18 the kernel
 *                uses a bitmap in LDS (any k); otherwise it sorts (k <= 4096).
 *   out_slots    device int32 [rows, k]: the row's distinct slots in
 *                ascending order, then -1.
 *   out_stats    device int32 [rows, 3] (nullable): distinct slots, distinct
 *                pages (slot / page_size), maximal runs of consecutive slots.
 * Errors as in indexer_score_topk. */
int sa_tidy_indices(const int32_t* idx, int32_t rows, int32_t T, int32_t k,
                    const int32_t* block_table, int32_t pages_per_seq, int32_t page_size,
                    int32_t max_slots, int32_t* out_slots, int32_t* out_stats, void* stream);

/* ------------------------------------------------------- ragged rows */

/* Workspace bytes for indexer_score_topk_ragged. */
int indexer_score_topk_ragged_ws(const sa_shape* s, size_t* ws_bytes);

/* DSA indexer over a batch of sequences of different lengths (PaperTrace
 * "2.2.2 MISA, LISA and ResMiSA", section 2.3, load and tail latency: each
 * row selects among its own min(k, t+1) positions; per-row lengths instead of
 * padding every row to the longest one).  Decode-style rows (T < 16) take
 * the decode scan; T >= 16 takes the fused prefill, each sequence's query
 * block placed at the end of its own history (chunked prefill of sequences
 * with different cached prefixes).
 *   seq_lens  device int32 [batch]: keys [0, seq_lens[b]) of sequence b are
 *             its history; its T query rows sit at positions
 *             seq_lens[b] - T + i (causal within the sequence).  Lengths are
 *             clamped to [T, L].  Work beyond a row's length is skipped.
 *   total_len host-side sum of the lengths, or 0 if unknown: it only sizes
 *             the decode scan's key chunks per workgroup (the result does not
 *             depend on it), so that a batch with a few long rows still
 *             spreads over the CUs; the prefill ignores it.
 *   s         L is the per-sequence capacity (the keys' row stride);
 *             causal_offset must be L - T.
 * Selection and outputs as in indexer_score_topk; other arguments,
 * ownership and errors likewise. */
int indexer_score_topk_ragged(const uint16_t* q, const float* w, const uint16_t* keys,
                              const int32_t* seq_lens, int64_t total_len, const sa_shape* s,
                              int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------- FP8 keys */

/* FP8 key cache (PaperTrace section 2.3, "from the formula to the FP8
 * cache": indexer keys are quantized in blocks to FP8 with one scale per
 * block; the query stays at the compute precision).  The block is one key
 * (its d = 128 values):
 *   scales[s] = max_x |k_{s,x}| / 448 in fp32 (1 for an all-zero key),
 *   codes[s, x] = OCP E4M3 code nearest to k_{s,x} / scales[s] (fp32
 *                 division; ties to the even code; |.| > 448 saturates).
 * keys: [batch, L, d] bf16 bit patterns (device); codes: [batch, L, d]
 * bytes; scales: [batch, L] fp32 (device, caller-owned).  d must be 128.
 * Errors: SA_EINVAL (NULL pointer, batch or L < 1), SA_EUNSUPPORTED
 * (d != 128), SA_EHIP. */
int sa_quantize_keys_fp8(const uint16_t* keys, int32_t batch, int32_t L, int32_t d,
                         uint8_t* codes, float* scales, void* stream);

/* Workspace bytes for indexer_score_topk_fp8 on this shape. */
int indexer_score_topk_fp8_ws(const sa_shape* s, size_t* ws_bytes);

/* DSA lightning indexer on an FP8 key cache (codes and scales as written by
 * sa_quantize_keys_fp8): the scores are those of the dequantized keys,
 *   I = sum_j w_j * ReLU(q_j . (scales[s] * e4m3(codes[s]))),
 * and the selection is as in indexer_score_topk.  The key stream is 132
 * bytes per key instead of 256.  Decode-style rows only: T must be < 16
 * (SA_EUNSUPPORTED otherwise; prefill rows on the FP8 cache take
 * indexer_score_topk_fp8q).  Other arguments, ownership and errors as in
 * indexer_score_topk. */
int indexer_score_topk_fp8(const uint16_t* q, const float* w, const uint8_t* codes,
                           const float* scales, const sa_shape* s, int32_t* out_idx,
                           float* out_score, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for indexer_score_topk_fp8_ragged. */
int indexer_score_topk_fp8_ragged_ws(const sa_shape* s, size_t* ws_bytes);

/* Ragged batches (as indexer_score_topk_ragged: seq_lens, total_len, the
 * capacity L with causal_offset = L - T) over an FP8 key cache.  q_fp8 = 0:
 * the scores of indexer_score_topk_fp8 (q bf16), decode-style rows (T < 16,
 * SA_EUNSUPPORTED otherwise); q_fp8 != 0: those of indexer_score_topk_fp8q
 * (q converted to E4M3, fp8 MFMA), any T (T >= 16: the fused prefill, each
 * sequence's rows at its own end).  Other arguments, ownership and errors as
 * in indexer_score_topk_fp8. */
int indexer_score_topk_fp8_ragged(const uint16_t* q, const float* w, const uint8_t* codes,
                                  const float* scales, const int32_t* seq_lens, int64_t total_len,
                                  int32_t q_fp8, const sa_shape* s, int32_t* out_idx,
                                  float* out_score, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for indexer_score_topk_fp8q on this shape (for T < 16 the
 * same as for indexer_score_topk_fp8; for T >= 16 the fused prefill's
 * survivor lists, as indexer_score_topk). */
int indexer_score_topk_fp8q_ws(const sa_shape* s, size_t* ws_bytes);

/* As indexer_score_topk_fp8, with the query converted to E4M3 as well, the
 * compute type of the fp8 matrix product (PaperTrace section 2.3: the query
 * is converted to the compute type in registers; its quantization error
 * adds to the key's).  Each head vector q_{t,j} is quantized by the rule of
 * sa_quantize_keys_fp8 (b_j = max|q_{t,j}| / 448, codes of q / b_j) inside
 * the kernel, and since b_j > 0 commutes with ReLU,
 *   I = scales[s] * sum_j fp32(w_j * b_j) * ReLU(e4m3(qc_j) . e4m3(codes[s])),
 * the dot product on the 16x16x128 fp8 MFMA with fp32 accumulation.  Rows
 * with T >= 16 per sequence take the fused prefill on the same arithmetic
 * (the query quantized per head in the kernel, the keys' codes and scales
 * staged in LDS, no score matrix written).  Same arguments, ownership and
 * errors as indexer_score_topk_fp8 otherwise; q stays bf16 in memory. */
int indexer_score_topk_fp8q(const uint16_t* q, const float* w, const uint8_t* codes,
                            const float* scales, const sa_shape* s, int32_t* out_idx,
                            float* out_score, void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------- pooling */

/* Block means of the keys, the cache-side state MISA (B = 1024) and HISA
 * (b = 128) score against.  Block m covers keys [m*block, min((m+1)*block, L)).
 * out: [batch, ceil(L/block), 2, d] bf16 bit patterns; per block the fp32
 * mean is stored as hi = bf16(mean) followed by lo = bf16(mean - hi), so
 * hi + lo carries the mean to about 2^-16 relative.  */
int sa_pool_blocks(const uint16_t* keys, int32_t batch, int32_t L, int32_t d, int32_t block,
                   uint16_t* out, void* stream);

/* Both pools in one pass over the keys: `large` must be a multiple of
 * `small`; outputs as sa_pool_blocks for each block size. */
int sa_pool_blocks2(const uint16_t* keys, int32_t batch, int32_t L, int32_t d, int32_t small,
                    int32_t large, uint16_t* out_small, uint16_t* out_large, void* stream);

/* --------------------------------------------------------------- MISA */

/* Workspace bytes for misa_route.  pooled_given: whether `pooled` will be
 * passed (non-NULL) to misa_route. */
int misa_route_ws(const sa_shape* s, int32_t block_B, int32_t h, int32_t k_prime,
                  int32_t pooled_given, size_t* ws_bytes);

/* MISA routed indexer ("MISA" summary page, method steps 1-6).
 *   block_B  pooling block B (e.g. 1024); a block's pooled key is the mean
 *            of its legal keys.
 *   h        active heads per query, 1 <= h <= H.  Router:
 *            A[j,m] = w_j * ReLU(q_j . pooled_m), E_j = mean_m |A[j,m]| over
 *            the blocks that intersect [0, t]; the h largest E are routed
 *            (ties -> lower head).
 *   k_prime  0: one stage -- top-k of the routed score
 *            Ihat[s] = sum_{j routed} w_j ReLU(q_j . k_s); out_score = Ihat.
 *            >= topk: MISA-dagger -- top-k' by Ihat, rescored with all H
 *            heads, top-k of that; out_score = I.
 *   pooled   NULL (pool inside the call) or sa_pool_blocks(keys, ..., B)
 *            output for these keys.
 *   out_heads [batch, T, h] routed heads, ascending (nullable).
 *   out_pool  [batch, T, k_prime] the k' pool, -1 padded (nullable; only for
 *             k_prime > 0).
 * Rows with T >= 16 per sequence (prefill) take the fused prefill kernel on
 * the routed heads' q rows: no score row is written; decode-style rows write
 * one O(L) routed score row per query into the workspace. */
int misa_route(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
               int32_t block_B, int32_t h, int32_t k_prime, const uint16_t* pooled,
               int32_t* out_heads, int32_t* out_pool, int32_t* out_idx, float* out_score,
               void* ws, size_t ws_bytes, void* stream);

/* misa_route in phases (SA_PHASE_SCAN / SA_PHASE_SELECT, see
 * indexer_score_topk_pooled_phase): the scan phase routes each row and
 * streams the keys on the routed heads (out_heads written there; with
 * pooled NULL it pools the keys first, into the workspace); the select phase
 * takes the top-k, or for k_prime > 0 the k' pool (out_pool), its rescoring
 * with all H heads and the top-k.  Only decode rows (T < 16) whose pooling
 * blocks are all whole (the routed scan's own routing) can be split:
 * SA_EUNSUPPORTED for other shapes unless phases is both bits.  The select
 * call must follow the scan call on the same stream order, with the same
 * arguments and workspace, untouched in between; nothing checks this.
 * Arguments and errors otherwise as in misa_route. */
int misa_route_phase(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
                     int32_t block_B, int32_t h, int32_t k_prime, const uint16_t* pooled,
                     int32_t* out_heads, int32_t* out_pool, int32_t* out_idx, float* out_score,
                     void* ws, size_t ws_bytes, int32_t phases, void* stream);

/* Workspace bytes for misa_route_fp8 (the same as for misa_route). */
int misa_route_fp8_ws(const sa_shape* s, int32_t block_B, int32_t h, int32_t k_prime,
                      int32_t pooled_given, size_t* ws_bytes);

/* misa_route over an FP8 key cache (PaperTrace section 2.3; codes and scales
 * as written by sa_quantize_keys_fp8): every stage reads key s as
 * scales[s] * e4m3(codes[s]) -- the pooled keys (when `pooled` is NULL; the
 * means in fp32), the routed scan (codes widened exactly to bf16, the scale
 * applied after the head sum) and MISA-dagger's rerank.  q stays bf16.
 * `pooled`, if given, holds the block means of the dequantized keys in the
 * sa_pool_blocks layout.  Decode-style rows only: T must be < 16
 * (SA_EUNSUPPORTED otherwise).  Other arguments, shapes, ownership and errors
 * as in misa_route. */
int misa_route_fp8(const uint16_t* q, const float* w, const uint8_t* codes, const float* scales,
                   const sa_shape* s, int32_t block_B, int32_t h, int32_t k_prime,
                   const uint16_t* pooled, int32_t* out_heads, int32_t* out_pool,
                   int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------- HISA */

/* Workspace bytes for hisa_coarse_fine.  reps_given: whether `reps` will be
 * passed. */
int hisa_coarse_fine_ws(const sa_shape* s, int32_t block_b, int32_t r, int32_t reps_given,
                        size_t* ws_bytes);

/* HISA block-then-token search (PaperTrace section 2.1; blog "Route 1:
 * HISA").  Block representatives (means of block_b keys; a block cut by the
 * causal bound is the mean of its legal keys) are scored with the full
 * indexer formula; the min(r, #legal blocks) best blocks are kept (ties ->
 * lower block); their legal tokens are rescored exactly and the token top-k
 * is returned with out_score = I.  Requires r * block_b >= topk (PaperTrace
 * section 2.3), else SA_EINVAL.
 *   reps       NULL or sa_pool_blocks(keys, ..., block_b) output.
 *   out_blocks [batch, T, r] kept blocks, -1 padded (nullable). */
int hisa_coarse_fine(const uint16_t* q, const float* w, const uint16_t* keys,
                     const sa_shape* s, int32_t block_b, int32_t r, const uint16_t* reps,
                     int32_t* out_blocks, int32_t* out_idx, float* out_score, void* ws,
                     size_t ws_bytes, void* stream);

/* Workspace bytes for hisa_coarse_fine_fp8 (the same as for hisa_coarse_fine). */
int hisa_coarse_fine_fp8_ws(const sa_shape* s, int32_t block_b, int32_t r, int32_t reps_given,
                            size_t* ws_bytes);

/* hisa_coarse_fine over an FP8 key cache: block representatives (when `reps`
 * is NULL) are the fp32 means of the dequantized keys, and the fine stage
 * rescores the kept blocks' tokens from the codes (widened exactly, the key's
 * scale applied after the head sum).  Other arguments, shapes, ownership and
 * errors as in hisa_coarse_fine. */
int hisa_coarse_fine_fp8(const uint16_t* q, const float* w, const uint8_t* codes,
                         const float* scales, const sa_shape* s, int32_t block_b, int32_t r,
                         const uint16_t* reps, int32_t* out_blocks, int32_t* out_idx,
                         float* out_score, void* ws, size_t ws_bytes, void* stream);

/* -------------------------------------------------------- MISA x HISA */

/* Workspace bytes for misa_hisa. */
int misa_hisa_ws(const sa_shape* s, int32_t block_B, int32_t h, int32_t block_b, int32_t r,
                 int32_t pooled_given, int32_t reps_given, size_t* ws_bytes);

/* MISA x HISA: the head axis and the token axis in series ("MISA" summary
 * page, core method point (1): routing heads is orthogonal to HISA's
 * block-to-token hierarchy and the two can be chained).
 *   1. MISA router on the pooled keys (blocks of block_B): the h heads with
 *      the largest E_j = mean_m |w_j ReLU(q_j . pooled_m)| (misa_route).
 *   2. HISA coarse stage with those heads only: block scores
 *      J_m = sum_{j routed} w_j ReLU(q_j . rep_m) over blocks of block_b
 *      (reps: block means), the r best blocks (ties -> lower block).
 *   3. Fine stage: every legal token of the kept blocks scored with all H
 *      heads, token top-k; out_score = I.
 * pooled / reps: NULL (pooled inside the call) or sa_pool_blocks output for
 * block_B / block_b.  out_heads [batch, T, h] ascending, out_blocks [batch,
 * T, r] (both nullable).  Requires 1 <= h <= H and r * block_b >= topk.
 * Other arguments, ownership and errors as in indexer_score_topk. */
int misa_hisa(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
              int32_t block_B, int32_t h, int32_t block_b, int32_t r, const uint16_t* pooled,
              const uint16_t* reps, int32_t* out_heads, int32_t* out_blocks, int32_t* out_idx,
              float* out_score, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------- LISA / ResMiSA */

/* Workspace bytes for lisa_score_topk. */
int lisa_score_topk_ws(const sa_shape* s, size_t* ws_bytes);

/* LISA linear score (PaperTrace "2.2.2 MISA, LISA and ResMiSA", section 3.1):
 * with the fused query g_t = sum_j w_j q_j (one key shared by every head),
 *   l[t,s] = g_t . k_s
 * for every legal key s <= t, then the top-k by l with the selection rules of
 * indexer_score_topk; out_score = l.  g is formed in fp32 and carried as a
 * bf16 hi/lo pair (~2^-16 relative).  Any T; arguments, ownership and errors
 * as in indexer_score_topk. */
int lisa_score_topk(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
                    int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                    void* stream);

/* Per-block key extrema, the cache-side state of ResMiSA's routing bound.
 * Block m covers keys [m*block, min((m+1)*block, L)).  out: [batch,
 * ceil(L/block), 2, d] bf16 bit patterns: per block the per-dimension maximum,
 * then the minimum (exact: extrema of bf16 values). */
int sa_block_extrema(const uint16_t* keys, int32_t batch, int32_t L, int32_t d, int32_t block,
                     uint16_t* out, void* stream);

/* Workspace bytes for resmisa_route.  extrema_given: whether `extrema` will
 * be passed (non-NULL) to resmisa_route. */
int resmisa_route_ws(const sa_shape* s, int32_t block, int32_t r, int32_t extrema_given,
                     size_t* ws_bytes);

/* ResMiSA / MISA-2 (same page, section 3.2): the shared linear score plus r
 * routed residual heads,
 *   R[t,s] = l[t,s] + sum_{h in A_t} w_h * ReLU(-(q_h . k_s)),
 * then the top-k by R (selection rules of indexer_score_topk; out_score = R).
 *   block    size of the blocks whose key extrema bound the residuals.
 *   r        residual heads per query, 0 <= r <= H; 4 + r must be <= 64
 *            unless r == H (SA_EUNSUPPORTED otherwise).  r = 0 is LISA,
 *            r = H the DSA score.  Routing: for every block b that
 *            intersects [0, t] (a block cut by the causal bound uses the
 *            extrema of its legal keys) and head h,
 *              U-[h,b] = sum_d (max(-q_hd,0) kmax_bd - max(q_hd,0) kmin_bd),
 *            S_h = |w_h| max_b ReLU(U-[h,b]); A_t = the r largest S_h
 *            (ties -> lower head).
 *   extrema  NULL (computed inside the call) or sa_block_extrema(keys, ...,
 *            block) output for these keys.
 *   out_heads [batch, T, r] routed heads, ascending (nullable).
 * Other arguments, ownership and errors as in indexer_score_topk. */
int resmisa_route(const uint16_t* q, const float* w, const uint16_t* keys, const sa_shape* s,
                  int32_t block, int32_t r, const uint16_t* extrema, int32_t* out_heads,
                  int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ diagnostics */

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* sa_last_error(void);

/* Per-kernel timing with HIP events recorded on the launch stream around
 * every kernel this library launches.  enable(1) resets the counters and
 * starts recording; enable(0) stops.  sa_profile_read synchronises the
 * recorded events and returns the summed duration and launch count of
 * kernel `id` (0 <= id < sa_kernel_count()). */
int sa_profile_enable(int32_t on);
int sa_profile_read(int32_t id, double* total_ms, int64_t* launches);
int32_t sa_kernel_count(void);
const char* sa_kernel_name(int32_t id);

#ifdef __cplusplus
}
#endif

#endif
