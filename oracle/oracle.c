/*
 * CPU oracle for the DSA lightning-indexer selector and its MISA / HISA
 * accelerations.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never does.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Arithmetic: every bf16 / fp32 input is widened exactly to fp64; all dot
 * products, head sums, block means and router statistics are fp64, summed in
 * the natural index order (dimension order, then head order).
 *
 * Sources (cited by page title and section):
 *  [PT]   PaperTrace, "2.2.2 MISA, LISA and ResMiSA: when the indexer becomes
 *         the new bottleneck" -- section 1 (DSA score), 2.1 (HISA / MISA),
 *         2.3 (acceptance procedure, budgets r*b >= k, min(k, t)),
 *         3.1 (two-head worked example, score 6; the fused query and
 *         LISA's linear score), 3.2 (ResMiSA: the shared linear expert, r
 *         residual heads routed by the coordinate-box bound; the box example
 *         U- = 9).
 *  [MISA] "MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
 *         Inference" (structured paper summary), section "method steps"
 *         (steps 1-6 and the two-stage MISA-dagger variant).
 *  [BLOG] "The new bottleneck of sparse attention: from DSA to indexer
 *         acceleration and KV offload", sections "Route 1: HISA" and
 *         "Route 2: MISA".
 *  [PT] section 2.3, "from the formula to the FP8 cache": indexer keys are
 *         quantized in blocks to FP8 with one scale per block; the query
 *         stays at the compute precision; the key error bound and the 2E < m
 *         set-stability condition.  The FP8 format is OCP E4M3 (sign, 4
 *         exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the
 *         subnormals m * 2^-9; 0x7F / 0xFF are NaN; largest finite 448).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - causal legality is s <= t, t = causal_offset + row;
 *  - ReLU(0) = 0;
 *  - ties in every top-k (tokens, heads, blocks, the k' pool) go to the lower
 *    index, i.e. a stable sort of index-ordered input by descending score;
 *  - a block's pooled key is the mean of its *legal* keys (s <= t and s < L);
 *  - MISA and HISA keys are shared across heads (one key head), so the head
 *    subscript some formulas attach to the key is dropped;
 *  - MISA routes by |A| but scores with the sign of w kept;
 *  - ResMiSA's blocks have a caller-given size; a block cut by the causal
 *    bound takes the extrema of its legal keys only; routed heads are the r
 *    largest S_h, ties to the lower head.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

static double bf16_to_f64(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    double score;
    int32_t idx;
} scored_t;

/* Order: larger score first; equal scores -> smaller index first. */
static int scored_cmp(const void* a, const void* b)
{
    const scored_t* x = (const scored_t*)a;
    const scored_t* y = (const scored_t*)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    if (x->idx < y->idx) return -1;
    if (x->idx > y->idx) return 1;
    return 0;
}

/* Sort all n candidates by (score desc, idx asc) and keep the first
 * min(k, n).  Returns how many were kept. */
static int select_top(scored_t* cand, int n, int k)
{
    qsort(cand, (size_t)n, sizeof(scored_t), scored_cmp);
    return n < k ? n : k;
}

/* z = q_j . key, fp64, summed in dimension order. */
static double dot_q_key(const uint16_t* qj, const double* key, int d)
{
    double z = 0.0;
    for (int x = 0; x < d; ++x) z += bf16_to_f64(qj[x]) * key[x];
    return z;
}

/* I = sum over the listed heads (ascending order as given) of
 * w_j * max(q_j . key, 0).  heads == NULL means all H heads.
 * [PT] section 1; the worked example of [PT] section 3.1 evaluates this form
 * (1*ReLU(6) + 0.5*ReLU(-3) = 6). */
static double indexer_score(const uint16_t* qrow, const float* wrow, const double* key,
                            int H, int d, const int32_t* heads, int nheads)
{
    double acc = 0.0;
    int count = heads ? nheads : H;
    for (int u = 0; u < count; ++u) {
        int j = heads ? heads[u] : u;
        double z = dot_q_key(qrow + (size_t)j * d, key, d);
        double r = z > 0.0 ? z : 0.0;
        acc += (double)wrow[j] * r;
    }
    return acc;
}

static void widen_key(const uint16_t* k, int d, double* out)
{
    for (int x = 0; x < d; ++x) out[x] = bf16_to_f64(k[x]);
}

/* Mean of keys [lo, hi) of one sequence, fp64, summed in index order. */
static void pool_mean(const uint16_t* Kseq, int d, int lo, int hi, double* out)
{
    for (int x = 0; x < d; ++x) out[x] = 0.0;
    for (int s = lo; s < hi; ++s) {
        const uint16_t* k = Kseq + (size_t)s * d;
        for (int x = 0; x < d; ++x) out[x] += bf16_to_f64(k[x]);
    }
    double c = (double)(hi - lo);
    for (int x = 0; x < d; ++x) out[x] /= c;
}

/* ------------------------------------------------------- thread fan-out */

typedef struct {
    int (*fn)(void* ctx, int r);
    void* ctx;
    int nrows;
    int next;
    int err;
    pthread_mutex_t mu;
} pool_t;

static void* worker(void* arg)
{
    pool_t* p = (pool_t*)arg;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        int r = p->next++;
        pthread_mutex_unlock(&p->mu);
        if (r >= p->nrows) break;
        int e = p->fn(p->ctx, r);
        if (e) {
            pthread_mutex_lock(&p->mu);
            if (!p->err) p->err = e;
            pthread_mutex_unlock(&p->mu);
        }
    }
    return NULL;
}

static int run_rows(int (*fn)(void*, int), void* ctx, int nrows, int nthreads)
{
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.nrows = nrows;
    p.next = 0;
    p.err = 0;
    pthread_mutex_init(&p.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows > 0 ? nrows : 1;
    if (nthreads == 1) {
        worker(&p);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
        if (!th) return ORACLE_ENOMEM;
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &p);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&p.mu);
    return p.err;
}

/* ------------------------------------------------------ problem access */

static int check_problem(const oracle_problem* p)
{
    if (!p || !p->q || !p->w) return ORACLE_EINVAL;
    if (!p->K && !(p->codes && p->scales)) return ORACLE_EINVAL;
    if (p->Bt < 1 || p->T < 1 || p->H < 1 || p->d < 1 || p->L < 1) return ORACLE_EINVAL;
    if (p->causal_offset < 0 || (long)p->causal_offset + p->T > p->L) return ORACLE_EINVAL;
    return 0;
}

static const uint16_t* qrow_of(const oracle_problem* p, int row)
{
    return p->q + (size_t)row * p->H * p->d;
}
static const float* wrow_of(const oracle_problem* p, int row)
{
    return p->w + (size_t)row * p->H;
}
static const uint16_t* kseq_of(const oracle_problem* p, int row)
{
    int b = row / p->T;
    return p->K + (size_t)b * p->L * p->d;
}
static int t_of(const oracle_problem* p, int row)
{
    return p->causal_offset + row % p->T;
}

/* Key s of row's sequence in fp64: the bf16 key, or with an FP8 cache its
 * dequantized value scale * e4m3(code) (exact in fp64). */
static void key_of(const oracle_problem* p, int row, int s, double* out)
{
    const int b = row / p->T;
    const size_t at = (size_t)b * p->L + (size_t)s;
    if (p->codes) {
        const double a = (double)p->scales[at];
        const uint8_t* c = p->codes + at * p->d;
        for (int x = 0; x < p->d; ++x) out[x] = a * oracle_fp8_e4m3_decode(c[x]);
    } else {
        widen_key(p->K + at * p->d, p->d, out);
    }
}

/* Mean of keys [lo, hi) of row's sequence, fp64, summed in index order. */
static void pool_mean_of(const oracle_problem* p, int row, int lo, int hi, double* key,
                         double* out)
{
    for (int x = 0; x < p->d; ++x) out[x] = 0.0;
    for (int s = lo; s < hi; ++s) {
        key_of(p, row, s, key);
        for (int x = 0; x < p->d; ++x) out[x] += key[x];
    }
    double c = (double)(hi - lo);
    for (int x = 0; x < p->d; ++x) out[x] /= c;
}

static void write_topk(const scored_t* c, int kept, int topk, int32_t* idx, double* score)
{
    for (int u = 0; u < topk; ++u) {
        if (u < kept) {
            idx[u] = c[u].idx;
            score[u] = c[u].score;
        } else {
            idx[u] = -1;
            score[u] = -INFINITY;
        }
    }
}

/* ---------------------------------------------------------------- DSA */

typedef struct {
    const oracle_problem* p;
    int topk;
    const int32_t* rows;
    int32_t* out_idx;
    double* out_score;
    double* out_rowscore;
} dsa_ctx;

/* [PT] sections 1 and 2.3: score every causal prefix token s <= t of the
 * row, then keep the min(k, t+1) highest. */
static int dsa_row(void* vctx, int r)
{
    dsa_ctx* c = (dsa_ctx*)vctx;
    const oracle_problem* p = c->p;
    int row = c->rows ? c->rows[r] : r;
    int t = t_of(p, row);
    int n = t + 1;
    const uint16_t* qrow = qrow_of(p, row);
    const float* wrow = wrow_of(p, row);
    scored_t* cand = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
    double* key = (double*)malloc(sizeof(double) * (size_t)p->d);
    if (!cand || !key) {
        free(cand);
        free(key);
        return ORACLE_ENOMEM;
    }
    double* rs = c->out_rowscore ? c->out_rowscore + (size_t)r * p->L : NULL;
    for (int s = 0; s < n; ++s) {
        key_of(p, row, s, key);
        cand[s].score = indexer_score(qrow, wrow, key, p->H, p->d, NULL, 0);
        cand[s].idx = s;
        if (rs) rs[s] = cand[s].score;
    }
    if (rs)
        for (int s = n; s < p->L; ++s) rs[s] = NAN;
    int kept = select_top(cand, n, c->topk);
    write_topk(cand, kept, c->topk, c->out_idx + (size_t)r * c->topk,
               c->out_score + (size_t)r * c->topk);
    free(cand);
    free(key);
    return 0;
}

int oracle_dsa(const oracle_problem* p, int topk, const int32_t* rows, int nrows,
               int32_t* out_idx, double* out_score, double* out_rowscore, int nthreads)
{
    int e = check_problem(p);
    if (e) return e;
    if (topk < 1 || !out_idx || !out_score) return ORACLE_EINVAL;
    if (!rows) nrows = p->Bt * p->T;
    dsa_ctx c = {p, topk, rows, out_idx, out_score, out_rowscore};
    return run_rows(dsa_row, &c, nrows, nthreads);
}

/* --------------------------------------------------------------- MISA */

typedef struct {
    const oracle_problem* p;
    int topk, B, h, kprime;
    const int32_t* rows;
    const int32_t* override_heads;
    const int32_t* override_pool;
    int32_t* out_heads;
    double* out_E;
    int32_t* out_pool;
    double* out_hatrow;
    int32_t* out_idx;
    double* out_score;
} misa_ctx;

static int misa_row(void* vctx, int r)
{
    misa_ctx* c = (misa_ctx*)vctx;
    const oracle_problem* p = c->p;
    const int H = p->H, d = p->d;
    int row = c->rows ? c->rows[r] : r;
    int t = t_of(p, row);
    int n = t + 1;
    const uint16_t* qrow = qrow_of(p, row);
    const float* wrow = wrow_of(p, row);

    int Mt = t / c->B + 1; /* blocks that intersect the legal prefix [0, t] */
    double* pooled = (double*)malloc(sizeof(double) * (size_t)Mt * d);
    double* E = (double*)malloc(sizeof(double) * (size_t)H);
    scored_t* hc = (scored_t*)malloc(sizeof(scored_t) * (size_t)H);
    int32_t* heads = (int32_t*)malloc(sizeof(int32_t) * (size_t)c->h);
    scored_t* cand = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
    double* key = (double*)malloc(sizeof(double) * (size_t)d);
    int32_t* pool = c->kprime ? (int32_t*)malloc(sizeof(int32_t) * (size_t)c->kprime) : NULL;
    if (!pooled || !E || !hc || !heads || !cand || !key || (c->kprime && !pool)) {
        free(pooled); free(E); free(hc); free(heads); free(cand); free(key); free(pool);
        return ORACLE_ENOMEM;
    }

    /* Step 1 [MISA]: block mean-pool of the keys, blocks of B; only legal keys
     * enter a block's mean. */
    for (int m = 0; m < Mt; ++m) {
        int lo = m * c->B;
        int hi = lo + c->B;
        if (hi > n) hi = n;
        pool_mean_of(p, row, lo, hi, key, pooled + (size_t)m * d);
    }
    /* Step 2 [MISA]: A_{j,m} = w_j * ReLU(q_j . pooled_m);
     * E_j = (1/M) * sum_m |A_{j,m}|. */
    for (int j = 0; j < H; ++j) {
        double acc = 0.0;
        for (int m = 0; m < Mt; ++m) {
            double z = dot_q_key(qrow + (size_t)j * d, pooled + (size_t)m * d, d);
            double a = (double)wrow[j] * (z > 0.0 ? z : 0.0);
            acc += fabs(a);
        }
        E[j] = acc / (double)Mt;
        hc[j].score = E[j];
        hc[j].idx = j;
    }
    /* Step 3 [MISA]: the h heads with the largest E (ties -> lower head). */
    if (c->override_heads) {
        for (int u = 0; u < c->h; ++u) heads[u] = c->override_heads[(size_t)r * c->h + u];
    } else {
        select_top(hc, H, c->h);
        for (int u = 0; u < c->h; ++u) heads[u] = hc[u].idx;
    }
    /* Heads are summed in ascending head order. */
    for (int a = 1; a < c->h; ++a)
        for (int b2 = a; b2 > 0 && heads[b2 - 1] > heads[b2]; --b2) {
            int32_t tmp = heads[b2];
            heads[b2] = heads[b2 - 1];
            heads[b2 - 1] = tmp;
        }
    if (c->out_heads)
        for (int u = 0; u < c->h; ++u) c->out_heads[(size_t)r * c->h + u] = heads[u];
    if (c->out_E)
        for (int j = 0; j < H; ++j) c->out_E[(size_t)r * H + j] = E[j];

    /* Step 4 [MISA]: routed score over the selected heads only. */
    double* hr = c->out_hatrow ? c->out_hatrow + (size_t)r * p->L : NULL;
    for (int s = 0; s < n; ++s) {
        key_of(p, row, s, key);
        cand[s].score = indexer_score(qrow, wrow, key, H, d, heads, c->h);
        cand[s].idx = s;
        if (hr) hr[s] = cand[s].score;
    }
    if (hr)
        for (int s = n; s < p->L; ++s) hr[s] = NAN;

    int32_t* oidx = c->out_idx + (size_t)r * c->topk;
    double* oscore = c->out_score + (size_t)r * c->topk;
    if (c->kprime == 0) {
        /* Step 5 [MISA]: token top-k by the routed score. */
        int kept = select_top(cand, n, c->topk);
        write_topk(cand, kept, c->topk, oidx, oscore);
    } else {
        /* MISA-dagger [MISA]: top-k' by the routed score, then rescore that
         * pool with all heads and keep the top-k. */
        int np = 0;
        if (c->override_pool) {
            for (int u = 0; u < c->kprime; ++u) {
                int32_t s = c->override_pool[(size_t)r * c->kprime + u];
                if (s >= 0) pool[np++] = s;
            }
        } else {
            int kept = select_top(cand, n, c->kprime);
            for (int u = 0; u < kept; ++u) pool[np++] = cand[u].idx;
        }
        if (c->out_pool) {
            int32_t* op = c->out_pool + (size_t)r * c->kprime;
            for (int u = 0; u < c->kprime; ++u) op[u] = u < np ? pool[u] : -1;
        }
        for (int u = 0; u < np; ++u) {
            int32_t s = pool[u];
            key_of(p, row, s, key);
            cand[u].score = indexer_score(qrow, wrow, key, H, d, NULL, 0);
            cand[u].idx = s;
        }
        int kept = select_top(cand, np, c->topk);
        write_topk(cand, kept, c->topk, oidx, oscore);
    }
    free(pooled); free(E); free(hc); free(heads); free(cand); free(key); free(pool);
    return 0;
}

int oracle_misa(const oracle_problem* p, int topk, int B, int h, int kprime,
                const int32_t* rows, int nrows, const int32_t* override_heads,
                const int32_t* override_pool, int32_t* out_heads, double* out_E,
                int32_t* out_pool, double* out_hatrow, int32_t* out_idx, double* out_score,
                int nthreads)
{
    int e = check_problem(p);
    if (e) return e;
    if (topk < 1 || B < 1 || h < 1 || h > p->H || !out_idx || !out_score) return ORACLE_EINVAL;
    if (kprime != 0 && kprime < topk) return ORACLE_EINVAL;
    if (!rows) nrows = p->Bt * p->T;
    misa_ctx c = {p, topk, B, h, kprime, rows, override_heads, override_pool,
                  out_heads, out_E, out_pool, out_hatrow, out_idx, out_score};
    return run_rows(misa_row, &c, nrows, nthreads);
}

/* --------------------------------------------------------------- HISA */

typedef struct {
    const oracle_problem* p;
    int topk, b, r;
    const int32_t* rows;
    const int32_t* override_blocks;
    const int32_t* coarse_heads;
    int hsel;
    int32_t* out_blocks;
    double* out_J;
    int32_t* out_idx;
    double* out_score;
} hisa_ctx;

/* [PT] section 2.1 and [BLOG] "Route 1: HISA": block representatives are the
 * mean of b keys; blocks are scored with the indexer formula; the r best
 * blocks are kept and their tokens are rescored exactly; token top-k.
 * With coarse_heads (per row, hsel heads in ascending order) the block scores
 * sum only those heads: the MISA x HISA composition ([MISA] "core method",
 * point (1): head routing and HISA's token hierarchy are orthogonal and can
 * run in series), whose fine stage still rescores with every head. */
static int hisa_row(void* vctx, int rr)
{
    hisa_ctx* c = (hisa_ctx*)vctx;
    const oracle_problem* p = c->p;
    const int H = p->H, d = p->d;
    int row = c->rows ? c->rows[rr] : rr;
    int t = t_of(p, row);
    int n = t + 1;
    const uint16_t* qrow = qrow_of(p, row);
    const float* wrow = wrow_of(p, row);
    int nb = t / c->b + 1; /* blocks that intersect [0, t] */
    int nbmax = (p->L + c->b - 1) / c->b;

    double* rep = (double*)malloc(sizeof(double) * (size_t)d);
    scored_t* bc = (scored_t*)malloc(sizeof(scored_t) * (size_t)nb);
    int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(c->r < nb ? c->r : nb) + 4);
    double* key = (double*)malloc(sizeof(double) * (size_t)d);
    if (!rep || !bc || !blocks || !key) {
        free(rep); free(bc); free(blocks); free(key);
        return ORACLE_ENOMEM;
    }
    double* J = c->out_J ? c->out_J + (size_t)rr * nbmax : NULL;
    for (int m = 0; m < nb; ++m) {
        int lo = m * c->b;
        int hi = lo + c->b;
        if (hi > n) hi = n;
        pool_mean_of(p, row, lo, hi, key, rep);
        const int32_t* ch = c->coarse_heads ? c->coarse_heads + (size_t)rr * c->hsel : NULL;
        bc[m].score = indexer_score(qrow, wrow, rep, H, d, ch, c->hsel);
        bc[m].idx = m;
        if (J) J[m] = bc[m].score;
    }
    if (J)
        for (int m = nb; m < nbmax; ++m) J[m] = NAN;

    int nsel = 0;
    if (c->override_blocks) {
        for (int u = 0; u < c->r; ++u) {
            int32_t m = c->override_blocks[(size_t)rr * c->r + u];
            if (m >= 0 && nsel < nb) blocks[nsel++] = m;
        }
    } else {
        int kept = select_top(bc, nb, c->r);
        for (int u = 0; u < kept; ++u) blocks[nsel++] = bc[u].idx;
    }
    if (c->out_blocks) {
        int32_t* ob = c->out_blocks + (size_t)rr * c->r;
        for (int u = 0; u < c->r; ++u) ob[u] = u < nsel ? blocks[u] : -1;
    }
    /* Fine stage: exact indexer score on every legal token of the kept
     * blocks. */
    int ncand = 0;
    scored_t* cand = (scored_t*)malloc(sizeof(scored_t) * (size_t)nsel * c->b + 1);
    if (!cand) {
        free(rep); free(bc); free(blocks); free(key);
        return ORACLE_ENOMEM;
    }
    for (int u = 0; u < nsel; ++u) {
        int lo = blocks[u] * c->b;
        int hi = lo + c->b;
        if (hi > n) hi = n;
        for (int s = lo; s < hi; ++s) {
            key_of(p, row, s, key);
            cand[ncand].score = indexer_score(qrow, wrow, key, H, d, NULL, 0);
            cand[ncand].idx = s;
            ++ncand;
        }
    }
    int kept = select_top(cand, ncand, c->topk);
    write_topk(cand, kept, c->topk, c->out_idx + (size_t)rr * c->topk,
               c->out_score + (size_t)rr * c->topk);
    free(rep); free(bc); free(blocks); free(key); free(cand);
    return 0;
}

int oracle_hisa(const oracle_problem* p, int topk, int b, int r, const int32_t* rows,
                int nrows, const int32_t* override_blocks, const int32_t* coarse_heads,
                int hsel, int32_t* out_blocks, double* out_J, int32_t* out_idx,
                double* out_score, int nthreads)
{
    int e = check_problem(p);
    if (e) return e;
    if (topk < 1 || b < 1 || r < 1 || !out_idx || !out_score) return ORACLE_EINVAL;
    if ((long)r * b < topk) return ORACLE_EINVAL; /* [PT] 2.3: r*b >= k */
    if (coarse_heads && (hsel < 1 || hsel > p->H)) return ORACLE_EINVAL;
    if (!rows) nrows = p->Bt * p->T;
    hisa_ctx c = {p, topk, b, r, rows, override_blocks, coarse_heads, coarse_heads ? hsel : 0,
                  out_blocks, out_J, out_idx, out_score};
    return run_rows(hisa_row, &c, nrows, nthreads);
}

/* ---------------------------------------------------------------- FP8 */

/* Value of an OCP E4M3 code. */
double oracle_fp8_e4m3_decode(uint8_t c)
{
    double sign = (c & 0x80) ? -1.0 : 1.0;
    int e = (c >> 3) & 15;
    int m = c & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return sign * ldexp((double)m, -9);
    return sign * ldexp(1.0 + m / 8.0, e - 7);
}

/* Nearest E4M3 code to x: round to nearest, ties to the even code (mantissa
 * bit 0 clear), magnitudes above 448 saturate to 448; the sign is kept
 * (a value that rounds to zero keeps it, -0 -> 0x80).  Plain search over the
 * 127 finite magnitudes. */
uint8_t oracle_fp8_e4m3_encode(float x)
{
    double a = fabs((double)x);
    uint8_t s = signbit(x) ? 0x80 : 0x00;
    int best = 0;
    double bd = a;  /* distance to code 0 */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(oracle_fp8_e4m3_decode((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    if (a >= 448.0) best = 0x7E;
    return (uint8_t)(s | best);
}

/* [PT] section 2.3: one scale per key (the block is the key's d = 128
 * values): a = max_x |k_x| / 448 in fp32 (1 for an all-zero key), codes
 * c_x = E4M3(k_x / a) with the division in fp32. */
static void quantize_one_key(const uint16_t* k, int d, uint8_t* codes, float* scale)
{
    float amax = 0.0f;
    for (int x = 0; x < d; ++x) {
        float v = (float)fabs(bf16_to_f64(k[x]));
        if (v > amax) amax = v;
    }
    float a = amax > 0.0f ? amax / 448.0f : 1.0f;
    *scale = a;
    for (int x = 0; x < d; ++x) {
        float v = (float)bf16_to_f64(k[x]) / a;
        codes[x] = oracle_fp8_e4m3_encode(v);
    }
}

typedef struct {
    const uint16_t* K;
    long n_keys;
    int d;
    uint8_t* codes;
    float* scales;
} quant_ctx;

enum { QUANT_KEYS_PER_TASK = 1024 };

static int quant_task(void* vctx, int r)
{
    const quant_ctx* c = (const quant_ctx*)vctx;
    long lo = (long)r * QUANT_KEYS_PER_TASK;
    long hi = lo + QUANT_KEYS_PER_TASK < c->n_keys ? lo + QUANT_KEYS_PER_TASK : c->n_keys;
    for (long s = lo; s < hi; ++s)
        quantize_one_key(c->K + (size_t)s * c->d, c->d, c->codes + (size_t)s * c->d,
                         c->scales + s);
    return 0;
}

int oracle_quantize_keys_fp8(const uint16_t* K, long n_keys, int d, uint8_t* codes,
                             float* scales, int nthreads)
{
    if (!K || !codes || !scales || n_keys < 0 || d < 1) return ORACLE_EINVAL;
    quant_ctx c = {K, n_keys, d, codes, scales};
    long ntask = (n_keys + QUANT_KEYS_PER_TASK - 1) / QUANT_KEYS_PER_TASK;
    if (ntask > 0x7fffffffL) return ORACLE_EINVAL;
    return run_rows(quant_task, &c, (int)ntask, nthreads);
}

typedef struct {
    const oracle_problem* p;
    const uint8_t* codes;
    const float* scales;
    int topk;
    const int32_t* rows;
    int32_t* out_idx;
    double* out_score;
    double* out_rowscore;
} dsa8_ctx;

/* DSA (as dsa_row) on the dequantized keys a_s * decode(c_s), exact in fp64. */
static int dsa8_row(void* vctx, int r)
{
    dsa8_ctx* c = (dsa8_ctx*)vctx;
    const oracle_problem* p = c->p;
    int row = c->rows ? c->rows[r] : r;
    int t = t_of(p, row);
    int n = t + 1;
    int b = row / p->T;
    const uint16_t* qrow = qrow_of(p, row);
    const float* wrow = wrow_of(p, row);
    scored_t* cand = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
    double* key = (double*)malloc(sizeof(double) * (size_t)p->d);
    if (!cand || !key) {
        free(cand);
        free(key);
        return ORACLE_ENOMEM;
    }
    double* rs = c->out_rowscore ? c->out_rowscore + (size_t)r * p->L : NULL;
    for (int s = 0; s < n; ++s) {
        size_t ks = (size_t)b * p->L + s;
        for (int x = 0; x < p->d; ++x)
            key[x] = (double)c->scales[ks] * oracle_fp8_e4m3_decode(c->codes[ks * p->d + x]);
        cand[s].score = indexer_score(qrow, wrow, key, p->H, p->d, NULL, 0);
        cand[s].idx = s;
        if (rs) rs[s] = cand[s].score;
    }
    if (rs)
        for (int s = n; s < p->L; ++s) rs[s] = NAN;
    int kept = select_top(cand, n, c->topk);
    write_topk(cand, kept, c->topk, c->out_idx + (size_t)r * c->topk,
               c->out_score + (size_t)r * c->topk);
    free(cand);
    free(key);
    return 0;
}

int oracle_dsa_fp8(const oracle_problem* p, const uint8_t* codes, const float* scales, int topk,
                   const int32_t* rows, int nrows, int32_t* out_idx, double* out_score,
                   double* out_rowscore, int nthreads)
{
    if (!p || !p->q || !p->w || !codes || !scales) return ORACLE_EINVAL;
    if (p->Bt < 1 || p->T < 1 || p->H < 1 || p->d < 1 || p->L < 1) return ORACLE_EINVAL;
    if (p->causal_offset < 0 || (long)p->causal_offset + p->T > p->L) return ORACLE_EINVAL;
    if (topk < 1 || !out_idx || !out_score) return ORACLE_EINVAL;
    if (!rows) nrows = p->Bt * p->T;
    dsa8_ctx c = {p, codes, scales, topk, rows, out_idx, out_score, out_rowscore};
    return run_rows(dsa8_row, &c, nrows, nthreads);
}

/* DSA on FP8 keys with the query converted to E4M3 as well ([PT] section
 * 2.3: the query is converted to the compute type of the fp8 product; its
 * quantization error adds to the key's).  Each head vector q_{t,j} is
 * quantized by the key rule of quantize_one_key (scale b_j = max|q|/448 in
 * fp32, codes of q/b_j), so the row's query is the dequantized
 * qhat_j = b_j * e4m3(qc_j); key s is khat_s = a_s * e4m3(c_s).  The score is
 * the plain indexer formula on those vectors, in fp64:
 *   I = sum_j w_j * max(qhat_j . khat_s, 0). */
static int dsa8q_row(void* vctx, int r)
{
    dsa8_ctx* c = (dsa8_ctx*)vctx;
    const oracle_problem* p = c->p;
    int row = c->rows ? c->rows[r] : r;
    int t = t_of(p, row);
    int n = t + 1;
    int b = row / p->T;
    const uint16_t* qrow = qrow_of(p, row);
    const float* wrow = wrow_of(p, row);
    scored_t* cand = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
    double* key = (double*)malloc(sizeof(double) * (size_t)p->d);
    double* qhat = (double*)malloc(sizeof(double) * (size_t)p->H * p->d);
    uint8_t* qc = (uint8_t*)malloc((size_t)p->d);
    if (!cand || !key || !qhat || !qc) {
        free(cand);
        free(key);
        free(qhat);
        free(qc);
        return ORACLE_ENOMEM;
    }
    for (int j = 0; j < p->H; ++j) {
        float bj;
        quantize_one_key(qrow + (size_t)j * p->d, p->d, qc, &bj);
        for (int x = 0; x < p->d; ++x)
            qhat[(size_t)j * p->d + x] = (double)bj * oracle_fp8_e4m3_decode(qc[x]);
    }
    double* rs = c->out_rowscore ? c->out_rowscore + (size_t)r * p->L : NULL;
    for (int s = 0; s < n; ++s) {
        size_t ks = (size_t)b * p->L + s;
        for (int x = 0; x < p->d; ++x)
            key[x] = (double)c->scales[ks] * oracle_fp8_e4m3_decode(c->codes[ks * p->d + x]);
        double acc = 0.0;
        for (int j = 0; j < p->H; ++j) {
            double z = 0.0;
            for (int x = 0; x < p->d; ++x) z += qhat[(size_t)j * p->d + x] * key[x];
            acc += (double)wrow[j] * (z > 0.0 ? z : 0.0);
        }
        cand[s].score = acc;
        cand[s].idx = s;
        if (rs) rs[s] = acc;
    }
    if (rs)
        for (int s = n; s < p->L; ++s) rs[s] = NAN;
    int kept = select_top(cand, n, c->topk);
    write_topk(cand, kept, c->topk, c->out_idx + (size_t)r * c->topk,
               c->out_score + (size_t)r * c->topk);
    free(cand);
    free(key);
    free(qhat);
    free(qc);
    return 0;
}

int oracle_dsa_fp8q(const oracle_problem* p, const uint8_t* codes, const float* scales, int topk,
                    const int32_t* rows, int nrows, int32_t* out_idx, double* out_score,
                    double* out_rowscore, int nthreads)
{
    if (!p || !p->q || !p->w || !codes || !scales) return ORACLE_EINVAL;
    if (p->Bt < 1 || p->T < 1 || p->H < 1 || p->d < 1 || p->L < 1) return ORACLE_EINVAL;
    if (p->causal_offset < 0 || (long)p->causal_offset + p->T > p->L) return ORACLE_EINVAL;
    if (topk < 1 || !out_idx || !out_score) return ORACLE_EINVAL;
    if (!rows) nrows = p->Bt * p->T;
    dsa8_ctx c = {p, codes, scales, topk, rows, out_idx, out_score, out_rowscore};
    return run_rows(dsa8q_row, &c, nrows, nthreads);
}

/* --------------------------------------------------------------- pool */

int oracle_pool(const uint16_t* K, int Bt, int L, int d, int block, double* out)
{
    if (!K || !out || Bt < 1 || L < 1 || d < 1 || block < 1) return ORACLE_EINVAL;
    int nb = (L + block - 1) / block;
    for (int b = 0; b < Bt; ++b) {
        const uint16_t* Kseq = K + (size_t)b * L * d;
        for (int m = 0; m < nb; ++m) {
            int lo = m * block;
            int hi = lo + block;
            if (hi > L) hi = L;
            pool_mean(Kseq, d, lo, hi, out + ((size_t)b * nb + m) * d);
        }
    }
    return 0;
}

/* ------------------------------------------------------ LISA / ResMiSA */

/* [PT] section 3.1: with one key shared by every head,
 * ReLU(x) = x + ReLU(-x) splits the score into a linear term and a
 * nonlinear correction, I = l + c with
 *   l = sum_j w_j (q_j . k) = g . k,   g = sum_j w_j q_j   (the fused query),
 *   c = sum_j w_j ReLU(-(q_j . k)).
 * LISA ranks by l alone.  [PT] section 3.2 (ResMiSA / MISA-2) keeps l for
 * every key and adds the corrections of r routed residual heads A:
 *   R = l + sum_{h in A} w_h ReLU(-(q_h . k)).
 * Routing bounds each head's possible correction over the legal history: for
 * a block of keys with per-dimension extrema [kmin_d, kmax_d] and
 * q+ = max(q, 0), q- = max(-q, 0),
 *   U-_h = sum_d (q-_{h,d} kmax_d - q+_{h,d} kmin_d) >= -(q_h . k)
 * for every key of the block, and S_h = |w_h| max_b ReLU(U-_{h,b}) over the
 * blocks that intersect [0, t], a cut block taking the extrema of its legal
 * keys only.  A = the r heads with the largest S_h (ties -> lower head). */

double oracle_box_bound(const double* q, const double* kmin, const double* kmax, int d);

/* g = sum_j w_j q_j in fp64, heads in order. */
static void fused_query(const uint16_t* qrow, const float* wrow, int H, int d, double* g)
{
    for (int x = 0; x < d; ++x) g[x] = 0.0;
    for (int j = 0; j < H; ++j)
        for (int x = 0; x < d; ++x) g[x] += (double)wrow[j] * bf16_to_f64(qrow[(size_t)j * d + x]);
}

static double dot_f64(const double* a, const double* b, int d)
{
    double z = 0.0;
    for (int x = 0; x < d; ++x) z += a[x] * b[x];
    return z;
}

typedef struct {
    const oracle_problem* p;
    int topk, block, r;
    const int32_t* rows;
    const int32_t* override_heads;
    int32_t* out_heads;
    double* out_S;
    double* out_rowscore;
    int32_t* out_idx;
    double* out_score;
} resmisa_ctx;

static int resmisa_row(void* vctx, int rr)
{
    resmisa_ctx* c = (resmisa_ctx*)vctx;
    const oracle_problem* p = c->p;
    const int H = p->H, d = p->d, r = c->r;
    int row = c->rows ? c->rows[rr] : rr;
    int t = t_of(p, row);
    int n = t + 1;
    const uint16_t* qrow = qrow_of(p, row);
    const float* wrow = wrow_of(p, row);
    const uint16_t* Kseq = kseq_of(p, row);

    double* g = (double*)malloc(sizeof(double) * (size_t)d);
    double* key = (double*)malloc(sizeof(double) * (size_t)d);
    double* kmax = (double*)malloc(sizeof(double) * (size_t)d);
    double* kmin = (double*)malloc(sizeof(double) * (size_t)d);
    double* S = (double*)malloc(sizeof(double) * (size_t)H);
    scored_t* hc = (scored_t*)malloc(sizeof(scored_t) * (size_t)H);
    int32_t* heads = (int32_t*)malloc(sizeof(int32_t) * (size_t)(r > 0 ? r : 1));
    scored_t* cand = (scored_t*)malloc(sizeof(scored_t) * (size_t)n);
    if (!g || !key || !kmax || !kmin || !S || !hc || !heads || !cand) {
        free(g); free(key); free(kmax); free(kmin); free(S); free(hc); free(heads); free(cand);
        return ORACLE_ENOMEM;
    }
    fused_query(qrow, wrow, H, d, g);

    if (r > 0) {
        /* Routing statistic S_h over the blocks intersecting [0, t]. */
        for (int j = 0; j < H; ++j) S[j] = 0.0;  /* max of ReLU(.) >= 0 */
        int nb = t / c->block + 1;
        for (int m = 0; m < nb; ++m) {
            int lo = m * c->block;
            int hi = lo + c->block;
            if (hi > n) hi = n;
            for (int x = 0; x < d; ++x) {
                kmax[x] = -INFINITY;
                kmin[x] = INFINITY;
            }
            for (int s = lo; s < hi; ++s)
                for (int x = 0; x < d; ++x) {
                    double v = bf16_to_f64(Kseq[(size_t)s * d + x]);
                    if (v > kmax[x]) kmax[x] = v;
                    if (v < kmin[x]) kmin[x] = v;
                }
            for (int j = 0; j < H; ++j) {
                widen_key(qrow + (size_t)j * d, d, key);
                double U = oracle_box_bound(key, kmin, kmax, d);
                double bound = fabs((double)wrow[j]) * (U > 0.0 ? U : 0.0);
                if (bound > S[j]) S[j] = bound;
            }
        }
        for (int j = 0; j < H; ++j) {
            hc[j].score = S[j];
            hc[j].idx = j;
        }
        if (c->override_heads) {
            for (int u = 0; u < r; ++u) heads[u] = c->override_heads[(size_t)rr * r + u];
        } else {
            select_top(hc, H, r);
            for (int u = 0; u < r; ++u) heads[u] = hc[u].idx;
        }
        /* ascending head order for the residual sum */
        for (int a = 1; a < r; ++a)
            for (int b2 = a; b2 > 0 && heads[b2 - 1] > heads[b2]; --b2) {
                int32_t tmp = heads[b2];
                heads[b2] = heads[b2 - 1];
                heads[b2 - 1] = tmp;
            }
        if (c->out_heads)
            for (int u = 0; u < r; ++u) c->out_heads[(size_t)rr * r + u] = heads[u];
        if (c->out_S)
            for (int j = 0; j < H; ++j) c->out_S[(size_t)rr * H + j] = S[j];
    }

    double* rs = c->out_rowscore ? c->out_rowscore + (size_t)rr * p->L : NULL;
    for (int s = 0; s < n; ++s) {
        widen_key(Kseq + (size_t)s * d, d, key);
        double R = dot_f64(g, key, d);  /* l = g . k */
        for (int u = 0; u < r; ++u) {
            int j = heads[u];
            double z = dot_q_key(qrow + (size_t)j * d, key, d);
            double neg = -z;
            R += (double)wrow[j] * (neg > 0.0 ? neg : 0.0);
        }
        cand[s].score = R;
        cand[s].idx = s;
        if (rs) rs[s] = R;
    }
    if (rs)
        for (int s = n; s < p->L; ++s) rs[s] = NAN;
    int kept = select_top(cand, n, c->topk);
    write_topk(cand, kept, c->topk, c->out_idx + (size_t)rr * c->topk,
               c->out_score + (size_t)rr * c->topk);
    free(g); free(key); free(kmax); free(kmin); free(S); free(hc); free(heads); free(cand);
    return 0;
}

int oracle_resmisa(const oracle_problem* p, int topk, int block, int r, const int32_t* rows,
                   int nrows, const int32_t* override_heads, int32_t* out_heads, double* out_S,
                   double* out_rowscore, int32_t* out_idx, double* out_score, int nthreads)
{
    int e = check_problem(p);
    if (e) return e;
    if (!p->K) return ORACLE_EINVAL; /* bf16 keys only */
    if (topk < 1 || r < 0 || r > p->H || (r > 0 && block < 1) || !out_idx || !out_score)
        return ORACLE_EINVAL;
    if (!rows) nrows = p->Bt * p->T;
    resmisa_ctx c = {p, topk, block, r, rows, override_heads, out_heads, out_S, out_rowscore,
                     out_idx, out_score};
    return run_rows(resmisa_row, &c, nrows, nthreads);
}

/* LISA: the linear score alone (ResMiSA with no residual head). */
int oracle_lisa(const oracle_problem* p, int topk, const int32_t* rows, int nrows,
                int32_t* out_idx, double* out_score, double* out_rowscore, int nthreads)
{
    return oracle_resmisa(p, topk, 0, 0, rows, nrows, NULL, NULL, NULL, out_rowscore, out_idx,
                          out_score, nthreads);
}

/* The routing bound of one head over one box: U- = sum_d (q-_d kmax_d -
 * q+_d kmin_d), fp64 inputs (exposed for the worked example of [PT] 3.2). */
double oracle_box_bound(const double* q, const double* kmin, const double* kmax, int d)
{
    double U = 0.0;
    for (int x = 0; x < d; ++x) {
        double qpos = q[x] > 0.0 ? q[x] : 0.0;
        double qneg = q[x] < 0.0 ? -q[x] : 0.0;
        U += qneg * kmax[x] - qpos * kmin[x];
    }
    return U;
}
