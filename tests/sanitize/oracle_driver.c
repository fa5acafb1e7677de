/*
 * Host driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of
 * the CPU oracle (oracle/oracle.c): every oracle entry point on small seeded
 * problems (several threads, causal rows, cut blocks, override inputs, FP8
 * keys) and on rejected arguments.  Exits non-zero on a failed check; the
 * sanitizers abort on any memory or undefined-behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9e3779b97f4a7c15ull;

static double uniform(void)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_state >> 11) / 9007199254740992.0;
}

static uint16_t bf16_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static int failures = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static void check_rows(const int32_t* idx, int nrows, int topk, const oracle_problem* p)
{
    for (int r = 0; r < nrows; ++r) {
        int t = p->causal_offset + r % p->T;
        for (int u = 0; u < topk; ++u) {
            int s = idx[(size_t)r * topk + u];
            CHECK(s == -1 || (s >= 0 && s <= t));
        }
    }
}

int main(void)
{
    enum { Bt = 2, T = 5, H = 6, D = 16, L = 97, OFF = L - T, TOPK = 9 };
    uint16_t* q = malloc(sizeof(uint16_t) * Bt * T * H * D);
    float* w = malloc(sizeof(float) * Bt * T * H);
    uint16_t* K = malloc(sizeof(uint16_t) * Bt * L * D);
    for (int i = 0; i < Bt * T * H * D; ++i) q[i] = bf16_of((float)(uniform() * 2 - 1));
    for (int i = 0; i < Bt * T * H; ++i) w[i] = (float)(uniform() * 2 - 1);
    for (int i = 0; i < Bt * L * D; ++i) K[i] = bf16_of((float)(uniform() * 2 - 1));
    oracle_problem p = {q, w, K, Bt, T, H, D, L, OFF, NULL, NULL};
    const int nrows = Bt * T;
    int32_t* idx = malloc(sizeof(int32_t) * nrows * 64);
    double* sc = malloc(sizeof(double) * nrows * 64);
    double* rs = malloc(sizeof(double) * nrows * L);

    CHECK(oracle_dsa(&p, TOPK, NULL, 0, idx, sc, rs, 3) == 0);
    check_rows(idx, nrows, TOPK, &p);
    int32_t rows[3] = {0, 4, 9};
    CHECK(oracle_dsa(&p, TOPK, rows, 3, idx, sc, NULL, 2) == 0);

    int32_t heads[10 * 3], pool[10 * 20];
    double E[10 * H], hat[10 * L];
    CHECK(oracle_misa(&p, TOPK, 16, 3, 0, NULL, 0, NULL, NULL, heads, E, NULL, hat, idx, sc, 4) == 0);
    check_rows(idx, nrows, TOPK, &p);
    CHECK(oracle_misa(&p, TOPK, 30, 3, 20, NULL, 0, NULL, NULL, heads, E, pool, NULL, idx, sc, 4) == 0);
    check_rows(idx, nrows, TOPK, &p);
    CHECK(oracle_misa(&p, TOPK, 30, 3, 20, NULL, 0, heads, pool, NULL, NULL, NULL, NULL, idx, sc, 1) == 0);

    int32_t blocks[10 * 4];
    double J[10 * 7];
    CHECK(oracle_hisa(&p, TOPK, 16, 4, NULL, 0, NULL, NULL, 0, blocks, J, idx, sc, 3) == 0);
    check_rows(idx, nrows, TOPK, &p);
    CHECK(oracle_hisa(&p, TOPK, 16, 4, NULL, 0, blocks, heads, 3, NULL, NULL, idx, sc, 3) == 0);

    double* pooled = malloc(sizeof(double) * Bt * 4 * D);
    CHECK(oracle_pool(K, Bt, L, D, 30, pooled) == 0);

    uint8_t* codes = malloc((size_t)Bt * L * D);
    float* scales = malloc(sizeof(float) * Bt * L);
    CHECK(oracle_quantize_keys_fp8(K, Bt * L, D, codes, scales, 3) == 0);
    CHECK(oracle_dsa_fp8(&p, codes, scales, TOPK, NULL, 0, idx, sc, rs, 2) == 0);
    check_rows(idx, nrows, TOPK, &p);
    CHECK(oracle_dsa_fp8q(&p, codes, scales, TOPK, NULL, 0, idx, sc, rs, 2) == 0);
    check_rows(idx, nrows, TOPK, &p);
    oracle_problem p8 = {q, w, NULL, Bt, T, H, D, L, OFF, codes, scales};
    CHECK(oracle_misa(&p8, TOPK, 16, 2, 0, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, idx, sc, 2) == 0);
    CHECK(oracle_hisa(&p8, TOPK, 16, 4, NULL, 0, NULL, NULL, 0, NULL, NULL, idx, sc, 2) == 0);
    for (int c = 0; c < 256; ++c) {
        double v = oracle_fp8_e4m3_decode((uint8_t)c);
        if (!isnan(v)) CHECK(oracle_fp8_e4m3_decode(oracle_fp8_e4m3_encode((float)v)) == v);
    }

    CHECK(oracle_lisa(&p, TOPK, NULL, 0, idx, sc, rs, 2) == 0);
    int32_t rheads[10 * 2];
    double S[10 * H];
    CHECK(oracle_resmisa(&p, TOPK, 8, 2, NULL, 0, NULL, rheads, S, rs, idx, sc, 3) == 0);
    check_rows(idx, nrows, TOPK, &p);
    CHECK(oracle_resmisa(&p, TOPK, 8, 0, NULL, 0, NULL, NULL, NULL, NULL, idx, sc, 1) == 0);
    double bq[2] = {1.0, -2.0}, kmin[2] = {-1.0, 0.0}, kmax[2] = {3.0, 4.0};
    CHECK(oracle_box_bound(bq, kmin, kmax, 2) == 9.0);

    /* rejected arguments */
    CHECK(oracle_dsa(NULL, TOPK, NULL, 0, idx, sc, NULL, 1) != 0);
    CHECK(oracle_dsa(&p, 0, NULL, 0, idx, sc, NULL, 1) != 0);
    oracle_problem bad = p;
    bad.causal_offset = L;
    CHECK(oracle_dsa(&bad, TOPK, NULL, 0, idx, sc, NULL, 1) != 0);
    CHECK(oracle_hisa(&p, 64, 4, 2, NULL, 0, NULL, NULL, 0, NULL, NULL, idx, sc, 1) != 0);
    CHECK(oracle_pool(K, Bt, L, D, 0, pooled) != 0);

    free(q);
    free(w);
    free(K);
    free(idx);
    free(sc);
    free(rs);
    free(pooled);
    free(codes);
    free(scales);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver ok\n");
    return 0;
}
