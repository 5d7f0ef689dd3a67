/* oracle_checks.c -- runs every oracle function on small ragged shapes with
 * exact-size heap buffers, so that AddressSanitizer sees any read or write
 * past an input or output.  Values are checked only where a cheap identity
 * holds (split partials sum to the projection, the table's offsets add up);
 * the oracle's numerics are pinned by the Python tests.  Exit 0 when clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int failures = 0;
#define EXPECT(c)                                                             \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "oracle_checks: line %d: %s\n", __LINE__, #c);    \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static uint32_t rng = 12345u;
static uint32_t next(void) {
    rng = rng * 1664525u + 1013904223u;
    return rng >> 8;
}

static uint16_t* bf16s(int64_t n) {
    uint16_t* p = malloc((size_t)n * sizeof *p);
    for (int64_t i = 0; i < n; ++i) {
        const double v = ((double)(next() % 2001) - 1000.0) / 997.0;
        p[i] = oracle_f64_to_bf16(v);
    }
    return p;
}

static uint8_t* bytes(int64_t n, uint32_t lo, uint32_t hi) {
    uint8_t* p = malloc((size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = (uint8_t)(lo + next() % (hi - lo + 1));
    return p;
}

static void projection_and_splits(int64_t M, int64_t N, int64_t K) {
    uint16_t* x = bf16s(M * K);
    uint16_t* W = bf16s(N * K);
    double* y = malloc((size_t)(M * N) * sizeof *y);
    double* a = malloc((size_t)(M * N) * sizeof *a);
    oracle_projection(M, N, K, x, W, y, a);
    oracle_projection(M, N, K, x, W, y, NULL);
    for (int64_t S = 1; S <= 9; S += 2) {
        double* P = malloc((size_t)(S * M * N) * sizeof *P);
        double* ys = malloc((size_t)(M * N) * sizeof *ys);
        oracle_splitk_partials(M, N, K, S, x, W, P);
        oracle_splitk_sum(S, M * N, P, ys);
        for (int64_t i = 0; i < M * N; ++i) EXPECT(fabs(ys[i] - y[i]) <= 1e-12 * (a[i] + 1.0));
        free(P);
        free(ys);
    }
    uint16_t* r = bf16s(M * N);
    double* o = malloc((size_t)(M * N) * sizeof *o);
    oracle_residual(M * N, r, y, o);
    uint16_t* enc = malloc((size_t)(M * N) * sizeof *enc);
    oracle_encode_bf16(M * N, o, enc);
    free(x), free(W), free(y), free(a), free(r), free(o), free(enc);
}

static void moe(int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K) {
    int32_t* ids = malloc((size_t)(T * topk) * sizeof *ids);
    for (int64_t i = 0; i < T * topk; ++i) ids[i] = (int32_t)(next() % (E + 2)) - 1;  /* some invalid */
    int32_t* counts = malloc((size_t)E * sizeof *counts);
    int32_t* offsets = malloc((size_t)(E + 1) * sizeof *offsets);
    int32_t* pairs = malloc((size_t)(T * topk) * sizeof *pairs);
    const int64_t invalid = oracle_moe_table(T, topk, E, ids, counts, offsets, pairs);
    EXPECT(offsets[0] == 0 && offsets[E] + invalid == T * topk);
    uint16_t* x = bf16s(T * K);
    uint16_t* W = bf16s(E * N * K);
    double* out = malloc((size_t)(T * topk * N) * sizeof *out);
    double* a = malloc((size_t)(T * topk * N) * sizeof *a);
    oracle_grouped(T, topk, E, N, K, x, W, ids, out, a);
    oracle_grouped(T, topk, E, N, K, x, W, ids, out, NULL);
    free(ids), free(counts), free(offsets), free(pairs), free(x), free(W), free(out), free(a);
}

static void router(int64_t T, int64_t E, int64_t k) {
    float* s = malloc((size_t)(T * E) * sizeof *s);
    for (int64_t i = 0; i < T * E; ++i) s[i] = (float)(next() % 7) - 3.0f;  /* many ties */
    s[0] = NAN;
    int32_t* ids = malloc((size_t)(T * k) * sizeof *ids);
    float* top = malloc((size_t)(T * k) * sizeof *top);
    oracle_router_topk(T, E, k, s, ids, top);
    oracle_router_topk(T, E, k, s, ids, NULL);
    for (int64_t i = 0; i < T * k; ++i) EXPECT(ids[i] >= 0 && ids[i] < E);
    free(s), free(ids), free(top);
}

static void lowp(int64_t M, int64_t N, int64_t K) {
    uint16_t* x = bf16s(M * K);
    double* y = malloc((size_t)(M * N) * sizeof *y);
    double* a = malloc((size_t)(M * N) * sizeof *a);
    if (K % 32 == 0) {
        uint8_t* q = bytes(N * K / 2, 0, 255);
        uint8_t* sc = bytes(N * K / 32, 0, 255);
        oracle_projection_mxfp4(M, N, K, x, q, sc, y, a);
        oracle_projection_mxfp4(M, N, K, x, q, sc, y, NULL);
        free(q), free(sc);
    }
    if (K % 16 == 0) {
        const int64_t nb = (N + 127) / 128, kb = (K + 127) / 128;
        uint8_t* q = bytes(N * K, 0, 255);
        float* sc = malloc((size_t)(nb * kb) * sizeof *sc);
        for (int64_t i = 0; i < nb * kb; ++i) sc[i] = 1e-3f * (float)(1 + next() % 100);
        oracle_projection_fp8(M, N, K, x, q, sc, y, a);
        oracle_projection_fp8(M, N, K, x, q, sc, y, NULL);
        free(q), free(sc);
    }
    for (int c = 0; c < 256; ++c) {
        (void)oracle_e4m3_to_f64((uint8_t)c);
        (void)oracle_e8m0_to_f64((uint8_t)c);
        if (c < 16) (void)oracle_e2m1_to_f64((uint8_t)c);
    }
    free(x), free(y), free(a);
}

int main(void) {
    for (int b = 0; b < 65536; ++b) (void)oracle_bf16_to_f64((uint16_t)b);
    projection_and_splits(1, 1, 8);
    projection_and_splits(3, 5, 40);
    projection_and_splits(2, 7, 200);
    projection_and_splits(5, 3, 8);     /* most splits empty */
    moe(3, 4, 7, 5, 24);
    moe(1, 8, 16, 3, 8);
    router(3, 9, 4);
    router(2, 40, 40);
    lowp(3, 130, 160);
    lowp(1, 5, 32);
    lowp(2, 129, 144);
    if (failures) fprintf(stderr, "oracle_checks: %d failures\n", failures);
    else printf("oracle_checks: ok\n");
    return failures ? 1 : 0;
}
