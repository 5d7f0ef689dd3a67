/*
 * oracle.c -- plain, slow CPU reference for the skinny decode projection.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it.  It shares no
 * code with the HIP library.  Declarations and the page citations are in
 * oracle.h; each definition below restates the reading it follows.
 *
 * Deliberately naive: one loop nest per definition, double accumulation,
 * no blocking, no threads, no reordering.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_f64(uint16_t bits)
{
    /* bfloat16 is the upper 16 bits of an IEEE-754 binary32: widen by
     * appending 16 zero fraction bits, then read the binary32 exactly. */
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

uint16_t oracle_f64_to_bf16(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000u : 0x0000u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);

    /* a lies in [2^E, 2^(E+1)).  bf16 keeps 8 significant bits, so the
     * spacing of representable values there is 2^(E-7); below the smallest
     * normal 2^-126 the spacing is fixed at 2^-133 (subnormals). */
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2 with f in [0.5, 1), so E = e2 - 1 */
    int E = e2 - 1;
    int spacing_exp = (E < -126) ? -133 : E - 7;
    double q = ldexp(1.0, spacing_exp);

    /* a / q is exact (power-of-two scale).  Round it to an integer, ties
     * to even. */
    double n = a / q;
    double lo = floor(n);
    double frac = n - lo;
    double r = lo;
    if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0))
        r = lo + 1.0;
    double rounded = r * q; /* exact: r <= 256 */

    /* Largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounded
     * beyond it overflows to infinity. */
    if (rounded > ldexp(2.0 - ldexp(1.0, -7), 127))
        return (uint16_t)(sign | 0x7F80u);

    float f = (float)rounded; /* exact: a bf16 value is a binary32 value */
    uint32_t word;
    memcpy(&word, &f, sizeof word);
    return (uint16_t)(sign | (word >> 16));
}

void oracle_encode_bf16(int64_t n, const double* v, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(v[i]);
}

void oracle_projection(int64_t M, int64_t N, int64_t K,
                       const uint16_t* x, const uint16_t* W,
                       double* y, double* abs_scale)
{
    /* y = x W^T with W stored [N, K]: output (m, n) is the dot product of
     * row m of x with row n of W, summed over k in ascending order. */
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            double abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double term = oracle_bf16_to_f64(x[m * K + k]) *
                              oracle_bf16_to_f64(W[n * K + k]);
                sum += term;
                abs_sum += fabs(term);
            }
            y[m * N + n] = sum;
            if (abs_scale)
                abs_scale[m * N + n] = abs_sum;
        }
    }
}

void oracle_splitk_partials(int64_t M, int64_t N, int64_t K, int64_t S,
                            const uint16_t* x, const uint16_t* W, double* P)
{
    /* The accumulation dimension is cut into S contiguous chunks of
     * c = 64 * ceil(K / (64*S)) elements -- ceil(K/S) rounded up to whole
     * groups of 64 (128-byte cache lines of bf16) -- the last one shorter,
     * or empty.  Each chunk is an ordinary projection over its k range. */
    int64_t chunk = 64 * ((K + 64 * S - 1) / (64 * S));
    for (int64_t s = 0; s < S; ++s) {
        int64_t k_begin = s * chunk;
        int64_t k_end = (s + 1) * chunk < K ? (s + 1) * chunk : K;
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t n = 0; n < N; ++n) {
                double sum = 0.0;
                for (int64_t k = k_begin; k < k_end; ++k)
                    sum += oracle_bf16_to_f64(x[m * K + k]) *
                           oracle_bf16_to_f64(W[n * K + k]);
                P[(s * M + m) * N + n] = sum;
            }
        }
    }
}

void oracle_splitk_sum(int64_t S, int64_t MN, const double* P, double* y)
{
    for (int64_t i = 0; i < MN; ++i) {
        double sum = 0.0;
        for (int64_t s = 0; s < S; ++s)
            sum += P[s * MN + i];
        y[i] = sum;
    }
}

void oracle_residual(int64_t MN, const uint16_t* r, const double* y, double* out)
{
    for (int64_t i = 0; i < MN; ++i)
        out[i] = oracle_bf16_to_f64(r[i]) + y[i];
}

int64_t oracle_moe_table(int64_t T, int64_t topk, int64_t E, const int32_t* ids,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_pairs)
{
    int64_t pairs = T * topk;
    int64_t invalid = 0;

    for (int64_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t p = 0; p < pairs; ++p) {
        int32_t e = ids[p];
        if (e < 0 || e >= E)
            ++invalid;
        else
            ++counts[e];
    }

    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];

    /* Expert by expert in ascending order, list that expert's pairs in
     * ascending p starting at its offset; unused tail slots stay -1. */
    for (int64_t p = 0; p < pairs; ++p)
        sorted_pairs[p] = -1;
    for (int64_t e = 0; e < E; ++e) {
        int32_t slot = offsets[e];
        for (int64_t p = 0; p < pairs; ++p) {
            if (ids[p] == e)
                sorted_pairs[slot++] = (int32_t)p;
        }
    }
    return invalid;
}

void oracle_grouped(int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K,
                    const uint16_t* x, const uint16_t* W, const int32_t* ids,
                    double* out, double* abs_scale)
{
    /* Each (token, choice) pair is a one-row projection against its chosen
     * expert's weight; a pair with an out-of-range id yields zeros. */
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < topk; ++j) {
            int64_t p = t * topk + j;
            int32_t e = ids[p];
            double* o = out + p * N;
            double* a = abs_scale ? abs_scale + p * N : 0;
            if (e < 0 || e >= E) {
                for (int64_t n = 0; n < N; ++n) {
                    o[n] = 0.0;
                    if (a)
                        a[n] = 0.0;
                }
                continue;
            }
            oracle_projection(1, N, K, x + t * K, W + (int64_t)e * N * K, o, a);
        }
    }
}

/* Router top-k: true when (a, ia) ranks before (b, ib) -- the larger score
 * first, equal scores by the lower expert id, a NaN score as -infinity. */
static int oracle_ranks_before(float a, int64_t ia, float b, int64_t ib)
{
    double da = isnan(a) ? -INFINITY : (double)a;
    double db = isnan(b) ? -INFINITY : (double)b;
    if (da != db)
        return da > db;
    return ia < ib;
}

void oracle_router_topk(int64_t T, int64_t E, int64_t k, const float* scores,
                        int32_t* ids, float* top_scores)
{
    /* Expert selection by router score (routed experts, Method details §3):
     * for each token, k times, the best expert not taken yet.  The ranking
     * is decided on the given fp32 scores. */
    unsigned char* taken = (unsigned char*)malloc(E > 0 ? (size_t)E : 1);
    for (int64_t t = 0; t < T; ++t) {
        const float* s = scores + t * E;
        memset(taken, 0, E > 0 ? (size_t)E : 1);
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || oracle_ranks_before(s[e], e, s[best], best))
                    best = e;
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
            if (top_scores)
                top_scores[t * k + j] = s[best];
        }
    }
    free(taken);
}

double oracle_e2m1_to_f64(uint8_t code)
{
    /* 4-bit float: sign bit 3, 2-bit exponent (bias 1), 1-bit mantissa. */
    const int sign = (code >> 3) & 1;
    const int e = (code >> 1) & 3;
    const int m = code & 1;
    double mag;
    if (e == 0)
        mag = m * 0.5;                             /* subnormal: 0 or 0.5 */
    else
        mag = ldexp(1.0 + m * 0.5, e - 1);         /* 1, 1.5, 2, 3, 4, 6 */
    return sign ? -mag : mag;
}

double oracle_e8m0_to_f64(uint8_t s)
{
    /* unsigned 8-bit exponent, no sign or mantissa; all ones is NaN */
    if (s == 255)
        return NAN;
    return ldexp(1.0, (int)s - 127);
}

void oracle_projection_mxfp4(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                             const uint8_t* Wq, const uint8_t* Ws, double* y,
                             double* abs_scale)
{
    /* Decode each weight from its nibble and its block's scale, then the
     * plain projection sum, k ascending. */
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint8_t byte = Wq[n * (K / 2) + k / 2];
                const uint8_t code = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
                const double w = oracle_e2m1_to_f64(code) * oracle_e8m0_to_f64(Ws[n * (K / 32) + k / 32]);
                const double term = oracle_bf16_to_f64(x[m * K + k]) * w;
                sum += term;
                abs_sum += fabs(term);
            }
            y[m * N + n] = sum;
            if (abs_scale)
                abs_scale[m * N + n] = abs_sum;
        }
    }
}

double oracle_e4m3_to_f64(uint8_t code)
{
    /* OCP 8-bit float E4M3 (the "fn" variant: finite, no infinity): bit 7
     * sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.  Exponent 0 is
     * subnormal, m/8 * 2^-6; exponent 15 with mantissa 7 is NaN (either
     * sign); every other code is the normal value 2^(e-7) * (1 + m/8). */
    const int sign = (code >> 7) & 1;
    const int e = (code >> 3) & 15;
    const int m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    const double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

void oracle_projection_fp8(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                           const uint8_t* Wq, const float* Ws, double* y, double* abs_scale)
{
    /* Each weight is its e4m3 code times the fp32 scale of its 128 x 128
     * block, then the plain projection sum, k ascending. */
    const int64_t KB = (K + 127) / 128;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double w = oracle_e4m3_to_f64(Wq[n * K + k]) * (double)Ws[(n / 128) * KB + k / 128];
                const double term = oracle_bf16_to_f64(x[m * K + k]) * w;
                sum += term;
                abs_sum += fabs(term);
            }
            y[m * N + n] = sum;
            if (abs_scale)
                abs_scale[m * N + n] = abs_sum;
        }
    }
}
