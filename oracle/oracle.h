/*
 * oracle.h -- plain, slow CPU reference for the skinny decode projection.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load this library.
 * It shares no code, header, table or helper with the HIP library, and
 * neither side includes or links the other.
 *
 * What it computes follows the method pages:
 *   - "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly"
 *     (deepnotes summary page), Method details §1 "Tune shapes for the
 *     workload": decode-time input projections, a small-matrix kernel at
 *     batch 1-2 and a split-K kernel (accumulation dimension split over more
 *     workers) at larger batch;
 *   - same page, Method details §2: the output projection fused with the
 *     attention residual add;
 *   - same page, Method details §3, and the French translation ("Hyper
 *     optimisation de Kimi K3 dans vLLM"), Partie 2 §4: routed experts, where
 *     expert selection decides which weights are read.
 * The pages give the operation, not its arithmetic; every reading taken where
 * they are silent is stated at the function it governs.
 *
 * Conventions
 *   bf16 values travel as raw 16-bit patterns (uint16_t), the upper half of
 *   an IEEE-754 binary32.  All arithmetic is IEEE double, summed in the
 *   order each comment states.  Matrices are dense and row-major:
 *   x [M,K], W [N,K] (the nn.Linear weight layout), y [M,N], so y = x W^T.
 *
 * Parity pins: every function here is pinned by CPU tests against
 * something other than itself (exact rational brute force, closed forms,
 * library routines, invariants).  The oracle has no function whose parity is
 * unpinned.
 */
#ifndef SKINNY_GEMM_ORACLE_H
#define SKINNY_GEMM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact value of a bf16 bit pattern (sign, 8-bit exponent, 7-bit fraction). */
double oracle_bf16_to_f64(uint16_t bits);

/* Round a double to the nearest bf16, ties to even; overflow gives +-inf,
 * NaN gives a quiet NaN with the input's sign. */
uint16_t oracle_f64_to_bf16(double v);

/* Element-wise oracle_f64_to_bf16 over n values. */
void oracle_encode_bf16(int64_t n, const double* v, uint16_t* out);

/* Projection y[m,n] = sum_k x[m,k] * W[n,k], k ascending, in double.
 * abs_scale[m,n] = sum_k |x[m,k] * W[n,k]| (the tolerance scale); may be NULL. */
void oracle_projection(int64_t M, int64_t N, int64_t K,
                       const uint16_t* x, const uint16_t* W,
                       double* y, double* abs_scale);

/* Split-K partial sums.  Chunk s covers k in [s*c, min(K, (s+1)*c)) with
 * c = 64*ceil(K/(64*S)) (ceil(K/S) rounded up to a multiple of 64, whole
 * 128-byte lines of bf16);
 * P[s,m,n] = sum over that chunk, k ascending.  A chunk that starts at or
 * past K is empty and holds 0. */
void oracle_splitk_partials(int64_t M, int64_t N, int64_t K, int64_t S,
                            const uint16_t* x, const uint16_t* W, double* P);

/* y[i] = P[0,i] + P[1,i] + ... + P[S-1,i], s ascending, over MN elements. */
void oracle_splitk_sum(int64_t S, int64_t MN, const double* P, double* y);

/* Residual add out[i] = r[i] + y[i] (r a bf16 pattern), in double. */
void oracle_residual(int64_t MN, const uint16_t* r, const double* y, double* out);

/* Per-expert token table for topk_ids [T, topk] over E experts.
 * Pair p = t*topk + j routes token t's j-th choice to expert ids[p].
 * counts[e]       = number of pairs with ids[p] == e                [E]
 * offsets[e]      = counts[0] + ... + counts[e-1], offsets[0] = 0   [E+1]
 * sorted_pairs    = the valid pairs grouped by expert, ascending e, and
 *                   ascending p inside each expert's segment; slots from
 *                   offsets[E] to T*topk-1 hold -1                  [T*topk]
 * Returns the number of pairs whose id lies outside [0, E). */
int64_t oracle_moe_table(int64_t T, int64_t topk, int64_t E, const int32_t* ids,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_pairs);

/* Grouped projection over routed experts: W is [E, N, K].
 * out[t,j,n] = sum_k x[t,k] * W[ids[t*topk+j], n, k] for a valid id, and 0
 * for an id outside [0, E).  abs_scale likewise (may be NULL). */
void oracle_grouped(int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K,
                    const uint16_t* x, const uint16_t* W, const int32_t* ids,
                    double* out, double* abs_scale);

/* Router top-k (routed experts: "Hyper Optimizing Kimi K3 in vLLM", Method
 * details §3 -- expert selection from the router scores decides which expert
 * weights are read).  scores [T,E] fp32 (the router projection's output);
 * for each token t, ids[t,j] (j < k <= E) is the expert of rank j: larger
 * score first, equal scores by the lower expert id, a NaN score ranking as
 * -infinity.  top_scores[t,j] = scores[t, ids[t,j]] (may be NULL).  The
 * ranking is decided on the fp32 values as given. */
void oracle_router_topk(int64_t T, int64_t E, int64_t k, const float* scores,
                        int32_t* ids, float* top_scores);

/* Block-scaled 4-bit weights.  The pages' later evaluation model ships
 * NVFP4 weights ("Hyper Optimizing Kimi K3 in vLLM", Experimental setup and
 * Supplementary details: a 4-bit float element format with per-block
 * scales).  The block-scaled 4-bit format MI355X handles natively is OCP
 * MXFP4: e2m1 elements, blocks of 32 consecutive elements along K, one e8m0
 * power-of-two scale per block.  That is the format read here.
 *
 * e2m1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.  Exponent 0
 * is subnormal (0 or 0.5); otherwise 2^(e-1) * (1 + m/2).  No Inf or NaN;
 * the largest magnitude is 6. */
double oracle_e2m1_to_f64(uint8_t code);

/* e8m0 scale: 2^(s - 127) for s in 0..254; s == 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t s);

/* Projection with MXFP4 weights (K a multiple of 32):
 *   Wq [N, K/2] bytes: element k of row n sits in byte n*K/2 + k/2, in the
 *                      low nibble for even k and the high nibble for odd k;
 *   Ws [N, K/32] e8m0 scales: block b of row n covers k in [32b, 32b+32).
 *   w[n,k] = e2m1(code[n,k]) * e8m0(Ws[n, k/32])
 *   y[m,n] = sum_k x[m,k] * w[n,k], k ascending, in double; abs_scale the
 *   sum of |x[m,k] * w[n,k]| (may be NULL). */
void oracle_projection_mxfp4(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                             const uint8_t* Wq, const uint8_t* Ws, double* y,
                             double* abs_scale);

/* FP8 weights with block scales (the block-scaled 8-bit weight format of
 * DeepSeek-V3-style checkpoints; a reading: the method pages name only a
 * 4-bit format for a later model).
 * e4m3: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
 * exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN;
 * no infinity.  The largest finite magnitude is 448. */
double oracle_e4m3_to_f64(uint8_t code);

/* y = x W^T for FP8 weights:
 *   Wq [N, K] e4m3 codes, one byte each, row-major;
 *   Ws [ceil(N/128), ceil(K/128)] fp32 scales, row-major: block (i, j)
 *      covers rows [128i, 128i+128) and k in [128j, 128j+128);
 *   w[n,k] = e4m3(Wq[n,k]) * Ws[n/128, k/128], then the plain sum, k
 *   ascending.  abs_scale (nullable) receives sum_k |x w|. */
void oracle_projection_fp8(int64_t M, int64_t N, int64_t K, const uint16_t* x,
                           const uint8_t* Wq, const float* Ws, double* y, double* abs_scale);

#ifdef __cplusplus
}
#endif

#endif
