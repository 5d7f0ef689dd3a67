/*
 * skinny_gemm.h -- C ABI of libskinny_gemm.so: the batch-1..64 decode linear
 * projection y = x W^T (+ fused residual add) and its routed-expert (MoE)
 * variant, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (method pages):
 *   [P] "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly"
 *       (deepnotes summary page), Method details:
 *       §1 "Tune shapes for the workload" -- decode input projections use a
 *          dedicated small-matrix kernel at batch 1-2 and a split-K kernel
 *          (the accumulation dimension spread over more compute units) at
 *          larger batch; every projection is tuned to a kernel size that
 *          fills the GPU;
 *       §2 "Overlap computation and communication" -- the output projection
 *          is fused with the attention residual add;
 *       §3 "Improve MoE scheduling and overlap" -- routed experts;
 *       §4 "Prefetching upcoming weights into cache" -- a side-stream kernel
 *          warms the next weights while memory bandwidth is idle.
 *   [F] "Hyper optimisation de Kimi K3 dans vLLM : aller vite et
 *       responsablement" (French translation of the same post): Partie 1
 *       §1-§4 (same four techniques); Partie 2 §1 (the selected path and the
 *       way back to the standard path must be observable); Partie 2 §3 (an
 *       early load may only read static weights); Partie 2 §4 (expert
 *       selection decides which weights are read).
 *   [D] "Qu'est-ce qui va suivre" on [F] and "Supplementary details" on [P]:
 *       prefill and mixed batches fall back transparently to the standard
 *       path; the specialised decode path covers up to 64 concurrent requests.
 *
 * Conventions shared by every call
 *   - sg_bf16 is a raw bfloat16 bit pattern.  All matrices are dense,
 *     row-major, contiguous, in device memory:
 *       x [M, K], W [N, K] (the nn.Linear weight layout), y/out/r [M, N].
 *     y[m, n] = sum_k x[m, k] * W[n, k], accumulated in fp32.
 *   - Every device pointer must be 16-byte aligned and K a multiple of 8
 *     (rows are read with 16-byte loads); otherwise SG_ERR_ALIGN.
 *   - Ownership: the caller allocates and owns every buffer, including the
 *     workspace.  The library allocates no device memory, holds no
 *     per-call state beyond atomic launch counters, never synchronises the
 *     device, and is safe to call from several host threads.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     null stream) and may be captured into a HIP graph.
 *   - Errors: every problem the host can see is reported before anything is
 *     launched; a launch failure returns SG_ERR_HIP.  No C++ exception
 *     crosses this interface.  Data errors found on the device (an expert id
 *     outside [0, E)) never trap: they are counted and their outputs zeroed.
 */
#ifndef SKINNY_GEMM_H
#define SKINNY_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t sg_bf16;

typedef enum {
    SG_OK = 0,
    SG_ERR_NULL = 1,        /* a required pointer is NULL                         */
    SG_ERR_SHAPE = 2,       /* a negative or over-limit size                      */
    SG_ERR_UNSUPPORTED = 3, /* outside the decode path (M > 64): caller falls back */
    SG_ERR_ALIGN = 4,       /* K % 8 != 0 or a pointer not 16-byte aligned       */
    SG_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required         */
    SG_ERR_PLAN = 6,        /* plan does not describe this problem, or bad choice */
    SG_ERR_HIP = 7          /* the HIP runtime refused a launch                   */
} sg_status;

/* Kernel identifiers; also the indices of the launch counters. */
typedef enum {
    SG_KERNEL_NONE = 0,         /* empty problem (M == 0 or N == 0): nothing runs  */
    SG_KERNEL_GEMV = 1,         /* small-matrix kernel, M <= 2                     */
    SG_KERNEL_SPLITK_VALU = 2,  /* split-K partial, vector-ALU dot, 3 <= M <= 7    */
    SG_KERNEL_SPLITK_MFMA = 3,  /* split-K partial, bf16 matrix cores, M >= 6 or 8 */
    SG_KERNEL_REDUCE = 4,       /* split-K deterministic reduction + epilogue      */
    SG_KERNEL_MOE_TABLE = 5,    /* per-expert token table                          */
    SG_KERNEL_GROUPED = 6,      /* grouped per-expert projection                   */
    SG_KERNEL_PREFETCH = 7,     /* side-stream weight prefetch                     */
    SG_KERNEL_ROUTER_TOPK = 8,  /* router top-k expert selection                   */
    SG_KERNEL_MXFP4 = 9,        /* projection with block-scaled 4-bit weights      */
    SG_KERNEL_FP8 = 10          /* projection with block-scaled 8-bit weights      */
} sg_kernel;

#define SG_NUM_COUNTERS 11
#define SG_MAX_M 64

/* Launch decision for one projection shape.  Produced by skinny_gemm_plan
 * (or skinny_gemm_plan_force) and passed unchanged to skinny_gemm /
 * skinny_gemm_residual. */
typedef struct {
    int32_t M, N, K;
    int32_t kernel;   /* sg_kernel of the main (first) launch                  */
    int32_t split_k;  /* S: number of K chunks; 1 = no split, no reduction     */
    int32_t k_chunk;  /* elements per K chunk: ceil(K/S) rounded up to a
                         multiple of 64 (whole 128-byte lines); chunk s
                         covers [s*k_chunk, min(K, (s+1)*k_chunk))          */
    int32_t tile_n;   /* rows of W per work item: small-matrix / VALU kernels,
                         rows per wave iteration; matrix cores: 16 for the
                         in-workgroup (team) kernel, 128 or 256 for the
                         chunk kernel (16 or 32 rows per wave)              */
    int32_t grid;     /* workgroups of the main launch                          */
    int32_t two_pass; /* 1: the S partials go through the workspace to a second,
                         reduction kernel; 0: they are added inside the main
                         kernel (S waves of one workgroup), or S == 1        */
    size_t workspace_bytes; /* device workspace the call needs (0 if none)      */
} sg_plan;

/* plan(M, N, K) -- pick the kernel and its tiling for y[M,N] = x[M,K] W[N,K]^T
 * ([P] Method details §1).  0 <= M <= 64: M <= 2 small-matrix kernel; larger
 * M split-K, on the vector ALU below 8 rows and on bf16 matrix cores from 8
 * rows -- from 6 rows where N/16 workgroups fill the GPU (measured
 * crossovers on MI355X); the split factor and row tiling come
 * from a per-compute-unit byte cost model, overridable by a tuned table.  M > 64 returns
 * SG_ERR_UNSUPPORTED (prefill-sized batches fall back, [D]); M == 0 or
 * N == 0 gives kernel SG_KERNEL_NONE.  Host-only: touches no GPU state.
 * Limits: 0 <= N <= 1<<20, 0 <= K <= 1<<20 (else SG_ERR_SHAPE).
 * The environment variable SKINNY_GEMM_TUNE_TABLE may name a text file of
 * entries checked before the built-in tuned table, read once per process:
 * one entry a line, "M_lo M_hi N K kernel split tile_n" (integers; 0 leaves
 * that choice to the planner; kernel an sg_kernel value up to
 * SG_KERNEL_SPLITK_MFMA; tile_n 0, 16, 128 or 256), '#' starts a comment.
 * A line that does not parse rejects the whole file (one warning on
 * stderr); an entry the planner cannot honour for a shape yields the
 * default plan. */
sg_status skinny_gemm_plan(int32_t M, int32_t N, int32_t K, sg_plan* out);

/* Same, but with the kernel, split factor, reduction mode and (matrix cores)
 * row tiling chosen by the caller (sweeps and tests).  kernel <= 0,
 * split_k <= 0 and tile_n <= 0 let the library choose; two_pass: 0 reduce
 * inside the main kernel, 1 second-pass reduction through the workspace,
 * < 0 let the library choose; tile_n (matrix cores only): 16 the team
 * kernel, 128 or 256 the chunk kernel.  SG_ERR_PLAN when the kernel cannot
 * run this shape (GEMV with M > 2, VALU split-K with M > 15 or with a chunk
 * whose x rows do not fit its registers, a chunk kernel whose x chunk does
 * not fit in LDS), when the split cannot be reduced in the requested mode,
 * or split_k > 64.  A forced split may leave trailing chunks empty; their
 * partials are 0. */
sg_status skinny_gemm_plan_force(int32_t M, int32_t N, int32_t K, int32_t kernel,
                                 int32_t split_k, int32_t two_pass, int32_t tile_n,
                                 sg_plan* out);

/* y = x W^T ([P] Method details §1).  Writes y_f32 [M,N] (fp32) and/or
 * y_bf16 [M,N] (the same fp32 value rounded to nearest even); at least one
 * must be non-NULL.  workspace: at least plan->workspace_bytes bytes, may be
 * NULL when that is 0; in two-pass plans the fp32 split-K partial sums
 * occupy its first bytes: P[S,M,N] for the vector-ALU kernel, P[S,N,Mp]
 * (Mp = 16*ceil(M/16), rows m >= M zero) for the matrix-core chunk kernel
 * (tile_n 128 or 256).  Split partials are always added
 * in ascending split order in fp32, without atomics: repeated calls give
 * identical bits.  Output buffers must not overlap the inputs. */
sg_status skinny_gemm(const sg_plan* plan, const sg_bf16* x, const sg_bf16* W,
                      float* y_f32, sg_bf16* y_bf16,
                      void* workspace, size_t workspace_bytes, void* stream);

/* skinny_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture that must not call hipMalloc, tight serving loops, harnesses
 * that forbid allocation).  Same plan, inputs, outputs, kernels and results
 * as skinny_gemm; the split-K partials of two-pass plans go to a scratch
 * array of SG_NOALLOC_MAX_WORKSPACE bytes inside the library, one per GPU,
 * held from the first call on that GPU until the process ends (the first call
 * on a device looks up its address there: the current device must be the
 * one the stream and buffers belong to).  A plan whose workspace_bytes
 * exceeds SG_NOALLOC_MAX_WORKSPACE returns SG_ERR_WORKSPACE (no launch).  The
 * call allocates nothing.  All calls on one GPU share its scratch array:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race on it and must be serialised by the caller. */
#define SG_NOALLOC_MAX_WORKSPACE ((size_t)16 << 20)
sg_status skinny_gemm_noalloc(const sg_plan* plan, const sg_bf16* x, const sg_bf16* W,
                              float* y_f32, sg_bf16* y_bf16, void* stream);

/* Fused residual epilogue ([P] Method details §2): out = r + x W^T, with the
 * fp32 accumulator added to r in fp32 and rounded once.  out_bf16 [M,N]
 * and/or out_f32 [M,N]; out_bf16 may be the same pointer as r (in place;
 * any other overlap is undefined).  Workspace as for skinny_gemm. */
sg_status skinny_gemm_residual(const sg_plan* plan, const sg_bf16* x, const sg_bf16* W,
                               const sg_bf16* r, sg_bf16* out_bf16, float* out_f32,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes grouped_skinny_gemm needs for this problem size. */
size_t grouped_skinny_gemm_workspace(int32_t T, int32_t E, int32_t topk, int32_t N, int32_t K);

/* Routed-expert projection for MoE decode ([P] Method details §3, [F]
 * Partie 2 §4).  x [T,K] bf16, W [E,N,K] bf16 (expert e at W + e*N*K),
 * topk_ids [T,topk] int32.  Pair p = t*topk + j sends token t to expert
 * ids[p]; out [T,topk,N] fp32 gets out[t,j,n] = sum_k x[t,k] W[ids[p],n,k].
 * Each selected expert's weights are read once per call however many tokens
 * chose it.  Optional outputs (NULL to skip), computed on the device:
 *   expert_offsets [E+1]: offsets[e] = number of valid pairs routed to
 *                         experts below e;
 *   sorted_pairs [T*topk]: valid pairs grouped by expert in ascending id,
 *                         ascending p inside a group, -1 after the last;
 *   invalid_count [1]:    pairs whose id is outside [0, E) -- their
 *                         out rows are zero-filled.
 * With all three NULL and T*topk <= 512 the call is one launch that builds
 * the table it needs in each workgroup (no table kernel; the workspace is
 * not touched); otherwise a table kernel runs first.  Both give the same
 * output bits.
 * Limits: 0 <= T <= 256, 1 <= topk <= 32, T*topk <= 4096, 1 <= E <= 4096,
 * 0 <= N <= 1<<20, 0 <= K <= 8192 (else SG_ERR_SHAPE). */
sg_status grouped_skinny_gemm(const sg_bf16* x, int32_t T, const sg_bf16* W, int32_t E,
                              int32_t N, int32_t K, const int32_t* topk_ids, int32_t topk,
                              float* out, int32_t* expert_offsets, int32_t* sorted_pairs,
                              int32_t* invalid_count,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Router top-k: the experts each token is routed to ([P] Method details §3:
 * expert selection decides which expert weights are read; the selection is
 * the step upstream of grouped_skinny_gemm).  scores [T,E] fp32 -- the
 * router projection, e.g. skinny_gemm with N = E -- in device memory;
 * topk_ids [T,k] int32 receives, for each token, the experts of rank
 * 0..k-1: the larger score first, equal scores by the lower expert id, a
 * NaN score ranking as -infinity (a total order: the ids of a token are
 * distinct).  topk_scores [T,k] fp32 (NULL to skip) receives the selected
 * scores as given.  Limits: 0 <= T <= 1<<20, 1 <= E <= 4096,
 * 1 <= k <= min(E, 32) (else SG_ERR_SHAPE); pointers 4-byte aligned. */
sg_status skinny_gemm_router_topk(const float* scores, int32_t T, int32_t E, int32_t k,
                                  int32_t* topk_ids, float* topk_scores, void* stream);

/* y = x W^T with block-scaled 4-bit weights.  The pages' later evaluation
 * model ships NVFP4 weights ([P] Experimental setup and Supplementary
 * details: 4-bit floats with per-block scales); the block-scaled 4-bit
 * format MI355X converts in hardware is OCP MXFP4, read here:
 *   W_codes  [N, K/2] bytes: e2m1 codes (bit 3 sign, bits 2..1 exponent with
 *            bias 1, bit 0 mantissa: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 *            negatives); element k of row n is in byte n*K/2 + k/2, low
 *            nibble for even k;
 *   W_scales [N, K/32] bytes: e8m0 scale of elements [32b, 32b+32) of row
 *            n, 2^(s-127); s == 255 is NaN (the row's outputs become NaN).
 *   W[n,k] = e2m1 * 2^(s-127);  y[m,n] = sum_k x[m,k] W[n,k] in fp32
 *   (the codes are converted at unit scale and each block's fp32 sum is
 *   multiplied by its scale, so every scale code 0..254 is exact down to
 *   fp32's subnormals, including weights outside bf16's range), then the
 *   epilogue of skinny_gemm_residual when r is given (out = bf16_RNE(fp32(r)
 *   + y), r may alias y_bf16) or of skinny_gemm otherwise.  The weight stream
 *   is a quarter of bf16's plus 1/16 for the scales.  M <= 8 runs on the
 *   vector ALU and 9 <= M <= 16 on bf16 matrix cores (one launch, the
 *   workspace is not used) where its grid of 16-row tiles (32-row from N =
 *   8161) is a whole multiple of 256 workgroups, and for 9 <= M <= 11 also
 *   where N > 5888; elsewhere from 9 rows, and for 17 <= M <= 64, the
 *   matrix-core chunk kernel runs (up to 16 rows only while its x chunk fits
 *   in LDS; a longer K takes the one-launch kernel) (x staged once per
 *   128 or 256 weight rows, K split between workgroups) and, when it splits
 *   K, the deterministic reduction: the fp32 partials need
 *   skinny_gemm_mxfp4_workspace(M, N, K) bytes of workspace (16-byte
 *   aligned; NULL when that is 0), summed in ascending split order.
 * Batch 1 to 64 is the decode path of [P] Method details.
 * Limits: 0 <= M <= 64 (M > 64: SG_ERR_UNSUPPORTED), 0 <= N <= 1<<20,
 * 0 <= K <= 1<<20 (else SG_ERR_SHAPE), K % 32 == 0 (SG_ERR_ALIGN); K <=
 * 32768 at M <= 2 and 16384 for 3 <= M <= 8, and from 17 rows a
 * split whose x chunk fits in LDS (any K up to 65536) (else
 * SG_ERR_UNSUPPORTED); a short
 * workspace: SG_ERR_WORKSPACE.  x, W_codes, r, outputs and the workspace
 * 16-byte aligned; W_scales any alignment. */
sg_status skinny_gemm_mxfp4(int32_t M, int32_t N, int32_t K, const sg_bf16* x,
                            const uint8_t* W_codes, const uint8_t* W_scales, const sg_bf16* r,
                            float* y_f32, sg_bf16* y_bf16, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Projection with FP8 weights and block scales (low-precision weights: [P]
 * Experimental setup and Supplementary details, the later evaluation model
 * ships 4-bit weights; the 8-bit format read here is the block-scaled FP8 of
 * DeepSeek-V3-style checkpoints).  W_codes [N, K] bytes, OCP E4M3 codes
 * (bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa; exponent
 * 0 subnormal; 0x7F and 0xFF are NaN; no infinity), row-major.  W_scales
 * [ceil(N/128), ceil(K/128)] fp32, row-major: w[n,k] = e4m3(code[n,k]) *
 * W_scales[n/128][k/128].  x [M, K] bf16; fp32 sums; y_f32 and/or y_bf16
 * [M, N] (at least one); r (nullable) bf16 [M, N] gives the fused residual
 * y = r + x W^T as for skinny_gemm_residual (y_bf16 may equal r).  A NaN
 * code or scale makes its outputs NaN.  M <= 4 runs on the vector ALU,
 * 5 <= M <= 7 on bf16 matrix cores (codes converted exactly to bf16, each
 * 128-column window's sum scaled once; one launch, no workspace), also 8 <=
 * M <= 11 where N/32 is a whole multiple of 256 (N = 8192); otherwise from 8
 * rows the matrix-core chunk kernel with the workspace and reduction of
 * skinny_gemm_mxfp4 (skinny_gemm_fp8_workspace bytes), up to 16 rows only
 * while its x chunk fits in LDS (a longer K takes the one-launch kernel).
 * Limits: 0 <= M <= 64, K % 16 == 0 (else SG_ERR_ALIGN), M * K <= 32768 at
 * M <= 2 (x staged in LDS) and K <= 16384 at M = 3, 4 (x in registers), any
 * K for 5 <= M <= 16, and from 17 rows a split whose x chunk fits in LDS
 * (any K up to 65536)
 * (else SG_ERR_UNSUPPORTED), N, K <= 1<<20; a short workspace:
 * SG_ERR_WORKSPACE.  x, W_codes, r, outputs and the workspace 16-byte
 * aligned, W_scales 4-byte aligned.  Allocates nothing. */
sg_status skinny_gemm_fp8(int32_t M, int32_t N, int32_t K, const sg_bf16* x,
                          const uint8_t* W_codes, const float* W_scales, const sg_bf16* r,
                          float* y_f32, sg_bf16* y_bf16, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace bytes skinny_gemm_fp8 (resp. skinny_gemm_mxfp4) needs for an
 * M x N x K projection: the fp32 split-K partials [S, N, 16*ceil(M/16)] of
 * the chunk kernel when the call runs it and it splits K; 0 otherwise (the
 * one-launch kernels, one split, or sizes the call rejects). */
size_t skinny_gemm_fp8_workspace(int32_t M, int32_t N, int32_t K);
size_t skinny_gemm_mxfp4_workspace(int32_t M, int32_t N, int32_t K);

/* One MoE decode step of a layer on one GPU, with the shared expert on its
 * own stream ([P] Method details §3; [F] Partie 1 §3: the shared expert runs
 * on a separate stream and its work overlaps the routing or the
 * routed-expert computation).
 *   on stream:       scores     = x W_router^T       (skinny_gemm, N = E)
 *                    topk_ids, topk_scores            (skinny_gemm_router_topk)
 *                    out        = routed projection   (grouped_skinny_gemm)
 *   on side_stream:  shared_out = x W_shared^T       (skinny_gemm, N = N_shared)
 * The side stream starts after the work already queued on `stream`
 * (fork_event is recorded on stream), so the shared expert overlaps the
 * routing phase -- router projection, top-k and token table, which leave
 * HBM mostly idle -- and the start of the routed projection; `stream` waits
 * for it at the end (join_event), so work queued on `stream` afterwards
 * sees every output.  side_stream NULL (or equal to stream): everything runs
 * on `stream` in the order above, the shared expert last.  The two events
 * are caller-owned hipEvent_t (timing may be disabled), required with a
 * side stream.  The outputs are identical either way.
 * flags & SG_MOE_STEP_FUSED_SHARED: the shared expert joins the router's
 * projection instead -- both read the same x, so they are one skinny GEMM,
 * one weight stream and one launch ([P] Method details §3 likewise merges
 * the projections that precede the experts into a single GEMM).  Then
 * W_router is [E + N_shared, K] (router rows, then the shared expert's),
 * `scores` is [T, E + N_shared] (columns [0,E) the router scores, columns
 * [E, E+N_shared) the shared expert's output), W_shared and shared_out are
 * ignored, and no side stream is used.  Outputs equal those of the other
 * modes to the projection tolerance (the fused GEMM may take another plan).
 * flags & SG_MOE_STEP_SHARED_IN_ROUTED: up to 4 tokens (E <= 512, N >= 1)
 * the routed-expert launch, which ranks the scores itself, also computes
 * shared_out: every wave streams its share of W_shared's rows while it ranks,
 * when no routed weight can be requested yet -- the overlap of [P] Method
 * details §3 inside one launch, two launches a step.  Larger steps run as
 * with side_stream NULL.  Buffers as in the default mode; no side stream is
 * used; ids and routed outputs equal the other modes' bit for bit, shared_out
 * to the projection tolerance.  Both flags together: SG_ERR_SHAPE.
 * Shapes: x [T,K], W_router [E,K], W_experts [E,N,K], W_shared [N_shared,K]
 * (bf16); scores [T,E], topk_scores [T,topk] (nullable), out [T,topk,N],
 * shared_out [T,N_shared] (fp32); topk_ids [T,topk] int32.  Pointers whose
 * extent is zero may be NULL; the others must be 16-byte aligned.
 * Limits: T > 64 -> SG_ERR_UNSUPPORTED; 1 <= E <= 4096, 1 <= topk <=
 * min(E, 32), 0 <= K <= 8192 (K % 8 == 0), 0 <= N, N_shared <= 1<<20 (else
 * SG_ERR_SHAPE / SG_ERR_ALIGN).  Workspace: skinny_moe_step_workspace bytes,
 * 16-byte aligned, used by the three projections and the token table. */
typedef struct {
    const sg_bf16* x;
    const sg_bf16* W_router;
    const sg_bf16* W_experts;
    const sg_bf16* W_shared;
    float* scores;
    int32_t* topk_ids;
    float* topk_scores;
    float* out;
    float* shared_out;
    int32_t T, K, E, topk, N, N_shared;
    int32_t flags;  /* 0, SG_MOE_STEP_FUSED_SHARED or SG_MOE_STEP_SHARED_IN_ROUTED */
} sg_moe_step;

#define SG_MOE_STEP_FUSED_SHARED 1
#define SG_MOE_STEP_SHARED_IN_ROUTED 2

/* Workspace bytes skinny_moe_step needs (0 if the sizes are rejected). */
size_t skinny_moe_step_workspace(int32_t T, int32_t K, int32_t E, int32_t topk, int32_t N,
                                 int32_t N_shared);

sg_status skinny_moe_step(const sg_moe_step* step, void* workspace, size_t workspace_bytes,
                          void* stream, void* side_stream, void* fork_event, void* join_event);

/* Side-stream weight prefetch ([P] Method details §4): reads
 * [W, W + bytes) so that a following projection finds it in the GPU's
 * caches (MI355X: 4 MB L2 per XCD, 256 MB Infinity Cache).  Reads only the
 * given static-weight range and writes nothing ([F] Partie 2 §3); the
 * caller orders it against other streams with events.  W 16-byte aligned,
 * bytes a multiple of 16. */
sg_status skinny_gemm_prefetch(const void* W, size_t bytes, void* stream);

/* Read-bandwidth probe (measurement only; computes and writes nothing).
 * Small-batch projections are bound by how fast weights stream from HBM
 * ([P] Method details §1); this call reads W [rows, row_bytes] with the load
 * shape of the M <= 2 projection kernel -- rows_per_iter (1 or 2) whole rows
 * per wave and iteration, 1 KB buffer loads with the non-temporal hint, grid
 * workgroups of 4 waves striding over the row groups -- and no arithmetic,
 * so its time is what that kernel's loads alone take on this GPU.  Pass the
 * plan's grid and tile_n (rows per iteration) of the projection to compare.
 * Limits: 0 <= rows, 16 <= row_bytes <= 16384, 1 <= grid <= 65536,
 * rows * row_bytes <= 2^40 (else SG_ERR_SHAPE); row_bytes % 16 == 0 and W
 * 16-byte aligned (SG_ERR_ALIGN); W NULL with rows > 0: SG_ERR_NULL.  Not
 * counted in the launch counters.  Asynchronous on `stream`. */
sg_status skinny_gemm_read_probe(const void* W, int32_t rows, int32_t row_bytes,
                                 int32_t rows_per_iter, int32_t grid, void* stream);

/* Text for a status code (static storage). */
const char* skinny_gemm_status_str(sg_status status);

/* Launch counters, indexed by sg_kernel: how many times each kernel was
 * launched since load or the last reset ([F] Partie 2 §1: which path ran
 * must be observable).  Process-wide, atomic. */
void skinny_gemm_get_counters(uint64_t launches[SG_NUM_COUNTERS]);
void skinny_gemm_reset_counters(void);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_GEMM_H */
