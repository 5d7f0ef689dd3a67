// api.cpp -- the C ABI of libskinny_gemm.so (declared in include/skinny_gemm.h).
//
// Every host-visible problem is rejected before any HIP call, so a rejected
// call has no side effects and never touches the GPU.  Accepted calls only
// enqueue kernels on the caller's stream: no allocation, no synchronisation,
// no memset (graph-capturable).  Which kernels ran is observable through
// process-wide launch counters, and SKINNY_GEMM_LOG=1 prints every launch
// decision to stderr ("Hyper optimisation de Kimi K3 dans vLLM", Partie 2
// §1: reviewers must be able to see when the optimised path is taken and how
// execution falls back to the standard one).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "launch.h"
#include "plan_internal.h"
#include "skinny_gemm.h"

namespace {

std::atomic<uint64_t> g_launches[SG_NUM_COUNTERS];

void count(int kernel) { g_launches[kernel].fetch_add(1, std::memory_order_relaxed); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("SKINNY_GEMM_LOG");
        return v && *v && *v != '0';
    }();
    return on;
}

const char* kernel_name(int k) {
    switch (k) {
        case SG_KERNEL_NONE: return "none";
        case SG_KERNEL_GEMV: return "gemv";
        case SG_KERNEL_SPLITK_VALU: return "splitk_valu";
        case SG_KERNEL_SPLITK_MFMA: return "splitk_mfma";
        case SG_KERNEL_REDUCE: return "reduce";
        case SG_KERNEL_MOE_TABLE: return "moe_table";
        case SG_KERNEL_GROUPED: return "grouped";
        case SG_KERNEL_PREFETCH: return "prefetch";
        case SG_KERNEL_FP8: return "fp8";
        case SG_KERNEL_ROUTER_TOPK: return "router_topk";
        case SG_KERNEL_MXFP4: return "mxfp4";
        default: return "?";
    }
}

sg_status projection(const sg_plan* p, const sg_bf16* x, const sg_bf16* W, const sg_bf16* r,
                     float* y_f32, sg_bf16* y_bf16, void* ws, size_t ws_bytes, void* stream,
                     bool residual) {
    if (!p) return SG_ERR_NULL;
    if (!sg::plan_matches(p)) return SG_ERR_PLAN;
    if (p->kernel == SG_KERNEL_NONE) return SG_OK;
    if (p->K > 0 && (!x || !W)) return SG_ERR_NULL;
    if (residual && !r) return SG_ERR_NULL;
    if (!y_f32 && !y_bf16) return SG_ERR_NULL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(r) || !aligned16(y_f32) || !aligned16(y_bf16))
        return SG_ERR_ALIGN;
    if (p->workspace_bytes > 0) {
        if (!ws || ws_bytes < p->workspace_bytes) return SG_ERR_WORKSPACE;
        if (!aligned16(ws)) return SG_ERR_ALIGN;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // start from a clean error state
    const sg::Epilogue fin{nullptr, y_f32, y_bf16, r};
    const bool split = p->two_pass != 0;
    const sg::Epilogue main_ep =
        split ? sg::Epilogue{static_cast<float*>(ws), nullptr, nullptr, nullptr} : fin;

    hipError_t err;
    const bool chunk = p->kernel == SG_KERNEL_SPLITK_MFMA && p->tile_n >= sg::kMfmaTileN;
    if (chunk)
        err = sg::launch_splitk_mfma(p->M, p->N, p->K, p->split_k, p->k_chunk, p->tile_n, x, W,
                                     main_ep, s);
    else if (p->kernel == SG_KERNEL_SPLITK_MFMA)
        err = sg::launch_mfma_team(p->M, p->N, p->K, p->split_k, p->k_chunk, x, W, main_ep, s);
    else
        err = sg::launch_rowdot(p->M, p->N, p->K, p->split_k, p->k_chunk, p->grid, split, x, W,
                                main_ep, s);
    if (err != hipSuccess) return SG_ERR_HIP;
    count(p->kernel);
    if (split) {
        if (chunk)
            err = sg::launch_reduce_tiles(static_cast<const float*>(ws), p->split_k, p->M, p->N,
                                          p->tile_n, fin, s);
        else
            err = sg::launch_reduce(static_cast<const float*>(ws), p->split_k,
                                    (int64_t)p->M * p->N, fin, s);
        if (err != hipSuccess) return SG_ERR_HIP;
        count(SG_KERNEL_REDUCE);
    }
    if (log_enabled())
        std::fprintf(stderr,
                     "[skinny_gemm] M=%d N=%d K=%d kernel=%s split_k=%d k_chunk=%d grid=%d%s%s\n",
                     p->M, p->N, p->K, kernel_name(p->kernel), p->split_k, p->k_chunk, p->grid,
                     split ? " +reduce pass" : (p->split_k > 1 ? " in-workgroup reduce" : ""),
                     residual ? " residual" : "");
    return SG_OK;
}

bool grouped_sizes_ok(int32_t T, int32_t E, int32_t topk, int32_t N, int32_t K) {
    if (T < 0 || T > 256 || topk < 1 || topk > 32 || (int64_t)T * topk > 4096) return false;
    if (E < 1 || E > 4096 || N < 0 || N > (1 << 20) || K < 0 || K > 8192) return false;
    return true;
}

}  // namespace

namespace sg {

sg_status router_topk_call(const float* scores, int64_t ld, int32_t T, int32_t E, int32_t k,
                           int32_t* topk_ids, float* topk_scores, void* stream) {
    if (T < 0 || T > (1 << 20) || E < 1 || E > 4096 || k < 1 || k > 32 || k > E || ld < E)
        return SG_ERR_SHAPE;
    if (T == 0) return SG_OK;
    if (!scores || !topk_ids) return SG_ERR_NULL;
    auto aligned4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (!aligned4(scores) || !aligned4(topk_ids) || !aligned4(topk_scores)) return SG_ERR_ALIGN;
    (void)hipGetLastError();
    if (launch_router_topk(scores, ld, T, E, k, topk_ids, topk_scores,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
        return SG_ERR_HIP;
    count(SG_KERNEL_ROUTER_TOPK);
    if (log_enabled())
        std::fprintf(stderr, "[skinny_gemm] router_topk T=%d E=%d k=%d ld=%lld\n", T, E, k,
                     (long long)ld);
    return SG_OK;
}

bool route_grouped_ok(int32_t T, int32_t E, int32_t k, int32_t N) {
    return T >= 1 && T <= kRouteFusedMaxT && E >= 1 && E <= kRouteFusedMaxExperts && k >= 1 &&
           k <= 32 && k <= E && N >= 1;
}

sg_status route_grouped_call(const float* scores, int64_t ld, int32_t T, int32_t E, int32_t k,
                             int32_t* topk_ids, float* topk_scores, const sg_bf16* x,
                             const sg_bf16* W, int32_t N, int32_t K, float* out,
                             const sg_bf16* W_shared, int32_t N_shared, float* shared_out,
                             void* stream) {
    if (!route_grouped_ok(T, E, k, N) || ld < E || K < 0 || K > 8192 || K % 8 != 0 ||
        N_shared < 0)
        return SG_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    if (launch_route_grouped(scores, ld, T, E, k, topk_ids, topk_scores, x, W, N, K, out,
                             W_shared, N_shared, shared_out,
                             static_cast<hipStream_t>(stream)) != hipSuccess)
        return SG_ERR_HIP;
    count(SG_KERNEL_GROUPED);
    if (log_enabled())
        std::fprintf(stderr,
                     "[skinny_gemm] router top-k + grouped (one launch) T=%d E=%d k=%d N=%d K=%d "
                     "N_shared=%d\n",
                     T, E, k, N, K, N_shared);
    return SG_OK;
}

}  // namespace sg

extern "C" {

sg_status skinny_gemm(const sg_plan* plan, const sg_bf16* x, const sg_bf16* W, float* y_f32,
                      sg_bf16* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
    return projection(plan, x, W, nullptr, y_f32, y_bf16, workspace, workspace_bytes, stream,
                      false);
}

sg_status skinny_gemm_residual(const sg_plan* plan, const sg_bf16* x, const sg_bf16* W,
                               const sg_bf16* r, sg_bf16* out_bf16, float* out_f32,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return projection(plan, x, W, r, out_f32, out_bf16, workspace, workspace_bytes, stream, true);
}

size_t grouped_skinny_gemm_workspace(int32_t T, int32_t E, int32_t topk, int32_t N, int32_t K) {
    if (!grouped_sizes_ok(T, E, topk, N, K)) return 0;
    return sg::grouped_workspace_bytes(E, T * topk);
}

sg_status grouped_skinny_gemm(const sg_bf16* x, int32_t T, const sg_bf16* W, int32_t E,
                              int32_t N, int32_t K, const int32_t* topk_ids, int32_t topk,
                              float* out, int32_t* expert_offsets, int32_t* sorted_pairs,
                              int32_t* invalid_count, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!grouped_sizes_ok(T, E, topk, N, K)) return SG_ERR_SHAPE;
    if (K % 8 != 0) return SG_ERR_ALIGN;
    if (T > 0 && (!topk_ids || (N > 0 && !out))) return SG_ERR_NULL;
    if (T > 0 && N > 0 && K > 0 && (!x || !W)) return SG_ERR_NULL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(topk_ids) || !aligned16(out) ||
        !aligned16(expert_offsets) || !aligned16(sorted_pairs) || !aligned16(invalid_count))
        return SG_ERR_ALIGN;
    const size_t need = sg::grouped_workspace_bytes(E, T * topk);
    if (!workspace || workspace_bytes < need) return SG_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SG_ERR_ALIGN;

    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    // No table output asked for and a small table: one fused launch builds
    // what it needs of the table in each workgroup.
    const bool fused = !expert_offsets && !sorted_pairs && !invalid_count &&
                       T * topk <= sg::kFusedMaxPairs && E <= sg::kFusedMaxExperts;
    if (fused) {
        if (T > 0 && N > 0) {
            if (sg::launch_grouped_fused(x, T, W, topk_ids, E, N, K, topk, out, s) != hipSuccess)
                return SG_ERR_HIP;
            count(SG_KERNEL_GROUPED);
        }
        if (log_enabled())
            std::fprintf(stderr, "[skinny_gemm] grouped (fused table) T=%d topk=%d E=%d N=%d K=%d\n",
                         T, topk, E, N, K);
        return SG_OK;
    }
    const sg::GroupedWorkspace g = sg::grouped_workspace_layout(workspace, E, T * topk);
    if (sg::launch_moe_table(topk_ids, T, topk, E, N, g, expert_offsets, sorted_pairs,
                             invalid_count, out, s) != hipSuccess)
        return SG_ERR_HIP;
    count(SG_KERNEL_MOE_TABLE);
    if (T > 0 && N > 0) {
        if (sg::launch_grouped(x, T, W, E, N, K, topk, g, out, s) != hipSuccess) return SG_ERR_HIP;
        count(SG_KERNEL_GROUPED);
    }
    if (log_enabled())
        std::fprintf(stderr, "[skinny_gemm] grouped T=%d topk=%d E=%d N=%d K=%d\n", T, topk, E, N,
                     K);
    return SG_OK;
}

sg_status skinny_gemm_router_topk(const float* scores, int32_t T, int32_t E, int32_t k,
                                  int32_t* topk_ids, float* topk_scores, void* stream) {
    return sg::router_topk_call(scores, E, T, E, k, topk_ids, topk_scores, stream);
}

}  // extern "C"

namespace {

size_t lowp_workspace(int fmt, int32_t M, int32_t N, int32_t K) {
    if (N < 1 || N > (1 << 20) || K < 0 || K > (1 << 20) || !sg::lowp_use_chunk(fmt, M, N))
        return 0;
    sg::LowpChunkPlan lp;
    return sg::lowp_chunk_plan(M, N, K, &lp) ? lp.workspace : 0;
}

}  // namespace

extern "C" {

size_t skinny_gemm_fp8_workspace(int32_t M, int32_t N, int32_t K) {
    return lowp_workspace(sg::kLowpFp8, M, N, K);
}

size_t skinny_gemm_mxfp4_workspace(int32_t M, int32_t N, int32_t K) {
    return lowp_workspace(sg::kLowpMxfp4, M, N, K);
}

}  // extern "C"

namespace {

// The chunk-kernel path shared by both formats: the split plan, the
// workspace check, then the chunk kernel (and the reduction when the plan
// splits K).
sg_status lowp_chunk_call(int fmt, int32_t M, int32_t N, int32_t K, const sg_bf16* x,
                          const void* W_codes, const void* W_scales, const sg_bf16* r,
                          float* y_f32, sg_bf16* y_bf16, void* workspace, size_t workspace_bytes,
                          void* stream) {
    sg::LowpChunkPlan lp;
    if (!sg::lowp_chunk_plan(M, N, K, &lp)) return SG_ERR_UNSUPPORTED;
    if (lp.workspace > 0) {
        if (!workspace || workspace_bytes < lp.workspace) return SG_ERR_WORKSPACE;
        if (!aligned16(workspace)) return SG_ERR_ALIGN;
    }
    (void)hipGetLastError();
    const sg::Epilogue fin{nullptr, y_f32, y_bf16, r};
    if (sg::launch_lowp_chunk(fmt, M, N, K, x, W_codes, W_scales, fin, workspace,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
        return SG_ERR_HIP;
    count(fmt == sg::kLowpFp8 ? SG_KERNEL_FP8 : SG_KERNEL_MXFP4);
    if (lp.S > 1) count(SG_KERNEL_REDUCE);
    if (log_enabled())
        std::fprintf(stderr, "[skinny_gemm] %s M=%d N=%d K=%d chunk kernel %d-row tiles S=%d%s%s\n",
                     fmt == sg::kLowpFp8 ? "fp8" : "mxfp4", M, N, K, 128 * lp.NT, lp.S,
                     lp.S > 1 ? " +reduce pass" : "", r ? " residual" : "");
    return SG_OK;
}

}  // namespace

extern "C" {

sg_status skinny_gemm_mxfp4(int32_t M, int32_t N, int32_t K, const sg_bf16* x,
                            const uint8_t* W_codes, const uint8_t* W_scales, const sg_bf16* r,
                            float* y_f32, sg_bf16* y_bf16, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (M < 0 || N < 0 || N > (1 << 20) || K < 0 || K > (1 << 20)) return SG_ERR_SHAPE;
    if (M > sg::kLowpMaxM) return SG_ERR_UNSUPPORTED;
    if (K % 32 != 0) return SG_ERR_ALIGN;
    bool chunk = sg::lowp_use_chunk(sg::kLowpMxfp4, M, N);
    sg::LowpChunkPlan lp;
    // up to 16 rows a K whose chunks do not fit in LDS goes to the matrix-core kernel
    if (chunk && M <= sg::kMxfp4MaxM && N > 0 && !sg::lowp_chunk_plan(M, N, K, &lp)) chunk = false;
    int nb, splits;
    if (M > 0 && !chunk && !sg::mxfp4_split(M, K, &nb, &splits)) return SG_ERR_UNSUPPORTED;
    if (chunk && N > 0 && !sg::lowp_chunk_plan(M, N, K, &lp)) return SG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return SG_OK;
    if (!y_f32 && !y_bf16) return SG_ERR_NULL;
    if (K > 0 && (!x || !W_codes || !W_scales)) return SG_ERR_NULL;
    if (!aligned16(x) || !aligned16(W_codes) || !aligned16(r) || !aligned16(y_f32) ||
        !aligned16(y_bf16))
        return SG_ERR_ALIGN;
    if (chunk)
        return lowp_chunk_call(sg::kLowpMxfp4, M, N, K, x, W_codes, W_scales, r, y_f32, y_bf16,
                               workspace, workspace_bytes, stream);
    (void)hipGetLastError();
    const sg::Epilogue ep{nullptr, y_f32, y_bf16, r};
    if (sg::launch_mxfp4(M, N, K, x, W_codes, W_scales, ep, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return SG_ERR_HIP;
    count(SG_KERNEL_MXFP4);
    if (log_enabled())
        std::fprintf(stderr, "[skinny_gemm] mxfp4 M=%d N=%d K=%d %s%s\n", M, N, K,
                     M >= sg::kMxfp4MfmaFromM ? "matrix cores" : "vector ALU",
                     r ? " residual" : "");
    return SG_OK;
}

sg_status skinny_gemm_fp8(int32_t M, int32_t N, int32_t K, const sg_bf16* x,
                          const uint8_t* W_codes, const float* W_scales, const sg_bf16* r,
                          float* y_f32, sg_bf16* y_bf16, void* workspace, size_t workspace_bytes,
                          void* stream) {
    if (M < 0 || N < 0 || N > (1 << 20) || K < 0 || K > (1 << 20)) return SG_ERR_SHAPE;
    if (K % 16 != 0) return SG_ERR_ALIGN;
    if (M > sg::kLowpMaxM) return SG_ERR_UNSUPPORTED;
    bool chunk = sg::lowp_use_chunk(sg::kLowpFp8, M, N);
    sg::LowpChunkPlan lp;
    // up to 16 rows a K whose chunks do not fit in LDS goes to the matrix-core kernel
    if (chunk && M <= sg::kFp8MaxM && N > 0 && !sg::lowp_chunk_plan(M, N, K, &lp)) chunk = false;
    if (M > 0 && !chunk && !sg::fp8_size_ok(M, K)) return SG_ERR_UNSUPPORTED;
    if (chunk && N > 0 && !sg::lowp_chunk_plan(M, N, K, &lp)) return SG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return SG_OK;
    if (!y_f32 && !y_bf16) return SG_ERR_NULL;
    if (K > 0 && (!x || !W_codes || !W_scales)) return SG_ERR_NULL;
    auto aligned4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
    if (!aligned16(x) || !aligned16(W_codes) || !aligned4(W_scales) || !aligned16(r) ||
        !aligned16(y_f32) || !aligned16(y_bf16))
        return SG_ERR_ALIGN;
    if (chunk)
        return lowp_chunk_call(sg::kLowpFp8, M, N, K, x, W_codes, W_scales, r, y_f32, y_bf16,
                               workspace, workspace_bytes, stream);
    int splits, chunk16, nch;
    if (!sg::fp8_split(M, N, K, &splits, &chunk16, &nch)) return SG_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    const sg::Epilogue ep{nullptr, y_f32, y_bf16, r};
    if (sg::launch_fp8(M, N, K, x, W_codes, W_scales, ep, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return SG_ERR_HIP;
    count(SG_KERNEL_FP8);
    if (log_enabled())
        std::fprintf(stderr, "[skinny_gemm] fp8 M=%d N=%d K=%d %s split_k=%d%s\n", M, N, K,
                     M >= sg::kFp8MfmaFromM ? "matrix cores" : "vector ALU", splits,
                     r ? " residual" : "");
    return SG_OK;
}

sg_status skinny_gemm_prefetch(const void* W, size_t bytes, void* stream) {
    if (bytes == 0) return SG_OK;
    if (!W) return SG_ERR_NULL;
    if (!aligned16(W) || bytes % 16 != 0) return SG_ERR_ALIGN;
    (void)hipGetLastError();
    if (sg::launch_prefetch(W, bytes, static_cast<hipStream_t>(stream)) != hipSuccess)
        return SG_ERR_HIP;
    count(SG_KERNEL_PREFETCH);
    return SG_OK;
}

sg_status skinny_gemm_read_probe(const void* W, int32_t rows, int32_t row_bytes,
                                 int32_t rows_per_iter, int32_t grid, void* stream) {
    if (rows < 0 || row_bytes < 16 || row_bytes > 16384 || grid < 1 || grid > 65536 ||
        (rows_per_iter != 1 && rows_per_iter != 2) ||
        (int64_t)rows * row_bytes > (int64_t(1) << 40))
        return SG_ERR_SHAPE;
    if (row_bytes % 16 != 0) return SG_ERR_ALIGN;
    if (rows == 0) return SG_OK;
    if (!W) return SG_ERR_NULL;
    if (!aligned16(W)) return SG_ERR_ALIGN;
    (void)hipGetLastError();
    if (sg::launch_read_probe(W, rows, row_bytes, rows_per_iter, grid,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
        return SG_ERR_HIP;
    return SG_OK;
}

const char* skinny_gemm_status_str(sg_status status) {
    switch (status) {
        case SG_OK: return "SG_OK";
        case SG_ERR_NULL: return "SG_ERR_NULL: a required pointer is NULL";
        case SG_ERR_SHAPE: return "SG_ERR_SHAPE: size negative or over the limit";
        case SG_ERR_UNSUPPORTED: return "SG_ERR_UNSUPPORTED: batch outside the decode path (M > 64)";
        case SG_ERR_ALIGN: return "SG_ERR_ALIGN: K % 8 != 0 or a pointer misaligned";
        case SG_ERR_WORKSPACE: return "SG_ERR_WORKSPACE: workspace missing or too small";
        case SG_ERR_PLAN: return "SG_ERR_PLAN: plan does not fit this problem";
        case SG_ERR_HIP: return "SG_ERR_HIP: kernel launch failed";
        default: return "unknown sg_status";
    }
}

void skinny_gemm_get_counters(uint64_t launches[SG_NUM_COUNTERS]) {
    if (!launches) return;
    for (int i = 0; i < SG_NUM_COUNTERS; ++i)
        launches[i] = g_launches[i].load(std::memory_order_relaxed);
}

void skinny_gemm_reset_counters(void) {
    for (int i = 0; i < SG_NUM_COUNTERS; ++i) g_launches[i].store(0, std::memory_order_relaxed);
}

}  // extern "C"
