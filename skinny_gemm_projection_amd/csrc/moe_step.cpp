// moe_step.cpp -- one MoE decode step of a layer: router projection, top-k,
// token table and routed-expert projection on the caller's stream, and the
// shared expert's projection on a side stream that overlaps them.
//
// The shared expert depends only on the layer input, so it can start as soon
// as the step does and run on a separate stream ("Hyper Optimizing Kimi K3 in
// vLLM" deepnotes page, Method details §3; French translation, Partie 1 §3).
// On one MI355X the window it fills is the routing phase: the router
// projection is a few MB, and the top-k and the start of the routed-expert
// launch (which builds its token table in LDS) occupy a handful of CUs, so
// HBM is mostly idle for several microseconds before the routed-expert
// weights start to stream.  Up to 4 tokens the top-k itself runs inside the
// routed-expert launch: every workgroup ranks the scores, so a step is two
// launches (router projection, routed experts).  The side stream forks from the
// caller's stream at entry and joins it at the end; the caller owns both
// streams and both events.  Host-side composition only: every step is one of
// the library's own calls, so the outputs are identical with and without the
// side stream.
//
// Measured on MI355X, the fork/join events of the side stream cost more than
// the overlap hides at batch 1.  The fused mode therefore takes the shared
// expert into the router's GEMM: same input, one weight stream of
// E + N_shared rows, one launch, and the top-k kernel reads the score columns
// through a row stride.  The SHARED_IN_ROUTED mode instead makes the overlap
// happen inside the routed-expert launch (up to 4 tokens): its waves stream
// the shared expert's rows while they rank, the window in which no routed
// weight can be requested yet.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_internal.h"
#include "skinny_gemm.h"

namespace {

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct StepLayout {
    sg_plan router{}, shared{};  // fused: router covers E + N_shared rows, shared is empty
    size_t router_ws = 0, grouped_ws = 0, shared_ws = 0, total = 0;
};

sg_status step_layout(int32_t T, int32_t K, int32_t E, int32_t topk, int32_t N,
                      int32_t N_shared, bool fused, StepLayout* L) {
    if (T < 0 || K < 0 || K > 8192 || E < 1 || E > 4096 || topk < 1 || topk > 32 || topk > E ||
        N < 0 || N > (1 << 20) || N_shared < 0 || N_shared > (1 << 20))
        return SG_ERR_SHAPE;
    if (T > 64) return SG_ERR_UNSUPPORTED;
    if (K % 8 != 0) return SG_ERR_ALIGN;
    sg_status st = skinny_gemm_plan(T, fused ? E + N_shared : E, K, &L->router);
    if (st != SG_OK) return st;
    st = skinny_gemm_plan(T, fused ? 0 : N_shared, K, &L->shared);
    if (st != SG_OK) return st;
    L->router_ws = align256(L->router.workspace_bytes);
    L->grouped_ws = align256(grouped_skinny_gemm_workspace(T, E, topk, N, K));
    L->shared_ws = align256(L->shared.workspace_bytes);
    L->total = L->router_ws + L->grouped_ws + L->shared_ws;
    return SG_OK;
}

}  // namespace

extern "C" {

size_t skinny_moe_step_workspace(int32_t T, int32_t K, int32_t E, int32_t topk, int32_t N,
                                 int32_t N_shared) {
    // the larger of the two modes' needs, so one buffer serves either
    StepLayout a, b;
    if (step_layout(T, K, E, topk, N, N_shared, false, &a) != SG_OK ||
        step_layout(T, K, E, topk, N, N_shared, true, &b) != SG_OK)
        return 0;
    return a.total > b.total ? a.total : b.total;
}

sg_status skinny_moe_step(const sg_moe_step* a, void* workspace, size_t workspace_bytes,
                          void* stream, void* side_stream, void* fork_event, void* join_event) {
    if (!a) return SG_ERR_NULL;
    if (a->flags & ~(SG_MOE_STEP_FUSED_SHARED | SG_MOE_STEP_SHARED_IN_ROUTED)) return SG_ERR_SHAPE;
    const bool fused = (a->flags & SG_MOE_STEP_FUSED_SHARED) != 0;
    const bool in_routed = (a->flags & SG_MOE_STEP_SHARED_IN_ROUTED) != 0;
    if (fused && in_routed) return SG_ERR_SHAPE;
    StepLayout L;
    sg_status st = step_layout(a->T, a->K, a->E, a->topk, a->N, a->N_shared, fused, &L);
    if (st != SG_OK) return st;
    if (a->T == 0) return SG_OK;

    // every check of the calls below, made here before the first launch
    const bool k_ = a->K > 0;
    const bool sep = !fused && a->N_shared > 0;  // a separate shared-expert projection
    if (!a->scores || !a->topk_ids || (k_ && (!a->x || !a->W_router))) return SG_ERR_NULL;
    if (a->N > 0 && (!a->out || (k_ && !a->W_experts))) return SG_ERR_NULL;
    if (sep && (!a->shared_out || (k_ && !a->W_shared))) return SG_ERR_NULL;
    const void* ptrs[] = {a->x,        a->W_router,  a->W_experts, sep ? a->W_shared : nullptr,
                          a->scores,   a->topk_ids,  a->topk_scores, a->out,
                          sep ? a->shared_out : nullptr};
    for (const void* p : ptrs)
        if (!aligned16(p)) return SG_ERR_ALIGN;
    if (!workspace || workspace_bytes < L.total) return SG_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SG_ERR_ALIGN;
    const bool overlap = sep && !in_routed && side_stream && side_stream != stream;
    if (overlap && (!fork_event || !join_event)) return SG_ERR_NULL;

    char* base = static_cast<char*>(workspace);
    void* router_ws = base;
    void* grouped_ws = base + L.router_ws;
    void* shared_ws = base + L.router_ws + L.grouped_ws;
    auto shared_expert = [&](void* s) {
        return skinny_gemm(&L.shared, a->x, a->W_shared, a->shared_out, nullptr, shared_ws,
                           L.shared_ws, s);
    };

    hipStream_t main_s = static_cast<hipStream_t>(stream);
    hipStream_t side_s = static_cast<hipStream_t>(side_stream);
    hipEvent_t fork = static_cast<hipEvent_t>(fork_event);
    hipEvent_t join = static_cast<hipEvent_t>(join_event);
    if (overlap) {
        if (hipEventRecord(fork, main_s) != hipSuccess) return SG_ERR_HIP;
        if (hipStreamWaitEvent(side_s, fork, 0) != hipSuccess) return SG_ERR_HIP;
        if ((st = shared_expert(side_stream)) != SG_OK) return st;
        if (hipEventRecord(join, side_s) != hipSuccess) return SG_ERR_HIP;
    }
    if ((st = skinny_gemm(&L.router, a->x, a->W_router, a->scores, nullptr, router_ws,
                          L.router_ws, stream)) != SG_OK)
        return st;
    const int64_t ld = fused ? (int64_t)a->E + a->N_shared : a->E;  // row stride of the scores
    bool shared_done = false;
    if (sg::route_grouped_ok(a->T, a->E, a->topk, a->N)) {
        // a few tokens: top-k and the routed experts in one launch, and in
        // SHARED_IN_ROUTED mode the shared expert too, streamed while it ranks
        const bool sh = in_routed && sep;
        if ((st = sg::route_grouped_call(a->scores, ld, a->T, a->E, a->topk, a->topk_ids,
                                         a->topk_scores, a->x, a->W_experts, a->N, a->K,
                                         a->out, sh ? a->W_shared : nullptr,
                                         sh ? a->N_shared : 0, sh ? a->shared_out : nullptr,
                                         stream)) != SG_OK)
            return st;
        shared_done = sh;
    } else {
        if ((st = sg::router_topk_call(a->scores, ld, a->T, a->E, a->topk, a->topk_ids,
                                       a->topk_scores, stream)) != SG_OK)
            return st;
        if ((st = grouped_skinny_gemm(a->x, a->T, a->W_experts, a->E, a->N, a->K, a->topk_ids,
                                      a->topk, a->out, nullptr, nullptr, nullptr, grouped_ws,
                                      L.grouped_ws, stream)) != SG_OK)
            return st;
    }
    if (overlap) return hipStreamWaitEvent(main_s, join, 0) == hipSuccess ? SG_OK : SG_ERR_HIP;
    return sep && !shared_done ? shared_expert(stream) : SG_OK;
}

}  // extern "C"
