// plan_internal.h -- planner and call entry points shared inside the library.
#pragma once

#include "skinny_gemm.h"

namespace sg {

// Plan for (M, N, K); kernel <= 0, split_k <= 0, two_pass < 0 and
// tile_n <= 0 let the planner choose.
sg_status make_plan(int32_t M, int32_t N, int32_t K, int32_t kernel, int32_t split_k,
                    int32_t two_pass, int32_t tile_n, sg_plan* out);

// True when *p is exactly what the planner produces for its own fields.
bool plan_matches(const sg_plan* p);

// The checked, counted and logged router top-k call behind
// skinny_gemm_router_topk, with a row stride (ld >= E elements) for scores
// that share their rows with other outputs (a fused router + shared-expert
// projection).
sg_status router_topk_call(const float* scores, int64_t ld, int32_t T, int32_t E, int32_t k,
                           int32_t* topk_ids, float* topk_scores, void* stream);

// Router top-k and the routed-expert projection as one launch (a few tokens,
// E <= 512, N >= 1; see launch_route_grouped): whether it applies, and the
// counted, logged call.  The caller has checked pointers and alignment.
bool route_grouped_ok(int32_t T, int32_t E, int32_t k, int32_t N);
sg_status route_grouped_call(const float* scores, int64_t ld, int32_t T, int32_t E, int32_t k,
                             int32_t* topk_ids, float* topk_scores, const sg_bf16* x,
                             const sg_bf16* W, int32_t N, int32_t K, float* out,
                             const sg_bf16* W_shared, int32_t N_shared, float* shared_out,
                             void* stream);

}  // namespace sg
