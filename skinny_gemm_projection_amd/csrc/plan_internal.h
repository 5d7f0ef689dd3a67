// plan_internal.h -- planner entry points shared inside the library.
#pragma once

#include "skinny_gemm.h"

namespace sg {

// Plan for (M, N, K); kernel <= 0, split_k <= 0, two_pass < 0 and
// tile_n <= 0 let the planner choose.
sg_status make_plan(int32_t M, int32_t N, int32_t K, int32_t kernel, int32_t split_k,
                    int32_t two_pass, int32_t tile_n, sg_plan* out);

// True when *p is exactly what the planner produces for its own fields.
bool plan_matches(const sg_plan* p);

}  // namespace sg
