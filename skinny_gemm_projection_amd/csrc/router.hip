// router.hip -- router top-k on gfx950: the experts each token is routed to,
// from its router scores.
//
// Expert selection decides which expert weights the routed-expert step reads
// ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Method details §3;
// French translation, Partie 2 §4).  The scores themselves are a skinny
// projection (the small-matrix or split-K path with N = number of experts);
// this kernel ranks them.  Rank order: the larger score first, equal scores
// by the lower expert id, a NaN score as -infinity -- a total order, so the
// selected ids are unique.
//
// One wavefront per token.  Lane l holds the scores of experts l, l+64, ...
// in registers.  Round j keeps, in each lane, the best of its experts that
// rank after the round j-1 winner, then DPP and permlane exchanges find the
// wave's best: k rounds of (E/64 compares + 6 exchanges), no LDS, no
// sorting, and nothing to reset between tokens.
#include "launch.h"

namespace sg {

namespace {

__device__ __forceinline__ bool ranks_before(float a, int ia, float b, int ib) {
    return a > b || (a == b && ia < ib);
}

__device__ __forceinline__ void keep_first(float& v, int& i, float ov, int oi) {
    if (ranks_before(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

template <int CTRL>
__device__ __forceinline__ void dpp_step(float& v, int& i) {
    const float ov = dpp<CTRL>(v);
    const int oi = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, true);
    keep_first(v, i, ov, oi);
}

// Every lane receives the wave's first-ranked (v, i): DPP exchanges inside
// 16-lane rows (partners l^1, l^2, the mirrored half row, the mirrored row),
// then row-pair and half-wave swaps -- all VALU, no LDS round trips.
__device__ __forceinline__ void wave_first(float& v, int& i) {
    dpp_step<0xB1>(v, i);   // quad_perm [1,0,3,2]
    dpp_step<0x4E>(v, i);   // quad_perm [2,3,0,1]
    dpp_step<0x141>(v, i);  // row_half_mirror
    dpp_step<0x140>(v, i);  // row_mirror
    {
        const auto pv = __builtin_amdgcn_permlane16_swap(as_u(v), as_u(v), false, false);
        const auto pi = __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false);
        v = as_f(pv[0]);
        i = (int)pi[0];
        keep_first(v, i, as_f(pv[1]), (int)pi[1]);
    }
    {
        const auto pv = __builtin_amdgcn_permlane32_swap(as_u(v), as_u(v), false, false);
        const auto pi = __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
        v = as_f(pv[0]);
        i = (int)pi[0];
        keep_first(v, i, as_f(pv[1]), (int)pi[1]);
    }
}

template <int PER>
__global__ __launch_bounds__(kBlock) void router_topk_kernel(const float* __restrict__ scores,
                                                             int T, int E, int k,
                                                             int32_t* __restrict__ ids,
                                                             float* __restrict__ top) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * kWavesPerBlock + wave_id_in_block();
    if (t >= T) return;
    const float* s = scores + (int64_t)t * E;
    float key[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = j * kWave + lane;
        const float v = e < E ? s[e] : -__builtin_inff();
        key[j] = v != v ? -__builtin_inff() : v;  // NaN ranks as -infinity
    }
    float prev = 0.0f;
    int prev_id = -1;  // -1: no winner yet
    int mine = 0;      // lane r keeps the round-r winner
    for (int r = 0; r < k; ++r) {
        float best = -__builtin_inff();
        int best_id = 0x7fffffff;  // ranks after every expert
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = j * kWave + lane;
            const bool after_prev = prev_id < 0 || ranks_before(prev, prev_id, key[j], e);
            if (e < E && after_prev && ranks_before(key[j], e, best, best_id)) {
                best = key[j];
                best_id = e;
            }
        }
        wave_first(best, best_id);
        if (lane == r) mine = best_id;
        prev = best;
        prev_id = best_id;
    }
    if (lane < k) {  // one parallel store (and read of the score as given, NaN kept)
        ids[(int64_t)t * k + lane] = mine;
        if (top) top[(int64_t)t * k + lane] = s[mine];
    }
}

}  // namespace

hipError_t launch_router_topk(const float* scores, int T, int E, int k, int32_t* ids,
                              float* top, hipStream_t stream) {
    const int grid = (T + kWavesPerBlock - 1) / kWavesPerBlock;
    const int per = (E + kWave - 1) / kWave;
#define SG_PER(p) \
    if (per <= p) { \
        router_topk_kernel<p><<<grid, kBlock, 0, stream>>>(scores, T, E, k, ids, top); \
        return hipGetLastError(); \
    }
    SG_PER(1) SG_PER(2) SG_PER(4) SG_PER(8) SG_PER(16) SG_PER(32) SG_PER(64)
#undef SG_PER
    return hipErrorInvalidValue;
}

}  // namespace sg
