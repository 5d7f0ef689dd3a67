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
// The order is carried by one 64-bit key per expert (topk_device.h).  One
// wavefront per token ranks its scores (wave_topk: DPP and permlane
// exchanges, no LDS); lane r keeps the round-r winner, and the k results
// leave in one parallel store.
#include "launch.h"
#include "topk_device.h"

namespace sg {

namespace {

template <int PER>
__global__ __launch_bounds__(kBlock) void router_topk_kernel(const float* __restrict__ scores,
                                                             int64_t ld, int T, int E, int k,
                                                             int32_t* __restrict__ ids,
                                                             float* __restrict__ top) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * kWavesPerBlock + wave_id_in_block();
    if (t >= T) return;
    const float* s = scores + t * ld;
    const uint64_t mine = wave_topk<PER>(s, E, k, lane);
    if (lane < k) {
        const int id = key_id(mine);
        ids[(int64_t)t * k + lane] = id;
        if (top) top[(int64_t)t * k + lane] = s[id];  // the score as given (NaN, -0 kept)
    }
}

}  // namespace

hipError_t launch_router_topk(const float* scores, int64_t ld, int T, int E, int k,
                              int32_t* ids, float* top, hipStream_t stream) {
    const int grid = (T + kWavesPerBlock - 1) / kWavesPerBlock;
    const int per = (E + kWave - 1) / kWave;
#define SG_PER(p) \
    if (per <= p) { \
        router_topk_kernel<p><<<grid, kBlock, 0, stream>>>(scores, ld, T, E, k, ids, top); \
        return hipGetLastError(); \
    }
    SG_PER(1) SG_PER(2) SG_PER(3) SG_PER(4) SG_PER(5) SG_PER(6) SG_PER(7) SG_PER(8)
    SG_PER(16) SG_PER(32) SG_PER(64)
#undef SG_PER
    return hipErrorInvalidValue;
}

}  // namespace sg
