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
// The order is carried by one 64-bit key per expert: the high word is the
// score's bits mapped so that unsigned order is float order (NaN mapped to
// -infinity first, -0 to +0), the low word is ~id, so that the lower id wins
// a tie.  Keys are distinct, so "ranks before" is one unsigned compare and
// the wave's first is a plain maximum.
//
// One wavefront per token; lane l holds the keys of experts l, l+64, ...
// in registers.  Up to 8 keys a lane: the lane sorts them once, then each
// of the k rounds takes the wave maximum of the lane heads (DPP and
// permlane exchanges, no LDS) and the winning lane pops its head.  More
// keys a lane: each round every lane rescans for its best key below the
// previous winner.  Lane r keeps the round-r winner; the k results leave in
// one parallel store.
#include "launch.h"

namespace sg {

namespace {

constexpr int kSortedPerLane = 8;  // presort up to this many keys per lane

__device__ __forceinline__ uint64_t rank_key(float v, int e) {
    if (v != v) v = -__builtin_inff();  // NaN ranks as -infinity
    if (v == 0.0f) v = 0.0f;            // -0 ties with +0
    uint32_t u = as_u(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }

__device__ __forceinline__ uint64_t join(uint32_t hi, uint32_t lo) {
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umax(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    return umax(v, join(hi, lo));
}

// Every lane receives the wave maximum: DPP exchanges inside 16-lane rows
// (partners l^1, l^2, the mirrored half row, the mirrored row), then
// row-pair and half-wave swaps.
__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
    v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_max<0x141>(v);  // row_half_mirror
    v = dpp_max<0x140>(v);  // row_mirror
    {
        const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
        const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        v = umax(join(ph[0], pl[0]), join(ph[1], pl[1]));
    }
    {
        const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
        const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        v = umax(join(ph[0], pl[0]), join(ph[1], pl[1]));
    }
    return v;
}

template <int PER>
__global__ __launch_bounds__(kBlock) void router_topk_kernel(const float* __restrict__ scores,
                                                             int64_t ld, int T, int E, int k,
                                                             int32_t* __restrict__ ids,
                                                             float* __restrict__ top) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * kWavesPerBlock + wave_id_in_block();
    if (t >= T) return;
    const float* s = scores + t * ld;
    // key 0 (below every real key) pads experts past E
    uint64_t key[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = j * kWave + lane;
        const float v = s[e < E ? e : E - 1];
        key[j] = e < E ? rank_key(v, e) : 0;
    }
    uint64_t mine = 0;
    if constexpr (PER <= kSortedPerLane) {
        // odd-even transposition sort, descending
#pragma unroll
        for (int r = 0; r < PER; ++r) {
#pragma unroll
            for (int j = r & 1; j + 1 < PER; j += 2) {
                const uint64_t a = key[j], b = key[j + 1];
                key[j] = umax(a, b);
                key[j + 1] = a > b ? b : a;
            }
        }
        for (int r = 0; r < k; ++r) {
            const uint64_t w = wave_max(key[0]);
            if (lane == r) mine = w;
            const uint64_t pop = key[0] == w ? ~0ull : 0;  // the winner lane shifts
#pragma unroll
            for (int j = 0; j + 1 < PER; ++j) key[j] = (key[j] & ~pop) | (key[j + 1] & pop);
            key[PER - 1] &= ~pop;
        }
    } else {
        uint64_t prev = ~0ull;  // ranks before every key
        for (int r = 0; r < k; ++r) {
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) best = key[j] < prev ? umax(best, key[j]) : best;
            prev = wave_max(best);
            if (lane == r) mine = prev;
        }
    }
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
