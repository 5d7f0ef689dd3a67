// topk_device.h -- the router's rank order and a wavefront's top-k, shared by
// the router top-k kernel and the routed-expert launch that ranks the scores
// itself (gfx950, wave64).
//
// Rank order ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Method
// details §3: the router picks the experts each token is sent to): the
// larger score first, equal scores by the lower expert id, a NaN score as
// -infinity -- a total order, so the selected ids are unique.  It is carried
// by one 64-bit key per expert: the high word is the score's bits mapped so
// that unsigned order is float order (NaN mapped to -infinity first, -0 to
// +0), the low word is ~id, so that the lower id wins a tie.  Keys are
// distinct, so "ranks before" is one unsigned compare and the wave's first
// is a plain maximum.
#pragma once

#include "sg_device.h"

namespace sg {

constexpr int kSortedPerLane = 8;  // presort up to this many keys per lane

__device__ __forceinline__ uint64_t rank_key(float v, int e) {
    if (v != v) v = -__builtin_inff();  // NaN ranks as -infinity
    if (v == 0.0f) v = 0.0f;            // -0 ties with +0
    uint32_t u = as_u(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }

__device__ __forceinline__ uint64_t join_u64(uint32_t hi, uint32_t lo) {
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    return umax64(v, join_u64(hi, lo));
}

// Every lane receives the wave maximum: DPP exchanges inside 16-lane rows
// (partners l^1, l^2, the mirrored half row, the mirrored row), then
// row-pair and half-wave swaps.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
    v = dpp_max64<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_max64<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_max64<0x141>(v);  // row_half_mirror
    v = dpp_max64<0x140>(v);  // row_mirror
    {
        const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
        const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        v = umax64(join_u64(ph[0], pl[0]), join_u64(ph[1], pl[1]));
    }
    {
        const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
        const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        v = umax64(join_u64(ph[0], pl[0]), join_u64(ph[1], pl[1]));
    }
    return v;
}

// The E scores s[0..E) a lane holds (PER >= ceil(E / 64)): lane l takes
// experts l, l+64, ....  Buffer loads with no branch (a score past E reads
// zero), all issued before any is used: written as a load per key under
// `e < E`, each load sat in its own branch with a wait right behind it, so
// the PER loads ran one after another.
template <int PER>
__device__ __forceinline__ void wave_topk_fetch(const float* __restrict__ s, int E, int lane,
                                                uint32_t (&v)[PER]) {
    const rsrc_t rs = make_rsrc(s, (uint32_t)E * 4u);
#pragma unroll
    for (int j = 0; j < PER; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(j * kWave + lane) * 4u, 0,
                                                    kCached);
}

// Their keys; key 0 (below every real key) pads experts past E.
template <int PER>
__device__ __forceinline__ void wave_topk_keys(const uint32_t (&v)[PER], int E, int lane,
                                               uint64_t (&key)[PER]) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = j * kWave + lane;
        const uint64_t kj = rank_key(as_f(v[j]), e);
        key[j] = e < E ? kj : 0;
    }
}

// The k first-ranked of the keys wave_topk_keys gave, computed by one whole
// wavefront: up to kSortedPerLane keys a lane are sorted once and each of
// the k rounds takes the wave maximum of the lane heads (the winning lane
// pops its head); with more, each round every lane rescans for its best key
// below the previous winner.  Returns, in lane r < k, the key of rank r.
template <int PER>
__device__ __forceinline__ uint64_t wave_topk_rank(uint64_t (&key)[PER], int k, int lane) {
    uint64_t mine = 0;
    if constexpr (PER <= kSortedPerLane) {
        // odd-even transposition sort, descending
#pragma unroll
        for (int r = 0; r < PER; ++r) {
#pragma unroll
            for (int j = r & 1; j + 1 < PER; j += 2) {
                const uint64_t a = key[j], b = key[j + 1];
                key[j] = umax64(a, b);
                key[j + 1] = a > b ? b : a;
            }
        }
        for (int r = 0; r < k; ++r) {
            const uint64_t w = wave_max64(key[0]);
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
            for (int j = 0; j < PER; ++j) best = key[j] < prev ? umax64(best, key[j]) : best;
            prev = wave_max64(best);
            if (lane == r) mine = prev;
        }
    }
    return mine;
}

// The k first-ranked of the E scores s[0..E): in lane r < k, the key of rank r.
template <int PER>
__device__ __forceinline__ uint64_t wave_topk(const float* __restrict__ s, int E, int k, int lane) {
    uint32_t v[PER];
    uint64_t key[PER];
    wave_topk_fetch<PER>(s, E, lane, v);
    wave_topk_keys<PER>(v, E, lane, key);
    return wave_topk_rank<PER>(key, k, lane);
}

}  // namespace sg
