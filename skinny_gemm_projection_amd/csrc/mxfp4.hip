// mxfp4.hip -- decode projection with block-scaled 4-bit weights on gfx950.
//
// The pages' later evaluation model ships NVFP4 weights ("Hyper Optimizing
// Kimi K3 in vLLM" deepnotes page, Experimental setup and Supplementary
// details): 4-bit floats with per-block scales, a quarter of the bf16 weight
// bytes for the same bandwidth-bound projection.  The block-scaled 4-bit
// format MI355X converts in hardware is OCP MXFP4: e2m1 codes, two a byte
// (low nibble first), one e8m0 power-of-two scale per 32 consecutive
// elements of a row.  Activations stay bf16 and sums fp32.
//
// Mapping (wave64, like the bf16 row-streaming kernel).  A wave owns one K
// chunk of whole W rows; lane l takes the 32-element blocks c*64 + l of the
// chunk, so one 16-byte load is exactly one block (coalesced: 1 KB of codes
// per instruction) and one byte load is its scale (64 consecutive bytes per
// instruction).  The block's 32 activations of every x row stay in
// registers for the wave's life.  Each code byte becomes two bf16 weights in
// one v_cvt_scalef32_pk_bf16_fp4, which applies the block scale on the way
// (the instruction reads its float operand's exponent field as an e8m0
// scale; e2m1 times a power of two is exact in bf16), and the pair meets the
// matching x pair in one v_dot2c_f32_bf16 per activation row.  A scale code
// 255 (NaN) is handled once per row, not per element: the row's partial
// becomes NaN before the lane reduction.
//
// Rows are grouped R per iteration, their R*M lane partials reduced
// together by the reduce-scatter of the bf16 kernel; S waves of a workgroup
// split K and add their partials in LDS in ascending chunk order.
#include "launch.h"

namespace sg {

namespace {

constexpr int kBlockElems = 32;  // elements per scale block = per 16-byte code load

// 32 products of one block: x pairs (16 dwords, xb[d] component j holds
// elements 8d+2j, 8d+2j+1) against the 32 codes of w (dword d, byte j holds
// the same two elements), each code pair converted with the block scale.
__device__ __forceinline__ float dot_block(const uint4 (&xb)[4], const uint4 w, float scale,
                                           float acc) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t xd[4] = {xb[d].x, xb[d].y, xb[d].z, xb[d].w};
        const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], scale, 0);
        const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], scale, 1);
        const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], scale, 2);
        const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], scale, 3);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[0]), w0, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[1]), w1, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[2]), w2, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[3]), w3, acc, false);
    }
    return acc;
}

constexpr int pad4(int v) { return (v + 3) / 4 * 4; }
constexpr int team_waves(int S) { return S > kWavesPerBlock ? S : kWavesPerBlock; }

template <int M, int NB, int R, int S>
__global__ __launch_bounds__(kWave * team_waves(S)) void mxfp4_rowdot_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ Wq, const uint8_t* __restrict__ Ws,
    int N, int KB, int chunk_b, int iters, Epilogue ep) {
    constexpr int kWaves = team_waves(S);
    constexpr int kTeams = kWaves / S;
    constexpr int V = pad4(R * M);
    __shared__ float red[2][kTeams][S][V];

    const int lane = threadIdx.x & (kWave - 1);
    const int wib = wave_id_in_block();
    const int team_in_block = wib / S;
    const int member = wib % S;
    const int team = blockIdx.x * kTeams + team_in_block;
    const int teams = gridDim.x * kTeams;

    // this wave's chunk: blocks [b0, b0 + len) of every row
    const int b0 = member * chunk_b;
    const int len = max(0, min(KB - b0, chunk_b));

    // activations: 4 x 16 bytes per block and row, zero past the chunk
    uint4 xr[M][NB][4];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const rsrc_t rx = make_rsrc(x + ((int64_t)m * KB + b0) * 4, (uint32_t)len * 64u);
#pragma unroll
        for (int c = 0; c < NB; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xr[m][c][q] = load16<kCached>(rx, (uint32_t)((c * kWave + lane) * 64 + q * 16));
    }

    const int groups = (N + R - 1) / R;
    for (int it = 0; it < iters; ++it) {
        const int g = team + it * teams;
        const int n0 = g * R;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.0f;
        if (g < groups) {
            uint4 wr[R][NB];
            uint32_t sc[R][NB];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = n0 + r;
                const bool ok = n < N;
                const int64_t row = (int64_t)(ok ? n : 0) * KB + b0;
                const rsrc_t rw = make_rsrc(Wq + row, ok ? (uint32_t)len * 16u : 0u);
                const rsrc_t rs = make_rsrc(Ws + row, ok ? (uint32_t)len : 0u);
#pragma unroll
                for (int c = 0; c < NB; ++c) {
                    wr[r][c] = load16<kStream>(rw, (uint32_t)(c * kWave + lane) * 16u);
                    sc[r][c] = __builtin_amdgcn_raw_buffer_load_b8(
                        rs, (uint32_t)(c * kWave + lane), 0, kStream);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                bool nan_scale = false;
                float scale[NB];
#pragma unroll
                for (int c = 0; c < NB; ++c) {
                    nan_scale |= sc[r][c] == 255u;
                    scale[c] = as_f(sc[r][c] << 23);  // e8m0 code in the exponent field
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float a = 0.0f;
#pragma unroll
                    for (int c = 0; c < NB; ++c) a = dot_block(xr[m][c], wr[r][c], scale[c], a);
                    acc[r * M + m] = nan_scale ? __builtin_nanf("") : a;
                }
            }
        }
        const float total = reduce_scatter<V>(acc, lane);
        const int v = scatter_index<V>(lane);
        const bool mine = v >= 0 && v < R * M;
        const int r = mine ? v / M : 0;
        const int m = mine ? v - r * M : 0;
        const int n = n0 + r;
        const bool live = mine && g < groups && n < N;
        if (S == 1) {
            if (live) store_final(ep, (int64_t)m * N + n, total);
        } else {
            const int buf = it & 1;
            if (mine) red[buf][team_in_block][member][v] = total;
            __syncthreads();
            if (member == 0 && live) {
                float sum = red[buf][team_in_block][0][v];
#pragma unroll
                for (int s = 1; s < S; ++s) sum += red[buf][team_in_block][s][v];
                store_final(ep, (int64_t)m * N + n, sum);
            }
        }
    }
}

constexpr int kResidentWaves = 2048;  // 256 CUs x 8 waves
constexpr int kRows = 8;              // rows per wave iteration: 8 x NB KB of codes in flight

template <int M, int NB, int S>
hipError_t launch_mns(int N, int KB, int chunk_b, const void* x, const void* Wq,
                      const uint8_t* Ws, const Epilogue& ep, hipStream_t stream) {
    constexpr int kTeams = team_waves(S) / S;
    const int groups = (N + kRows - 1) / kRows;
    const int cap = kResidentWaves / S;
    const int teams_needed = groups < cap ? groups : cap;
    const int grid = (teams_needed + kTeams - 1) / kTeams;
    const int teams = grid * kTeams;
    const int iters = (groups + teams - 1) / teams;
    mxfp4_rowdot_kernel<M, NB, kRows, S><<<grid, kWave * team_waves(S), 0, stream>>>(
        static_cast<const uint4*>(x), static_cast<const uint4*>(Wq), Ws, N, KB, chunk_b, iters,
        ep);
    return hipGetLastError();
}

template <int M, int NB>
hipError_t launch_mn(int S, int N, int KB, int chunk_b, const void* x, const void* Wq,
                     const uint8_t* Ws, const Epilogue& ep, hipStream_t stream) {
    switch (S) {
        case 1: return launch_mns<M, NB, 1>(N, KB, chunk_b, x, Wq, Ws, ep, stream);
        case 2: return launch_mns<M, NB, 2>(N, KB, chunk_b, x, Wq, Ws, ep, stream);
        case 4: return launch_mns<M, NB, 4>(N, KB, chunk_b, x, Wq, Ws, ep, stream);
        case 8: return launch_mns<M, NB, 8>(N, KB, chunk_b, x, Wq, Ws, ep, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int M>
hipError_t launch_m(int NB, int S, int N, int KB, int chunk_b, const void* x, const void* Wq,
                    const uint8_t* Ws, const Epilogue& ep, hipStream_t stream) {
    // x registers: 16 * M * NB VGPRs, kept at 64 (128 from M = 5)
    if (NB == 4) {
        if constexpr (M == 1) return launch_mn<M, 4>(S, N, KB, chunk_b, x, Wq, Ws, ep, stream);
    } else if (NB == 2) {
        if constexpr (M <= 2) return launch_mn<M, 2>(S, N, KB, chunk_b, x, Wq, Ws, ep, stream);
    } else if (NB == 1) {
        return launch_mn<M, 1>(S, N, KB, chunk_b, x, Wq, Ws, ep, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mxfp4_split(int M, int K, int* nb, int* splits) {
    const int KB = K / kBlockElems;
    const int nb_max = M == 1 ? 4 : (M == 2 ? 2 : 1);
    int NB = 1;
    while (NB < nb_max && NB * kWave < KB) NB *= 2;
    int S = 1;
    while (S * NB * kWave < KB) S *= 2;
    *nb = NB;
    *splits = S;
    return S <= kMxfp4MaxSplit;
}

hipError_t launch_mxfp4(int M, int N, int K, const void* x, const void* Wq, const uint8_t* Ws,
                        const Epilogue& ep, hipStream_t stream) {
    const int KB = K / kBlockElems;
    int NB, S;
    if (!mxfp4_split(M, K, &NB, &S)) return hipErrorInvalidValue;
    const int chunk_b = NB * kWave;  // blocks per wave: lanes x blocks per lane
    switch (M) {
#define SG_CASE(m) \
    case m: return launch_m<m>(NB, S, N, KB, chunk_b, x, Wq, Ws, ep, stream);
        SG_CASE(1) SG_CASE(2) SG_CASE(3) SG_CASE(4) SG_CASE(5) SG_CASE(6) SG_CASE(7) SG_CASE(8)
#undef SG_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sg
