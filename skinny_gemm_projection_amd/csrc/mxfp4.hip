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
// one v_cvt_scalef32_pk_bf16_fp4 at unit scale (every e2m1 value is exact in
// bf16), the pair meets the matching x pair in one v_dot2c_f32_bf16 per
// activation row, and the block's fp32 sum is then multiplied by its scale
// 2^(s-127) in one fma into the row's total.  Scaling the sum rather than
// the converted weights keeps every valid scale code exact: the weights of
// codes 0..1 would be subnormal and those of codes 253..254 could overflow
// bf16, while a power-of-two product of an fp32 sum is exact down to fp32's
// subnormals.  The scale code 255 (NaN) becomes a NaN factor, so the row's
// total is NaN.
//
// Rows are grouped R per iteration, their R*M lane partials reduced
// together by the reduce-scatter of the bf16 kernel; S waves of a workgroup
// split K and add their partials in LDS in ascending chunk order.
//
// From 9 rows of batch the VALU dots (16*M per block and row) outgrow the
// weight stream, and a matrix-core kernel takes over (up to 16 rows of x,
// one MFMA m-tile).  Lane (col, grp) of a wave on a 16-row tile loads block
// grp of a 128-element window of row col (16 bytes) and its scale byte.  Four
// lane-row swaps (permlane32 then permlane16) transpose the 4 x 4 dwords of
// the four lane groups of a column, so that for step t every lane of column
// col holds 8 codes of the same block 4w + t: one v_mfma_f32_16x16x32_bf16
// step is then exactly one scale block, converted at unit scale straight into
// B operand layout.  Its 16x16 result is multiplied by the block scale of
// each column and added to the accumulator in fp32 (one fma per output), the
// same exact scaling as the vector kernel; two more swaps gather the four
// scale bytes of a column into each of its lanes.  The matching A operand is
// x[m][window + 32*t + 8*grp ..+8).  x of each window is loaded as 4 rows x
// 256 bytes per instruction into a swizzled per-wave LDS tile and read back
// in operand layout (reading the operands straight from L2, 16 rows x 64
// bytes per instruction, was 10-25% slower).  S waves of a workgroup split K
// over the tile (8 windows in flight each) and add their 16x16 tiles in LDS
// in ascending order.  Every workgroup still reads all of x from L2 -- at 16
// rows four x bytes per code byte -- and that traffic, not HBM, bounds the
// kernel; through M = 8 the VALU kernel is as fast or faster.
#include "launch.h"

namespace sg {

namespace {

constexpr int kBlockElems = 32;  // elements per scale block = per 16-byte code load

// e8m0 scale code -> its fp32 value 2^(s-127): the code is the exponent
// field for 1 <= s <= 254, s = 0 is the fp32 subnormal 2^-127 and s = 255
// is NaN.
__device__ __forceinline__ float e8m0_value(uint32_t s) {
    return as_f(s == 0u ? 0x00400000u : s == 255u ? 0x7FC00000u : s << 23);
}

// The fp32 sum of the 32 products of one block at unit scale: x pairs (16
// dwords, xb[d] component j holds elements 8d+2j, 8d+2j+1) against the 32
// codes of w (dword d, byte j holds the same two elements).
__device__ __forceinline__ float dot_block(const uint4 (&xb)[4], const uint4 w) {
    constexpr float kUnit = 1.0f;  // exponent field 127: scale 2^0
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t xd[4] = {xb[d].x, xb[d].y, xb[d].z, xb[d].w};
        const bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], kUnit, 0);
        const bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], kUnit, 1);
        const bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], kUnit, 2);
        const bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], kUnit, 3);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[0]), w0, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[1]), w1, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[2]), w2, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[3]), w3, acc, false);
    }
    return acc;
}

constexpr int pad4(int v) { return (v + 3) / 4 * 4; }
constexpr int team_waves(int S) { return S > kWavesPerBlock ? S : kWavesPerBlock; }

// Rows whose M partials one lane reduce-scatter finishes (at most 64 values).
constexpr int reduce_rows(int M, int R) {
    int rb = 1;
    while (rb * 2 <= R && rb * 2 * M <= 64) rb *= 2;
    return rb;
}

template <int M, int NB, int R, int S>
__global__ __launch_bounds__(kWave * team_waves(S)) void mxfp4_rowdot_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ Wq, const uint8_t* __restrict__ Ws,
    int N, int KB, int chunk_b, int iters, Epilogue ep) {
    constexpr int kWaves = team_waves(S);
    constexpr int kTeams = kWaves / S;
    constexpr int RB = reduce_rows(M, R);  // rows per reduce-scatter
    static_assert(R % RB == 0, "whole reduction batches");
    constexpr int V = pad4(RB * M);
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
        // all R rows' codes and scales are requested with the first batch; the
        // dots of each batch of RB rows are formed right before its reduction
        uint4 wr[R][NB];
        uint32_t sc[R][NB];
#pragma unroll
        for (int q = 0; q < R / RB; ++q) {  // batches of RB rows
            float part[V];
#pragma unroll
            for (int v = 0; v < V; ++v) part[v] = 0.0f;
            if (g < groups) {
                if (q == 0) {
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
                    // At 2 to 4 rows of x every row's loads leave before the
                    // first dot: left to itself the scheduler issued the
                    // later rows' loads between the earlier rows' dots,
                    // behind their waits.  Interleaved A/B on MI355X:
                    // 8192 x 7168 M = 2 9.60 -> 9.05 us, 4096 x 7168 M = 2 /
                    // 4 6.13 / 7.65 -> 5.94 / 7.37 us; at M = 1 mixed
                    // (-0.27 to +0.34 us over five shapes), at M = 8 slower
                    // (8192 x 7168 18.43 -> 18.92 us).
                    if constexpr (M >= 2 && M <= 4) __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const int r = q * RB + i;
                    float scale[NB];
#pragma unroll
                    for (int c = 0; c < NB; ++c) scale[c] = e8m0_value(sc[r][c]);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        float a = 0.0f;
#pragma unroll
                        for (int c = 0; c < NB; ++c)
                            a = __builtin_fmaf(dot_block(xr[m][c], wr[r][c]), scale[c], a);
                        part[i * M + m] = a;
                    }
                }
            }
            const float total = reduce_scatter<V>(part, lane);
            const int v = scatter_index<V>(lane);
            const bool mine = v >= 0 && v < RB * M;
            const int r = mine ? q * RB + v / M : 0;
            const int m = mine ? v % M : 0;
            const int n = n0 + r;
            const bool live = mine && g < groups && n < N;
            if (S == 1) {
                if (live) store_final(ep, (int64_t)m * N + n, total);
            } else {
                const int buf = (it * (R / RB) + q) & 1;
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
}

// Matrix-core kernel: one workgroup of S waves per NT 16-row tiles of W;
// wave s takes windows [s*chunk_w, (s+1)*chunk_w) of 128 elements (4
// blocks), D of them in flight at a time.  With NT = 2 each x operand read
// serves two row tiles, halving the x bytes per code byte.  Two windows in
// flight: interleaved A/B on MI355X against 8 (and 4), K = 7168: N = 4096
// M = 9 / 12 / 16 11.44 / 11.98 / 12.65 -> 11.18 / 11.55 / 12.07 us (4:
// 11.44 / 11.88 / 12.41), N = 2048 M = 16 12.02 -> 11.41 us, N = 5888
// M = 12 21.51 -> 19.27 us (4: 18.89).
constexpr int kMfmaWindows = 2;

template <int NT, int S>
__global__ __launch_bounds__(kWave * S) void mxfp4_mfma_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ Wq, const uint8_t* __restrict__ Ws,
    int M, int N, int KB, int chunk_w, Epilogue ep) {
    constexpr int D = kMfmaWindows;
    __shared__ f32x4_t red[S > 1 ? S : 1][NT][kWave];
    __shared__ uint4 xtiles[S][256];  // per wave: x of one window, 16 rows x 16 pieces

    const int lane = threadIdx.x & (kWave - 1);
    const int col = lane & 15, grp = lane >> 4;
    const int s = wave_id_in_block();
    const int n0 = blockIdx.x * 16 * NT;
    const int rows = min(16 * NT, N - n0);
    const int K8 = KB * 4;  // 16-byte pieces of an x row
    const int KW = (KB + 3) / 4;
    const int w0 = s * chunk_w;
    const int w1 = min(KW, w0 + chunk_w);

    // wave-uniform descriptors over the tiles' codes and scales and over x:
    // rows past N and x rows past M read zero
    const rsrc_t rw = make_rsrc(Wq + (int64_t)n0 * KB, (uint32_t)rows * KB * 16u);
    const rsrc_t rs = make_rsrc(Ws + (int64_t)n0 * KB, (uint32_t)rows * KB);
    const rsrc_t rx = make_rsrc(x, (uint32_t)M * K8 * 16u);
    constexpr uint32_t kOut = 0xFFFFFFF0u;  // past any range: reads zero

    // x of a window goes through the wave's LDS tile: load i reads row
    // 4i + grp, piece col ^ (4i + grp) of the window (4 rows x 256 bytes per
    // instruction), into slot col of that row; the A operand of step t,
    // piece 4t + grp of row col, is read back from slot (4t + grp) ^ col.
    uint4* xt = xtiles[s];
    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int wb = w0; wb < w1; wb += D) {
        uint4 wv[D][NT], xa[D][4];
        uint32_t sc[D][NT];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int w = wb + d;
            const int b = 4 * w + grp;  // this lane's block of its rows
            const bool ok = w < w1 && b < KB;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const uint32_t blk = (uint32_t)((16 * nt + col) * KB + b);
                wv[d][nt] = load16<kStream>(rw, ok ? blk * 16u : kOut);
                sc[d][nt] = __builtin_amdgcn_raw_buffer_load_b8(rs, ok ? blk : kOut, 0, kStream);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * i + grp;
                const int piece = 16 * w + (col ^ r);  // of the x row
                const bool xok = w < w1 && piece < K8;
                xa[d][i] = load16<kCached>(rx, xok ? (uint32_t)(r * K8 + piece) * 16u : kOut);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xt[(4 * i + grp) * 16 + col] = xa[d][i];
            __builtin_amdgcn_wave_barrier();
            uint32_t wd[NT][4];
            float scale[NT][4];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                // lane (col, grp) holds dword t of block grp (T[grp][t]); after
                // the swaps wd[t] holds T[t][grp]: dword grp of block t
                const auto p02 = __builtin_amdgcn_permlane32_swap(wv[d][nt].x, wv[d][nt].z, false, false);
                const auto p13 = __builtin_amdgcn_permlane32_swap(wv[d][nt].y, wv[d][nt].w, false, false);
                const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
                const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
                wd[nt][0] = q01[0];
                wd[nt][1] = q01[1];
                wd[nt][2] = q23[0];
                wd[nt][3] = q23[1];
                // byte t of `all` = the scale code of block t of row col
                const uint32_t mine = sc[d][nt] << (8 * grp);
                const auto g16 = __builtin_amdgcn_permlane16_swap(mine, mine, false, false);
                const uint32_t pair = g16[0] | g16[1];  // rows 0,1: bytes 0,1; rows 2,3: bytes 2,3
                const auto g32 = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
                const uint32_t all = g32[0] | g32[1];
#pragma unroll
                for (int t = 0; t < 4; ++t) scale[nt][t] = e8m0_value((all >> (8 * t)) & 0xFFu);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 a = xt[col * 16 + ((4 * t + grp) ^ col)];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    constexpr float kUnit = 1.0f;  // convert at scale 2^0
                    const uint4 b = {
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 0)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 2)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 3))};
                    const f32x4_t blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                        f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[nt][v] = __builtin_fmaf(blk[v], scale[nt][t], acc[nt][v]);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    if (S > 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[s][nt][lane] = acc[nt];
        __syncthreads();
        if (s != 0) return;
#pragma unroll
        for (int j = 1; j < S; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] += red[j][nt][lane];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * nt + col;
        if (r >= rows) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * grp + v;
            if (m < M) store_final(ep, (int64_t)m * N + n0 + r, acc[nt][v]);
        }
    }
}

// Row tiles per wave for the matrix-core kernel: two once the 32-row tiles
// alone give every CU a workgroup (as in the FP8 matrix-core kernel).
constexpr int kCus = 256;  // compute units
int mxfp4_mfma_nt(int N) { return (N + 31) / 32 >= kCus ? 2 : 1; }

constexpr int kResidentWaves = 2048;  // 256 CUs x 8 waves

// Rows per wave iteration (R * NB KB of codes in flight per wave): 8, and at
// M = 1 4 where the 8-row groups would leave resident teams without one, so
// that a short matrix still fills the GPU.  Measured on MI355X with full
// occupancy (K = 7168 and 8192): 8 rows at every M (4 and 16 were slower;
// 16 rows at M >= 7 also halve the resident waves).  The 4-row rule at M = 1
// (interleaved A/B): 2048 x 7168 4.77 -> 3.99 us, 4096 x 7168 5.40 -> 5.13
// us, 6144 x 7168 6.75 -> 6.65 us, 4096 x 4096 4.78 -> 3.98 us, 1024 x 1024
// 3.30 -> 2.78 us; at M = 2 mixed (2048 x 7168 5.26 -> 4.61, 4096 x 7168
// 5.97 -> 6.26 us), at M = 4, 8 slower (2048 x 7168 5.35 -> 5.69, 7.28 ->
// 7.93 us).
constexpr int kMxfp4Rows = 8;
constexpr int kMxfp4RowsShort = 4;

template <int M, int NB, int S, int kRows>
hipError_t launch_mnsr(int N, int KB, int chunk_b, const void* x, const void* Wq,
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

template <int M, int NB, int S>
hipError_t launch_mns(int N, int KB, int chunk_b, const void* x, const void* Wq,
                      const uint8_t* Ws, const Epilogue& ep, hipStream_t stream) {
    if constexpr (M == 1) {
        const int cap = kResidentWaves / S;  // resident teams
        if ((N + kMxfp4Rows - 1) / kMxfp4Rows < cap)
            return launch_mnsr<M, NB, S, kMxfp4RowsShort>(N, KB, chunk_b, x, Wq, Ws, ep, stream);
    }
    return launch_mnsr<M, NB, S, kMxfp4Rows>(N, KB, chunk_b, x, Wq, Ws, ep, stream);
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
    if (NB == 2) {
        if constexpr (M <= 2) return launch_mn<M, 2>(S, N, KB, chunk_b, x, Wq, Ws, ep, stream);
    } else if (NB == 1) {
        return launch_mn<M, 1>(S, N, KB, chunk_b, x, Wq, Ws, ep, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

void mxfp4_mfma_split(int N, int K, int* splits, int* chunk_w) {
    const int KW = (K / kBlockElems + 3) / 4;
    const int rows = 16 * mxfp4_mfma_nt(N);
    const int tiles = (N + rows - 1) / rows;
    int S = 1;
    while (S < 8 && S < KW && tiles * S < kResidentWaves) S *= 2;
    *splits = S;
    *chunk_w = KW > 0 ? (KW + S - 1) / S : 0;
}

bool mxfp4_split(int M, int K, int* nb, int* splits) {
    if (M >= kMxfp4MfmaFromM) {  // matrix-core kernel: any K (team split of windows)
        *nb = 0;
        *splits = 0;
        return true;
    }
    const int KB = K / kBlockElems;
    // Blocks per lane: at most 2 for one or two rows of x, so one row's K is
    // split over two waves of a team (2048 waves instead of 1024 at N = 8192).
    // Measured on MI355X at M = 1 against 4 blocks a lane (K whole per wave):
    // 8192x7168 7.65 -> 7.30 us, 4096x7168 6.41 -> 5.19 us, 7168x8192
    // 7.64 -> 7.44 us.  At M = 2, one block a lane was slower (8.7 -> 9.2 us).
    const int nb_max = M <= 2 ? 2 : 1;
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
    if (M >= kMxfp4MfmaFromM) {
        int S, chunk_w;
        mxfp4_mfma_split(N, K, &S, &chunk_w);
        const int NT = mxfp4_mfma_nt(N);
        const int grid = (N + 16 * NT - 1) / (16 * NT);
        const uint4* xp = static_cast<const uint4*>(x);
        const uint4* wp = static_cast<const uint4*>(Wq);
#define SG_S(nt, v) \
    if (NT == nt && S == v) { \
        mxfp4_mfma_kernel<nt, v><<<grid, kWave * v, 0, stream>>>(xp, wp, Ws, M, N, KB, chunk_w, \
                                                                ep); \
        return hipGetLastError(); \
    }
        SG_S(1, 1) SG_S(1, 2) SG_S(1, 4) SG_S(1, 8) SG_S(2, 1) SG_S(2, 2) SG_S(2, 4) SG_S(2, 8)
#undef SG_S
        return hipErrorInvalidValue;
    }
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
