// fp8.hip -- projection with 8-bit float (e4m3) weights and one fp32 scale per
// 128 x 128 block of W, on gfx950.
//
// Small-batch decode streams every weight once, so fewer weight bytes is time
// saved ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Experimental setup
// and Supplementary details: the later evaluation model ships low-precision
// weights).  8-bit weights halve the bf16 stream.  The format read here is the
// block-scaled FP8 of DeepSeek-V3-style checkpoints (a reading; the pages name
// only a 4-bit format): OCP E4M3 codes, W [N, K] one byte each, and scales
// [ceil(N/128), ceil(K/128)] fp32, w[n,k] = e4m3(code) * scale[n/128][k/128].
//
// Mapping (the bf16 row-streaming kernel's, with 16 codes a lane).  A wave
// owns one K chunk of R rows: lane l loads the 16-byte units c*64 + l of the
// chunk of each row (1 KB of one row per load instruction, non-temporal, ragged
// tails read zero through the buffer bounds).  Each wave keeps the 16
// activations of each of its units in registers: at M <= 2 x is staged once
// per workgroup in LDS and read from there; from M = 3 (K split over teams of
// waves) each wave loads its chunk of x straight from L2, which measured
// faster (4096 x 7168, M = 4: 9.7 -> 9.0 us; at M = 2 the LDS staging was
// faster, 12.5 against 13.1 us at 8192 x 7168).  The first row group's codes
// are requested right behind x (at M = 1 this measured 11.3 -> 10.8 us at
// 8192 x 7168, once the LDS copy of x stopped waiting for the codes), and
// teams of 4 or 8 waves request each next group before their reduction.  A
// unit's codes become bf16 pairs with v_cvt_scalef32_pk_bf16_fp8
// (scale 1: exact, every e4m3 value is a bf16 value) and meet their x pairs in
// v_dot2; the unit's sum is multiplied by its block scale (a unit of 16 codes
// never straddles a 128-column block) and accumulated in fp32.  R divides 128
// and groups start at multiples of R, so the R rows of a group share their
// row block of scales.  The R*M lane sums are reduced by the lane
// reduce-scatter; a team of S waves (one K chunk each) adds its partials in
// LDS in ascending chunk order, and the first wave runs the epilogue.
#include <type_traits>

#include "launch.h"

namespace sg {

namespace {

constexpr int kUnitCodes = 16;  // e4m3 codes per 16-byte lane load
// Rows per wave iteration (divides 128).  At one row of x, two: half the
// codes in flight per wave at once (with four, every wave requests its whole
// share of the matrix at the start).  Interleaved A/B on MI355X against
// four: 8192 x 7168 10.94 -> 10.78 us, 4096 x 7168 6.72 -> 6.56 us, 18432 x
// 7168 22.19 -> 21.38 us, 2048 x 7168 5.33 -> 4.41 us; one row was mixed
// (7168 x 8192 11.01 -> 10.74, 4096 x 7168 6.56 -> 6.69 us).  At M = 2
// equal, at M = 3, 4 slower (4096 x 7168 8.05 / 8.78 -> 8.42 / 9.01 us).
constexpr int fp8_rows(int M) { return M == 1 ? 2 : 4; }

constexpr int pad4(int v) { return (v + 3) / 4 * 4; }
constexpr int team_block_waves(int S) { return S > kWavesPerBlock ? S : kWavesPerBlock; }
// x of the batch staged in LDS (M <= 2) or loaded by each wave from L2
constexpr bool fp8_x_in_lds(int M) { return M <= 2; }

// Sum of one 16-code unit times its 16 activations (two 16-byte pieces of x):
// dword d of the codes holds elements 4d..4d+3, low byte first; x dword j
// holds elements 2j, 2j+1.
__device__ __forceinline__ float dot_unit(const uint4 w, const uint4 xa, const uint4 xb) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const uint32_t xd[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[d], 1.0f, false);
        const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[d], 1.0f, true);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[2 * d]), lo, acc,
                                              false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xd[2 * d + 1]), hi,
                                              acc, false);
    }
    return acc;
}

// x staging loads per thread of the vector kernel (x [M, 2*K16] pieces over
// the workgroup; LDS holds this many rounds of the workgroup's threads).
constexpr int fp8_stage_loads(int M, int NCH, int S) {
    return (2 * M * NCH * S + team_block_waves(S) - 1) / team_block_waves(S);
}

template <int M, int NCH, int S>
__global__ __launch_bounds__(kWave * team_block_waves(S)) void fp8_rowdot_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ Wq, const float* __restrict__ Ws,
    int N, int K16, int KB, int chunk16, int iters, Epilogue ep) {
    constexpr int R = fp8_rows(M);
    constexpr int kWaves = team_block_waves(S);
    constexpr int kTeams = kWaves / S;
    constexpr int V = pad4(R * M);
    __shared__ float red[2][kTeams][S][V];
    extern __shared__ uint4 xs[];  // x [M, 2*K16]: 16-byte pieces of 8 bf16

    const int lane = threadIdx.x & (kWave - 1);
    const int wib = wave_id_in_block();
    const int team_in_block = wib / S;
    const int member = wib % S;
    const int team = blockIdx.x * kTeams + team_in_block;
    const int teams = gridDim.x * kTeams;
    const int u0 = member * chunk16;                 // first unit of this wave's chunk
    const int len = max(0, min(K16 - u0, chunk16));  // units in the chunk
    const int K8 = 2 * K16;                          // x pieces per row

    const int groups = (N + R - 1) / R;
    uint4 wr[R][NCH];
    float sc[NCH];
    // codes and scales of the group of R rows starting at row g * R
    auto load_group = [&](int g) {
        const int n0 = g * R;
        // the group's rows share one 128-row block of scales (a group past
        // the end reads the last block; its sums are never stored)
        // Chunks start on 128-column blocks (u0 is a multiple of 8 units), so
        // the chunk's scales are the ceil(len / 8) words from u0 / 8; lanes
        // past them read zero, and lanes past len inside the last block read
        // its scale for codes that read zero.
        const rsrc_t rsc = make_rsrc(Ws + (int64_t)(min(n0, N - 1) / 128) * KB + u0 / 8,
                                     (uint32_t)((len + 7) / 8) * 4u);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int u = c * kWave + lane;  // 8 units = 128 columns
            sc[c] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rsc, (uint32_t)(u / 8) * 4u, 0, kCached));
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = n0 + r;
            const rsrc_t rs = make_rsrc(Wq + (int64_t)min(n, N - 1) * K16 + u0,
                                        n < N ? (uint32_t)len * 16u : 0u);
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                wr[r][c] = load16<kStream>(rs, (uint32_t)(c * kWave + lane) * 16u);
        }
    };

    uint4 xr[M][NCH][2];
    auto read_x_lds = [&]() {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int u = c * kWave + lane;
                const bool in = u < len;
                xr[m][c][0] = in ? xs[m * K8 + 2 * (u0 + u)] : make_uint4(0, 0, 0, 0);
                xr[m][c][1] = in ? xs[m * K8 + 2 * (u0 + u) + 1] : make_uint4(0, 0, 0, 0);
            }
    };
    if constexpr (fp8_x_in_lds(M)) {
        // x into registers first, then the first group's codes behind it:
        // loads return in order, so the LDS copy waits for x only.  The copy
        // is unconditional (the LDS buffer holds every staged slot): copied
        // under a bounds test, an x load was moved into that branch, behind
        // the code loads, and the barrier then waited for all of them.
        constexpr int kThreads = kWave * kWaves;
        constexpr int kStage = fp8_stage_loads(M, NCH, S);  // >= M*K8 / kThreads
        const int total = M * K8;
        const rsrc_t rx = make_rsrc(x, (uint32_t)total * 16u);
        uint4 stage[kStage];
#pragma unroll
        for (int j = 0; j < kStage; ++j)
            stage[j] = load16<kCached>(rx, (uint32_t)(threadIdx.x + j * kThreads) * 16u);
        load_group(team);
#pragma unroll
        for (int j = 0; j < kStage; ++j) xs[threadIdx.x + j * kThreads] = stage[j];
        __syncthreads();
        read_x_lds();
    } else {
        // the 32 bytes of x of each of the lane's units, zero past the chunk
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const rsrc_t rx = make_rsrc(x + (int64_t)m * K8 + 2 * u0, (uint32_t)len * 32u);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const uint32_t off = (uint32_t)(c * kWave + lane) * 32u;
                xr[m][c][0] = load16<kCached>(rx, off);
                xr[m][c][1] = load16<kCached>(rx, off + 16u);
            }
        }
        load_group(team);
    }

    // One iteration over the group whose codes are in wr / sc: the dot
    // products, then (if `next`) the next group's codes requested, then the
    // reduction and the stores, which the new loads overlap.  A group past
    // the end reads zero through the buffer bounds and stores nothing; no
    // load sits behind a branch.  The codes of the first group are requested
    // behind x, above.
    auto iteration = [&](int it, auto next) {
        const int g = team + it * teams;
        const int n0 = g * R;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float a = 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    a = fmaf(dot_unit(wr[r][c], xr[m][c][0], xr[m][c][1]), sc[c], a);
                acc[r * M + m] = a;
            }
        if constexpr (decltype(next)::value) {
            // kept behind the dot products: hoisted above them, the loads
            // would need a second set of code registers
            __builtin_amdgcn_sched_barrier(0);
            load_group(g + teams);
        }
        const float tot = reduce_scatter<V>(acc, lane);
        const int v = scatter_index<V>(lane);
        const bool mine = v >= 0 && v < R * M;
        const int r = mine ? v / M : 0;
        const int m = mine ? v - r * M : 0;
        const int n = n0 + r;
        const bool live = mine && g < groups && n < N;
        if (S == 1) {
            if (live) store_final(ep, (int64_t)m * N + n, tot);
        } else {
            // the S chunk partials added in ascending chunk order
            const int buf = it & 1;
            if (mine) red[buf][team_in_block][member][v] = tot;
            __syncthreads();
            if (member == 0 && live) {
                float sum = red[buf][team_in_block][0][v];
#pragma unroll
                for (int s = 1; s < S; ++s) sum += red[buf][team_in_block][s][v];
                store_final(ep, (int64_t)m * N + n, sum);
            }
        }
    };
    if constexpr (S >= 4) {
        // The last iteration is peeled off the loop: with the loads it
        // consumes issued either before the loop or in its last trip, each
        // row's dot products still wait for that row's codes only.  (Separate
        // straight-line paths for one and two iterations cost the M = 1 kernel
        // 140 registers.)  8192 x 7168, M = 3: 13.5 -> 12.3 us.
        for (int it = 0; it < iters - 1; ++it) iteration(it, std::true_type{});
        iteration(iters - 1, std::false_type{});
    } else {
        // A lone wave or a pair: each iteration requests its own codes at the
        // top.  The early request measured slower for a lone wave (18432 x
        // 7168, M = 1: 23.1 against 22.1 us) and no faster for a pair (7168 x
        // 8192, M = 2: 12.4 / 12.6 us).  The first iteration is peeled, its
        // codes requested with x.
        iteration(0, std::false_type{});
        for (int it = 1; it < iters; ++it) {
            load_group(team + it * teams);
            iteration(it, std::false_type{});
        }
    }
}

// Matrix-core kernel (kFp8MfmaFromM <= M <= 16: x is one 16-row A tile of
// v_mfma_f32_16x16x32_bf16, rows past M zero).  A workgroup of S waves owns
// NT 16-row tiles of W; wave s takes the 128-column windows [s*chunk_w,
// (s+1)*chunk_w), D of them in flight.  Lane (col, grp) loads the 32 codes
// k = 128w + 32grp .. +32 of row n0 + 16nt + col (two 16-byte loads per row
// tile); k step t of the window takes codes 8t .. 8t+7 of them, converted to
// bf16 (exact) as the B operand, against x[m][128w + 32grp + 8t .. +8) as the
// A operand, so A and B agree on the k of every operand slot.  x of a window
// goes through the wave's LDS tile (4 rows x 256 bytes per load instruction,
// the piece index XOR-swizzled by row so the operand reads hit 16 different
// bank groups); with NT = 2 each A operand read serves two row tiles, halving
// the x traffic per code byte.  A window lies inside one 128 x 128 scale
// block (16 NT divides 128, so the tiles' rows share a row block): its 4
// products are summed first and the sum is multiplied by that one scale.
// The S partial tiles are added in LDS in ascending wave order.
constexpr int kF8Windows = 4;  // windows in flight per wave

template <int NT, int S>
__global__ __launch_bounds__(kWave * S) void fp8_mfma_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ Wq, const float* __restrict__ Ws,
    int M, int N, int K16, int KB, int chunk_w, Epilogue ep) {
    constexpr int D = kF8Windows;
    __shared__ f32x4_t red[S > 1 ? S : 1][NT][kWave];
    __shared__ uint4 xtiles[S][256];  // per wave: x of one window, 16 rows x 16 pieces

    const int lane = threadIdx.x & (kWave - 1);
    const int col = lane & 15, grp = lane >> 4;
    const int s = wave_id_in_block();
    const int n0 = blockIdx.x * 16 * NT;
    const int rows = min(16 * NT, N - n0);
    const int K8 = 2 * K16;        // 16-byte pieces of an x row
    const int KW = (K16 + 7) / 8;  // 128-column windows (8 units of 16 codes)
    const int w0 = s * chunk_w;
    const int w1 = min(KW, w0 + chunk_w);

    // wave-uniform descriptors: codes of the tiles' rows (rows past N read
    // zero), and x (rows past M read zero)
    const rsrc_t rw = make_rsrc(Wq + (int64_t)n0 * K16, (uint32_t)rows * K16 * 16u);
    const rsrc_t rx = make_rsrc(x, (uint32_t)M * K8 * 16u);
    const float* __restrict__ srow = Ws + (int64_t)(n0 / 128) * KB;
    constexpr uint32_t kOut = 0xFFFFFFF0u;  // past any range: reads zero

    uint4* xt = xtiles[s];
    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int wb = w0; wb < w1; wb += D) {
        uint4 wv[D][NT][2], xa[D][4];
        float sc[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int w = wb + d;
            const bool live = w < w1;
            const int u = 8 * w + 2 * grp;  // first unit of this lane in its rows
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const bool ok = live && u + j < K16;
                    const uint32_t off = (uint32_t)((16 * nt + col) * K16 + u + j) * 16u;
                    wv[d][nt][j] = load16<kStream>(rw, ok ? off : kOut);
                }
            sc[d] = live ? srow[w] : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * i + grp;
                const int piece = 16 * w + (col ^ r);  // of the x row
                const bool ok = live && piece < K8;
                xa[d][i] = load16<kCached>(rx, ok ? (uint32_t)(r * K8 + piece) * 16u : kOut);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xt[(4 * i + grp) * 16 + col] = xa[d][i];
            __builtin_amdgcn_wave_barrier();
            f32x4_t part[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) part[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 a = xt[col * 16 + ((4 * grp + t) ^ col)];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    // codes 8t .. 8t+7: dwords 2t, 2t+1 of the lane's 32, low byte first
                    const uint4 q = wv[d][nt][t / 2];
                    const uint32_t lo = (t & 1) ? q.z : q.x;
                    const uint32_t hi = (t & 1) ? q.w : q.y;
                    const uint4 b = {
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
                    part[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), part[nt],
                        0, 0, 0);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[nt][v] = fmaf(part[nt][v], sc[d], acc[nt][v]);
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

// Row tiles per wave: two once the 32-row tiles alone give every CU a
// workgroup (measured at K = 7168: 8192 rows M = 8 18.5 -> 16.7 us, M = 16
// 20.9 -> 17.7 us; at 4096 rows the 128 workgroups left half the CUs idle,
// M = 8 10.8 -> 20.1 us).
constexpr int kCus = 256;  // compute units
int fp8_mfma_nt(int N) { return (N + 31) / 32 >= kCus ? 2 : 1; }

// Lane loads per row (x registers: 8*M*NCH VGPRs) allowed at batch size M.
constexpr int fp8_nch_cap(int M) { return M == 1 ? 8 : (M == 2 ? 4 : 2); }

constexpr int kResident = 2048;  // 256 CUs x 8 waves

template <int M, int NCH, int S>
hipError_t launch_mns(int N, int K16, int chunk16, const void* x, const void* Wq,
                      const float* Ws, const Epilogue& ep, hipStream_t stream) {
    constexpr int kTeams = team_block_waves(S) / S;
    const int groups = (N + fp8_rows(M) - 1) / fp8_rows(M);
    const int cap = kResident / S;
    int teams = groups < cap ? groups : cap;
    const int its = (groups + teams - 1) / teams;
    teams = (groups + its - 1) / its;  // every team the same number of row groups
    const int grid = (teams + kTeams - 1) / kTeams;
    const int iters = (groups + grid * kTeams - 1) / (grid * kTeams);
    const int KB = (K16 * kUnitCodes + 127) / 128;
    // the staged x and its padding to whole staging rounds
    const size_t lds =
        fp8_x_in_lds(M) ? (size_t)fp8_stage_loads(M, NCH, S) * kWave * team_block_waves(S) * 16
                        : 0;
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fp8_rowdot_kernel<M, NCH, S>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    fp8_rowdot_kernel<M, NCH, S><<<grid, kWave * team_block_waves(S), lds, stream>>>(
        static_cast<const uint4*>(x), static_cast<const uint4*>(Wq), Ws, N, K16, KB, chunk16,
        iters, ep);
    return hipGetLastError();
}

template <int M, int NCH>
hipError_t launch_mn(int S, int N, int K16, int chunk16, const void* x, const void* Wq,
                     const float* Ws, const Epilogue& ep, hipStream_t stream) {
    switch (S) {
        case 1: return launch_mns<M, NCH, 1>(N, K16, chunk16, x, Wq, Ws, ep, stream);
        case 2: return launch_mns<M, NCH, 2>(N, K16, chunk16, x, Wq, Ws, ep, stream);
        case 4: return launch_mns<M, NCH, 4>(N, K16, chunk16, x, Wq, Ws, ep, stream);
        case 8: return launch_mns<M, NCH, 8>(N, K16, chunk16, x, Wq, Ws, ep, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int M>
hipError_t launch_m(int nch, int S, int N, int K16, int chunk16, const void* x, const void* Wq,
                    const float* Ws, const Epilogue& ep, hipStream_t stream) {
    switch (nch) {
        case 1: return launch_mn<M, 1>(S, N, K16, chunk16, x, Wq, Ws, ep, stream);
        case 2:
            if constexpr (fp8_nch_cap(M) >= 2)
                return launch_mn<M, 2>(S, N, K16, chunk16, x, Wq, Ws, ep, stream);
            break;
        case 4:
            if constexpr (fp8_nch_cap(M) >= 4)
                return launch_mn<M, 4>(S, N, K16, chunk16, x, Wq, Ws, ep, stream);
            break;
        case 8:
            if constexpr (fp8_nch_cap(M) >= 8)
                return launch_mn<M, 8>(S, N, K16, chunk16, x, Wq, Ws, ep, stream);
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

}  // namespace

void fp8_mfma_split(int N, int K, int* splits, int* chunk_w) {
    const int KW = (K / kUnitCodes + 7) / 8;
    const int rows = 16 * fp8_mfma_nt(N);
    const int tiles = (N + rows - 1) / rows;
    int S = 1;
    while (S < 8 && S < KW && tiles * S < kResident) S *= 2;
    *splits = S;
    *chunk_w = KW > 0 ? (KW + S - 1) / S : 0;
}

bool fp8_size_ok(int M, int K) {
    if (M < 1 || M > kFp8MaxM || K < 0) return false;
    if (M >= kFp8MfmaFromM) return true;  // matrix-core kernel: windows split over a team
    // x in registers: a team of at most 8 waves, NCH units of 16 codes per lane
    return fp8_x_in_lds(M) ? (int64_t)M * K <= kFp8MaxMK
                           : K <= 8 * kWave * kUnitCodes * fp8_nch_cap(M);
}

bool fp8_split(int M, int N, int K, int* splits, int* chunk16, int* nch) {
    if (!fp8_size_ok(M, K) || K % kUnitCodes != 0) return false;
    if (M >= kFp8MfmaFromM) {  // matrix-core kernel: windows of 8 units, nch unused
        int chunk_w;
        fp8_mfma_split(N, K, splits, &chunk_w);
        *chunk16 = 8 * chunk_w;
        *nch = 0;
        return true;
    }
    const int K16 = K / kUnitCodes;
    // The smallest split whose chunks fit the lane loads and leave no wave
    // without a chunk (within the size limits above one always exists).
    for (int S = 1; S <= 8; S *= 2) {
        // chunks of whole 128-byte lines (8 units)
        const int c16 = (K16 + 8 * S - 1) / (8 * S) * 8;
        const int n = next_pow2((c16 + kWave - 1) / kWave);
        if (n <= fp8_nch_cap(M) && (S == 1 || (int64_t)(S - 1) * c16 < K16)) {
            *splits = S;
            *chunk16 = c16;
            *nch = n < 1 ? 1 : n;
            return true;
        }
    }
    return false;
}

hipError_t launch_fp8(int M, int N, int K, const void* x, const void* Wq, const float* Ws,
                      const Epilogue& ep, hipStream_t stream) {
    const int K16 = K / kUnitCodes;
    if (M >= kFp8MfmaFromM) {
        if (!fp8_size_ok(M, K) || K % kUnitCodes != 0) return hipErrorInvalidValue;
        int S, chunk_w;
        fp8_mfma_split(N, K, &S, &chunk_w);
        const int KB = (K + 127) / 128;
        const int NT = fp8_mfma_nt(N);
        const int grid = (N + 16 * NT - 1) / (16 * NT);
        const uint4* xp = static_cast<const uint4*>(x);
        const uint4* wp = static_cast<const uint4*>(Wq);
#define SG_S(nt, v) \
    if (NT == nt && S == v) { \
        fp8_mfma_kernel<nt, v><<<grid, kWave * v, 0, stream>>>(xp, wp, Ws, M, N, K16, KB, \
                                                              chunk_w, ep); \
        return hipGetLastError(); \
    }
        SG_S(1, 1) SG_S(1, 2) SG_S(1, 4) SG_S(1, 8) SG_S(2, 1) SG_S(2, 2) SG_S(2, 4) SG_S(2, 8)
#undef SG_S
        return hipErrorInvalidValue;
    }
    int S, chunk16, nch;
    if (!fp8_split(M, N, K, &S, &chunk16, &nch)) return hipErrorInvalidValue;
    switch (M) {
        case 1: return launch_m<1>(nch, S, N, K16, chunk16, x, Wq, Ws, ep, stream);
        case 2: return launch_m<2>(nch, S, N, K16, chunk16, x, Wq, Ws, ep, stream);
        case 3: return launch_m<3>(nch, S, N, K16, chunk16, x, Wq, Ws, ep, stream);
        case 4: return launch_m<4>(nch, S, N, K16, chunk16, x, Wq, Ws, ep, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sg
