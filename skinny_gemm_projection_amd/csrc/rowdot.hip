// rowdot.hip -- row-streaming vector-ALU projection kernel for gfx950.
//
// Serves the small-matrix path (M <= 2, "Hyper Optimizing Kimi K3 in vLLM"
// deepnotes page, Method details §1: a dedicated kernel at batch 1-2) and
// vector-ALU split-K (same section: the accumulation dimension is spread
// over more compute units), which the planner picks for 3 <= M <= 7 (6 and 7
// only where the matrix-core team kernel would not fill the GPU) and which a
// forced plan can run up to M = 15: there the batch is too small for a
// matrix-core tile to be a real dense contraction.
//
// Mapping (MI355X, wave64).  A wave owns one K chunk of whole W rows: lane l
// reads the 16-byte pieces c*64 + l (c < nch) of the chunk, so each load
// instruction covers 1 KB of contiguous weights; loads are raw buffer loads
// with the non-temporal hint (ragged tails read zero in hardware).  The
// matching x pieces of all M activation rows stay in registers for the
// wave's life, so each weight byte is fetched from HBM exactly once.  Lanes
// multiply with v_dot2c_f32_bf16 (exact bf16 products, fp32 sums).
//
// The R*M lane partials of one iteration are reduced together by a
// reduce-scatter: v_permlane32_swap and v_permlane16_swap halve the set
// twice and four DPP steps finish inside 16-lane rows -- about 2.5 VALU ops
// per output instead of 11 for one full reduction per output.
//
// Split-K inside a workgroup.  S waves form a team: they take the same rows,
// each its own K chunk, and after each iteration the S partial sums of every
// output are added in LDS in ascending chunk order (a fixed order: identical
// bits on every run) by the team's first wave, which then runs the epilogue.
// Teams stride over row groups persistent-style, the grid sized to the
// chip's resident wave slots.  A plan may instead send the S partials
// through a workspace to the separate reduction kernel (two-pass mode).
#include "launch.h"

namespace sg {

namespace {

template <int NCH, int POLICY, bool GUARD>
__device__ __forceinline__ void load_pieces(uint4 (&dst)[NCH], rsrc_t r, int nch, int lane) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (!GUARD) {
            dst[c] = load16<POLICY>(r, (uint32_t)(c * kWave + lane) * 16u);
        } else {
            dst[c] = make_uint4(0, 0, 0, 0);
            if (c < nch) dst[c] = load16<POLICY>(r, (uint32_t)(c * kWave + lane) * 16u);
        }
    }
}

constexpr int pad4(int v) { return (v + 3) / 4 * 4; }
constexpr int block_waves(int S) { return S > kWavesPerBlock ? S : kWavesPerBlock; }

// XS: the workgroup stages all of x once in LDS (dynamic, M*K8 pieces)
// instead of every wave reading its own copy from L2 -- measured on MI355X,
// those per-wave x reads cost 1-2 us of a 59-117 MB projection.  Each thread
// loads its share of x, the first group's weight loads are queued right
// behind, and only the x part is waited for before the LDS copy and the
// barrier; each wave then reads its own chunk of x from LDS.
template <int M, int NCH, int R, int S, bool GUARD, bool TWO_PASS, bool XS>
__global__ __launch_bounds__(kWave * block_waves(S)) void rowdot_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ W, int N, int K8, int splits,
    int chunk8, int iters, Epilogue ep) {
    static_assert(!XS || !TWO_PASS, "x staging: in-workgroup teams only");
    // Teams of S waves (S == 1 in two-pass mode, where a wave's chunk comes
    // from its global index instead).
    constexpr int kWaves = block_waves(S);
    constexpr int kTeams = kWaves / S;
    constexpr int V = pad4(R * M);
    __shared__ float red[2][kTeams][S][V];
    // From M = 6 up the rows of the next group are requested as soon as the
    // dot products have consumed this group's registers -- before the lane
    // reduction and the team barrier -- so the wave keeps weight loads in
    // flight across the iteration boundary.  Measured on MI355X at K=7168,
    // N=4096: M=6 13.3 -> 12.9 us, M=7 14.2 -> 13.5 us; at M <= 5 and on the
    // unsplit M <= 2 kernels it was neutral or slower (M=5 12.0 -> 12.4 us).
    constexpr bool kPipe = M >= 6;

    const int lane = threadIdx.x & (kWave - 1);
    const int wib = wave_id_in_block();
    const int team_in_block = wib / S;
    const int member = wib % S;
    int chunk, team, teams;
    if (TWO_PASS) {
        const int wave = blockIdx.x * kWaves + wib;
        chunk = wave % splits;
        team = wave / splits;
        teams = (gridDim.x * kWaves) / splits;
        if (team >= teams) return;  // remainder waves; this mode has no barriers
    } else {
        chunk = member;
        team = blockIdx.x * kTeams + team_in_block;
        teams = gridDim.x * kTeams;
    }

    const int k0 = chunk * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));
    const int nch = (len + kWave - 1) / kWave;
    const uint32_t bytes = (uint32_t)len * 16u;

    const int groups = (N + R - 1) / R;
    uint4 xr[M][NCH];
    uint4 wr[R][NCH];
    auto load_w = [&](int g) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = g * R + r;
            const rsrc_t rs = make_rsrc(W + (int64_t)min(n, N - 1) * K8 + k0, n < N ? bytes : 0u);
            load_pieces<NCH, kStream, GUARD>(wr[r], rs, nch, lane);
        }
    };
    if constexpr (XS) {
        extern __shared__ uint4 xs[];  // x [M, K8] pieces
        constexpr int kThreads = kWave * kWaves;
        constexpr int kStage = (M * NCH * S + kWaves - 1) / kWaves;  // >= M*K8 / kThreads
        const int total = M * K8;
        const rsrc_t rx = make_rsrc(x, (uint32_t)total * 16u);
        uint4 stage[kStage];
#pragma unroll
        for (int j = 0; j < kStage; ++j)
            stage[j] = load16<kCached>(rx, (uint32_t)(threadIdx.x + j * kThreads) * 16u);
        if (team < groups) load_w(team);  // the first iteration's rows, behind x
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int i = threadIdx.x + j * kThreads;
            if (i < total) xs[i] = stage[j];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int p = c * kWave + lane;
                xr[m][c] = p < len ? xs[m * K8 + k0 + p] : make_uint4(0, 0, 0, 0);
            }
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m)
            load_pieces<NCH, kCached, GUARD>(xr[m], make_rsrc(x + (int64_t)m * K8 + k0, bytes),
                                             nch, lane);
        if (kPipe && team < groups) load_w(team);
    }

    // Every wave of a block runs the same number of iterations (the team
    // barrier below needs it); a group past the end contributes nothing.
    for (int it = 0; it < iters; ++it) {
        const int g = team + it * teams;
        const int n0 = g * R;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.0f;
        if (g < groups) {
            if (!kPipe && (!XS || it > 0)) load_w(g);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float a = 0.0f;
#pragma unroll
                    for (int c = 0; c < NCH; ++c) a = dot8(xr[m][c], wr[r][c], a);
                    acc[r * M + m] = a;
                }
        }
        if (kPipe && it + 1 < iters && g + teams < groups) load_w(g + teams);
        const float total = reduce_scatter<V>(acc, lane);
        const int v = scatter_index<V>(lane);
        const bool mine = v >= 0 && v < R * M;
        const int r = mine ? v / M : 0;
        const int m = mine ? v - r * M : 0;
        const int n = n0 + r;
        const bool live = mine && g < groups && n < N;
        if (TWO_PASS) {
            if (live) ep.partial[((int64_t)chunk * M + m) * N + n] = total;
        } else if (S == 1) {
            if (live) store_final(ep, (int64_t)m * N + n, total);
        } else {
            // Team reduction in LDS: the S chunk partials added in ascending order.
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

// x staging loads per thread of the streaming kernel (LDS slots: 256 times
// this): all of x, M * K8 <= M * NCH * 64 * S pieces.
constexpr int rowstream_stage_loads(int M, int NCH, int S) {
    return (M * NCH * kWave * S + kBlock - 1) / kBlock;
}

// Streaming projection kernel for the vector ALU with x staged in LDS.  A
// team of S waves (S = 1, 2 or 4 in a workgroup of 4 waves) takes ITERS
// rows, one per step, the grid's teams striding over N; member s of a team
// covers K chunk s of each row ([s*chunk8, (s+1)*chunk8) pieces).  Two row
// buffers keep the next row's loads in flight while the current row is
// multiplied, reduced and stored.  Every step is unrolled, so each wait is
// for exactly the row it needs (behind a loop header the compiler would wait
// for every load in flight), and every load is issued: pieces past a chunk
// or a row past N read zero through the buffer bounds (a branch around a
// load would also make the compiler wait for all of them).  With S > 1 the
// members' sums of a step meet in LDS and the first member adds them in
// ascending chunk order (one barrier a step; the barrier waits for LDS
// only, not for the row loads in flight) -- the same order on every run.
template <int M, int NCH, int S, int ITERS>
__global__ __launch_bounds__(kBlock) void rowstream_kernel(const uint4* __restrict__ x,
                                                           const uint4* __restrict__ W, int N,
                                                           int K8, int chunk8, Epilogue ep) {
    static_assert(S == 1 || S == 2 || S == 4, "a team fits in the 4-wave workgroup");
    constexpr int V = pad4(M);
    constexpr int kTeams = kWavesPerBlock / S;  // teams per workgroup
    constexpr int kStage = rowstream_stage_loads(M, NCH, S);
    __shared__ float red[S > 1 ? 2 : 1][kTeams][S][V];
    const int lane = threadIdx.x & (kWave - 1);
    const int wib = wave_id_in_block();
    const int team_in_block = wib / S;
    const int member = wib - team_in_block * S;
    const int team = blockIdx.x * kTeams + team_in_block;
    const int teams = gridDim.x * kTeams;
    const int k0 = member * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));  // pieces of this member's chunk
    const uint32_t bytes = (uint32_t)len * 16u;
    const int v = scatter_index<V>(lane);  // the output a lane holds after a row's reduction
    const bool stores = member == 0;        // the first member finishes the outputs
    // Residual values of the outputs this lane stores, requested first: read
    // inside a step, each would wait for every row load in flight.  Buffer
    // loads (no branch) keep the compiler from sinking them to their use,
    // into 32-bit slots (packed 16-bit halves would serialise the loads), and
    // converted at their use, so that nothing waits for them before then.
    uint32_t rv[ITERS];
    if (ep.r) {
        const rsrc_t rr = make_rsrc(ep.r, (uint32_t)M * (uint32_t)N * 2u);
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int n = team + it * teams;
            const bool mine = stores && v >= 0 && v < M && n < N;
            rv[it] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                rr, mine ? (uint32_t)(v * N + n) * 2u : 0xFFFFFFF0u, 0, kCached);
        }
    }
    uint4 wr[2][NCH];
    auto load_row = [&](int it, uint4 (&dst)[NCH]) {
        const int n = team + it * teams;
        const rsrc_t rs =
            make_rsrc(W + (int64_t)min(n, N - 1) * K8 + k0, n < N ? bytes : 0u);
        load_pieces<NCH, kStream, false>(dst, rs, NCH, lane);
    };
    // x: each thread stages its share; the first two rows are requested right
    // behind it.  The LDS copy is unconditional (the buffer holds every staged
    // slot) so that no x load moves into a branch behind the row loads.
    extern __shared__ uint4 xs[];  // x [M, K8] pieces, then padding
    const int pieces = M * K8;
    const rsrc_t rx = make_rsrc(x, (uint32_t)pieces * 16u);
    uint4 stage[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j)
        stage[j] = load16<kCached>(rx, (uint32_t)(threadIdx.x + j * kBlock) * 16u);
    load_row(0, wr[0]);
    if (ITERS > 1) load_row(1, wr[1]);
#pragma unroll
    for (int j = 0; j < kStage; ++j) xs[threadIdx.x + j * kBlock] = stage[j];
    __syncthreads();
    uint4 xr[M][NCH];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int p = c * kWave + lane;
            xr[m][c] = p < len ? xs[m * K8 + k0 + p] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int b = it & 1;
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float a = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) a = dot8(xr[m][c], wr[b][c], a);
            acc[m] = a;
        }
        if (it + 2 < ITERS) load_row(it + 2, wr[b]);  // the buffer just consumed
        float sum = reduce_scatter<V>(acc, lane);
        const int n = team + it * teams;
        if constexpr (S > 1) {
            // the step's partials meet in LDS; two buffers, so a member that
            // runs ahead writes the other one (one barrier a step suffices)
            if (v >= 0) red[b][team_in_block][member][v] = sum;
            __syncthreads();
            if (stores && v >= 0) {
                sum = red[b][team_in_block][0][v];
#pragma unroll
                for (int q = 1; q < S; ++q) sum += red[b][team_in_block][q][v];
            }
        }
        if (stores && v >= 0 && v < M && n < N) {
            const float val = ep.r ? sum + __builtin_bit_cast(float, rv[it] << 16) : sum;
            const int64_t i = (int64_t)v * N + n;
            if (ep.y_f32) ep.y_f32[i] = val;
            if (ep.y_bf16) ep.y_bf16[i] = f32_to_bf16(val);
        }
    }
}

int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Two rows in flight per wave, except M=2 with more than 8 chunks, where the
// second row's registers would cut occupancy below 3 waves per SIMD.
constexpr int rows_per_iter(int M, int NCH) { return (M == 2 && NCH > 8) ? 1 : 2; }

}  // namespace

int rowdot_nch_cap(int M) {
    // x registers 4*M*NCH VGPRs, kept within 128.
    if (M <= 2) return 16;
    if (M <= 4) return 8;
    if (M <= 8) return 4;
    return 2;
}

int rowdot_rows_per_iter(int M, int nch) {
    const int c = nch < 1 ? 1 : nch;
    return rows_per_iter(M, M <= 2 ? c : next_pow2(c));
}

bool rowdot_team_split_ok(int M, int S) { return S == 1 || S == 2 || S == 4 || (S == 8 && M >= 5); }

int rowdot_block_threads(int S, bool two_pass) {
    return kWave * (two_pass ? kWavesPerBlock : block_waves(S));
}

// 256 CUs x 8 waves.  Measured on MI355X: twice as many (a second round of
// workgroups) was slower on every shape (7168 x 8192, M=2: 18.9 -> 20.0 us).
int rowdot_resident_waves(int, int) { return 2048; }

int rowdot_grid(int M, int N, int K, int S, int k_chunk, bool two_pass) {
    (void)K;
    const int nch = (k_chunk + kLaneSpan - 1) / kLaneSpan;
    const int R = rowdot_rows_per_iter(M, nch);
    const int groups = (N + R - 1) / R;
    const int resident = rowdot_resident_waves(M, nch);
    if (two_pass) {
        const int cap = (resident + S - 1) / S;
        const int Q = groups < cap ? groups : cap;
        return (S * Q + kWavesPerBlock - 1) / kWavesPerBlock;
    }
    const int teams_per_block = block_waves(S) / S;
    const int cap_teams = resident / S;
    int teams = groups < cap_teams ? groups : cap_teams;
    // as few teams as give every team the same number of row groups: a
    // ragged last round leaves part of the grid idle (measured: 7168 x 8192,
    // M = 1, 20.4 -> 19.9 us)
    const int its = (groups + teams - 1) / teams;
    teams = (groups + its - 1) / its;
    return (teams + teams_per_block - 1) / teams_per_block;
}

// Teams stage x in LDS while it fits in kStageMax (two 4-wave workgroups of
// a CU then still fit in its 160 KB).
constexpr size_t kStageMax = 64 * 1024;

// Rows a team of the streaming kernel takes (the unrolled step count): as
// many teams as the chip keeps resident waves for, each the same number of
// rows; teams of S > 1 waves round it up to a power of two (the compiled
// step counts), with the team count then trimmed to match.
static int rowstream_iters(int N, int S) {
    const int resident = rowdot_resident_waves(1, 0) / S;
    const int teams = N < resident ? N : resident;
    const int its = (N + teams - 1) / teams;
    return S == 1 ? its : next_pow2(its);
}

// Loads per row of a team member: exact for S = 1 (up to 16), else the
// power of two the launch is compiled for.
static int rowstream_nch(int K, int S) {
    const int chunk = 64 * ((K + 64 * S - 1) / (64 * S));  // the plan's k_chunk
    const int nch = (chunk + kLaneSpan - 1) / kLaneSpan;
    return S == 1 ? nch : next_pow2(nch);
}

bool rowstream_plan(int M, int N, int K, int S, bool two_pass, int* grid) {
    if (M < 1 || two_pass || K <= 0 || N < 1 || (size_t)M * K * 2 > kStageMax) return false;
    const int nch = rowstream_nch(K, S);
    const int its = rowstream_iters(N, S);
    if (M <= 2) {  // one K chunk: x of the whole row in registers
        if (S != 1 || nch > 16 || its > kRowstreamMaxIters) return false;
    } else {       // M = 3, 4: teams of 2 or 4 waves on K chunks
        if (M > 4 || (S != 2 && S != 4) || nch < 2 || nch > 8 || its < 2 ||
            its > kRowstreamMaxTeamIters)
            return false;
    }
    const int teams = (N + its - 1) / its;
    const int per_block = kWavesPerBlock / S;
    if (grid) *grid = (teams + per_block - 1) / per_block;
    return true;
}

template <int M, int NCH, int S, bool GUARD, bool XS = false>
static hipError_t launch_mns(int N, int K, int splits, int k_chunk, int grid, bool two_pass,
                             const void* x, const void* W, const Epilogue& ep,
                             hipStream_t stream) {
    const int K8 = K / kPiece;
    const int chunk8 = k_chunk / kPiece;
    constexpr int R = rows_per_iter(M, NCH);
    const int groups = (N + R - 1) / R;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    constexpr bool kStreamOne = M <= 2 && S == 1 && XS && !GUARD;
    constexpr bool kStreamTeam = (M == 3 || M == 4) && (S == 2 || S == 4) && XS &&
                                 (NCH == 2 || NCH == 4 || NCH == 8);
    if constexpr (kStreamOne || kStreamTeam) {
        int g = 0;
        if (rowstream_plan(M, N, K, splits, two_pass, &g)) {
            const int its = rowstream_iters(N, S);
            const size_t lds = (size_t)rowstream_stage_loads(M, NCH, S) * kBlock * 16;
            switch (its) {
#define SG_ITERS(i)                                                                         \
    case i:                                                                                 \
        rowstream_kernel<M, NCH, S, i><<<g, kBlock, lds, stream>>>(xp, wp, N, K8, chunk8, ep); \
        return hipGetLastError();
                SG_ITERS(2) SG_ITERS(4)
#undef SG_ITERS
                case 1:
                    if constexpr (kStreamOne) {
                        rowstream_kernel<M, NCH, S, 1><<<g, kBlock, lds, stream>>>(xp, wp, N, K8,
                                                                                 chunk8, ep);
                        return hipGetLastError();
                    }
                    break;
                case 3:
                    if constexpr (kStreamOne) {
                        rowstream_kernel<M, NCH, S, 3><<<g, kBlock, lds, stream>>>(xp, wp, N, K8,
                                                                                 chunk8, ep);
                        return hipGetLastError();
                    }
                    break;
                case 8:
                    if constexpr (kStreamTeam) {
                        rowstream_kernel<M, NCH, S, 8><<<g, kBlock, lds, stream>>>(xp, wp, N, K8,
                                                                                 chunk8, ep);
                        return hipGetLastError();
                    }
                    break;
                default: break;
            }
        }
    }
    if (two_pass) {
        const int teams = (grid * kWavesPerBlock) / splits;
        const int iters = (groups + teams - 1) / teams;
        rowdot_kernel<M, NCH, R, 1, GUARD, true, false>
            <<<grid, kWave * kWavesPerBlock, 0, stream>>>(xp, wp, N, K8, splits, chunk8, iters, ep);
    } else {
        const int teams = grid * (block_waves(S) / S);
        const int iters = (groups + teams - 1) / teams;
        const size_t lds = XS ? (size_t)M * K8 * 16 : 0;  // staged x
        rowdot_kernel<M, NCH, R, S, GUARD, false, XS>
            <<<grid, kWave * block_waves(S), lds, stream>>>(xp, wp, N, K8, S, chunk8, iters, ep);
    }
    return hipGetLastError();
}

// Team splits compiled per batch size: up to 8 waves per team (a 512-thread
// workgroup keeps 256 VGPRs per lane); larger splits use the two-pass mode.
template <int M>
constexpr bool team_split_compiled(int S) {
    return S == 1 || S == 2 || S == 4 || (S == 8 && M >= 5);
}


template <int M, int NCH, int S, bool GUARD>
static hipError_t launch_team(int N, int K, int k_chunk, int grid, const void* x, const void* W,
                              const Epilogue& ep, hipStream_t stream) {
    if ((size_t)M * K * 2 <= kStageMax)
        return launch_mns<M, NCH, S, GUARD, true>(N, K, S, k_chunk, grid, false, x, W, ep, stream);
    return launch_mns<M, NCH, S, GUARD, false>(N, K, S, k_chunk, grid, false, x, W, ep, stream);
}

template <int M, int NCH, bool GUARD>
static hipError_t launch_mn(int N, int K, int S, int k_chunk, int grid, bool two_pass,
                            const void* x, const void* W, const Epilogue& ep, hipStream_t stream) {
    if (two_pass)
        return launch_mns<M, NCH, 1, GUARD>(N, K, S, k_chunk, grid, true, x, W, ep, stream);
    switch (S) {
        case 1: return launch_team<M, NCH, 1, GUARD>(N, K, k_chunk, grid, x, W, ep, stream);
        case 2: return launch_team<M, NCH, 2, GUARD>(N, K, k_chunk, grid, x, W, ep, stream);
        case 4: return launch_team<M, NCH, 4, GUARD>(N, K, k_chunk, grid, x, W, ep, stream);
        case 8:
            if constexpr (team_split_compiled<M>(8))
                return launch_team<M, NCH, 8, GUARD>(N, K, k_chunk, grid, x, W, ep, stream);
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

template <int M>
static hipError_t launch_m(int nch, int N, int K, int S, int k_chunk, int grid, bool two_pass,
                           const void* x, const void* W, const Epilogue& ep, hipStream_t stream) {
    if constexpr (M <= 2) {
        // The unsplit small-matrix path gets an exact chunk count: no guarded loads.
        if (!two_pass && S == 1) {
            switch (nch < 1 ? 1 : nch) {
#define SG_NCH(c) \
    case c: return launch_mns<M, c, 1, false, true>(N, K, 1, k_chunk, grid, false, x, W, ep, stream);
                SG_NCH(1) SG_NCH(2) SG_NCH(3) SG_NCH(4) SG_NCH(5) SG_NCH(6) SG_NCH(7) SG_NCH(8)
                SG_NCH(9) SG_NCH(10) SG_NCH(11) SG_NCH(12) SG_NCH(13) SG_NCH(14) SG_NCH(15)
                SG_NCH(16)
#undef SG_NCH
                default: return hipErrorInvalidValue;
            }
        }
    }
    switch (next_pow2(nch < 1 ? 1 : nch)) {
        case 1: return launch_mn<M, 1, true>(N, K, S, k_chunk, grid, two_pass, x, W, ep, stream);
        case 2: return launch_mn<M, 2, true>(N, K, S, k_chunk, grid, two_pass, x, W, ep, stream);
        case 4:
            if constexpr (M <= 8)
                return launch_mn<M, 4, true>(N, K, S, k_chunk, grid, two_pass, x, W, ep, stream);
            break;
        case 8:
            if constexpr (M <= 4)
                return launch_mn<M, 8, true>(N, K, S, k_chunk, grid, two_pass, x, W, ep, stream);
            break;
        case 16:
            if constexpr (M <= 2)
                return launch_mn<M, 16, true>(N, K, S, k_chunk, grid, two_pass, x, W, ep, stream);
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_rowdot(int M, int N, int K, int S, int k_chunk, int grid, bool two_pass,
                         const void* x, const void* W, const Epilogue& ep, hipStream_t stream) {
    const int nch = (k_chunk + kLaneSpan - 1) / kLaneSpan;
    switch (M) {
#define SG_CASE(m) \
    case m: return launch_m<m>(nch, N, K, S, k_chunk, grid, two_pass, x, W, ep, stream);
        SG_CASE(1) SG_CASE(2) SG_CASE(3) SG_CASE(4) SG_CASE(5) SG_CASE(6) SG_CASE(7) SG_CASE(8)
        SG_CASE(9) SG_CASE(10) SG_CASE(11) SG_CASE(12) SG_CASE(13) SG_CASE(14) SG_CASE(15)
#undef SG_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sg
