// splitk_mfma.hip -- split-K projection on bf16 matrix cores (gfx950).
//
// For batches of 16 and more rows the activation tile is a real dense
// contraction, so the partial products run on v_mfma_f32_16x16x32_bf16
// ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Method details §1:
// split-K at larger batch; the accumulation dimension is spread over more
// compute units).
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane (col = lane % 16,
// grp = lane / 16) supplies 8 consecutive k of one row of each operand, and
// D = A * B leaves lane (col, grp) the outputs (m = 16*mt + 4*grp + v,
// n = n0 + col), v = 0..3.  M is padded to 16*MT rows of x with zeros.  The
// k order inside a 32-wide step is free (the sum is over k), so A and B only
// have to agree on which 8 k values each lane group supplies.
//
// Two kernels:
//  * chunk kernel (default): a workgroup of 8 waves owns 128 rows of W and
//    one K chunk; the x chunk is staged in LDS once.  Loading the B operand
//    straight from HBM would read 16 rows x 64 bytes per instruction, which
//    streams about 20% slower than whole 256-byte row segments, so each wave
//    loads W as 4 rows x 256 bytes per instruction (16 pieces of 16 bytes of
//    each of its 16 rows per "round"), writes the round to a 4 KB LDS tile
//    of its own and reads it back in operand layout.  Slot c of row r in the
//    tile holds piece c ^ r (an XOR swizzle), so the operand read -- 16
//    different rows at one piece each -- hits 16 different bank groups.
//    Partials go to the [S, M, N] workspace and the deterministic reduction
//    kernel adds them (two-pass split-K).  The grid's column-tile count is
//    padded to a multiple of the 8 XCDs: workgroups are dispatched to XCDs
//    round-robin by linear id, so all S splits of a column tile run on one
//    XCD and the tiled reduction finds their partials in that XCD's L2.
//  * team kernel: S waves of one workgroup split K over a 16-row tile (the
//    same weight streaming), read x straight from L2, and add their S
//    partial tiles in LDS in ascending split order (no workspace, no second
//    pass).

#include "launch.h"

namespace sg {

namespace {

constexpr int kChunkWaves = 8;
constexpr int kTileSlots = 256;       // weight tile of one wave: 4 KB
constexpr int kXLoadsPerThread = 16;  // x staging loads per thread (LDS bound)

// Geometry of the chunk kernel for NT row tiles (16 rows each) per wave: a
// round covers 16/NT pieces of each of the wave's 16*NT rows (4 KB), loaded
// by 4 instructions of 4*NT rows x (256/NT) bytes.
template <int NT>
struct ChunkGeom {
    static constexpr int kRows = 16 * NT;                  // W rows per wave
    static constexpr int kRoundPieces = 16 / NT;           // pieces per row per round
    static constexpr int kSteps = kRoundPieces / 4;        // 32-wide k steps per round
    static constexpr int kRowsPerLoad = kWave / kRoundPieces;
    static constexpr int kWgRows = kRows * kChunkWaves;    // W rows per workgroup
    // Tile slot of (row, piece): row-major [kRows][kRoundPieces] with the
    // piece XOR-swizzled so that the 16 rows one operand load reads fall in
    // 16 different 16-byte bank groups.
    __device__ static int swz(int row) {
        return NT == 1 ? (row & 15) : ((row >> 1) & (kRoundPieces - 1));
    }
};

// Row pitch (16-byte units) of the staged x chunk: whole rounds plus one, odd,
// so the 16 rows read by one operand load fall in 16 different bank groups.
__host__ __device__ inline int x_pitch(int chunk8, int round_pieces) {
    return (chunk8 + round_pieces - 1) / round_pieces * round_pieces + 1;
}

template <int MT, int NT, int DR>
__global__ __launch_bounds__(kWave * kChunkWaves) void splitk_mfma_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ W, int M, int N, int K8, int chunk8,
    Epilogue ep) {
    using G = ChunkGeom<NT>;
    constexpr int RP = G::kRoundPieces;
    extern __shared__ uint4 lds[];
    constexpr uint32_t kOff = 0xFFFFFFF0u;  // past any descriptor range: reads zero
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = wave_id_in_block();
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int s = blockIdx.y;
    const int k0 = s * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));  // pieces of this chunk
    // whole rounds: x is staged as zeros past len and the weights past len
    // load as zeros, so every k step of a round runs unconditionally
    const int lenr = (len + RP - 1) / RP * RP;
    const int pitch = x_pitch(chunk8, RP);
    uint4* xs = lds;                                  // [16*MT][pitch]
    uint4* tile = lds + 16 * MT * pitch + wv * kTileSlots;

    if (blockIdx.x * G::kWgRows >= N) return;  // padding column of the grid
    const int row0 = blockIdx.x * G::kWgRows + wv * G::kRows;
    // wave-uniform by construction; readfirstlane keeps the descriptor scalar
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(G::kRows, N - row0)));
    const rsrc_t wrs = make_rsrc(W + (int64_t)row0 * K8, (uint32_t)rows * (uint32_t)K8 * 16u);
    // Load i of a round reads row i*kRowsPerLoad + lane/RP; slot lane%RP of
    // that row carries piece slot ^ swz(row).
    const int lrow = lane / RP;
    const int lslot = lane % RP;
    uint32_t woff[4];
    int wpiece[4];
    bool wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = i * G::kRowsPerLoad + lrow;
        wpiece[i] = lslot ^ G::swz(r);
        wrow[i] = r < rows;
        woff[i] = ((uint32_t)r * K8 + k0 + wpiece[i]) * 16u;
    }
    auto load_round = [&](int rd, uint4 (&w)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = wrow[i] && (rd * RP + wpiece[i] < len);
            w[i] = load16<kStream>(wrs, ok ? woff[i] + (uint32_t)rd * (RP * 16u) : kOff);
        }
    };

    // x loads go out first (they hit L2 and return early), then the first DR
    // weight rounds, then the x values are written to LDS: waiting for the x
    // loads does not wait for the weight stream.
    const int xtotal = 16 * MT * lenr;
    const int div = max(lenr, RP);
    const int step_rows = (kWave * kChunkWaves) / div;  // idx += 512 moves this many rows
    const int step_p = (kWave * kChunkWaves) - step_rows * div;  // ... and this many pieces
    const int nx = (xtotal + kWave * kChunkWaves - 1) / (kWave * kChunkWaves);  // <= 16
    const rsrc_t xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);
    uint4 xv[kXLoadsPerThread];
    int xdst[kXLoadsPerThread];  // LDS slot of each staged piece, -1 if none
    {
        int row = tid / div;
        int p = tid - row * div;
#pragma unroll
        for (int j = 0; j < kXLoadsPerThread; ++j) {
            if (j < nx) {  // workgroup-uniform
                const int idx = tid + j * kWave * kChunkWaves;
                const bool ok = idx < xtotal && row < M && p < len;
                xv[j] = load16<kCached>(xrs, ok ? ((uint32_t)row * K8 + k0 + p) * 16u : kOff);
                xdst[j] = idx < xtotal ? row * pitch + p : -1;
                row += step_rows;
                p += step_p;
                if (p >= div) {
                    p -= div;
                    ++row;
                }
            }
        }
    }
    uint4 wb[DR][4];
#pragma unroll
    for (int d = 0; d < DR; ++d) load_round(d, wb[d]);
#pragma unroll
    for (int j = 0; j < kXLoadsPerThread; ++j)
        if (j < nx && xdst[j] >= 0) xs[xdst[j]] = xv[j];  // zeros past M and len
    __syncthreads();

    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    int bslot[NT][G::kSteps];  // tile slot of this lane's B operand per (row tile, k step)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int t = 0; t < G::kSteps; ++t) {
            const int r = 16 * nt + col;
            bslot[nt][t] = r * RP + ((4 * t + grp) ^ G::swz(r));
        }
    const int rounds = (len + RP - 1) / RP;
    for (int r0 = 0; r0 < rounds; r0 += DR) {
#pragma unroll
        for (int d = 0; d < DR; ++d) {
            const int rd = r0 + d;
            if (rd < rounds) {  // wave-uniform
                // Within one wave LDS operations run in order, so the tile can
                // be rewritten right after the previous round's reads.
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tile[(i * G::kRowsPerLoad + lrow) * RP + lslot] = wb[d][i];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int t = 0; t < G::kSteps; ++t) {
                    const int p = rd * RP + 4 * t + grp;  // < lenr < pitch
                    uint4 a[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) a[mt] = xs[(mt * 16 + col) * pitch + p];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const uint4 b = tile[bslot[nt][t]];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, a[mt]), __builtin_bit_cast(bf16x8_t, b),
                                acc[nt][mt], 0, 0, 0);
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
            load_round(rd + DR, wb[d]);  // past the chunk: no memory access
        }
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * nt + col;
        if (r >= rows) continue;
        const int n = row0 + r;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = mt * 16 + grp * 4 + v;
                if (m < M) {
                    if (ep.partial)
                        ep.partial[((int64_t)s * M + m) * N + n] = acc[nt][mt][v];
                    else
                        store_final(ep, (int64_t)m * N + n, acc[nt][mt][v]);
                }
            }
        }
    }
}

// Team kernel: the S waves of one workgroup share a 16-row tile of W and
// split K between them (wave s streams chunk s).  The weights arrive as in
// the chunk kernel -- 4 rows x 256 bytes per load, transposed through a
// per-wave LDS tile -- while the x operands of each k step are loaded
// straight from L2 into the same register ring (x is small and every
// workgroup reads all of it; at MT row tiles that is MT times the weight
// bytes, so the planner uses this kernel for M <= 16).  There is no barrier
// in the main loop.  At the end the S partial tiles are added in LDS in
// ascending split order (deterministic) and wave w finishes the outputs o
// with o % S == w: no workspace and no second kernel.
template <int MT, int S, int DR>
__global__ __launch_bounds__(kWave * S) void mfma_team_kernel(const uint4* __restrict__ x,
                                                              const uint4* __restrict__ W, int M,
                                                              int N, int K8, int chunk8,
                                                              Epilogue ep) {
    constexpr int OUT = MT * 4;  // accumulator floats per lane
    constexpr int RP = 16;       // pieces per row per round
    constexpr uint32_t kOff = 0xFFFFFFF0u;  // past any descriptor range: reads zero
    __shared__ uint4 tiles[S][kTileSlots];
    __shared__ float red[S][OUT][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int s = wave_id_in_block();
    const int col = lane & 15;
    const int grp = lane >> 4;
    uint4* tile = tiles[s];
    const int row0 = blockIdx.x * 16;
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(16, N - row0)));
    const int k0 = s * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));  // pieces of this wave's chunk
    const int rounds = (len + RP - 1) / RP;

    const rsrc_t wrs = make_rsrc(W + (int64_t)row0 * K8, (uint32_t)rows * (uint32_t)K8 * 16u);
    const rsrc_t xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);
    // weights: load i of a round reads row 4i + grp, slot col = piece col ^ row
    uint32_t woff[4];
    int wpiece[4];
    bool wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + grp;
        wpiece[i] = col ^ r;
        wrow[i] = r < rows;
        woff[i] = ((uint32_t)r * K8 + k0 + wpiece[i]) * 16u;
    }
    // x: the A operand of step t is piece 16*rd + 4t + grp of row 16*mt + col
    uint32_t xoff[MT];
    bool xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + col;
        xrow[mt] = m < M;
        xoff[mt] = ((uint32_t)m * K8 + k0 + grp) * 16u;
    }
    auto load_round = [&](int rd, uint4 (&w)[4], uint4 (&a)[4][MT]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = wrow[i] && (rd * RP + wpiece[i] < len);
            w[i] = load16<kStream>(wrs, ok ? woff[i] + (uint32_t)rd * (RP * 16u) : kOff);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bool ok = xrow[mt] && (rd * RP + 4 * t + grp < len);
                a[t][mt] = load16<kCached>(
                    xrs, ok ? xoff[mt] + (uint32_t)(rd * RP + 4 * t) * 16u : kOff);
            }
    };

    uint4 wb[DR][4];
    uint4 xb[DR][4][MT];
#pragma unroll
    for (int d = 0; d < DR; ++d) load_round(d, wb[d], xb[d]);
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int r0 = 0; r0 < rounds; r0 += DR) {
#pragma unroll
        for (int d = 0; d < DR; ++d) {
            const int rd = r0 + d;
            if (rd < rounds) {  // wave-uniform
#pragma unroll
                for (int i = 0; i < 4; ++i) tile[(4 * i + grp) * RP + col] = wb[d][i];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint4 b = tile[col * RP + ((4 * t + grp) ^ col)];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, xb[d][t][mt]),
                            __builtin_bit_cast(bf16x8_t, b), acc[mt], 0, 0, 0);
                }
                __builtin_amdgcn_wave_barrier();
            }
            load_round(rd + DR, wb[d], xb[d]);  // past the chunk: no memory access
        }
    }

    const int n = row0 + col;
    if (S == 1) {
        if (col >= rows) return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = mt * 16 + grp * 4 + v;
                if (m < M) store_final(ep, (int64_t)m * N + n, acc[mt][v]);
            }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[s][mt * 4 + v][lane] = acc[mt][v];
    __syncthreads();
    if (col >= rows) return;
#pragma unroll
    for (int o = 0; o < OUT; ++o) {
        if (o % S != s) continue;
        float sum = red[0][o][lane];
#pragma unroll
        for (int q = 1; q < S; ++q) sum += red[q][o][lane];
        const int m = (o / 4) * 16 + grp * 4 + (o % 4);
        if (m < M) store_final(ep, (int64_t)m * N + n, sum);
    }
}

}  // namespace

bool mfma_team_split_ok(int S) { return S == 1 || S == 2 || S == 4 || S == 8; }

hipError_t launch_mfma_team(int M, int N, int K, int S, int k_chunk, const void* x,
                            const void* W, const Epilogue& ep, hipStream_t stream) {
    const int grid = (N + 15) / 16;
    const int K8 = K / kPiece;
    const int chunk8 = k_chunk / kPiece;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const int MT = (M + 15) / 16;
    constexpr int DR = 2;  // rounds in flight per wave
#define SG_TEAM(mt, sp) \
    if (MT == mt && S == sp) { \
        mfma_team_kernel<mt, sp, DR><<<grid, kWave * sp, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); \
        return hipGetLastError(); \
    }
    SG_TEAM(1, 1) SG_TEAM(1, 2) SG_TEAM(1, 4) SG_TEAM(1, 8)
    SG_TEAM(2, 1) SG_TEAM(2, 2) SG_TEAM(2, 4) SG_TEAM(2, 8)
    SG_TEAM(3, 1) SG_TEAM(3, 2) SG_TEAM(3, 4) SG_TEAM(3, 8)
    SG_TEAM(4, 1) SG_TEAM(4, 2) SG_TEAM(4, 4) SG_TEAM(4, 8)
#undef SG_TEAM
    return hipErrorInvalidValue;
}

int mfma_grid_tiles(int N, int tile_n) {
    const int tiles = (N + tile_n - 1) / tile_n;
    return (tiles + kXcds - 1) / kXcds * kXcds;
}

size_t mfma_chunk_lds_bytes(int M, int k_chunk, int tile_n) {
    const int MT = (M + 15) / 16;
    const int round_pieces = tile_n == 2 * kMfmaTileN ? 8 : 16;
    return (size_t)16 * MT * x_pitch(k_chunk / kPiece, round_pieces) * 16 +
           (size_t)kChunkWaves * kTileSlots * 16;
}

hipError_t launch_splitk_mfma(int M, int N, int K, int S, int k_chunk, int tile_n, const void* x,
                              const void* W, const Epilogue& ep, hipStream_t stream) {
    const int NT = tile_n / kMfmaTileN;
    if (NT != 1 && NT != 2) return hipErrorInvalidValue;
    const dim3 grid(mfma_grid_tiles(N, tile_n), S);
    const int K8 = K / kPiece;
    const int chunk8 = k_chunk / kPiece;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const int MT = (M + 15) / 16;
    const size_t lds = mfma_chunk_lds_bytes(M, k_chunk, tile_n);
    if (lds > kMfmaMaxLds) return hipErrorInvalidValue;
    // x staging: 16*MT*(pitch - 1) pieces at most over the workgroup's threads
    if ((size_t)16 * MT * (x_pitch(chunk8, 16 / NT) - 1) >
        (size_t)kXLoadsPerThread * kWave * kChunkWaves)
        return hipErrorInvalidValue;
    constexpr int DR = 2;  // weight rounds in flight per wave (8 loads)
#define SG_CHUNK(mt, nt) \
    if (MT == mt && NT == nt) { \
        hipError_t e = hipFuncSetAttribute( \
            reinterpret_cast<const void*>(&splitk_mfma_kernel<mt, nt, DR>), \
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
        if (e != hipSuccess) return e; \
        splitk_mfma_kernel<mt, nt, DR><<<grid, kWave * kChunkWaves, lds, stream>>>( \
            xp, wp, M, N, K8, chunk8, ep); \
        return hipGetLastError(); \
    }
    SG_CHUNK(1, 1) SG_CHUNK(2, 1) SG_CHUNK(3, 1) SG_CHUNK(4, 1)
    SG_CHUNK(1, 2) SG_CHUNK(2, 2) SG_CHUNK(3, 2) SG_CHUNK(4, 2)
#undef SG_CHUNK
    return hipErrorInvalidValue;
}

}  // namespace sg
