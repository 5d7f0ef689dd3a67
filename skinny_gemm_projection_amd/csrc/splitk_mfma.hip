// splitk_mfma.hip -- split-K projection on bf16 matrix cores (gfx950).
//
// From 8 rows of batch up the activation tile is dense enough that the
// partial products run on v_mfma_f32_16x16x32_bf16
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
//  * chunk kernel (default): a workgroup of 8 waves owns 128 (or 256) rows
//    of W and one K chunk, processed in rounds; x of each round is staged in
//    a double-buffered LDS block while the previous round is multiplied.
//    Loading the B operand straight from HBM would read 16 rows x 64 bytes
//    per instruction, which streams about 20% slower than whole 256-byte row
//    segments, so each wave loads W as 4 rows x 256 bytes (or 8 x 128) per
//    instruction, writes the round to a 4 KB LDS tile of its own and reads
//    it back in operand layout.  Slot c of row r in the tile holds piece
//    c ^ swz(r) (an XOR swizzle), so the operand read -- 16 different rows
//    at one piece each -- hits 16 different bank groups.  Partials go to the
//    [S, N, 16*ceil(M/16)] workspace and the deterministic reduction kernel adds them
//    (two-pass split-K).  The grid's column-tile count is padded to a
//    multiple of the 8 XCDs: workgroups are dispatched to XCDs round-robin
//    by linear id, so all S splits of a column tile run on one XCD and the
//    tiled reduction finds their partials in that XCD's L2.
//  * team kernel: S waves of one workgroup split K over a 16-row tile (the
//    same weight streaming), read x straight from L2, and add their S
//    partial tiles in LDS in ascending split order (no workspace, no second
//    pass).

#include "launch.h"

namespace sg {

namespace {

constexpr int kChunkWaves = 8;
constexpr int kChunkThreads = kWave * kChunkWaves;
constexpr int kTileSlots = 256;  // weight tile of one wave: 4 KB

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

constexpr int kXLoadsMax = 16;  // x staging loads per thread and phase

// Chunk kernel.  A workgroup of 8 waves owns 128*NT rows of W and one K
// chunk, processed in rounds of 16/NT pieces.  Each wave streams its own
// 16*NT weight rows, DR rounds in flight in a register ring, transposed
// through its own LDS tile into operand layout; the waves run independently
// except at phase boundaries.  x is staged in LDS by phases of `phase`
// pieces: when the whole chunk fits (one phase) it is staged once before
// the loop and the loop has no barrier at all; otherwise two phase buffers
// alternate -- x of the next phase is loaded into registers while the
// current phase is multiplied, written to the other buffer at its end, and
// one barrier per phase publishes it.
template <int MT, int NT, int DR, bool PHASED, int ROUNDS>
__global__ __launch_bounds__(kChunkThreads) void splitk_mfma_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ W, int M, int N, int K8, int chunk8,
    int phase, Epilogue ep) {
    using G = ChunkGeom<NT>;
    constexpr int RP = G::kRoundPieces;
    constexpr int XROWS = 16 * MT;
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
    const int rounds = (len + RP - 1) / RP;        // workgroup-uniform
    const int pr = phase / RP;                      // rounds per phase
    // PHASED == false: the launcher made the phase cover every chunk
    const int nphases = PHASED ? (rounds + pr - 1) / pr : 1;
    const int xp = phase + 1;                       // odd row pitch of a phase buffer
    const int xslots = XROWS * xp;
    uint4* xs = lds;                                // [1 or 2][XROWS][xp]
    uint4* tile = lds + (nphases > 1 ? 2 : 1) * xslots + wv * kTileSlots;

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

    // x of a phase: thread t stages the pieces t, t+512, ... of the phase's
    // XROWS x phase block (row = idx / phase, piece = idx % phase); past M or
    // the chunk they are zeros.  At most kXLoadsMax per thread (the launcher
    // sizes `phase` so).
    const rsrc_t xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);
    const int xtotal = XROWS * phase;
    const int nx = (xtotal + kChunkThreads - 1) / kChunkThreads;  // workgroup-uniform
    const int step_rows = kChunkThreads / phase;                   // idx += 512 in rows ...
    const int step_p = kChunkThreads - step_rows * phase;          // ... and pieces
    const int row_t = tid / phase;
    const int p_t = tid - row_t * phase;
    uint4 xv[kXLoadsMax];
    auto load_x = [&](int ph) {
        int row = row_t, p = p_t;
#pragma unroll
        for (int j = 0; j < kXLoadsMax; ++j) {
            if (j < nx) {
                const int idx = tid + j * kChunkThreads;
                const int kp = ph * phase + p;  // piece within the chunk
                const bool ok = idx < xtotal && row < M && kp < len;
                xv[j] = load16<kCached>(xrs, ok ? ((uint32_t)row * K8 + k0 + kp) * 16u : kOff);
                row += step_rows;
                p += step_p;
                if (p >= phase) {
                    p -= phase;
                    ++row;
                }
            }
        }
    };
    auto store_x = [&](int buf) {
        int row = row_t, p = p_t;
#pragma unroll
        for (int j = 0; j < kXLoadsMax; ++j) {
            if (j < nx) {
                const int idx = tid + j * kChunkThreads;
                if (idx < xtotal) xs[buf * xslots + row * xp + p] = xv[j];
                row += step_rows;
                p += step_p;
                if (p >= phase) {
                    p -= phase;
                    ++row;
                }
            }
        }
    };

    // x loads first (they hit L2 and return early), then the weight
    // prologue, then the x stores: waiting for x does not wait for weights.
    load_x(0);
    uint4 wb[DR][4];
#pragma unroll
    for (int d = 0; d < DR; ++d) load_round(d, wb[d]);
    store_x(0);
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
    // One round: the weights of round rd into the wave's LDS tile, its k
    // steps against the staged x, then the loads of round rd + DR into the
    // freed registers (past the chunk: no memory access).
    auto round_step = [&](int rd, uint4 (&w)[4]) {
        const int ph = PHASED ? rd / pr : 0;
        const int rin = rd - ph * pr;  // round within the phase
        const bool next = PHASED && ph + 1 < nphases;
        if (next && rin == 0) load_x(ph + 1);
        // Within one wave LDS operations run in order, so the tile can be
        // rewritten right after the previous round's reads.
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[(i * G::kRowsPerLoad + lrow) * RP + lslot] = w[i];
        __builtin_amdgcn_wave_barrier();
        const uint4* xb = xs + (ph & 1) * xslots + rin * RP;
#pragma unroll
        for (int t = 0; t < G::kSteps; ++t) {
            const int p = 4 * t + grp;
            uint4 a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt] = xb[(mt * 16 + col) * xp + p];
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
        if (ROUNDS == 0 || rd + DR < ROUNDS) load_round(rd + DR, w);
        if (next && (rin == pr - 1)) {
            // The other buffer was last read in phase ph - 1, which every wave
            // finished before the previous phase barrier.
            store_x((ph + 1) & 1);
            __syncthreads();
        }
        // (unrolled) keeps the next round's LDS copy below these loads, so
        // that it waits for its own round only
        if constexpr (ROUNDS > 0) __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (ROUNDS > 0) {
        // One x phase of ROUNDS * RP pieces a row (zeros past the chunk): a
        // round past a shorter last chunk reads zero x and zero weights and
        // adds exactly 0, so no round is guarded and every round is unrolled.
        // Behind the loop header below the compiler waited for every load in
        // flight at the top of each trip.
        static_assert(!PHASED, "unrolled rounds need the whole chunk of x staged");
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) round_step(rd, wb[rd % DR]);
    } else {
        for (int r0 = 0; r0 < rounds; r0 += DR) {
#pragma unroll
            for (int d = 0; d < DR; ++d) {
                const int rd = r0 + d;
                if (rd < rounds) round_step(rd, wb[d]);  // workgroup-uniform
            }
        }
    }

    if (ep.partial) {
        // Partials as [S, N, 16*MT]: the 4 consecutive m a lane holds leave as
        // one 16-byte store (rows m >= M carry the zeros of the padded x).
        // Measured on MI355X against 4-byte stores into [S, M, N]: K=7168,
        // N=4096, M=64 15.9 -> 15.2 us for this kernel.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int r = 16 * nt + col;
            if (r >= rows) continue;
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(
                ep.partial + ((int64_t)s * N + row0 + r) * XROWS + grp * 4);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) dst[mt * 4] = acc[nt][mt];
        }
        return;
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
                if (m < M) store_final(ep, (int64_t)m * N + n, acc[nt][mt][v]);
            }
        }
    }
}

// Team kernel: the S waves of one workgroup share NT 16-row tiles of W and
// split K between them (wave s streams chunk s).  The weights arrive as in
// the chunk kernel -- 4 rows x 256 bytes per load, transposed through a
// per-wave LDS tile -- while the x operands of each k step are loaded
// straight from L2 into the same register ring (x is small and every
// workgroup reads all of it; at MT row tiles that is MT / NT times the
// weight bytes, so the planner uses this kernel for M <= 16).  With NT = 2
// each x operand read serves both tiles.  There is no barrier in the main
// loop.  At the end the S partial tiles are added in LDS in ascending split
// order (deterministic) and wave w finishes the outputs o with o % S == w:
// no workspace and no second kernel.  ROUNDS > 0 (at least the rounds of
// any wave's chunk) unrolls every round: behind the loop header the compiler
// waited for every load in flight (the prologue and the loop body filled the
// round buffers in different registers), so each trip drained the stream.
template <int MT, int S, int DR, int NT, int ROUNDS>
__global__ __launch_bounds__(kWave * S) void mfma_team_kernel(const uint4* __restrict__ x,
                                                              const uint4* __restrict__ W, int M,
                                                              int N, int K8, int chunk8,
                                                              Epilogue ep) {
    constexpr int OUT = MT * 4;  // accumulator floats per lane and tile
    constexpr int RP = 16;       // pieces per row per round
    constexpr uint32_t kOff = 0xFFFFFFF0u;  // past any descriptor range: reads zero
    // x tiles in LDS too, where the workgroup's LDS allows (all but MT = 4, S = 8)
    constexpr bool XT =
        (size_t)S * (kTileSlots * 16 * (NT + MT) + NT * OUT * kWave * 4) <= kMfmaMaxLds;
    __shared__ uint4 tiles[S][NT][kTileSlots];
    __shared__ uint4 xtiles[XT ? S : 1][XT ? MT : 1][XT ? kTileSlots : 1];
    __shared__ float red[S][NT * OUT][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int s = wave_id_in_block();
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int row0 = blockIdx.x * 16 * NT;
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(16 * NT, N - row0)));
    const int k0 = s * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));  // pieces of this wave's chunk
    const int rounds = (len + RP - 1) / RP;

    const rsrc_t wrs = make_rsrc(W + (int64_t)row0 * K8, (uint32_t)rows * (uint32_t)K8 * 16u);
    const rsrc_t xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);
    // weights: load i of a round reads row 16*nt + 4i + grp, slot col =
    // piece col ^ (4i + grp)
    uint32_t woff[NT][4];
    int wpiece[4];
    bool wrow[NT][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wpiece[i] = col ^ (4 * i + grp);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * nt + 4 * i + grp;
            wrow[nt][i] = r < rows;
            woff[nt][i] = ((uint32_t)r * K8 + k0 + wpiece[i]) * 16u;
        }
    // x goes the same way as the weights: load i of a round reads row
    // 16*mt + 4i + grp of x, slot col = piece col ^ (4i + grp), into the
    // wave's x tile; the A operand of step t (piece 4t + grp of row
    // 16*mt + col) is then read back like the B operand.  Whole 256-byte
    // row segments per instruction, instead of 16 rows x 64 bytes.
    // (Without x tiles: the A operand of step t, piece 16*rd + 4t + grp of
    // row 16*mt + col, straight from L2.)
    uint32_t xoff[4][MT];
    bool xrow[4][MT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = XT ? mt * 16 + 4 * i + grp : mt * 16 + col;
            const int piece = XT ? wpiece[i] : grp + 4 * i;
            xrow[i][mt] = m < M;
            xoff[i][mt] = ((uint32_t)m * K8 + k0 + piece) * 16u;
        }
    auto load_round = [&](int rd, uint4 (&w)[NT][4], uint4 (&a)[4][MT]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = wrow[nt][i] && (rd * RP + wpiece[i] < len);
                w[nt][i] =
                    load16<kStream>(wrs, ok ? woff[nt][i] + (uint32_t)rd * (RP * 16u) : kOff);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int piece = XT ? wpiece[i] : grp + 4 * i;
                const bool ok = xrow[i][mt] && (rd * RP + piece < len);
                a[i][mt] = load16<kCached>(xrs, ok ? xoff[i][mt] + (uint32_t)rd * (RP * 16u) : kOff);
            }
    };

    uint4 wb[DR][NT][4];
    uint4 xb[DR][4][MT];
#pragma unroll
    for (int d = 0; d < DR; ++d) load_round(d, wb[d], xb[d]);
    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // One round: the weights (and x) of round rd into the wave's LDS tiles,
    // its 4 k steps, then the loads of round rd + DR into the freed
    // registers (past the chunk: no memory access).
    auto round_step = [&](int rd, uint4 (&w)[NT][4], uint4 (&a)[4][MT]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) tiles[s][nt][(4 * i + grp) * RP + col] = w[nt][i];
            if constexpr (XT) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    xtiles[s][mt][(4 * i + grp) * RP + col] = a[i][mt];
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int slot = col * RP + ((4 * t + grp) ^ col);
            uint4 b[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b[nt] = tiles[s][nt][slot];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 av = XT ? xtiles[XT ? s : 0][XT ? mt : 0][XT ? slot : 0] : a[t][mt];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, b[nt]),
                        acc[nt][mt], 0, 0, 0);
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (ROUNDS == 0 || rd + DR < ROUNDS) load_round(rd + DR, w, a);
        // keeps the next round's LDS copy below these loads, so that it
        // waits for its own round only
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (ROUNDS > 0) {
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) round_step(rd, wb[rd % DR], xb[rd % DR]);
    } else {
        // rounds padded to whole multiples of DR: a padded round reads zero
        // and adds exactly 0
        const int rounds_p = (rounds + DR - 1) / DR * DR;
        for (int r0 = 0; r0 < rounds_p; r0 += DR) {
#pragma unroll
            for (int d = 0; d < DR; ++d) round_step(r0 + d, wb[d], xb[d]);
        }
    }

    if (S == 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int r = 16 * nt + col;
            if (r >= rows) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = mt * 16 + grp * 4 + v;
                    if (m < M) store_final(ep, (int64_t)m * N + row0 + r, acc[nt][mt][v]);
                }
        }
        return;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[s][nt * OUT + mt * 4 + v][lane] = acc[nt][mt][v];
    __syncthreads();
#pragma unroll
    for (int o = 0; o < NT * OUT; ++o) {
        if (o % S != s) continue;
        const int nt = o / OUT;
        const int r = 16 * nt + col;
        if (r >= rows) continue;
        float sum = red[0][o][lane];
#pragma unroll
        for (int q = 1; q < S; ++q) sum += red[q][o][lane];
        const int oo = o - nt * OUT;
        const int m = (oo / 4) * 16 + grp * 4 + (oo % 4);
        if (m < M) store_final(ep, (int64_t)m * N + row0 + r, sum);
    }
}

}  // namespace

bool mfma_team_split_ok(int S) { return S == 1 || S == 2 || S == 4 || S == 8; }

// Two tiles a wave (sharing each x operand read) measured faster only from 12
// rows, and slower by 18-49 % at every M when the row pitch is a multiple of
// 8 KB (K a multiple of 4096).  Interleaved A/B on MI355X, two tiles against
// one: 8192x7168 M = 4 / 8 / 16 20.37 / 19.43 / 20.45 against 20.21 / 19.24
// / 21.87 us; 16384x5120 M = 16 29.3 against 31.1; 8192x4096 M = 8 17.58
// against 12.09; 8192x8192 M = 16 28.07 against 23.83.
int mfma_team_tiles_per_wave(int M, int N, int K) {
    return M >= kMfmaTeamTwoTilesFromM && M <= 16 && N >= kMfmaTeamTwoTilesFromN &&
                   K % 4096 != 0
               ? 2
               : 1;
}

int mfma_team_grid(int M, int N, int K) {
    const int rows = 16 * mfma_team_tiles_per_wave(M, N, K);
    return (N + rows - 1) / rows;
}

hipError_t launch_mfma_team(int M, int N, int K, int S, int k_chunk, const void* x,
                            const void* W, const Epilogue& ep, hipStream_t stream) {
    const int grid = mfma_team_grid(M, N, K);
    const int NT = mfma_team_tiles_per_wave(M, N, K);
    const int K8 = K / kPiece;
    const int chunk8 = k_chunk / kPiece;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const int MT = (M + 15) / 16;
    // rounds in flight per wave; measured on MI355X, 3 or 4 were slower (K=7168,
    // N=4096, M=8: 12.4 us at 2, 14.4 at 3, 15.0 at 4, in the loop form), and
    // so was 1 (8192x7168 M = 8 19.17 -> 20.45 us, 7168x8192 M = 12 21.23 ->
    // 22.68 us)
    constexpr int DR = 2;
    // Up to 8 rounds a wave (K <= 8192 over 8 waves): every round unrolled.
    // Measured on MI355X (interleaved A/B against the loop): 4096x7168 M = 8
    // / 16 12.34 / 13.52 -> 10.92 / 12.19 us, 8192x7168 21.21 / 22.14 ->
    // 19.13 / 20.33 us, 7168x8192 22.53 / 24.16 -> 20.13 / 22.70 us.  3 or 4
    // rounds in flight stayed slower (8192x7168 M = 8: 19.4 / 19.9 us).
    const int rounds = (chunk8 + 15) / 16;
#define SG_TEAM_R(mt, nt, r) \
    if (MT == mt && S == 8 && NT == nt && rounds == r) { \
        mfma_team_kernel<mt, 8, DR, nt, r><<<grid, kWave * 8, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); \
        return hipGetLastError(); \
    }
    SG_TEAM_R(1, 1, 1) SG_TEAM_R(1, 1, 2) SG_TEAM_R(1, 1, 3) SG_TEAM_R(1, 1, 4)
    SG_TEAM_R(1, 1, 5) SG_TEAM_R(1, 1, 6) SG_TEAM_R(1, 1, 7) SG_TEAM_R(1, 1, 8)
    SG_TEAM_R(1, 2, 1) SG_TEAM_R(1, 2, 2) SG_TEAM_R(1, 2, 3) SG_TEAM_R(1, 2, 4)
    SG_TEAM_R(1, 2, 5) SG_TEAM_R(1, 2, 6) SG_TEAM_R(1, 2, 7) SG_TEAM_R(1, 2, 8)
#undef SG_TEAM_R
#define SG_TEAM(mt, sp, nt) \
    if (MT == mt && S == sp && NT == nt) { \
        mfma_team_kernel<mt, sp, DR, nt, 0><<<grid, kWave * sp, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); \
        return hipGetLastError(); \
    }
    SG_TEAM(1, 1, 1) SG_TEAM(1, 2, 1) SG_TEAM(1, 4, 1) SG_TEAM(1, 8, 1)
    SG_TEAM(1, 1, 2) SG_TEAM(1, 2, 2) SG_TEAM(1, 4, 2) SG_TEAM(1, 8, 2)
    SG_TEAM(2, 1, 1) SG_TEAM(2, 2, 1) SG_TEAM(2, 4, 1) SG_TEAM(2, 8, 1)
    SG_TEAM(3, 1, 1) SG_TEAM(3, 2, 1) SG_TEAM(3, 4, 1) SG_TEAM(3, 8, 1)
    SG_TEAM(4, 1, 1) SG_TEAM(4, 2, 1) SG_TEAM(4, 4, 1) SG_TEAM(4, 8, 1)
#undef SG_TEAM
    return hipErrorInvalidValue;
}

int mfma_grid_tiles(int N, int tile_n) {
    const int tiles = (N + tile_n - 1) / tile_n;
    return (tiles + kXcds - 1) / kXcds * kXcds;
}

// Pieces of x staged per phase for a chunk kernel launch: the whole chunk
// (rounded to whole rounds) in one buffer when that fits in LDS and in the
// staging registers, else the largest whole number of rounds for which two
// buffers fit.  0 if not even one round fits.
static int chunk_phase(int M, int k_chunk, int tile_n) {
    const int MT = (M + 15) / 16;
    const int xrows = 16 * MT;
    const int rp = tile_n == 2 * kMfmaTileN ? 8 : 16;
    const size_t budget = kMfmaMaxLds - (size_t)kChunkWaves * kTileSlots * 16;  // after W tiles
    const int chunk8 = k_chunk / kPiece;
    const int whole = (chunk8 + rp - 1) / rp * rp;
    const int max_stage = kXLoadsMax * kChunkThreads / xrows;  // staging registers
    if (whole >= rp && whole <= max_stage && (size_t)xrows * (whole + 1) * 16 <= budget)
        return whole;
    int ph = 0;
    for (int p = rp; p <= whole && p <= max_stage; p += rp)
        if ((size_t)2 * xrows * (p + 1) * 16 <= budget) ph = p;
    return ph;
}

size_t mfma_chunk_lds_bytes(int M, int k_chunk, int tile_n) {
    const int MT = (M + 15) / 16;
    const int ph = chunk_phase(M, k_chunk, tile_n);
    if (ph == 0) return kMfmaMaxLds + 1;  // cannot run
    const int chunk8 = k_chunk / kPiece;
    const int rp = tile_n == 2 * kMfmaTileN ? 8 : 16;
    const int whole = (chunk8 + rp - 1) / rp * rp;
    const int buffers = ph >= whole ? 1 : 2;
    return (size_t)buffers * 16 * MT * (ph + 1) * 16 + (size_t)kChunkWaves * kTileSlots * 16;
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
    const int phase = chunk_phase(M, k_chunk, tile_n);
    const size_t lds = mfma_chunk_lds_bytes(M, k_chunk, tile_n);
    if (phase == 0 || lds > kMfmaMaxLds) return hipErrorInvalidValue;
    // weight rounds in flight per wave (8 loads); 3 or 4 measured slower on
    // MI355X (K=7168, N=4096, M=64: 18.5 us at 2, 18.8 at 3, 19.6 at 4; with
    // every round unrolled 17.0 / 17.0 / 18.4 us), and 1 too (M = 20 / 64
    // 14.07 / 17.06 -> 15.09 / 18.17 us)
    constexpr int DR = 2;
    const int whole = (chunk8 + 16 / NT - 1) / (16 / NT) * (16 / NT);
    const bool phased = phase < whole;
    // One x phase and 4 to 8 rounds (128-row tiles) or 14 / 16 rounds
    // (256-row tiles, K = 7168 or 8192 over 8 splits): every round unrolled.
    // Interleaved A/B on MI355X against the loop: 4096x7168 M = 17 / 32 / 64
    // 14.98 / 15.11 / 18.23 -> 14.07 / 14.18 / 17.00 us, 8192x7168 M = 64
    // 30.33 -> 28.96 us.
    const int rounds = whole / (16 / NT);
#define SG_CHUNK_R(mt, nt, r) \
    if (MT == mt && NT == nt && !phased && rounds == r) { \
        hipError_t e = hipFuncSetAttribute( \
            reinterpret_cast<const void*>(&splitk_mfma_kernel<mt, nt, DR, false, r>), \
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
        if (e != hipSuccess) return e; \
        splitk_mfma_kernel<mt, nt, DR, false, r><<<grid, kChunkThreads, lds, stream>>>( \
            xp, wp, M, N, K8, chunk8, phase, ep); \
        return hipGetLastError(); \
    }
    SG_CHUNK_R(1, 1, 4) SG_CHUNK_R(2, 1, 4) SG_CHUNK_R(3, 1, 4) SG_CHUNK_R(4, 1, 4)
    SG_CHUNK_R(1, 1, 5) SG_CHUNK_R(2, 1, 5) SG_CHUNK_R(3, 1, 5) SG_CHUNK_R(4, 1, 5)
    SG_CHUNK_R(1, 1, 6) SG_CHUNK_R(2, 1, 6) SG_CHUNK_R(3, 1, 6) SG_CHUNK_R(4, 1, 6)
    SG_CHUNK_R(1, 1, 7) SG_CHUNK_R(2, 1, 7) SG_CHUNK_R(3, 1, 7) SG_CHUNK_R(4, 1, 7)
    SG_CHUNK_R(1, 1, 8) SG_CHUNK_R(2, 1, 8) SG_CHUNK_R(3, 1, 8) SG_CHUNK_R(4, 1, 8)
    SG_CHUNK_R(1, 2, 14) SG_CHUNK_R(2, 2, 14) SG_CHUNK_R(3, 2, 14) SG_CHUNK_R(4, 2, 14)
    SG_CHUNK_R(1, 2, 16) SG_CHUNK_R(2, 2, 16) SG_CHUNK_R(3, 2, 16) SG_CHUNK_R(4, 2, 16)
#undef SG_CHUNK_R
#define SG_CHUNK(mt, nt, ph) \
    if (MT == mt && NT == nt && phased == ph) { \
        hipError_t e = hipFuncSetAttribute( \
            reinterpret_cast<const void*>(&splitk_mfma_kernel<mt, nt, DR, ph, 0>), \
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
        if (e != hipSuccess) return e; \
        splitk_mfma_kernel<mt, nt, DR, ph, 0><<<grid, kChunkThreads, lds, stream>>>( \
            xp, wp, M, N, K8, chunk8, phase, ep); \
        return hipGetLastError(); \
    }
    SG_CHUNK(1, 1, false) SG_CHUNK(2, 1, false) SG_CHUNK(3, 1, false) SG_CHUNK(4, 1, false)
    SG_CHUNK(1, 2, false) SG_CHUNK(2, 2, false) SG_CHUNK(3, 2, false) SG_CHUNK(4, 2, false)
    SG_CHUNK(1, 1, true) SG_CHUNK(2, 1, true) SG_CHUNK(3, 1, true) SG_CHUNK(4, 1, true)
    SG_CHUNK(1, 2, true) SG_CHUNK(2, 2, true) SG_CHUNK(3, 2, true) SG_CHUNK(4, 2, true)
#undef SG_CHUNK
    return hipErrorInvalidValue;
}

}  // namespace sg
