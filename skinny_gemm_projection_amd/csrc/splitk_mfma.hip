// splitk_mfma.hip -- split-K projection on bf16 matrix cores (gfx950).
//
// For batches of 16 and more rows the activation tile is a real dense
// contraction, so the partial products run on v_mfma_f32_16x16x32_bf16
// ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Method details §1:
// split-K at larger batch; the accumulation dimension is spread over more
// compute units).
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane (col = lane % 16,
// grp = lane / 16) supplies 8 consecutive k of one row of each operand, so a
// 32-wide k step of a 16-row W tile is one 16-byte load per lane (16 rows x
// 64 contiguous bytes per instruction) and D = A * B leaves lane (col, grp)
// the outputs (m = 16*mt + 4*grp + v, n = n0 + col), v = 0..3.  M is padded
// to 16*MT rows of x with zeros.
//
// Two kernels share that inner step:
//  * chunk kernel (default): a workgroup of 8 waves owns 128 rows of W and
//    one K chunk; the x chunk is staged in LDS once, then each wave streams
//    its 16 rows barrier-free.  Partials go to the [S, M, N] workspace and
//    the deterministic reduction kernel adds them (two-pass split-K).
//  * team kernel: S waves of one workgroup split K over a 16-row tile, read
//    x straight from L2, and add their S partial tiles in LDS in ascending
//    split order (no workspace, no second pass).

#include "launch.h"

namespace sg {

namespace {

// Chunk kernel (two-pass split-K).  A workgroup of 8 waves owns 128 rows of
// W and one K chunk.  It first stages the x chunk of all M rows (padded to
// 16*MT) in LDS once -- rows padded by 16 bytes against bank conflicts --
// then each wave streams its own 16 rows with no further barrier: D k-steps
// of its B operands stay in flight in a register ring and the A operands come
// from LDS.  x is read from L2 once per 128 rows.  The W loads use the default
// cache policy: each instruction covers only half of 16 cache lines (the next
// k step covers the other half), and for that pattern it measures faster than
// the streaming (nt) policy.
constexpr int kChunkWaves = 8;
constexpr int kChunkRows = 16 * kChunkWaves;

template <int MT, int D>
__global__ __launch_bounds__(kWave * kChunkWaves) void splitk_mfma_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ W, int M, int N, int K8, int chunk8,
    Epilogue ep) {
    extern __shared__ uint4 xs[];  // [16*MT][pitch], pitch = round4(chunk8) + 1
    constexpr uint32_t kOff = 0xFFFFFFF0u;
    const int pitch = (chunk8 + 3) / 4 * 4 + 1;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = wave_id_in_block();
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int s = blockIdx.y;
    const int k0 = s * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));
    const int lenr = (len + 3) / 4 * 4;  // whole k-steps; pieces past len staged as 0


    const int row0 = blockIdx.x * kChunkRows + wv * 16;
    const int rows = max(0, min(16, N - row0));
    const bool n_ok = col < rows;
    const rsrc_t wrs = make_rsrc(W + (int64_t)row0 * K8, (uint32_t)rows * (uint32_t)K8 * 16u);
    const uint32_t w_lane = ((uint32_t)col * K8 + k0 + grp) * 16u;
    const int steps = (len + 3) / 4;

    uint4 wb[D];
    auto load_w = [&](int t) {
        const bool ok = n_ok && (t * 4 + grp < len);
        return load16<kCached>(wrs, ok ? w_lane + (uint32_t)t * 64u : kOff);
    };
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // The first D weight steps go out before x is staged, so HBM streaming
    // starts at once and overlaps the staging.
#pragma unroll
    for (int d = 0; d < D; ++d) wb[d] = load_w(d);

    // Stage x[0..16*MT) x pieces [k0, k0+lenr) into LDS (zeros past M or len).
    {
        const rsrc_t xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);
        const int total = 16 * MT * lenr;
        for (int idx = tid; idx < total; idx += kWave * kChunkWaves) {
            const int row = idx / lenr;
            const int p = idx - row * lenr;
            const uint32_t off =
                (row < M && p < len) ? ((uint32_t)row * K8 + k0 + p) * 16u : kOff;
            xs[row * pitch + p] = load16<kCached>(xrs, off);
        }
    }
    __syncthreads();

    for (int t0 = 0; t0 < steps; t0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int t = t0 + d;
            const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, wb[d]);
            if (t < steps) {  // wave-uniform; p < lenr < pitch stays inside the row
                const int p = t * 4 + grp;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint4 a = xs[(mt * 16 + col) * pitch + p];
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, a), bop, acc[mt], 0, 0, 0);
                }
            }
            wb[d] = load_w(t + D);
        }
    }

    if (!n_ok) return;
    const int n = row0 + col;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = mt * 16 + grp * 4 + v;
            if (m < M) {
                if (ep.partial)
                    ep.partial[((int64_t)s * M + m) * N + n] = acc[mt][v];
                else
                    store_final(ep, (int64_t)m * N + n, acc[mt][v]);
            }
        }
    }
}

// Team kernel: S waves of one workgroup share a 16-row tile of W and split
// K between them; all M rows of x (padded to 16*MT) go through each wave.
// There is no barrier in the main loop: every wave keeps D k-steps of its W
// operand (nt buffer loads from HBM) and of its x operands (buffer loads,
// L2-resident) in flight in a register ring, refilling a slot right after
// the matrix ops that consumed it.  Steps past the chunk read zeros and add
// nothing.  At the end the S partial tiles are added in LDS in ascending
// split order (deterministic) and wave w finishes the outputs o with
// o % S == w.
template <int MT, int S, int D>
__global__ __launch_bounds__(kWave * S) void mfma_team_kernel(const uint4* __restrict__ x,
                                                              const uint4* __restrict__ W, int M,
                                                              int N, int K8, int chunk8,
                                                              Epilogue ep) {
    constexpr int OUT = MT * 4;  // accumulator floats per lane
    constexpr uint32_t kOff = 0xFFFFFFF0u;  // past any descriptor range: reads zero
    __shared__ float red[S][OUT][kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int s = wave_id_in_block();
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int row0 = blockIdx.x * 16;
    const int rows = max(0, min(16, N - row0));
    const bool n_ok = col < rows;
    const int k0 = s * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));  // pieces of this wave's chunk
    const int steps = (len + 3) / 4;                // 32-wide k steps

    const rsrc_t wrs = make_rsrc(W + (int64_t)row0 * K8, (uint32_t)rows * (uint32_t)K8 * 16u);
    const rsrc_t xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);
    const uint32_t w_lane = ((uint32_t)col * K8 + k0 + grp) * 16u;
    uint32_t x_lane[MT];
    bool x_ok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + col;
        x_ok[mt] = m < M;
        x_lane[mt] = ((uint32_t)m * K8 + k0 + grp) * 16u;
    }

    uint4 wb[D];
    uint4 xb[D][MT];
    auto load_step = [&](int t, uint4& w, uint4 (&xv)[MT]) {
        const bool ok = t * 4 + grp < len;
        w = load16<kStream>(wrs, (n_ok && ok) ? w_lane + (uint32_t)t * 64u : kOff);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            xv[mt] = load16<kCached>(xrs, (x_ok[mt] && ok) ? x_lane[mt] + (uint32_t)t * 64u : kOff);
    };

    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < D; ++d) load_step(d, wb[d], xb[d]);
    for (int t0 = 0; t0 < steps; t0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, wb[d]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, xb[d][mt]), bop, acc[mt], 0, 0, 0);
            load_step(t0 + d + D, wb[d], xb[d]);
        }
    }

    const int n = row0 + col;
    if (S == 1) {
        if (!n_ok) return;
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
    if (!n_ok) return;
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
    constexpr int D = 8;
#define SG_TEAM(mt, sp) \
    if (MT == mt && S == sp) { \
        mfma_team_kernel<mt, sp, D><<<grid, kWave * sp, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); \
        return hipGetLastError(); \
    }
    SG_TEAM(1, 1) SG_TEAM(1, 2) SG_TEAM(1, 4) SG_TEAM(1, 8)
    SG_TEAM(2, 1) SG_TEAM(2, 2) SG_TEAM(2, 4) SG_TEAM(2, 8)
    SG_TEAM(3, 1) SG_TEAM(3, 2) SG_TEAM(3, 4) SG_TEAM(3, 8)
    SG_TEAM(4, 1) SG_TEAM(4, 2) SG_TEAM(4, 4) SG_TEAM(4, 8)
#undef SG_TEAM
    return hipErrorInvalidValue;
}

size_t mfma_chunk_lds_bytes(int M, int k_chunk) {
    const int MT = (M + 15) / 16;
    const int pitch = (k_chunk / kPiece + 3) / 4 * 4 + 1;
    return (size_t)16 * MT * pitch * 16;
}

hipError_t launch_splitk_mfma(int M, int N, int K, int S, int k_chunk, const void* x,
                              const void* W, const Epilogue& ep, hipStream_t stream) {
    const dim3 grid((N + kChunkRows - 1) / kChunkRows, S);
    const int K8 = K / kPiece;
    const int chunk8 = k_chunk / kPiece;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const int MT = (M + 15) / 16;
    const size_t lds = mfma_chunk_lds_bytes(M, k_chunk);
    constexpr int D = 8;
#define SG_CHUNK(mt) \
    if (MT == mt) { \
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&splitk_mfma_kernel<mt, D>), \
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
        if (e != hipSuccess) return e; \
        splitk_mfma_kernel<mt, D><<<grid, kWave * kChunkWaves, lds, stream>>>(xp, wp, M, N, K8, \
                                                                             chunk8, ep); \
        return hipGetLastError(); \
    }
    SG_CHUNK(1) SG_CHUNK(2) SG_CHUNK(3) SG_CHUNK(4)
#undef SG_CHUNK
    return hipErrorInvalidValue;
}

}  // namespace sg
