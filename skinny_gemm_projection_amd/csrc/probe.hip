// probe.hip -- read-bandwidth probe for gfx950: the small-matrix kernel's
// weight stream with no arithmetic.
//
// Small-batch projections are limited by how fast the weights stream from
// HBM ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Method details §1).
// The peak in the datasheet is not what a single kernel of one projection's
// size can reach: the launch, the ramp while the first waves issue their
// loads, and the tail while the last ones drain all count.  This kernel
// reads a [rows, row_bytes] matrix with exactly the load shape of the M <= 2
// kernel in rowdot.hip -- a wave takes R whole rows per iteration, each row
// as row_bytes / 1 KB buffer loads of 64 lanes x 16 bytes with the
// non-temporal hint, waves striding over row groups on the same grid -- and
// folds the data into one word per lane that is stored only when `never` is
// nonzero (the host passes 0, so nothing is written, but the compiler cannot
// drop the loads).  Its time is the best the projection's loads can do on
// this GPU; the projection's own time above it is its arithmetic, reduction
// and stores.
#include "launch.h"

namespace sg {

namespace {

template <int NCH, int R>
__global__ __launch_bounds__(kBlock) void read_probe_kernel(const uint4* __restrict__ W, int rows,
                                                            int row16, int iters, int never,
                                                            uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = blockIdx.x * kWavesPerBlock + wave_id_in_block();
    const int waves = gridDim.x * kWavesPerBlock;
    const uint32_t bytes = (uint32_t)row16 * 16u;
    uint32_t fold = 0;
    for (int it = 0; it < iters; ++it) {
        uint4 v[R][NCH];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int64_t n = ((int64_t)wave + (int64_t)it * waves) * R + q;
            // rows past the end get an empty descriptor: their loads read zero
            const int64_t row = n < rows ? n : rows - 1;
            const rsrc_t r = make_rsrc(W + row * row16, n < rows ? bytes : 0u);
#pragma unroll
            for (int c = 0; c < NCH; ++c) v[q][c] = load16<kStream>(r, (uint32_t)(c * kWave + lane) * 16u);
        }
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int c = 0; c < NCH; ++c) fold ^= v[q][c].x ^ v[q][c].y ^ v[q][c].z ^ v[q][c].w;
    }
    if (never) sink[(int64_t)blockIdx.x * kBlock + threadIdx.x] = fold;
}

template <int R>
hipError_t launch_probe_r(int nch, const uint4* W, int rows, int row16, int grid,
                          hipStream_t stream) {
    const int groups = (rows + R - 1) / R;
    const int waves = grid * kWavesPerBlock;
    const int iters = (groups + waves - 1) / waves;
    switch (nch) {
#define SG_PROBE(c)                                                                            \
    case c:                                                                                    \
        read_probe_kernel<c, R><<<grid, kBlock, 0, stream>>>(W, rows, row16, iters, 0, nullptr); \
        return hipGetLastError();
        SG_PROBE(1) SG_PROBE(2) SG_PROBE(3) SG_PROBE(4) SG_PROBE(5) SG_PROBE(6) SG_PROBE(7)
        SG_PROBE(8) SG_PROBE(9) SG_PROBE(10) SG_PROBE(11) SG_PROBE(12) SG_PROBE(13)
        SG_PROBE(14) SG_PROBE(15) SG_PROBE(16)
#undef SG_PROBE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_read_probe(const void* W, int rows, int row_bytes, int rows_per_iter, int grid,
                             hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int row16 = row_bytes / 16;
    const int nch = (row16 + kWave - 1) / kWave;
    const uint4* wp = static_cast<const uint4*>(W);
    if (rows_per_iter == 1) return launch_probe_r<1>(nch, wp, rows, row16, grid, stream);
    if (rows_per_iter == 2) return launch_probe_r<2>(nch, wp, rows, row16, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace sg
