// prefetch.hip -- side-stream weight prefetch for gfx950.
//
// Small-batch decode is bound by how fast weights stream from HBM, and some
// phases (communication, on the pages) leave that bandwidth idle; a kernel
// on a side stream can use those windows to pull the next projection's
// weights into the caches ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page,
// Method details §4).  On MI355X the target is the 256 MB Infinity Cache
// (MALL) in front of HBM, which holds a whole 117 MB weight matrix.
//
// The kernel reads only the static weight range it is given -- never
// activations, whose producer may not have finished (the pages report a
// compiler moving activation reads above a wait and restrict early loads to
// static weights; French translation, Partie 2 §3).  The loaded values are
// folded into one word per lane that is stored only when `never` is nonzero;
// the host always passes 0, so nothing is written, but the compiler cannot
// drop the loads.
#include "launch.h"

namespace sg {

namespace {

// Each wave reads kPrefetchUnroll consecutive 1 KB blocks per step (64 lanes
// x 16 bytes, one buffer load each), the waves striding over the range.
// Measured on MI355X over a 117 MB matrix: 19.1 us against 23.9 us for a
// grid-stride loop of per-thread 16-byte loads.  The loads use the default
// cache policy: with the non-temporal hint the data does not stay in the
// Infinity Cache (the following projection ran no faster than on a cold
// matrix), and warming that cache is the point.
constexpr int kPrefetchUnroll = 8;
constexpr uint32_t kPrefetchSpan = kPrefetchUnroll * kWave * 16;  // bytes per wave step
constexpr int kPrefetchGrid = 1024;                                 // 256 CUs x 4 workgroups

__global__ __launch_bounds__(kBlock) void prefetch_kernel(const uint8_t* __restrict__ src,
                                                          uint64_t bytes, int never,
                                                          uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint64_t wave = (uint64_t)blockIdx.x * kWavesPerBlock + wave_id_in_block();
    const uint64_t waves = (uint64_t)gridDim.x * kWavesPerBlock;
    uint32_t fold = 0;
    for (uint64_t base = wave * kPrefetchSpan; base < bytes; base += waves * kPrefetchSpan) {
        // a descriptor per step keeps every offset 32-bit for any range size;
        // loads past the step's end (the range's last partial step) read zero
        const uint64_t left = bytes - base;
        const rsrc_t r = make_rsrc(src + base, (uint32_t)(left < kPrefetchSpan ? left : kPrefetchSpan));
        uint4 v[kPrefetchUnroll];
#pragma unroll
        for (int u = 0; u < kPrefetchUnroll; ++u)
            v[u] = load16<kCached>(r, (uint32_t)(u * kWave + lane) * 16u);
#pragma unroll
        for (int u = 0; u < kPrefetchUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (never) sink[(int64_t)blockIdx.x * kBlock + threadIdx.x] = fold;
}

}  // namespace

hipError_t launch_prefetch(const void* W, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    const uint64_t steps = (bytes + kPrefetchSpan - 1) / kPrefetchSpan;
    const uint64_t blocks = (steps + kWavesPerBlock - 1) / kWavesPerBlock;
    const int grid = blocks < (uint64_t)kPrefetchGrid ? (int)blocks : kPrefetchGrid;
    prefetch_kernel<<<grid, kBlock, 0, stream>>>(static_cast<const uint8_t*>(W), (uint64_t)bytes,
                                                 0, nullptr);
    return hipGetLastError();
}

}  // namespace sg
