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

constexpr int kPrefetchUnroll = 8;

__global__ __launch_bounds__(kBlock) void prefetch_kernel(const uint4* __restrict__ src,
                                                          int64_t n16, int never,
                                                          uint32_t* __restrict__ sink) {
    uint32_t fold = 0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (; i + (kPrefetchUnroll - 1) * stride < n16; i += kPrefetchUnroll * stride) {
        uint4 v[kPrefetchUnroll];
#pragma unroll
        for (int u = 0; u < kPrefetchUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kPrefetchUnroll; ++u) fold ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        fold ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (never) sink[(int64_t)blockIdx.x * kBlock + threadIdx.x] = fold;
}

}  // namespace

hipError_t launch_prefetch(const void* W, size_t bytes, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    const int64_t per_block = (int64_t)kBlock * kPrefetchUnroll;
    int64_t grid = (n16 + per_block - 1) / per_block;
    if (grid > 1024) grid = 1024;  // 256 CUs x 4 workgroups
    prefetch_kernel<<<(unsigned)grid, kBlock, 0, stream>>>(static_cast<const uint4*>(W), n16, 0,
                                                           nullptr);
    return hipGetLastError();
}

}  // namespace sg
