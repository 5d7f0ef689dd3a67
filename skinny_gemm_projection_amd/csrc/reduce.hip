// reduce.hip -- deterministic second pass of split-K.
//
// y[i] = P[0, i] + P[1, i] + ... + P[S-1, i], added in ascending s in fp32 (no
// atomics, so every run gives the same bits), followed by the final
// epilogue: optional residual add (fp32(r) + y, rounded once to bf16 -- the
// output projection fused with the residual, "Hyper Optimizing Kimi K3 in
// vLLM" deepnotes page, Method details §2) and fp32 and/or bf16 stores.
// Each thread owns 4 consecutive outputs (16-byte partial loads when the
// row-major M*N plane keeps them aligned).
#include "launch.h"

namespace sg {

namespace {

// All S partial loads of a thread are issued before any is added (S <= 64,
// in batches of 16), so the pass costs about one memory round trip.
__global__ __launch_bounds__(kBlock) void splitk_reduce_kernel(const float* __restrict__ P, int S,
                                                               int64_t MN, Epilogue ep) {
    constexpr int kBatch = 16;
    const int64_t i0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4;
    if (i0 >= MN) return;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if ((MN & 3) == 0) {
        for (int s0 = 0; s0 < S; s0 += kBatch) {
            float4 part[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (s0 + j < S)
                    part[j] = reinterpret_cast<const float4*>(P + (int64_t)(s0 + j) * MN + i0)[0];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (s0 + j < S) {
                    if (s0 + j == 0) {
                        acc[0] = part[j].x;
                        acc[1] = part[j].y;
                        acc[2] = part[j].z;
                        acc[3] = part[j].w;
                    } else {
                        acc[0] += part[j].x;
                        acc[1] += part[j].y;
                        acc[2] += part[j].z;
                        acc[3] += part[j].w;
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float a = 0.0f;
            if (i0 + j < MN) {
                a = P[i0 + j];
                for (int s = 1; s < S; ++s) a += P[(int64_t)s * MN + i0 + j];
            }
            acc[j] = a;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (i0 + j < MN) store_final(ep, i0 + j, acc[j]);
}

// Tiled form for the chunk kernel's partials, laid out [S, N, MP] (MP = 16 *
// ceil(M/16); rows m >= M are zeros).  blockIdx.x is the chunk kernel's
// column tile and the grid's x extent is the chunk kernel's (padded to a
// multiple of 8), so linear workgroup ids -- and with them XCDs -- match
// those of the workgroups that wrote the tile; blockIdx.y picks a slice of
// kRedCols columns of the tile.  Thread (c, q) of a workgroup owns the four
// rows 4q..4q+3 of column c: it loads that float4 of every split -- all S
// issued before any is added (batches of 16) -- adds them in ascending s and
// writes the four outputs; consecutive lanes take consecutive columns, so
// each store instruction covers whole runs of a row of y.
constexpr int kRedCols = 16;  // 256 workgroups at N = 4096 with 128-row tiles

__global__ __launch_bounds__(kBlock) void splitk_reduce_tiles_kernel(const float* __restrict__ P,
                                                                     int S, int M, int MP, int N,
                                                                     int tile_n, Epilogue ep) {
    constexpr int kBatch = 16;
    const int c = threadIdx.x % kRedCols;
    const int q = threadIdx.x / kRedCols;  // float4 of the column
    const int n = blockIdx.x * tile_n + blockIdx.y * kRedCols + c;
    if (n >= N || 4 * q >= M) return;
    const int64_t plane4 = (int64_t)N * (MP / 4);
    const float4* src = reinterpret_cast<const float4*>(P) + (int64_t)n * (MP / 4) + q;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int s0 = 0; s0 < S; s0 += kBatch) {
        float4 part[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (s0 + j < S) part[j] = src[(s0 + j) * plane4];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (s0 + j < S) {
                if (s0 + j == 0) {
                    acc = part[j];
                } else {
                    acc.x += part[j].x;
                    acc.y += part[j].y;
                    acc.z += part[j].z;
                    acc.w += part[j].w;
                }
            }
        }
    }
    const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (4 * q + i < M) store_final(ep, (int64_t)(4 * q + i) * N + n, v[i]);
}

}  // namespace

hipError_t launch_reduce_tiles(const float* P, int S, int M, int N, int tile_n,
                               const Epilogue& ep, hipStream_t stream) {
    const int MP = mfma_partial_rows(M);
    if (tile_n % kRedCols != 0 || kRedCols * (MP / 4) > kBlock) return hipErrorInvalidValue;
    const dim3 grid(mfma_grid_tiles(N, tile_n), tile_n / kRedCols);
    splitk_reduce_tiles_kernel<<<grid, kBlock, 0, stream>>>(P, S, M, MP, N, tile_n, ep);
    return hipGetLastError();
}

hipError_t launch_reduce(const float* P, int S, int64_t MN, const Epilogue& ep,
                         hipStream_t stream) {
    const int64_t threads = (MN + 3) / 4;
    const int64_t grid = (threads + kBlock - 1) / kBlock;
    splitk_reduce_kernel<<<dim3((unsigned)grid), kBlock, 0, stream>>>(P, S, MN, ep);
    return hipGetLastError();
}

}  // namespace sg
