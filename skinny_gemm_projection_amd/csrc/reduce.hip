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

// Tiled form: blockIdx.x is the chunk kernel's column tile (tile_n outputs
// of a row), blockIdx.y a block of rows; each thread owns 4 consecutive
// columns of one row.  The grid's x extent is the chunk kernel's (padded to a
// multiple of 8), so linear workgroup ids -- and with them XCDs -- match those
// of the workgroups that wrote the tile.
__global__ __launch_bounds__(kBlock) void splitk_reduce_tiles_kernel(const float* __restrict__ P,
                                                                     int S, int M, int N,
                                                                     int tile_n, Epilogue ep) {
    constexpr int kBatch = 16;
    const int per_row = tile_n / 4;  // threads per row of the tile
    const int m = blockIdx.y * (kBlock / per_row) + threadIdx.x / per_row;
    const int n0 = blockIdx.x * tile_n + (threadIdx.x % per_row) * 4;
    if (m >= M || n0 >= N) return;
    const int64_t plane = (int64_t)M * N;
    const int64_t i0 = (int64_t)m * N + n0;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if ((N & 3) == 0) {  // n0 + 3 < N and 16-byte aligned
        for (int s0 = 0; s0 < S; s0 += kBatch) {
            float4 part[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (s0 + j < S) part[j] = reinterpret_cast<const float4*>(P + (s0 + j) * plane + i0)[0];
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
            if (n0 + j < N) {
                a = P[i0 + j];
                for (int s = 1; s < S; ++s) a += P[s * plane + i0 + j];
            }
            acc[j] = a;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (n0 + j < N) store_final(ep, i0 + j, acc[j]);
}

}  // namespace

hipError_t launch_reduce_tiles(const float* P, int S, int M, int N, int tile_n,
                               const Epilogue& ep, hipStream_t stream) {
    if (tile_n % 4 != 0 || tile_n / 4 > kBlock || kBlock % (tile_n / 4) != 0)
        return hipErrorInvalidValue;
    const int rows_per_block = kBlock / (tile_n / 4);
    const dim3 grid(mfma_grid_tiles(N, tile_n), (M + rows_per_block - 1) / rows_per_block);
    splitk_reduce_tiles_kernel<<<grid, kBlock, 0, stream>>>(P, S, M, N, tile_n, ep);
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
