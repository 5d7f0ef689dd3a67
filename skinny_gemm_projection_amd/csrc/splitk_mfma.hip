// splitk_mfma.hip -- split-K projection on bf16 matrix cores (gfx950).
//
// For batches of 16 and more rows the activation tile is a real dense
// contraction, so the partial products run on v_mfma_f32_16x16x32_bf16
// ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Method details §1:
// split-K at larger batch; the accumulation dimension is spread over more
// compute units).
//
// Mapping.  Grid = (ceil(N / 64), S): a workgroup owns 64 rows of W and one K
// chunk; each of its 4 waves owns 16 of those rows and every 16-row tile of
// x (M padded to 16*MT).  For one 32-wide k step a lane (col = lane % 16,
// grp = lane / 16) loads the 16 bytes W[n0 + col][k + 8*grp .. +8] straight
// from HBM into its B operand (16 rows x 64 contiguous bytes per
// instruction), and reads the matching x bytes for each m tile from LDS as
// its A operand.  The x chunk is staged through LDS in 256-wide K blocks
// (double buffered, rows padded by 16 bytes against bank conflicts); the W
// loads of the next block are issued before the current block's matrix ops.
// Each W byte is read from HBM once; x is read once per workgroup.
// D = A * B gives lane (col, grp) the outputs (m = 16*mt + 4*grp + v,
// n = n0 + col), v = 0..3.
#include "launch.h"

namespace sg {

namespace {

constexpr int kKB8 = 32;             // 16-byte pieces per K block (256 elements)
constexpr int kPitch8 = kKB8 + 1;    // LDS row pitch in pieces (+16 B pad)
constexpr int kSteps = kKB8 / 4;     // 32-wide k steps per K block

template <int MT>
__global__ __launch_bounds__(kBlock) void splitk_mfma_kernel(const uint4* __restrict__ x,
                                                             const uint4* __restrict__ W,
                                                             int M, int N, int K8, int chunk8,
                                                             Epilogue ep) {
    constexpr int ROWS = 16 * MT;
    constexpr int XPT = ROWS * kKB8 / kBlock;  // x pieces staged per thread per block
    __shared__ uint4 xs[2][ROWS * kPitch8];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = wave_id_in_block();
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int s = blockIdx.y;
    const int n = blockIdx.x * kMfmaTileN + wv * 16 + col;
    const bool n_ok = n < N;
    const int k0 = s * chunk8;
    const int len = max(0, min(K8 - k0, chunk8));
    const int nblocks = (len + kKB8 - 1) / kKB8;

    // One buffer descriptor per wave over its 16 rows of W (rows past N lie
    // beyond the descriptor's range); a lane's piece outside its row's chunk
    // (the K tail) or in a row past N gets an offset past the range, so the
    // hardware returns zeros without a branch.
    const int row0 = blockIdx.x * kMfmaTileN + wv * 16;
    const int rows = max(0, min(16, N - row0));
    const rsrc_t wr = make_rsrc(W + (int64_t)row0 * K8, (uint32_t)rows * (uint32_t)K8 * 16u);
    const uint32_t lane_base = ((uint32_t)col * (uint32_t)K8 + (uint32_t)k0) * 16u;
    const rsrc_t xr = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);

    auto load_w = [&](int b, uint4 (&w)[kSteps]) {
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            const int p = b * kKB8 + t * 4 + grp;
            const uint32_t off = (n_ok && p < len) ? lane_base + (uint32_t)p * 16u : 0xFFFFFFF0u;
            w[t] = load16<kStream>(wr, off);
        }
    };
    auto load_x = [&](int b, uint4 (&xv)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int idx = tid + i * kBlock;
            const int row = idx / kKB8;
            const int p = b * kKB8 + idx % kKB8;
            const uint32_t off = (row < M && p < len)
                                     ? ((uint32_t)row * (uint32_t)K8 + (uint32_t)(k0 + p)) * 16u
                                     : 0xFFFFFFF0u;
            xv[i] = load16(xr, off);
        }
    };
    auto store_x = [&](int buf, const uint4 (&xv)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int idx = tid + i * kBlock;
            xs[buf][(idx / kKB8) * kPitch8 + idx % kKB8] = xv[i];
        }
    };

    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    uint4 wcur[kSteps], wnxt[kSteps];
    uint4 xv[XPT];
    if (nblocks > 0) {
        load_w(0, wcur);
        load_x(0, xv);
        store_x(0, xv);
    }
    __syncthreads();

    for (int b = 0; b < nblocks; ++b) {
        const int cur = b & 1;
        const bool more = b + 1 < nblocks;
        if (more) {
            load_w(b + 1, wnxt);
            load_x(b + 1, xv);
        }
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, wcur[t]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 a = xs[cur][(mt * 16 + col) * kPitch8 + t * 4 + grp];
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, a), bop, acc[mt], 0, 0, 0);
            }
        }
        if (more) store_x(cur ^ 1, xv);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kSteps; ++t) wcur[t] = wnxt[t];
    }

    if (!n_ok) return;
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

}  // namespace

hipError_t launch_splitk_mfma(int M, int N, int K, int S, int k_chunk, const void* x,
                              const void* W, const Epilogue& ep, hipStream_t stream) {
    const dim3 grid((N + kMfmaTileN - 1) / kMfmaTileN, S);
    const int K8 = K / kPiece;
    const int chunk8 = k_chunk / kPiece;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const int MT = (M + 15) / 16;
    switch (MT) {
        case 1: splitk_mfma_kernel<1><<<grid, kBlock, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); break;
        case 2: splitk_mfma_kernel<2><<<grid, kBlock, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); break;
        case 3: splitk_mfma_kernel<3><<<grid, kBlock, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); break;
        case 4: splitk_mfma_kernel<4><<<grid, kBlock, 0, stream>>>(xp, wp, M, N, K8, chunk8, ep); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sg
