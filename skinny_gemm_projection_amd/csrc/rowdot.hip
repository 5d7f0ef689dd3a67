// rowdot.hip -- row-streaming vector-ALU projection kernel for gfx950.
//
// Serves the small-matrix path (M <= 2, "Hyper Optimizing Kimi K3 in vLLM"
// deepnotes page, Method details §1: a dedicated kernel at batch 1-2) and the
// split-K partials for 3 <= M <= 15 (same section: the accumulation dimension
// is spread over more compute units), where the batch is too small for a
// matrix-core tile to be a real dense contraction.
//
// Mapping (MI355X, wave64): one wavefront owns one K chunk of whole W rows.
// Lane l reads the 16-byte pieces c*64 + l (c = 0..nch-1) of the chunk, so
// every load instruction of the wave covers 1 KB of contiguous weights and a
// row's chunk is fully in flight after nch instructions.  The matching x
// pieces for all M activation rows stay in registers for the wave's whole
// life; each weight byte is fetched from HBM exactly once.  A lane multiplies
// its pieces with v_dot2c_f32_bf16 (exact bf16 products, fp32 accumulation),
// and the 64 lane partials of a row are summed with DPP row steps plus four
// cross-row reads.  Waves stride over rows R at a time, persistent-style,
// with the grid sized to the resident wave slots of the chip.
#include "launch.h"

namespace sg {

namespace {

// Lane `lane` loads pieces c*64 + lane (c < nch) of a buffer of `bytes`
// bytes; pieces past the end read as zero.  `nch` is wave-uniform, so the
// guards are scalar branches and all loads of a row issue back to back.
template <int NCH, int POLICY>
__device__ __forceinline__ void load_pieces(uint4 (&dst)[NCH], rsrc_t r, int nch, int lane) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        dst[c] = make_uint4(0, 0, 0, 0);
        if (c < nch) dst[c] = load16<POLICY>(r, (uint32_t)(c * kWave + lane) * 16u);
    }
}

template <int M, int NCH, int R>
__global__ __launch_bounds__(kBlock) void rowdot_kernel(const uint4* __restrict__ x,
                                                        const uint4* __restrict__ W, int N,
                                                        int K8, int S, int chunk8,
                                                        int waves_per_split, Epilogue ep) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = blockIdx.x * kWavesPerBlock + wave_id_in_block();
    const int s = wave % S;
    const int q = wave / S;
    if (q >= waves_per_split) return;

    const int k0 = s * chunk8;                     // first piece of this chunk
    const int len = max(0, min(K8 - k0, chunk8));  // pieces in the chunk
    const int nch = (len + kWave - 1) / kWave;     // lane-pieces per row
    const uint32_t bytes = (uint32_t)len * 16u;

    uint4 xr[M][NCH];
#pragma unroll
    for (int m = 0; m < M; ++m)
        load_pieces<NCH, kCached>(xr[m], make_rsrc(x + (int64_t)m * K8 + k0, bytes), nch, lane);

    for (int n0 = q * R; n0 < N; n0 += waves_per_split * R) {
        uint4 wr[R][NCH];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = n0 + r;
            const rsrc_t rs = make_rsrc(W + (int64_t)min(n, N - 1) * K8 + k0, n < N ? bytes : 0u);
            load_pieces<NCH, kStream>(wr[r], rs, nch, lane);
        }
        float acc[R][M];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float a = 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    if (c < nch) a = dot8(xr[m][c], wr[r][c], a);
                acc[r][m] = wave_sum(a);
            }
        }
        // Lane r*M + m stores output (m, n0 + r); the totals are wave-uniform.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = n0 + r;
            if (n >= N) break;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if (lane == r * M + m) {
                    if (ep.partial)
                        ep.partial[((int64_t)s * M + m) * N + n] = acc[r][m];
                    else
                        store_final(ep, (int64_t)m * N + n, acc[r][m]);
                }
            }
        }
    }
}

int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Two rows in flight per wave unless that pushes the wave past 256 VGPRs
// (occupancy below 2 waves per SIMD): (M=2, 16 chunks) and M >= 9.
constexpr int rows_per_iter(int M, int NCH) { return (M >= 9 || (M == 2 && NCH > 8)) ? 1 : 2; }

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

int rowdot_resident_waves(int, int) { return 2048; }  // 256 CUs x 8 waves

int rowdot_grid(int M, int N, int K, int S, int k_chunk) {
    const int nch = (k_chunk + kLaneSpan - 1) / kLaneSpan;
    const int R = rowdot_rows_per_iter(M, nch);
    const int want = (N + R - 1) / R;
    const int cap = (rowdot_resident_waves(M, nch) + S - 1) / S;
    const int Q = want < cap ? want : cap;
    (void)K;
    return (S * Q + kWavesPerBlock - 1) / kWavesPerBlock;
}

template <int M, int NCH>
static hipError_t launch_mn(int N, int K, int S, int k_chunk, int grid, const void* x,
                            const void* W, const Epilogue& ep, hipStream_t stream) {
    const int K8 = K / kPiece;
    const int chunk8 = k_chunk / kPiece;
    constexpr int R = rows_per_iter(M, NCH);
    const int waves_per_split = (grid * kWavesPerBlock) / S;
    rowdot_kernel<M, NCH, R><<<grid, kBlock, 0, stream>>>(static_cast<const uint4*>(x),
                                                         static_cast<const uint4*>(W), N, K8, S,
                                                         chunk8, waves_per_split, ep);
    return hipGetLastError();
}

template <int M>
static hipError_t launch_m(int nch, int N, int K, int S, int k_chunk, int grid, const void* x,
                           const void* W, const Epilogue& ep, hipStream_t stream) {
    if constexpr (M <= 2) {
        // The small-matrix path gets an exact chunk count: no guarded loads.
        switch (nch < 1 ? 1 : nch) {
#define SG_NCH(c) \
    case c: return launch_mn<M, c>(N, K, S, k_chunk, grid, x, W, ep, stream);
            SG_NCH(1) SG_NCH(2) SG_NCH(3) SG_NCH(4) SG_NCH(5) SG_NCH(6) SG_NCH(7) SG_NCH(8)
            SG_NCH(9) SG_NCH(10) SG_NCH(11) SG_NCH(12) SG_NCH(13) SG_NCH(14) SG_NCH(15) SG_NCH(16)
#undef SG_NCH
            default: return hipErrorInvalidValue;
        }
    }
    const int NCH = next_pow2(nch < 1 ? 1 : nch);
    switch (NCH) {
        case 1: return launch_mn<M, 1>(N, K, S, k_chunk, grid, x, W, ep, stream);
        case 2: return launch_mn<M, 2>(N, K, S, k_chunk, grid, x, W, ep, stream);
        case 4:
            if constexpr (M <= 8) return launch_mn<M, 4>(N, K, S, k_chunk, grid, x, W, ep, stream);
            break;
        case 8:
            if constexpr (M <= 4) return launch_mn<M, 8>(N, K, S, k_chunk, grid, x, W, ep, stream);
            break;
        case 16:
            if constexpr (M <= 2) return launch_mn<M, 16>(N, K, S, k_chunk, grid, x, W, ep, stream);
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_rowdot(int M, int N, int K, int S, int k_chunk, int grid, const void* x,
                         const void* W, const Epilogue& ep, hipStream_t stream) {
    const int nch = (k_chunk + kLaneSpan - 1) / kLaneSpan;
    // The waves-per-split count is derived from the grid, which the plan
    // computed with rowdot_grid; the remainder waves of the last block exit.
    switch (M) {
#define SG_CASE(m) \
    case m: return launch_m<m>(nch, N, K, S, k_chunk, grid, x, W, ep, stream);
        SG_CASE(1) SG_CASE(2) SG_CASE(3) SG_CASE(4) SG_CASE(5) SG_CASE(6) SG_CASE(7) SG_CASE(8)
        SG_CASE(9) SG_CASE(10) SG_CASE(11) SG_CASE(12) SG_CASE(13) SG_CASE(14) SG_CASE(15)
#undef SG_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sg
