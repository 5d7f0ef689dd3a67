// plan.cpp -- plan(M, N, K): kernel and tiling choice for one projection shape.
//
// The pages pick a different kernel per batch size -- a dedicated
// small-matrix kernel at batch 1-2, split-K for larger batches -- and tune
// each projection to a kernel size that fills the GPU ("Hyper Optimizing
// Kimi K3 in vLLM" deepnotes page, Method details §1).  On MI355X:
//   M <= 2        row-streaming VALU kernel, no split while the x chunk fits
//                 in registers (K <= 8192), fused epilogue;
//   3 <= M <= 15  the same kernel on K chunks (split-K), the split sized so
//                 the M x-rows of a chunk fit in 128 VGPRs, then the
//                 deterministic reduction;
//   16 <= M <= 64 bf16 matrix-core split-K, split chosen so the grid covers
//                 the 256 compute units without the fp32 partials growing
//                 large next to the weights, then the reduction.
// A small table measured on MI355X overrides the split factor for known
// shapes.  Everything here is host arithmetic; no GPU call is made.
#include <cstdlib>

#include "launch.h"
#include "plan_internal.h"
#include "skinny_gemm.h"

namespace {

constexpr int32_t kMaxNK = 1 << 20;
constexpr int32_t kMaxSplit = 64;
constexpr int kComputeUnits = 256;

// Split factors measured on MI355X (bench sweeps); {M_lo, M_hi, N, K, S}.
struct Tuned {
    int32_t m_lo, m_hi, n, k, split;
};
constexpr Tuned kTuned[] = {
    {0, 0, 0, 0, 0},  // sentinel
};

bool split_ok(int32_t S) { return S >= 1 && S <= kMaxSplit; }

// Chunk width: ceil(K / S) rounded up to whole 16-byte groups (8 bf16), so
// every chunk starts on a 16-byte boundary; the last chunk is the shorter one.
int32_t chunk_of(int32_t K, int32_t S) {
    const int64_t groups = ((int64_t)K / 8 + S - 1) / S;
    return (int32_t)(8 * groups);
}

// No chunk of an automatic plan is empty.
bool no_empty_chunk(int32_t K, int32_t S) { return K == 0 || (int64_t)(S - 1) * chunk_of(K, S) < K; }

int nch_of(int32_t chunk) { return (chunk + sg::kLaneSpan - 1) / sg::kLaneSpan; }

bool rowdot_fits(int32_t M, int32_t K, int32_t S) {
    return nch_of(chunk_of(K, S)) <= sg::rowdot_nch_cap(M);
}

// Smallest split that keeps the rowdot x registers within the cap for M,
// preferring one a workgroup can reduce by itself (no second pass).
int32_t rowdot_split(int32_t M, int32_t K) {
    for (int32_t S = 1; S <= 8; S *= 2)
        if (sg::rowdot_team_split_ok(M, S) && no_empty_chunk(K, S) && rowdot_fits(M, K, S))
            return S;
    for (int32_t S = 1; S <= kMaxSplit; ++S)
        if (no_empty_chunk(K, S) && rowdot_fits(M, K, S)) return S;
    return -1;
}

bool mfma_chunk_fits(int32_t M, int32_t K, int32_t S) {
    return sg::mfma_chunk_lds_bytes(M, chunk_of(K, S)) <= sg::kMfmaMaxLds;
}

// Split for the matrix-core chunk kernel.  Cost model in bytes per compute
// unit: the weight bytes of the busiest unit -- ceil(tiles*S / 256) workgroups
// of 128 rows x K/S each -- plus the partials written and read back
// (2 * S*M*N*4 bytes spread over the 256 units).  Among the splits whose x
// chunk fits in LDS, the cheapest wins (ties: the smaller split).
int32_t mfma_split(int32_t M, int32_t N, int32_t K) {
    const int64_t tiles = (N + sg::kMfmaTileN - 1) / sg::kMfmaTileN;
    int32_t best = -1;
    int64_t best_cost = 0;
    for (int32_t S = 1; S <= kMaxSplit; ++S) {
        if (!no_empty_chunk(K, S)) break;
        if (!mfma_chunk_fits(M, K, S)) continue;
        const int64_t per_unit = (tiles * S + kComputeUnits - 1) / kComputeUnits;
        const int64_t w_bytes = per_unit * sg::kMfmaTileN * 2 * (int64_t)chunk_of(K, S);
        const int64_t p_bytes = 8 * (int64_t)S * M * N / kComputeUnits;
        const int64_t cost = w_bytes + p_bytes;
        if (best < 0 || cost < best_cost) {
            best = S;
            best_cost = cost;
        }
    }
    return best;
}

int32_t tuned_split(int32_t M, int32_t N, int32_t K) {
    for (const Tuned& t : kTuned)
        if (t.split > 0 && M >= t.m_lo && M <= t.m_hi && N == t.n && K == t.k) return t.split;
    return -1;
}

}  // namespace

namespace sg {

sg_status make_plan(int32_t M, int32_t N, int32_t K, int32_t kernel, int32_t split_k,
                    int32_t two_pass, sg_plan* out) {
    if (!out) return SG_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || N > kMaxNK || K > kMaxNK) return SG_ERR_SHAPE;
    if (M > SG_MAX_M) return SG_ERR_UNSUPPORTED;
    if (K % 8 != 0) return SG_ERR_ALIGN;

    sg_plan p{};
    p.M = M;
    p.N = N;
    p.K = K;
    if (M == 0 || N == 0) {
        if (kernel > 0 && kernel != SG_KERNEL_NONE) return SG_ERR_PLAN;
        p.kernel = SG_KERNEL_NONE;
        p.split_k = 1;
        p.k_chunk = K;
        p.two_pass = 0;
        *out = p;
        return SG_OK;
    }

    if (kernel <= 0) {
        kernel = M <= 2 ? SG_KERNEL_GEMV : (M < 16 ? SG_KERNEL_SPLITK_VALU : SG_KERNEL_SPLITK_MFMA);
        if (split_k <= 0) split_k = tuned_split(M, N, K);
    }

    switch (kernel) {
        case SG_KERNEL_GEMV:
            if (M > 2) return SG_ERR_PLAN;
            [[fallthrough]];
        case SG_KERNEL_SPLITK_VALU: {
            if (M > 15) return SG_ERR_PLAN;
            if (split_k <= 0) split_k = rowdot_split(M, K);
            if (!split_ok(split_k)) return SG_ERR_PLAN;
            if (!rowdot_fits(M, K, split_k)) return SG_ERR_PLAN;
            const bool team_ok = rowdot_team_split_ok(M, split_k);
            if (two_pass < 0) two_pass = (split_k > 1 && !team_ok) ? 1 : 0;
            if (two_pass == 0 && !team_ok) return SG_ERR_PLAN;
            if (split_k == 1) two_pass = 0;
            p.k_chunk = chunk_of(K, split_k);
            const int R = rowdot_rows_per_iter(M, nch_of(p.k_chunk));
            p.tile_n = R;
            p.grid = rowdot_grid(M, N, K, split_k, p.k_chunk, two_pass != 0);
            break;
        }
        case SG_KERNEL_SPLITK_MFMA: {
            // Default: the chunk kernel, its S partials summed by the second
            // pass.  two_pass == 0 asks for the team kernel (S in 1, 2, 4, 8
            // reduced inside the workgroup).
            if (two_pass == 0) {
                if (split_k <= 0) split_k = 8;
                while (split_k > 1 && !no_empty_chunk(K, split_k)) split_k /= 2;
                if (!mfma_team_split_ok(split_k)) return SG_ERR_PLAN;
                p.k_chunk = chunk_of(K, split_k);
                p.tile_n = kMfmaTeamTileN;
                p.grid = (N + kMfmaTeamTileN - 1) / kMfmaTeamTileN;
                two_pass = 0;
                break;
            }
            if (split_k <= 0) split_k = mfma_split(M, N, K);
            if (!split_ok(split_k)) return SG_ERR_PLAN;
            if (!mfma_chunk_fits(M, K, split_k)) {
                // x chunk too large for LDS: the team kernel, if allowed
                if (two_pass > 0 || !mfma_team_split_ok(split_k)) return SG_ERR_PLAN;
                p.k_chunk = chunk_of(K, split_k);
                p.tile_n = kMfmaTeamTileN;
                p.grid = (N + kMfmaTeamTileN - 1) / kMfmaTeamTileN;
                two_pass = 0;
                break;
            }
            two_pass = split_k > 1 ? 1 : 0;
            p.k_chunk = chunk_of(K, split_k);
            p.tile_n = kMfmaTileN;
            p.grid = mfma_grid_tiles(N) * split_k;
            break;
        }
        default:
            return SG_ERR_PLAN;
    }
    p.kernel = kernel;
    p.split_k = split_k;
    p.two_pass = two_pass;
    p.workspace_bytes =
        two_pass ? ((size_t)split_k * M * N * sizeof(float) + 255) / 256 * 256 : 0;
    *out = p;
    return SG_OK;
}

bool plan_matches(const sg_plan* p) {
    // The matrix-core path has two kernels; the plan's tile width says which
    // one it was made for (the team kernel is requested with two_pass == 0).
    int32_t request = p->two_pass;
    if (p->kernel == SG_KERNEL_SPLITK_MFMA) request = p->tile_n == kMfmaTileN ? 1 : 0;
    sg_plan q;
    if (make_plan(p->M, p->N, p->K, p->kernel, p->split_k, request, &q) != SG_OK) return false;
    return q.kernel == p->kernel && q.split_k == p->split_k && q.k_chunk == p->k_chunk &&
           q.tile_n == p->tile_n && q.grid == p->grid && q.two_pass == p->two_pass &&
           q.workspace_bytes == p->workspace_bytes;
}

}  // namespace sg

extern "C" sg_status skinny_gemm_plan(int32_t M, int32_t N, int32_t K, sg_plan* out) {
    return sg::make_plan(M, N, K, 0, 0, -1, out);
}

extern "C" sg_status skinny_gemm_plan_force(int32_t M, int32_t N, int32_t K, int32_t kernel,
                                            int32_t split_k, int32_t two_pass, sg_plan* out) {
    return sg::make_plan(M, N, K, kernel <= 0 ? 0 : kernel, split_k, two_pass < 0 ? -1 : two_pass,
                         out);
}
