// plan.cpp -- plan(M, N, K): kernel and tiling choice for one projection shape.
//
// The pages pick a different kernel per batch size -- a dedicated
// small-matrix kernel at batch 1-2, split-K for larger batches -- and tune
// each projection to a kernel size that fills the GPU ("Hyper Optimizing
// Kimi K3 in vLLM" deepnotes page, Method details §1).  On MI355X:
//   M <= 2        row-streaming VALU kernel, no split while the x chunk fits
//                 in registers (K <= 8192), fused epilogue;
//   3 <= M <= 7   the same kernel on K chunks (split-K), the split sized so
//                 the M x-rows of a chunk fit in its registers, reduced
//                 inside the workgroup when the split allows (from M = 6 only
//                 where the team kernel's grid does not fill the GPU);
//   8 <= M <= 64  bf16 matrix-core split-K: up to 16 rows the team kernel
//                 (K split over the waves of a workgroup, reduced in LDS)
//                 when N/16 workgroups fill the GPU; otherwise the chunk
//                 kernel, split factor and row tiling from a
//                 per-compute-unit byte cost model, then the deterministic
//                 reduction kernel.
// A small table measured on MI355X overrides the split factor for known
// shapes, and a text file named by SKINNY_GEMM_TUNE_TABLE can add entries
// ahead of it.  Everything here is host arithmetic; no GPU call is made.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "launch.h"
#include "plan_internal.h"
#include "skinny_gemm.h"

namespace {

constexpr int32_t kMaxNK = 1 << 20;
constexpr int32_t kMaxSplit = 64;
constexpr int kComputeUnits = 256;
// Smallest batch planned on the matrix cores.  Measured on MI355X (K=7168,
// N=4096): from M=8 up the VALU kernel's v_dot2 work per weight byte, M/2
// instructions per bf16 pair, outgrows the weight stream (M=8: 15.0 us VALU
// against 13.8 us MFMA; M=12: 20.7 against 14.0), while at M <= 6 the VALU
// kernel, which needs no second pass, is faster (M=4: 12.8 against 13.8).
constexpr int32_t kMfmaFromM = 8;
constexpr int32_t kTeamUpToM = 16;
// Where its grid of N/16 workgroups fills the compute units, the matrix-core
// team kernel beats the vector-ALU kernels from 3 rows for 4096 <= K <= 8192
// (at most 8 rounds a wave, every round unrolled).  Interleaved A/B on
// MI355X, team against the vector-ALU plan: 4096x7168 M = 3 / 4 / 5 10.83 /
// 10.87 / 10.87 against 11.02 / 11.39 / 12.01 us, 8192x7168 19.26 / 19.20 /
// 19.18 against 19.53 / 20.72 / 21.00 us, 4096x4096 M = 3 7.15 against 7.61
// us.  Outside that range it starts at 6 rows: with longer K (the loop form)
// it lost at 5 rows (4096x7168 before the unrolling: M = 6 12.3 against
// 12.9 us, M = 5 12.3 against 11.9 us), and at short K the streaming kernel
// stays ahead up to 5 rows (4096x2048: M = 3 / 5 5.19 / 5.76 against 5.98 /
// 6.01 us).
// The team kernel's grid of N/16 workgroups counts as filling the GPU from
// 160 workgroups (N >= 2545), five eighths of the compute units.  Interleaved
// A/B on MI355X, team against the plan of a 256-workgroup threshold (vector
// ALU below 8 rows, chunk kernel from 8), K = 7168: N = 2560 M = 3 / 8 / 16
// 9.72 / 11.02 / 11.00 -> 8.96 / 9.64 / 10.93 us, N = 3072 M = 4 / 8 10.26 /
// 11.28 -> 9.54 / 10.00 us (M = 16 11.26 against 11.42), N = 3584 M = 6 / 8 /
// 16 12.14 / 12.96 / 12.93 -> 10.19 / 10.42 / 11.78 us; 3072 x 4096 M = 8
// 8.38 -> 6.74 us.  At N = 2048 (128 workgroups) the other plans stay ahead
// (M = 3 / 16 7.56 / 9.04 against 8.59 / 10.50 us).
constexpr int32_t kTeamMinTiles = 160;
constexpr int32_t kTeamFromM = 3;
constexpr int32_t kTeamFromMOtherK = 6;
constexpr int32_t kTeamFromMMinK = 4096;
constexpr int32_t kTeamFromMMaxK = 8192;

// Choices measured on MI355X for known projection shapes, overriding the
// defaults: {M_lo, M_hi, N, K, kernel (0: default), split (0: default),
// matrix-core tile width (0: default)}.
struct Tuned {
    int32_t m_lo, m_hi, n, k, kernel, split, tile_n;
};
constexpr Tuned kTuned[] = {
    // 64-row batches on the 117 MB projections: 256-row workgroups in 8
    // splits (32.9 us at 8192 -> 7168, 29.8 us at 7168 -> 8192) beat the
    // cost model's pick of 9 splits (41.4 us) and 128-row tiles (35.7 us)
    {33, 64, 7168, 8192, SG_KERNEL_SPLITK_MFMA, 8, 256},
    {33, 64, 8192, 7168, SG_KERNEL_SPLITK_MFMA, 8, 256},
    // the MoE step's router + shared-expert GEMM (384 + 2048 rows) at one or
    // two tokens: 2 rows a wave on the streaming kernel leave its 304
    // workgroups uneven over 256 compute units; teams of 4 waves on K chunks
    // measured 7.8 / 8.0 us against 8.6 / 9.1 us (M = 1 / 2)
    {1, 2, 2432, 7168, SG_KERNEL_GEMV, 4, 0},
};

bool split_ok(int32_t S) { return S >= 1 && S <= kMaxSplit; }

// Chunk width: ceil(K / S) rounded up to whole 128-byte cache lines (64
// bf16), so every chunk starts on a line boundary of each weight row; the
// last chunk is the shorter one.  (With 16-byte granularity a chunk edge
// splits a line between two workgroups, often on different XCDs, and the
// weight stream measured 20-50% more HBM traffic than the weight bytes.)
int32_t chunk_of(int32_t K, int32_t S) {
    const int64_t lines = ((int64_t)K + 64 * (int64_t)S - 1) / (64 * (int64_t)S);
    return (int32_t)(64 * lines);
}

// No chunk of an automatic plan is empty.
bool no_empty_chunk(int32_t K, int32_t S) { return K == 0 || (int64_t)(S - 1) * chunk_of(K, S) < K; }

int nch_of(int32_t chunk) { return (chunk + sg::kLaneSpan - 1) / sg::kLaneSpan; }

bool rowdot_fits(int32_t M, int32_t K, int32_t S) {
    return nch_of(chunk_of(K, S)) <= sg::rowdot_nch_cap(M);
}

// Smallest split that keeps the rowdot x registers within the cap for M,
// preferring one a workgroup can reduce by itself (no second pass).
int32_t rowdot_split(int32_t M, int32_t N, int32_t K) {
    int32_t S0 = -1;
    for (int32_t S = 1; S <= 8 && S0 < 0; S *= 2)
        if (sg::rowdot_team_split_ok(M, S) && no_empty_chunk(K, S) && rowdot_fits(M, K, S))
            S0 = S;
    if (S0 < 0) {
        for (int32_t S = 1; S <= kMaxSplit; ++S)
            if (no_empty_chunk(K, S) && rowdot_fits(M, K, S)) return S;
        return -1;
    }
    // Few rows (a router's 384 experts, a 1024-row matrix): the row groups
    // alone leave most compute units idle, so split K over more waves of
    // each team while the teams still fit the resident wave slots.
    const int64_t groups = (N + 1) / 2;
    for (int32_t S = 2 * S0; S <= 4; S *= 2) {
        if (groups * S > sg::rowdot_resident_waves(M, 1)) break;
        if (!sg::rowdot_team_split_ok(M, S) || !no_empty_chunk(K, S)) break;
        if (groups * S0 >= kComputeUnits * 2) break;  // already two waves per CU
        S0 = S;
    }
    return S0;
}

bool mfma_chunk_fits(int32_t M, int32_t K, int32_t S, int32_t tile_n) {
    return sg::mfma_chunk_lds_bytes(M, chunk_of(K, S), tile_n) <= sg::kMfmaMaxLds;
}

// Cost of a chunk-kernel plan in bytes per compute unit: the weight bytes of
// the busiest unit -- ceil(tiles*S / 256) workgroups of tile_n rows x K/S --
// plus half the x bytes those workgroups stage from L2 into LDS, plus a
// tenth of the x operand bytes read back from LDS (MT/NT per weight byte),
// plus the partials written and read back (2 * S*M*N*4 bytes over the 256
// units).
int64_t mfma_cost(int32_t M, int32_t N, int32_t K, int32_t S, int32_t tile_n) {
    const int64_t tiles = (N + tile_n - 1) / tile_n;
    const int64_t per_unit = (tiles * S + kComputeUnits - 1) / kComputeUnits;
    const int64_t chunk = chunk_of(K, S);
    const int64_t w_bytes = per_unit * tile_n * 2 * chunk;
    const int64_t x_bytes = per_unit * M * chunk;
    const int64_t mt = (M + 15) / 16, nt = tile_n / sg::kMfmaTileN;
    const int64_t lds_bytes = w_bytes * mt / nt / 10;
    const int64_t p_bytes = 8 * (int64_t)S * M * N / kComputeUnits;
    return w_bytes + x_bytes + lds_bytes + p_bytes;
}

// Split and tile width for the matrix-core chunk kernel: the cheapest pair
// whose x chunk fits in LDS (ties: the smaller split, then 128-row tiles).
// Splits that cut K into equal whole-line chunks are preferred: on MI355X a
// ragged split measured slower than the equal split next to it despite a
// shorter chunk (K=8192, M=16: 9 splits 26.2 us, 8 splits 25.2 us).  A
// forced split or tile width narrows the search.  False if nothing fits.
bool mfma_choose(int32_t M, int32_t N, int32_t K, int32_t force_split, int32_t force_tile,
                 int32_t* split, int32_t* tile_n) {
    for (int pass = 0; pass < 2; ++pass) {  // 0: equal chunks only, 1: any
        bool found = false;
        int64_t best_cost = 0;
        for (int32_t t = sg::kMfmaTileN; t <= 2 * sg::kMfmaTileN; t *= 2) {
            if (force_tile > 0 && t != force_tile) continue;
            for (int32_t S = 1; S <= kMaxSplit; ++S) {
                if (force_split > 0 && S != force_split) continue;
                if (force_split <= 0 && !no_empty_chunk(K, S)) break;
                if (pass == 0 && force_split <= 0 && K % (64 * S) != 0) continue;
                if (!mfma_chunk_fits(M, K, S, t)) continue;
                const int64_t cost = mfma_cost(M, N, K, S, t);
                if (!found || cost < best_cost) {
                    found = true;
                    best_cost = cost;
                    *split = S;
                    *tile_n = t;
                }
            }
        }
        if (found) return true;
    }
    return false;
}

// Entries from the file SKINNY_GEMM_TUNE_TABLE names, read once per process.
// One entry a line, seven integers: M_lo M_hi N K kernel split tile_n (0 for
// "the planner's choice", as in kTuned; kernel is an sg_kernel value); text
// after '#' is a comment.  A line that does not parse, or an entry out of
// range, rejects the whole file: the built-in table alone applies and one
// warning goes to stderr.
std::vector<Tuned> g_user_tuned;
std::once_flag g_user_tuned_once;

bool parse_tuned_line(const char* line, Tuned* t, bool* empty) {
    char buf[512];
    std::strncpy(buf, line, sizeof buf - 1);
    buf[sizeof buf - 1] = '\0';
    if (char* hash = std::strchr(buf, '#')) *hash = '\0';
    long v[7];
    int n = 0;
    char* p = buf;
    while (n < 8) {
        char* end = nullptr;
        const long x = std::strtol(p, &end, 10);
        if (end == p) break;
        if (n < 7) v[n] = x;
        ++n;
        p = end;
    }
    for (; *p; ++p)
        if (*p != ' ' && *p != '\t' && *p != '\r' && *p != '\n') return false;  // stray text
    *empty = n == 0;
    if (n == 0) return true;
    if (n != 7) return false;
    const bool ok = v[0] >= 1 && v[0] <= v[1] && v[1] <= SG_MAX_M && v[2] >= 1 &&
                    v[2] <= kMaxNK && v[3] >= 0 && v[3] <= kMaxNK && v[4] >= 0 &&
                    v[4] <= SG_KERNEL_SPLITK_MFMA && v[5] >= 0 && v[5] <= kMaxSplit &&
                    (v[6] == 0 || v[6] == sg::kMfmaTeamTileN || v[6] == sg::kMfmaTileN ||
                     v[6] == 2 * sg::kMfmaTileN);
    if (!ok) return false;
    *t = Tuned{(int32_t)v[0], (int32_t)v[1], (int32_t)v[2], (int32_t)v[3],
               (int32_t)v[4], (int32_t)v[5], (int32_t)v[6]};
    return true;
}

void load_user_tuned() {
    const char* path = std::getenv("SKINNY_GEMM_TUNE_TABLE");
    if (!path || !*path) return;
    FILE* f = std::fopen(path, "r");
    if (!f) {
        std::fprintf(stderr, "[skinny_gemm] SKINNY_GEMM_TUNE_TABLE=%s: cannot open; ignored\n",
                     path);
        return;
    }
    std::vector<Tuned> rows;
    char line[512];
    int lineno = 0;
    bool bad = false;
    while (std::fgets(line, sizeof line, f)) {
        ++lineno;
        Tuned t{};
        bool empty = false;
        if (std::strlen(line) == sizeof line - 1 || !parse_tuned_line(line, &t, &empty)) {
            std::fprintf(stderr, "[skinny_gemm] SKINNY_GEMM_TUNE_TABLE=%s line %d: expected "
                                 "M_lo M_hi N K kernel split tile_n; file ignored\n",
                         path, lineno);
            bad = true;
            break;
        }
        if (!empty) rows.push_back(t);
    }
    std::fclose(f);
    if (!bad) g_user_tuned.swap(rows);
}

// The first matching entry: the user's file, then the built-in table.
const Tuned* tuned_for(int32_t M, int32_t N, int32_t K) {
    std::call_once(g_user_tuned_once, load_user_tuned);
    for (const Tuned& t : g_user_tuned)
        if (M >= t.m_lo && M <= t.m_hi && N == t.n && K == t.k) return &t;
    for (const Tuned& t : kTuned)
        if (M >= t.m_lo && M <= t.m_hi && N == t.n && K == t.k) return &t;
    return nullptr;
}

}  // namespace

namespace sg {

namespace {

sg_status make_plan_impl(int32_t M, int32_t N, int32_t K, int32_t kernel, int32_t split_k,
                         int32_t two_pass, int32_t tile_n, bool use_tuned, sg_plan* out);

}  // namespace

sg_status make_plan(int32_t M, int32_t N, int32_t K, int32_t kernel, int32_t split_k,
                    int32_t two_pass, int32_t tile_n, sg_plan* out) {
    const sg_status st = make_plan_impl(M, N, K, kernel, split_k, two_pass, tile_n, true, out);
    // A tuned entry the planner cannot honour for this shape (a user table's
    // split that leaves an empty chunk, say) gives way to the default plan.
    if (st == SG_ERR_PLAN && kernel <= 0 && split_k <= 0 && tile_n <= 0 &&
        tuned_for(M, N, K) != nullptr)
        return make_plan_impl(M, N, K, kernel, split_k, two_pass, tile_n, false, out);
    return st;
}

namespace {

sg_status make_plan_impl(int32_t M, int32_t N, int32_t K, int32_t kernel, int32_t split_k,
                         int32_t two_pass, int32_t tile_n, bool use_tuned, sg_plan* out) {
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
        const bool team_fills = (N + kMfmaTeamTileN - 1) / kMfmaTeamTileN >= kTeamMinTiles;
        const bool team_k = K >= kTeamFromMMinK && K <= kTeamFromMMaxK;
        const int32_t mfma_from =
            team_fills ? (team_k ? kTeamFromM : kTeamFromMOtherK) : kMfmaFromM;
        kernel = M <= 2 ? SG_KERNEL_GEMV
                        : (M < mfma_from ? SG_KERNEL_SPLITK_VALU : SG_KERNEL_SPLITK_MFMA);
        if (const Tuned* t = use_tuned ? tuned_for(M, N, K) : nullptr) {
            if (t->kernel > 0) kernel = t->kernel;
            if (split_k <= 0 && t->split > 0) split_k = t->split;
            if (tile_n <= 0 && t->tile_n > 0) tile_n = t->tile_n;
        }
    }

    switch (kernel) {
        case SG_KERNEL_GEMV:
            if (M > 2) return SG_ERR_PLAN;
            [[fallthrough]];
        case SG_KERNEL_SPLITK_VALU: {
            if (M > 15) return SG_ERR_PLAN;
            if (split_k <= 0) split_k = rowdot_split(M, N, K);
            if (!split_ok(split_k)) return SG_ERR_PLAN;
            if (!rowdot_fits(M, K, split_k)) return SG_ERR_PLAN;
            const bool team_ok = rowdot_team_split_ok(M, split_k);
            if (two_pass < 0) two_pass = (split_k > 1 && !team_ok) ? 1 : 0;
            if (two_pass == 0 && !team_ok) return SG_ERR_PLAN;
            if (split_k == 1) two_pass = 0;
            p.k_chunk = chunk_of(K, split_k);
            int g = 0;
            if (rowstream_plan(M, N, K, split_k, two_pass != 0, &g)) {
                p.tile_n = 1;  // the streaming kernel: one row per step
                p.grid = g;
            } else {
                p.tile_n = rowdot_rows_per_iter(M, nch_of(p.k_chunk));
                p.grid = rowdot_grid(M, N, K, split_k, p.k_chunk, two_pass != 0);
            }
            break;
        }
        case SG_KERNEL_SPLITK_MFMA: {
            // Default: the chunk kernel, its S partials summed by the second
            // pass.  two_pass == 0 asks for the team kernel (S in 1, 2, 4, 8
            // reduced inside the workgroup).
            // Up to 16 rows (one x row tile) the team kernel -- no
            // workspace, no second launch -- when its grid of N/16
            // workgroups fills the compute units (kTeamMinTiles).  Measured on MI355X with
            // x through the per-wave LDS tile: K=7168, N=4096, M=16 13.5 us
            // against 14.3 us for the chunk kernel and its reduction; from
            // M=20 (two row tiles) the chunk kernel wins (16.6 against 15.4).
            // With twice as many 16-row tiles as compute units (N >= 8161)
            // each wave of the team kernel takes two tiles and reads each x
            // operand once for both; that keeps it ahead of the chunk kernel
            // up to 16 rows: K=7168, N=8192, M = 12 / 16 22.0 / 22.2 us
            // against 22.5 / 22.6 us (chunk); residual M = 16 22.3 against
            // 22.9.  (With one tile a wave it lost there from 12 rows: 23.1
            // / 24.1 us.)
            const int32_t team_tiles = (N + kMfmaTeamTileN - 1) / kMfmaTeamTileN;
            const bool team_auto = two_pass < 0 && tile_n == 0 && M <= kTeamUpToM &&
                                   team_tiles >= kTeamMinTiles &&
                                   (split_k <= 0 || mfma_team_split_ok(split_k));
            const bool team_asked = two_pass == 0 || tile_n == kMfmaTeamTileN || team_auto;
            int32_t S = 0, t = 0;
            if (!team_asked && tile_n != 0 && tile_n != kMfmaTileN && tile_n != 2 * kMfmaTileN)
                return SG_ERR_PLAN;
            if (!team_asked && mfma_choose(M, N, K, split_k, tile_n, &S, &t)) {
                split_k = S;
                two_pass = S > 1 ? 1 : 0;
                p.k_chunk = chunk_of(K, S);
                p.tile_n = t;
                p.grid = mfma_grid_tiles(N, t) * S;
                break;
            }
            // team kernel: asked for, or the x chunk would not fit in LDS
            if (two_pass > 0 || (tile_n != 0 && tile_n != kMfmaTeamTileN)) return SG_ERR_PLAN;
            if (split_k <= 0) {
                split_k = 8;
                while (split_k > 1 && !no_empty_chunk(K, split_k)) split_k /= 2;
            }
            if (!mfma_team_split_ok(split_k)) return SG_ERR_PLAN;
            p.k_chunk = chunk_of(K, split_k);
            p.tile_n = kMfmaTeamTileN;
            p.grid = mfma_team_grid(M, N, K);
            two_pass = 0;
            break;
        }
        default:
            return SG_ERR_PLAN;
    }
    p.kernel = kernel;
    p.split_k = split_k;
    p.two_pass = two_pass;
    // chunk-kernel partials are [S, N, M padded to whole 16-row tiles]; the
    // vector-ALU kernel's are [S, M, N]
    const bool chunk = kernel == SG_KERNEL_SPLITK_MFMA && p.tile_n >= kMfmaTileN;
    const size_t rows = chunk ? (size_t)mfma_partial_rows(M) : (size_t)M;
    p.workspace_bytes =
        two_pass ? ((size_t)split_k * rows * N * sizeof(float) + 255) / 256 * 256 : 0;
    *out = p;
    return SG_OK;
}

}  // namespace

bool plan_matches(const sg_plan* p) {
    // The matrix-core path has two kernels; the plan's tile width says which
    // one (and which row tiling) it was made for.
    int32_t request = p->two_pass;
    int32_t tile = 0;
    if (p->kernel == SG_KERNEL_SPLITK_MFMA) {
        request = p->tile_n == kMfmaTeamTileN ? 0 : 1;
        tile = p->tile_n;
    }
    sg_plan q;
    if (make_plan(p->M, p->N, p->K, p->kernel, p->split_k, request, tile, &q) != SG_OK)
        return false;
    return q.kernel == p->kernel && q.split_k == p->split_k && q.k_chunk == p->k_chunk &&
           q.tile_n == p->tile_n && q.grid == p->grid && q.two_pass == p->two_pass &&
           q.workspace_bytes == p->workspace_bytes;
}

}  // namespace sg

extern "C" sg_status skinny_gemm_plan(int32_t M, int32_t N, int32_t K, sg_plan* out) {
    return sg::make_plan(M, N, K, 0, 0, -1, 0, out);
}

extern "C" sg_status skinny_gemm_plan_force(int32_t M, int32_t N, int32_t K, int32_t kernel,
                                            int32_t split_k, int32_t two_pass, int32_t tile_n,
                                            sg_plan* out) {
    return sg::make_plan(M, N, K, kernel <= 0 ? 0 : kernel, split_k, two_pass < 0 ? -1 : two_pass,
                         tile_n < 0 ? 0 : tile_n, out);
}
