// launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/skinny_gemm.h).  Each launcher
// checks nothing: the C-ABI layer has validated every argument before.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sg_device.h"

namespace sg {

// Largest chunk count (x registers: M * nch * 4 VGPRs) the row-streaming
// VALU kernel is instantiated for at a given M; nch = ceil(k_chunk / 512).
int rowdot_nch_cap(int M);
// Rows each wavefront handles per iteration in the row-streaming kernel.
int rowdot_rows_per_iter(int M, int nch);
// Wavefront slots the row-streaming kernel aims to keep resident.
int rowdot_resident_waves(int M, int nch);

// Whether an S-way split can be reduced inside one workgroup (a team of S
// waves) by the row-streaming kernel at batch size M.
bool rowdot_team_split_ok(int M, int S);
int rowdot_block_threads(int S, bool two_pass);
// Whether a vector-ALU plan runs the streaming kernel -- one row per step,
// the next row's loads in flight -- and its grid: M <= 2 with one K chunk,
// or M = 3, 4 with teams of 2 or 4 waves on K chunks; x staged in LDS.
constexpr int kRowstreamMaxIters = 4;      // rows a wave, M <= 2
constexpr int kRowstreamMaxTeamIters = 8;  // rows a team, M = 3, 4
bool rowstream_plan(int M, int N, int K, int S, bool two_pass, int* grid);

// Row-streaming VALU kernel (small-matrix path and VALU split-K).
// x [M, K], W [N, K]; split s covers pieces [s*chunk8, min(K8, (s+1)*chunk8)).
// two_pass: write split partials to ep.partial ([S, M, N]) instead of
// reducing them inside the workgroup.
hipError_t launch_rowdot(int M, int N, int K, int S, int k_chunk, int grid, bool two_pass,
                         const void* x, const void* W, const Epilogue& ep,
                         hipStream_t stream);
int rowdot_grid(int M, int N, int K, int S, int k_chunk, bool two_pass);

// bf16 matrix-core split-K (8 <= M <= 64, any M >= 1 when forced).
// Team kernel: S waves (S in {1,2,4,8}) of one workgroup split K over a
// 16-row tile and add their partials in LDS; grid ceil(N/16).
constexpr int kMfmaTeamTileN = 16;
// From this many rows, 12 to 16 batch rows and a row pitch that is not a
// multiple of 8 KB, each wave of the team kernel takes two 16-row tiles,
// sharing every x operand read between them.
constexpr int kMfmaTeamTwoTilesFromN = 8161;
constexpr int kMfmaTeamTwoTilesFromM = 12;
int mfma_team_tiles_per_wave(int M, int N, int K);
int mfma_team_grid(int M, int N, int K);  // workgroups of the team kernel's launch
bool mfma_team_split_ok(int S);
hipError_t launch_mfma_team(int M, int N, int K, int S, int k_chunk, const void* x,
                            const void* W, const Epilogue& ep, hipStream_t stream);
// Chunk kernel: workgroups of tile_n rows (128: 16 per wave, or 256: 32 per
// wave sharing each x operand load) x one K chunk, the x chunk staged in LDS;
// partials to ep.partial ([S, N, mfma_partial_rows(M)], rows m >= M zero) for
// the reduction kernel when S > 1; grid (mfma_grid_tiles(N, tile_n), S).
constexpr int kMfmaTileN = 128;  // W rows per workgroup with 16 rows per wave
constexpr size_t kMfmaMaxLds = 160 * 1024;
constexpr int kXcds = 8;         // MI355X: 8 XCDs, each with its own L2
inline int mfma_partial_rows(int M) { return 16 * ((M + 15) / 16); }
size_t mfma_chunk_lds_bytes(int M, int k_chunk, int tile_n);
// Column tiles of the chunk kernel's grid: ceil(N/tile_n) padded to a
// multiple of kXcds (the padding workgroups exit at once).
int mfma_grid_tiles(int N, int tile_n);
hipError_t launch_splitk_mfma(int M, int N, int K, int S, int k_chunk, int tile_n,
                              const void* x, const void* W, const Epilogue& ep,
                              hipStream_t stream);

// Deterministic split-K reduction: y[i] = P[0,i] + ... + P[S-1,i] (s
// ascending, fp32), then the final epilogue.
hipError_t launch_reduce(const float* P, int S, int64_t MN, const Epilogue& ep,
                         hipStream_t stream);
// The same sum for partials made by the chunk kernel ([S, N, Mp] layout):
// one workgroup per (column tile, 16-column slice), laid out so it runs on the
// XCD that wrote the tile's partials.
hipError_t launch_reduce_tiles(const float* P, int S, int M, int N, int tile_n,
                               const Epilogue& ep, hipStream_t stream);

// Per-expert token table.  ws points at the grouped workspace (layout in
// GroupedWorkspace).
struct GroupedWorkspace {
    int32_t* counts;       // [E]
    int32_t* offsets;      // [E+1]
    int32_t* sorted;       // [P]
    int32_t* invalid;      // [1]
    int32_t* active;       // [E]   experts with counts > 0, ascending
    int32_t* num_active;   // [1]
};
GroupedWorkspace grouped_workspace_layout(void* ws, int E, int P);
size_t grouped_workspace_bytes(int E, int P);

hipError_t launch_moe_table(const int32_t* ids, int T, int topk, int E, int N,
                            const GroupedWorkspace& g, int32_t* user_offsets,
                            int32_t* user_sorted, int32_t* user_invalid, float* out,
                            hipStream_t stream);

constexpr int kGroupedRowsPerWave = 8;  // even: rows go two at a time
constexpr int kGroupedTileN = kGroupedRowsPerWave * kWavesPerBlock;  // 32 rows per item
// Fused table + grouped projection for small tables when no table output is
// asked for: P = T * topk <= kFusedMaxPairs, E <= kFusedMaxExperts (LDS:
// (P + 2E) ints per workgroup).
constexpr int kFusedMaxPairs = 512;
constexpr int kFusedMaxExperts = 4096;
hipError_t launch_grouped_fused(const void* x, int T, const void* W, const int32_t* ids, int E,
                                int N, int K, int topk, float* out, hipStream_t stream);
// Router top-k and the fused grouped projection in one launch, for a few
// tokens: 1 <= T <= kRouteFusedMaxT, E <= kRouteFusedMaxExperts (at most 8
// keys a lane), N >= 1.  ids [T, k] (and top [T, k] when non-null) are
// written as by launch_router_topk.  With N_shared > 0 the launch also
// writes shared_out [T, N_shared] = x W_shared^T, streamed while it ranks.
constexpr int kRouteFusedMaxT = kWavesPerBlock;  // one ranking wave per token
constexpr int kRouteFusedMaxExperts = 512;
hipError_t launch_route_grouped(const float* scores, int64_t ld, int T, int E, int k,
                                int32_t* ids, float* top, const void* x, const void* W, int N,
                                int K, float* out, const void* W_shared, int N_shared,
                                float* shared_out, hipStream_t stream);
hipError_t launch_grouped(const void* x, int T, const void* W, int E, int N, int K, int topk,
                          const GroupedWorkspace& g, float* out, hipStream_t stream);

hipError_t launch_prefetch(const void* W, size_t bytes, hipStream_t stream);
// Read-bandwidth probe: the M <= 2 kernel's load shape over a [rows,
// row_bytes] matrix with no arithmetic (probe.hip).
hipError_t launch_read_probe(const void* W, int rows, int row_bytes, int rows_per_iter, int grid,
                             hipStream_t stream);

// Projection with FP8 e4m3 weights: codes [N, K], fp32 scales [ceil(N/128),
// ceil(K/128)] (one per 128 x 128 block).  1 <= M <= kFp8MaxM, K % 16 == 0;
// at M <= 2, M * K <= kFp8MaxMK (the LDS that stages x); at M = 3, 4 x
// stays in the registers of a team of at most 8 waves: K <= 16384.  From
// kFp8MfmaFromM rows the matrix-core kernel runs (any K, M <= 16).  fp8_split: the K split (S waves a team, chunk in
// 16-code units, loads per row; 0 loads for the matrix-core kernel) the
// kernel runs, false if the shape is outside those limits.
constexpr int kFp8MaxM = 16;
constexpr int kFp8MfmaFromM = 5;  // from here the matrix-core kernel
constexpr int64_t kFp8MaxMK = 32768;
bool fp8_size_ok(int M, int K);
bool fp8_split(int M, int N, int K, int* splits, int* chunk16, int* nch);
hipError_t launch_fp8(int M, int N, int K, const void* x, const void* Wq, const float* Ws,
                      const Epilogue& ep, hipStream_t stream);

// Projection with MXFP4 weights (1 <= M <= kMxfp4MaxM, K % 32 == 0):
// Wq [N, K/2] e2m1 codes, Ws [N, K/32] e8m0 scales.  Below kMxfp4MfmaFromM
// rows the VALU kernel runs; mxfp4_split gives its blocks per lane and team
// split for (M, K), false when K needs more than kMxfp4MaxSplit waves per
// row.  From kMxfp4MfmaFromM rows the matrix-core kernel runs (any K).
constexpr int kMxfp4MaxM = 16;
constexpr int kMxfp4MfmaFromM = 9;  // measured: the VALU kernel is faster through M = 8
constexpr int kMxfp4MaxSplit = 8;
bool mxfp4_split(int M, int K, int* nb, int* splits);
hipError_t launch_mxfp4(int M, int N, int K, const void* x, const void* Wq, const uint8_t* Ws,
                        const Epilogue& ep, hipStream_t stream);

// Projection with low-precision weights for 17 <= M <= 64 (both formats):
// workgroups of 128 * NT weight rows x one K chunk, x staged in LDS, fp32
// partials [S, N, 16*MT] through the workspace and the tiled reduction when
// S > 1.  FP8: Wq [N, K] e4m3 codes, Ws fp32 [ceil(N/128), ceil(K/128)];
// MXFP4: Wq [N, K/2], Ws [N, K/32] e8m0.
constexpr int kLowpFp8 = 0;
constexpr int kLowpMxfp4 = 1;
constexpr int kLowpMaxM = 64;
// Whether a format's M x N projection runs the chunk kernel (else the
// one-launch kernels of fp8.hip / mxfp4.hip, which take up to 16 rows).
bool lowp_use_chunk(int fmt, int M, int N);
struct LowpChunkPlan {
    int MT, NT, S, chunk, pitch;
    size_t lds, workspace;
};
bool lowp_chunk_plan(int M, int N, int K, LowpChunkPlan* p);
hipError_t launch_lowp_chunk(int fmt, int M, int N, int K, const void* x, const void* Wq,
                             const void* Ws, const Epilogue& fin, void* ws, hipStream_t stream);

// Router top-k: ids [T,k] (and their scores) from fp32 scores, row t at
// scores + t*ld (ld >= E); E <= 4096, k <= 32 (checked by the caller).
hipError_t launch_router_topk(const float* scores, int64_t ld, int T, int E, int k,
                              int32_t* ids, float* top, hipStream_t stream);

}  // namespace sg
