// lowp_chunk.hip -- projection with block-scaled 8-bit (FP8 e4m3) or 4-bit
// (MXFP4) weights for batches of 12 to 64 rows, on gfx950 matrix cores.
//
// The decode path the pages describe covers batch 1 to 64 ("Hyper Optimizing
// Kimi K3 in vLLM" deepnotes page, Method details: batch 1-64 decode; §1:
// split-K at larger batch) and their later model ships low-precision weights
// (Experimental setup and Supplementary details).  The one-launch FP8 and
// MXFP4 kernels (up to 16 rows) give each workgroup one or two 16-row weight
// tiles and read all of x from L2 per workgroup; as M grows that x traffic
// reaches and passes the code bytes, so from 12 rows (FP8, and MXFP4 on wide
// matrices; MXFP4 from 17 rows otherwise) this kernel uses the bf16 chunk
// kernel's shape instead:
//
//  * a workgroup of 8 waves owns 128 (NT = 1) or 256 (NT = 2) weight rows --
//    16 * NT per wave -- and one K chunk (a whole number of 128-element
//    windows); the x rows of the chunk (M padded to 16 * MT rows) are staged
//    once in LDS, so x is read once per 128 or 256 weight rows;
//  * each lane decodes its codes straight into B operand layout: FP8 lane
//    (col, grp) holds 32 codes of row col per window (k 32*grp .. +32), four
//    steps of v_mfma_f32_16x16x32_bf16 take 8 each, and the window's sum is
//    scaled once by its 128 x 128 block scale; MXFP4 lane (col, grp) loads
//    block grp of the window, permlane swaps transpose the four lane groups of
//    a column so that step t is exactly block t, and each step's result is
//    scaled by its block scale (codes converted at unit scale: exact for
//    every scale code);
//  * with S > 1 chunks the fp32 partials go to the workspace as
//    [S, N, 16 * MT] and the tiled reduction kernel adds them in ascending
//    chunk order (deterministic), as for the bf16 chunk kernel.
#include "launch.h"

namespace sg {

namespace {

constexpr int kLpWaves = 8;
constexpr int kLpThreads = kWave * kLpWaves;
constexpr int kLpWindow = 128;              // elements per window (one FP8 scale block)
constexpr int kLpXLoads = 16;               // x staging loads per thread (at most)
constexpr uint32_t kLpOut = 0xFFFFFFF0u;    // past any descriptor range: reads zero
constexpr int kLpPadSlots = kWave;          // LDS slots past the x rows (whole-chunk copy)

// e8m0 scale code -> 2^(s-127): the exponent field for 1..254, the fp32
// subnormal 2^-127 for 0, NaN for 255.
__device__ __forceinline__ float lp_e8m0(uint32_t s) {
    return as_f(s == 0u ? 0x00400000u : s == 255u ? 0x7FC00000u : s << 23);
}

template <int FMT, int MT, int NT, int D, bool ALL>
__global__ __launch_bounds__(kLpThreads) void lowp_chunk_kernel(
    const uint4* __restrict__ x, const uint8_t* __restrict__ Wq, const void* __restrict__ Ws,
    int M, int N, int K, int chunk, int pitch, Epilogue ep) {
    constexpr bool kFp8 = FMT == kLowpFp8;
    // ALL: the wave's whole chunk (at most D windows) is one batch, requested
    // behind x and consumed with no loop (FP8, one 16-row tile a wave).
    constexpr bool kHoist = kFp8 && MT <= 2;
    static_assert(!ALL || kHoist, "the whole-chunk batch is requested behind x");
    constexpr int XR = 16 * MT;
    extern __shared__ uint4 xs[];  // [XR][pitch] pieces of the chunk's x rows

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = wave_id_in_block();
    const int col = lane & 15, grp = lane >> 4;
    const int K8 = K / kPiece;
    const int k0 = blockIdx.y * chunk;
    const int len = max(0, min(K - k0, chunk));      // elements of this chunk
    const int windows = (len + kLpWindow - 1) / kLpWindow;
    const int w00 = k0 / kLpWindow;                   // first window of the chunk
    if (blockIdx.x * 128 * NT >= N) return;           // padding column of the grid
    const int row0 = blockIdx.x * 128 * NT + wv * 16 * NT;
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(16 * NT, N - row0)));

    // ---- weight codes of the wave's 16 * NT rows
    // FP8: rows of K/16 units of 16 codes; scales [ceil(N/128)][ceil(K/128)].
    // MXFP4: rows of K/32 blocks of 32 codes (16 bytes); scales [N][K/32].
    const int KU = kFp8 ? K / 16 : K / 32;  // 16-byte units per row
    const rsrc_t rw = make_rsrc(Wq + (int64_t)row0 * KU * 16, (uint32_t)rows * KU * 16u);
    const int KB = (K + kLpWindow - 1) / kLpWindow;
    const float* __restrict__ fsc = static_cast<const float*>(Ws) + (int64_t)(row0 / 128) * KB;
    const uint8_t* __restrict__ bsc = static_cast<const uint8_t*>(Ws);
    const rsrc_t rsc = make_rsrc(bsc + (int64_t)row0 * KU, (uint32_t)rows * KU);

    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    constexpr int UPW = kFp8 ? 2 : 1;  // 16-byte code loads per lane, window and tile
    struct Batch {
        uint4 wq[D][NT][UPW];
        uint32_t sb[D][NT];
        float sf[D];
    };
    // codes (and scales) of windows wb .. wb+D-1 of the chunk
    auto load_batch = [&](Batch& bt, int wb) {
        auto& wq = bt.wq;
        auto& sb = bt.sb;
        auto& sf = bt.sf;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int w = wb + d;
            const bool live = w < windows;
            const int gw = w00 + w;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int r = 16 * nt + col;
#pragma unroll
                for (int j = 0; j < UPW; ++j) {
                    // FP8: units 8*gw + 2*grp + j; MXFP4: block 4*gw + grp
                    const int u = kFp8 ? 8 * gw + 2 * grp + j : 4 * gw + grp;
                    const bool ok = live && u < KU;
                    wq[d][nt][j] =
                        load16<kStream>(rw, ok ? ((uint32_t)r * KU + u) * 16u : kLpOut);
                }
                if (!kFp8) {
                    const int b = 4 * gw + grp;
                    sb[d][nt] = __builtin_amdgcn_raw_buffer_load_b8(
                        rsc, live && b < KU ? (uint32_t)(r * KU + b) : kLpOut, 0, kStream);
                }
            }
            if (kFp8) sf[d] = live && rows > 0 ? fsc[gw] : 0.0f;  // no scale row past N
        }
    };

    Batch first;  // the early batch (kHoist)
    // ---- x of the chunk into LDS: row r, piece p at xs[r * pitch + p]
    {
        const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K8 * 16u);
        const int P8 = chunk / kPiece;
        const int total = XR * P8;
        if constexpr (ALL) {
            // A chunk of at most D = 8 windows (1024 elements): 4 * MT loads a
            // thread.  The copy has no branch (slots past the chunk's x go to
            // a padding slot per lane after the rows), its slots come from a
            // 24-bit product (with the 64-bit multiply-add the compiler chose,
            // the unused high half of its addend was a register a code load
            // writes, and the copy waited for that load), and scheduling
            // barriers keep the x loads ahead of the code loads.
            constexpr int XL = 4 * MT;
            uint4 v[XL];
            int dst[XL];
#pragma unroll
            for (int j = 0; j < XL; ++j) {
                const int idx = tid + j * kLpThreads;
                const int r = idx / P8, p = idx - r * P8;
                const bool ok = idx < total && r < M && p * kPiece < len;
                v[j] = load16<kCached>(rx, ok ? ((uint32_t)r * K8 + k0 / kPiece + p) * 16u : kLpOut);
                dst[j] = idx < total ? (int)__umul24((unsigned)r, (unsigned)pitch) + p
                                     : XR * pitch + lane;
            }
            __builtin_amdgcn_sched_barrier(0);
            load_batch(first, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < XL; ++j) xs[dst[j]] = v[j];
        } else {
            uint4 v[kLpXLoads];
#pragma unroll
            for (int j = 0; j < kLpXLoads; ++j) {
                const int idx = tid + j * kLpThreads;
                const int r = idx / P8, p = idx - r * P8;
                const bool ok = idx < total && r < M && p * kPiece < len;
                v[j] = load16<kCached>(rx, ok ? ((uint32_t)r * K8 + k0 / kPiece + p) * 16u : kLpOut);
            }
            // FP8 up to 32 rows: the first windows' codes are requested right
            // behind x (only the x loads are waited for before the LDS copy and
            // the barrier).  Measured on MI355X this pays there (4096 x 7168,
            // M = 16: 12.1 -> 11.5 us) and loses at 64 rows and for MXFP4.
            if constexpr (kHoist) load_batch(first, 0);
#pragma unroll
            for (int j = 0; j < kLpXLoads; ++j) {
                const int idx = tid + j * kLpThreads;
                const int r = idx / P8, p = idx - r * P8;
                if (idx < total) xs[r * pitch + p] = v[j];
            }
        }
    }
    __syncthreads();

    // windows wb .. wb+D-1 from the registers load_batch(wb) filled
    auto compute_batch = [&](const Batch& bt, int wb) {
        const auto& wq = bt.wq;
        const auto& sf = bt.sf;
        const auto& sb = bt.sb;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int w = wb + d;
            if (w >= windows) break;  // wave-uniform
            const uint4* xw = xs + w * (kLpWindow / kPiece);  // window's first piece
            if constexpr (kFp8) {
                f32x4_t part[NT][MT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) part[nt][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint4 a[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) a[mt] = xw[(16 * mt + col) * pitch + 4 * grp + t];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        // codes 8t .. 8t+7 of the lane's 32, low byte first
                        const uint4 q = wq[d][nt][t / 2];
                        const uint32_t lo = (t & 1) ? q.z : q.x;
                        const uint32_t hi = (t & 1) ? q.w : q.y;
                        const uint4 b = {
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            part[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, a[mt]), __builtin_bit_cast(bf16x8_t, b),
                                part[nt][mt], 0, 0, 0);
                    }
                }
                // a window lies in one 128 x 128 scale block of the wave's rows
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[nt][mt][v] = __builtin_fmaf(part[nt][mt][v], sf[d], acc[nt][mt][v]);
            } else {
                uint32_t wd[NT][4];
                float scale[NT][4];
                uint32_t out_of_range = 0;  // a scale code of this lane outside [64, 190]
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    // lane (col, grp) holds dword t of block grp; after the
                    // swaps wd[t] is dword grp of block t
                    const uint4 q = wq[d][nt][0];
                    const auto p02 = __builtin_amdgcn_permlane32_swap(q.x, q.z, false, false);
                    const auto p13 = __builtin_amdgcn_permlane32_swap(q.y, q.w, false, false);
                    const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
                    const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
                    wd[nt][0] = q01[0];
                    wd[nt][1] = q01[1];
                    wd[nt][2] = q23[0];
                    wd[nt][3] = q23[1];
                    // byte t of `all`: the scale code of block t of row col
                    const uint32_t mine = sb[d][nt] << (8 * grp);
                    const auto g16 = __builtin_amdgcn_permlane16_swap(mine, mine, false, false);
                    const uint32_t pair = g16[0] | g16[1];
                    const auto g32 = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
                    const uint32_t all = g32[0] | g32[1];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t code = (all >> (8 * t)) & 0xFFu;
                        scale[nt][t] = lp_e8m0(code);
                        out_of_range |= code - 64u > 126u;
                    }
                }
                // Every scale of the window in [64, 190] (the wave agrees): the
                // codes convert exactly at their block's scale (any code in
                // [2, 252] would: 0.5 * 2^(s-127) is a normal bf16 and
                // 6 * 2^(s-127) below bf16's largest) and the steps accumulate
                // on the matrix cores, with no fp32 scaling after each.  The
                // narrower range keeps the weights, and so the products and
                // partial sums the matrix cores form, 2^60 away from fp32's
                // subnormal and overflow limits for any x of ordinary size.
                // Otherwise each step's sum, formed at unit scale, is scaled by
                // its block's 2^(s-127) before it is added (exact for every
                // scale code).
                const bool at_scale = __builtin_amdgcn_ballot_w64(out_of_range != 0) == 0;
                if (at_scale) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        uint4 a[MT];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) a[mt] = xw[(16 * mt + col) * pitch + 4 * t + grp];
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            const float sc = scale[nt][t];
                            const uint4 b = {
                                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], sc, 0)),
                                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], sc, 1)),
                                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], sc, 2)),
                                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], sc, 3))};
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
                                acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8_t, a[mt]), __builtin_bit_cast(bf16x8_t, b),
                                    acc[nt][mt], 0, 0, 0);
                        }
                    }
                } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint4 a[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) a[mt] = xw[(16 * mt + col) * pitch + 4 * t + grp];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        constexpr float kUnit = 1.0f;
                        const uint4 b = {
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 0)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 1)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 2)),
                            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[nt][t], kUnit, 3))};
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            const f32x4_t blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, a[mt]), __builtin_bit_cast(bf16x8_t, b),
                                f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                acc[nt][mt][v] = __builtin_fmaf(blk[v], scale[nt][t], acc[nt][mt][v]);
                        }
                    }
                }
                }
            }
        }
    };

    // a batch issued before the barrier is consumed outside the loop: behind
    // a loop header the compiler would wait for all of its loads at once
    if constexpr (kHoist) compute_batch(first, 0);
    if constexpr (!ALL) {
        for (int wb = kHoist ? D : 0; wb < windows; wb += D) {
            Batch bt;
            load_batch(bt, wb);
            compute_batch(bt, wb);
        }
    }

    if (ep.partial) {
        // partials [S, N, XR]: the 4 consecutive m a lane holds as one 16-byte store
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int r = 16 * nt + col;
            if (r >= rows) continue;
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(
                ep.partial + ((int64_t)blockIdx.y * N + row0 + r) * XR + grp * 4);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) dst[mt * 4] = acc[nt][mt];
        }
        return;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * nt + col;
        if (r >= rows) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 16 * mt + 4 * grp + v;
                if (m < M) store_final(ep, (int64_t)m * N + row0 + r, acc[nt][mt][v]);
            }
    }
}

constexpr int kLpCus = 256;
constexpr size_t kLpLdsMax = 144 * 1024;  // x staging (the kernel uses no other LDS)

// Two 16-row tiles a wave while their 256-row workgroups, 8 splits each,
// still give three quarters of the compute units one.
int lowp_nt(int N) { return ((N + 255) / 256) * 8 >= 3 * kLpCus / 4 ? 2 : 1; }

}  // namespace

// Measured on MI355X (K = 7168 or 8192, N = 4096..8192): from 12 rows the
// chunk kernel beats the FP8 matrix-core kernel (N = 7168, K = 8192, M = 16:
// 21.9 -> 17.8 us; N = 4096, K = 7168, M = 16: 12.3 -> 11.5 us) and, where a
// wave takes two tiles, the MXFP4 one (N = 8192, M = 16: 19.5 -> 18.0 us); at
// N = 4096 the one-launch MXFP4 kernels stay ahead up to 16 rows (M = 12:
// 12.0 against 12.9 us).
// FP8 from 8 rows too, except where the FP8 matrix-core kernel takes two
// 16-row tiles a wave over a whole multiple of 256 workgroups (N = 8192):
// there it stays ahead to 11 rows (8192 x 7168 M = 8 16.99 against 17.86
// us); elsewhere the chunk kernel was ahead or level at 8 and 11 rows
// (K = 7168: N = 2048 M = 8 10.39 -> 9.37 us, N = 6144 17.82 -> 15.69 us,
// N = 4096 M = 11 11.46 -> 10.75 us, N = 18432 M = 11 41.96 -> 34.72 us,
// N = 3072 M = 8 10.65 / 10.58 us).
bool lowp_use_chunk(int fmt, int M, int N) {
    if (M > kLowpMaxM || M < 8) return false;
    if (fmt == kLowpFp8) {
        if (M >= 12) return true;
        const bool two_tiles = (N + 31) / 32 >= kLpCus;  // the matrix-core kernel's rule
        return !(two_tiles && ((N + 31) / 32) % kLpCus == 0);
    }
    // MXFP4 from 17 rows, from 12 where a wave takes two tiles, and from 9
    // where the MXFP4 matrix-core kernel's grid of 16- or 32-row tiles is not
    // a whole multiple of 256 workgroups.  Interleaved A/B, K = 7168 unless
    // noted, against the matrix-core kernel: N = 5888 M = 9 / 16 18.51 /
    // 20.50 -> 15.25 / 15.34 us, N = 12288 M = 9 28.97 -> 24.31 us, 7168 x
    // 8192 M = 9 20.07 -> 18.57 us, N = 2048 M = 16 11.42 -> 10.02 us; the
    // one loss N = 3072 M = 9 10.86 -> 11.25 us.
    if (M >= 17 || (M >= 12 && lowp_nt(N) == 2)) return true;
    const int t16 = (N + 15) / 16, t32 = (N + 31) / 32;
    const int tiles = t32 >= kLpCus ? t32 : t16;  // the matrix-core kernel's rule
    return M >= 9 && tiles % kLpCus != 0;
}

bool lowp_chunk_plan(int M, int N, int K, LowpChunkPlan* p) {
    if (M < 1 || M > kLowpMaxM || N < 1 || K < 0) return false;
    const int MT = (M + 15) / 16;
    const int XR = 16 * MT;
    if (K == 0) {  // outputs are r (or zero): one launch, nothing to stage
        *p = LowpChunkPlan{MT, 1, 1, kLpWindow, kLpWindow / kPiece + 1,
                           ((size_t)XR * (kLpWindow / kPiece + 1) + kLpPadSlots) * 16, 0};
        return true;
    }
    const int NT = lowp_nt(N);
    const int tiles = mfma_grid_tiles(N, 128 * NT);
    const int windows = (K + kLpWindow - 1) / kLpWindow;
    // The split whose busiest compute unit has the least to do: ceil(grid /
    // 256) workgroups of ceil(windows / S) windows each, plus one window's
    // worth a workgroup for staging x and writing its partials (without it,
    // N = 5888 took S = 56, one window a workgroup: MXFP4 M = 16 37.8 us);
    // a tie goes to the smaller split (fewer partials).  Only splits whose x chunk fits in LDS
    // (and the staging registers) and that leave no chunk empty.  The first
    // split to reach 256 workgroups, taken before, overshot to 264-304 where
    // the tiles do not divide 256, and the compute units holding two
    // workgroups set the time (FP8, K = 7168, M = 16: N = 3072 14.1 us at
    // S = 12 against 10.4 at S = 8; N = 6144 22.1 against 17.3 us).
    int best = 0;
    int64_t best_cost = INT64_MAX;
    for (int S = 1; S <= 64 && S <= windows; ++S) {
        const int wpw = (windows + S - 1) / S;
        const int chunk = kLpWindow * wpw;
        if ((int64_t)(S - 1) * chunk >= K) continue;  // an empty chunk
        const size_t lds = ((size_t)XR * (chunk / kPiece + 1) + kLpPadSlots) * 16;
        if (lds > kLpLdsMax || XR * (chunk / kPiece) > kLpXLoads * kLpThreads) continue;
        const int64_t cost = ((int64_t)tiles * S + kLpCus - 1) / kLpCus * (wpw + 1);
        if (cost < best_cost) {
            best = S;
            best_cost = cost;
        }
    }
    if (best == 0) return false;
    const int chunk = kLpWindow * ((windows + best - 1) / best);
    p->MT = MT;
    p->NT = NT;
    p->S = best;
    p->chunk = chunk;
    p->pitch = chunk / kPiece + 1;  // odd row pitch: the 16 rows of an operand read spread banks
    p->lds = ((size_t)XR * p->pitch + kLpPadSlots) * 16;
    p->workspace = best > 1 ? ((size_t)best * N * XR * sizeof(float) + 255) / 256 * 256 : 0;
    return true;
}

hipError_t launch_lowp_chunk(int fmt, int M, int N, int K, const void* x, const void* Wq,
                             const void* Ws, const Epilogue& fin, void* ws, hipStream_t stream) {
    LowpChunkPlan p;
    if (!lowp_chunk_plan(M, N, K, &p)) return hipErrorInvalidValue;
    const dim3 grid(mfma_grid_tiles(N, 128 * p.NT), p.S);
    const Epilogue ep = p.S > 1 ? Epilogue{static_cast<float*>(ws), nullptr, nullptr, nullptr} : fin;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint8_t* wp = static_cast<const uint8_t*>(Wq);
    // windows in flight per wave: FP8 up to 32 rows 2, from 33 rows 4; MXFP4 2.
    // Interleaved A/B on MI355X, FP8 4 -> 2 windows: 8192 x 7168 M = 32
    // 20.32 -> 19.76 us, 4096 x 7168 M = 32 12.61 -> 12.29 us, 2048 x 7168
    // M = 24 14.84 -> 13.85 us; at M = 64 2 was slower (4096 x 7168 14.84 ->
    // 15.13 us, 8192 x 7168 25.33 -> 25.71 us).
    constexpr int kD8 = 2, kD8Wide = 4, kD4 = 2;
    // FP8 with one 16-row tile and one x row tile a wave and 7 or 8 windows a
    // wave (K = 7168 or 8192 over 8 splits): the whole chunk is one batch.
    // Interleaved A/B on MI355X: 4096 x 7168 M = 12 / 16 11.41 / 11.43 ->
    // 10.71 / 10.76 us; with two tiles a wave or from 17 rows it was slower
    // (8192 x 7168 M = 16 17.94 -> 18.17 us, 4096 x 7168 M = 64 14.81 ->
    // 16.00 us).
    const int wpw = p.chunk / kLpWindow;
    const bool all = fmt == kLowpFp8 && p.MT == 1 && p.NT == 1 && (wpw == 7 || wpw == 8);
#define SG_LP(f, mt, nt, d, a)                                                                    \
    if (fmt == f && p.MT == mt && p.NT == nt && all == a) {                                       \
        auto* kern = &lowp_chunk_kernel<f, mt, nt, d, a>;                                         \
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                   \
                                           hipFuncAttributeMaxDynamicSharedMemorySize,            \
                                           (int)p.lds);                                           \
        if (e != hipSuccess) return e;                                                            \
        kern<<<grid, kLpThreads, p.lds, stream>>>(xp, wp, Ws, M, N, K, p.chunk, p.pitch, ep);    \
        e = hipGetLastError();                                                                    \
        if (e != hipSuccess) return e;                                                            \
        return p.S > 1 ? launch_reduce_tiles(static_cast<const float*>(ws), p.S, M, N, 128 * nt, \
                                             fin, stream)                                         \
                       : hipSuccess;                                                              \
    }
    SG_LP(kLowpFp8, 1, 1, 8, true)
    SG_LP(kLowpFp8, 1, 1, kD8, false) SG_LP(kLowpFp8, 2, 1, kD8, false)
    SG_LP(kLowpFp8, 3, 1, kD8Wide, false) SG_LP(kLowpFp8, 4, 1, kD8Wide, false)
    SG_LP(kLowpFp8, 1, 2, kD8, false) SG_LP(kLowpFp8, 2, 2, kD8, false)
    SG_LP(kLowpFp8, 3, 2, kD8Wide, false) SG_LP(kLowpFp8, 4, 2, kD8Wide, false)
    SG_LP(kLowpMxfp4, 1, 1, kD4, false) SG_LP(kLowpMxfp4, 2, 1, kD4, false)
    SG_LP(kLowpMxfp4, 3, 1, kD4, false) SG_LP(kLowpMxfp4, 4, 1, kD4, false)
    SG_LP(kLowpMxfp4, 1, 2, kD4, false) SG_LP(kLowpMxfp4, 2, 2, kD4, false)
    SG_LP(kLowpMxfp4, 3, 2, kD4, false) SG_LP(kLowpMxfp4, 4, 2, kD4, false)
#undef SG_LP
    return hipErrorInvalidValue;
}

}  // namespace sg
