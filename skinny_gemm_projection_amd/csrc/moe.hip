// moe.hip -- routed-expert (MoE) decode: per-expert token table and the
// grouped per-expert projection, for gfx950.
//
// The pages replace the stock MoE GEMMs with custom low-latency kernels and
// note that expert selection decides which weights get read ("Hyper
// Optimizing Kimi K3 in vLLM" deepnotes page, Method details §3 and
// Supplementary details §1; French translation, Partie 2 §4).  Here the
// selection is turned into a table on the device, and every selected
// expert's weight matrix is then streamed from HBM once per call, however
// many tokens chose it.  No host synchronisation: the number of active
// experts is only known on the device, so the grouped kernel reads it there.
#include <algorithm>

#include "launch.h"
#include "topk_device.h"

namespace sg {

namespace {

constexpr int kTableThreads = 1024;
constexpr int kTableWaves = kTableThreads / kWave;
constexpr int kMaxPairs = 4096;
constexpr int kMaxExperts = 4096;

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

// Exclusive prefix sums of a and b over the threads of the workgroup (in
// thread order); *total_a / *total_b receive the sums.  Two barriers.
__device__ __forceinline__ void block_exclusive_scan2(int a, int b, int* ex_a, int* ex_b,
                                                      int* total_a, int* total_b,
                                                      int (*s_wave)[kTableWaves]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int ia = wave_inclusive_scan(a);
    const int ib = wave_inclusive_scan(b);
    if (lane == kWave - 1) {
        s_wave[0][wv] = ia;
        s_wave[1][wv] = ib;
    }
    __syncthreads();
    int base_a = 0, base_b = 0, ta = 0, tb = 0;
    for (int w = 0; w < kTableWaves; ++w) {  // 16 LDS broadcast reads
        const int va = s_wave[0][w], vb = s_wave[1][w];
        if (w < wv) {
            base_a += va;
            base_b += vb;
        }
        ta += va;
        tb += vb;
    }
    *ex_a = base_a + ia - a;
    *ex_b = base_b + ib - b;
    *total_a = ta;
    *total_b = tb;
}

// One workgroup builds the table.
//  1. counts[e] by LDS integer atomics; ids outside [0, E) are left out
//     (their number is P minus the counts' sum);
//  2. offsets (exclusive scan of counts) and the ascending list of active
//     experts (exclusive scan of counts > 0), by wave-level scans;
//  3. every valid pair p is dropped into its expert's segment at a slot
//     taken with an LDS atomic (arbitrary order) ...
//  4. ... and then moved to offsets[e] + (number of pairs of the segment
//     with a smaller p), which orders every segment by ascending p.  A
//     thread does work proportional to its segment's length.
// Output rows of invalid pairs are zero-filled.
__global__ __launch_bounds__(kTableThreads) void moe_table_kernel(
    const int32_t* __restrict__ ids, int P, int E, int N, GroupedWorkspace g,
    int32_t* user_offsets, int32_t* user_sorted, int32_t* user_invalid, float* out) {
    __shared__ int32_t s_ids[kMaxPairs];
    __shared__ int32_t s_tmp[kMaxPairs];     // scan scratch first, then the unordered segments
    __shared__ int32_t s_cnt[kMaxExperts];  // counts, then fill cursors
    __shared__ int32_t s_off[kMaxExperts];
    int (*s_wave)[kTableWaves] = reinterpret_cast<int (*)[kTableWaves]>(s_tmp);

    const int tid = threadIdx.x;
    for (int p = tid; p < P; p += kTableThreads) s_ids[p] = ids[p];
    for (int e = tid; e < E; e += kTableThreads) s_cnt[e] = 0;
    __syncthreads();

    for (int p = tid; p < P; p += kTableThreads) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();

    // Thread t owns experts 4t .. 4t+3 (E <= 4096).
    int c[4];
    int sum_c = 0, sum_a = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        c[j] = (e < E) ? s_cnt[e] : 0;
        sum_c += c[j];
        sum_a += c[j] > 0;
    }
    int pc, pa, total, num_active;
    block_exclusive_scan2(sum_c, sum_a, &pc, &pa, &total, &num_active, s_wave);
    const int invalid = P - total;  // pairs whose id is outside [0, E)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        if (e < E) {
            g.counts[e] = c[j];
            g.offsets[e] = pc;
            if (user_offsets) user_offsets[e] = pc;
            s_off[e] = pc;
            s_cnt[e] = pc;  // fill cursor
            if (c[j] > 0) g.active[pa++] = e;
            pc += c[j];
        }
    }
    if (tid == 0) {
        g.offsets[E] = total;
        if (user_offsets) user_offsets[E] = total;
        *g.num_active = num_active;
        *g.invalid = invalid;
        if (user_invalid) *user_invalid = invalid;
    }
    __syncthreads();  // every thread is past its reads of s_wave (aliasing s_tmp)

    for (int p = tid; p < P; p += kTableThreads) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) s_tmp[atomicAdd(&s_cnt[e], 1)] = p;
    }
    __syncthreads();

    for (int i = tid; i < total; i += kTableThreads) {
        const int p = s_tmp[i];
        const int e = s_ids[p];
        const int lo = s_off[e];
        const int hi = s_cnt[e];  // the fill cursor stopped at the segment's end
        int rank = 0;
        for (int j = lo; j < hi; ++j) rank += s_tmp[j] < p;
        g.sorted[lo + rank] = p;
        if (user_sorted) user_sorted[lo + rank] = p;
    }
    for (int i = total + tid; i < P; i += kTableThreads) {
        g.sorted[i] = -1;
        if (user_sorted) user_sorted[i] = -1;
    }

    if (invalid > 0) {  // rare: zero-fill the output rows of out-of-range ids
        for (int p = 0; p < P; ++p) {
            const int e = s_ids[p];
            if (e < 0 || e >= E)
                for (int n = tid; n < N; n += kTableThreads) out[(int64_t)p * N + n] = 0.0f;
        }
    }
}

// A whole row (K8 16-byte pieces) as NCH lane-pieces; pieces past the row
// read as zero through the buffer bounds, and only the wave-uniform chunk
// count guards the loads.
template <int NCH, int POLICY>
__device__ __forceinline__ void load_row(uint4 (&dst)[NCH], const uint4* __restrict__ src,
                                         int K8, int lane) {
    const rsrc_t r = make_rsrc(src, (uint32_t)K8 * 16u);
    const int nch = (K8 + kWave - 1) / kWave;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        dst[c] = make_uint4(0, 0, 0, 0);
        if (c < nch) dst[c] = load16<POLICY>(r, (uint32_t)(c * kWave + lane) * 16u);
    }
}

template <int NCH>
__device__ __forceinline__ float dot_row(const uint4 (&a)[NCH], const uint4 (&b)[NCH]) {
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) s = dot8(a[c], b[c], s);
    return s;
}

// The wave's kGroupedRowsPerWave rows of expert W_e for one routed pair (the
// common case of one token per expert): one row per step with two row
// buffers, so the next row's loads are in flight while the current one is
// multiplied, reduced and stored -- the small-matrix streaming kernel's
// structure.  Every step is unrolled (each wait covers one row), and rows
// past N read as zero and are not stored, with no branch that would end the
// sequence early.  x_row is the token's activation row, out_row the pair's
// output row.
template <int NCH>
__device__ __forceinline__ void stream_rows_one_pair(const uint4* __restrict__ x_row,
                                                     const uint4* __restrict__ We, int nbase,
                                                     int N, int K8, int lane,
                                                     float* __restrict__ out_row) {
    const int v = scatter_index<4>(lane);  // 0: this lane stores the step's sum
    // Every one of the NCH loads is issued (pieces past the row read zero
    // through the buffer bounds): a branch around a load would make the
    // compiler wait for all loads in flight before the first row's dots.
    // Measured on MI355X: dispatching to the exact load count (K8 / 64
    // rounded up, 14 at K = 7168) instead of this power of two was slower
    // (E = 384, 2048 x 7168: T = 1 37.2 -> 38.9 us, T = 64 1268 -> 1298 us).
    auto load_unguarded = [&](uint4 (&dst)[NCH], const uint4* src, int pieces, int policy_stream) {
        const rsrc_t r = make_rsrc(src, (uint32_t)pieces * 16u);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            dst[c] = policy_stream ? load16<kStream>(r, (uint32_t)(c * kWave + lane) * 16u)
                                   : load16<kCached>(r, (uint32_t)(c * kWave + lane) * 16u);
    };
    uint4 xa[NCH];
    uint4 wr[2][NCH];
    load_unguarded(xa, x_row, K8, 0);
    auto load_w = [&](int i, uint4 (&dst)[NCH]) {
        const int n = nbase + i;
        const bool ok = n < N;
        load_unguarded(dst, We + (int64_t)(ok ? n : 0) * K8, ok ? K8 : 0, 1);
    };
    load_w(0, wr[0]);
    load_w(1, wr[1]);
#pragma unroll
    for (int i = 0; i < kGroupedRowsPerWave; ++i) {
        const int b = i & 1;
        float acc[4] = {dot_row<NCH>(xa, wr[b]), 0.0f, 0.0f, 0.0f};
        if (i + 2 < kGroupedRowsPerWave) load_w(i + 2, wr[b]);  // the buffer just consumed
        const float total = reduce_scatter<4>(acc, lane);
        const int n = nbase + i;
        if (v == 0 && n < N) out_row[n] = total;
    }
}

// Persistent grid over work items (active expert, tile of kGroupedTileN rows
// of its W).  Each wave takes kGroupedRowsPerWave rows of the tile.  With
// one token routed to the expert (the common case) they stream one row per
// step with the next row in flight (stream_rows_one_pair; measured on
// MI355X at E = 384, 2048 x 7168: T = 1 38.3 -> 37.2 us, T = 16 468 -> 465
// us against the loop below).  With more tokens the rows go two at a time
// (2 x up to 16 x 1 KB loads in flight), stay in registers while the
// tokens' x rows (L2-resident) stream past them, and the two sums of a
// (row pair, token) are reduced together by one lane reduce-scatter, so each
// weight byte is still fetched from HBM once.
template <int NCH>
__global__ __launch_bounds__(kBlock) void grouped_kernel(const uint4* __restrict__ x,
                                                         const uint4* __restrict__ W, int N,
                                                         int K8, int topk, int tiles,
                                                         GroupedWorkspace g,
                                                         float* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = wave_id_in_block();
    const int items = *g.num_active * tiles;
    const int v = scatter_index<4>(lane);  // this lane's row (0 or 1) of the sums, or -1/2/3

    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int e = g.active[item / tiles];
        const int tile = item - (item / tiles) * tiles;
        const int seg = g.offsets[e];
        const int cnt = g.offsets[e + 1] - seg;
        const uint4* __restrict__ We = W + (int64_t)e * N * K8;
        const int nbase = tile * kGroupedTileN + wv * kGroupedRowsPerWave;

        uint4 xa[NCH], w0[NCH], w1[NCH];
        auto load_w = [&](uint4 (&dst)[NCH], int n) {
            const bool ok = n < N;
            load_row<NCH, kStream>(dst, We + (int64_t)(ok ? n : 0) * K8, ok ? K8 : 0, lane);
        };
        auto load_x = [&](int p) {
            load_row<NCH, kCached>(xa, x + (int64_t)(p / topk) * K8, K8, lane);
        };
        auto finish = [&](int n, int p) {
            float acc[4] = {dot_row<NCH>(xa, w0), dot_row<NCH>(xa, w1), 0.0f, 0.0f};
            const float total = reduce_scatter<4>(acc, lane);
            if (v == 0 || v == 1) {
                const int row = n + v;
                if (row < N) out[(int64_t)p * N + row] = total;
            }
        };
        if (cnt == 1) {
            const int p = g.sorted[seg];
            stream_rows_one_pair<NCH>(x + (int64_t)(p / topk) * K8, We, nbase, N, K8, lane,
                                      out + (int64_t)p * N);
        } else {
#pragma unroll 1
            for (int i = 0; i < kGroupedRowsPerWave; i += 2) {
                const int n = nbase + i;
                if (n >= N) break;
                load_w(w0, n);
                load_w(w1, n + 1);
#pragma unroll 1
                for (int c = 0; c < cnt; ++c) {
                    const int p = g.sorted[seg + c];
                    load_x(p);
                    finish(n, p);
                }
            }
        }
    }
}

// Fused form for small routing tables (P = T * topk <= kFusedMaxPairs), used
// when the caller asks for none of the table outputs: every workgroup builds
// the part of the table it needs in LDS -- the ascending list of active
// experts, from the ids -- and each wave finds an expert's pairs, in
// ascending p, with ballots over the ids.  This drops the table kernel's
// launch and the grouped kernel's chain of dependent reads of its output
// (one token: 8 experts, 235 MB, the table alone was about 4 us under the
// profiler).  Work items, per-(pair, row) arithmetic and outputs are those
// of grouped_kernel; output rows of ids outside [0, E) are zero-filled here.
//
// The body runs once the workgroup's ids are in s_ids[0, P): the caller
// stores them, and the body's first barrier publishes them.
template <int NCH>
__device__ __forceinline__ void grouped_lds_table(const uint4* __restrict__ x,
                                                  const uint4* __restrict__ W,
                                                  const int32_t* s_ids, int32_t* s_flag,
                                                  int32_t* s_active, int32_t* s_wave, int P,
                                                  int E, int N, int K8, int topk, int tiles,
                                                  float* __restrict__ out) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = wave_id_in_block();

    for (int e = tid; e < E; e += kBlock) s_flag[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += kBlock) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) s_flag[e] = 1;  // every writer stores the same value
    }
    __syncthreads();
    // thread t scans experts [t * per, (t + 1) * per)
    const int per = (E + kBlock - 1) / kBlock;
    const int e0 = tid * per;
    int mine = 0;
    for (int j = 0; j < per; ++j) mine += (e0 + j < E) ? s_flag[e0 + j] : 0;
    const int incl = wave_inclusive_scan(mine);
    if (lane == kWave - 1) s_wave[wv] = incl;
    __syncthreads();
    int base = 0, num_active = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
        base += w < wv ? s_wave[w] : 0;
        num_active += s_wave[w];
    }
    int pos = base + incl - mine;
    for (int j = 0; j < per; ++j)
        if (e0 + j < E && s_flag[e0 + j]) s_active[pos++] = e0 + j;
    __syncthreads();

    // zero-fill the output rows of out-of-range ids, spread over the workgroups
    for (int p = blockIdx.x; p < P; p += gridDim.x) {
        const int e = s_ids[p];
        if (e < 0 || e >= E)
            for (int n = tid; n < N; n += kBlock) out[(int64_t)p * N + n] = 0.0f;
    }

    const int items = num_active * tiles;
    const int v = scatter_index<4>(lane);  // this lane's row (0 or 1) of the sums, or -1/2/3
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int e = s_active[item / tiles];
        const int tile = item - (item / tiles) * tiles;
        const uint4* __restrict__ We = W + (int64_t)e * N * K8;
        const int nbase = tile * kGroupedTileN + wv * kGroupedRowsPerWave;
        // this expert's pairs: count them, and the first (ascending p)
        int cnt = 0, first = -1;
        for (int b = 0; b < P; b += kWave) {
            const uint64_t m = __ballot(b + lane < P && s_ids[b + lane] == e);
            if (first < 0 && m) first = b + __builtin_ctzll(m);
            cnt += __popcll(m);
        }

        uint4 xa[NCH], w0[NCH], w1[NCH];
        auto load_w = [&](uint4 (&dst)[NCH], int n) {
            const bool ok = n < N;
            load_row<NCH, kStream>(dst, We + (int64_t)(ok ? n : 0) * K8, ok ? K8 : 0, lane);
        };
        auto load_x = [&](int p) {
            load_row<NCH, kCached>(xa, x + (int64_t)(p / topk) * K8, K8, lane);
        };
        auto finish = [&](int n, int p) {
            float acc[4] = {dot_row<NCH>(xa, w0), dot_row<NCH>(xa, w1), 0.0f, 0.0f};
            const float total = reduce_scatter<4>(acc, lane);
            if (v == 0 || v == 1) {
                const int row = n + v;
                if (row < N) out[(int64_t)p * N + row] = total;
            }
        };
        if (cnt == 1) {
            stream_rows_one_pair<NCH>(x + (int64_t)(first / topk) * K8, We, nbase, N, K8, lane,
                                      out + (int64_t)first * N);
        } else {
#pragma unroll 1
            for (int i = 0; i < kGroupedRowsPerWave; i += 2) {
                const int n = nbase + i;
                if (n >= N) break;
                load_w(w0, n);
                load_w(w1, n + 1);
#pragma unroll 1
                for (int b = 0; b < P; b += kWave) {
                    uint64_t m = __ballot(b + lane < P && s_ids[b + lane] == e);
                    while (m) {
                        const int p = b + __builtin_ctzll(m);
                        m &= m - 1;
                        load_x(p);
                        finish(n, p);
                    }
                }
            }
        }
    }
}

// LDS of the fused launches: ids [P], expert flags [E], active experts [E].
template <int NCH>
__global__ __launch_bounds__(kBlock) void grouped_fused_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ W, const int32_t* __restrict__ ids,
    int P, int E, int N, int K8, int topk, int tiles, float* __restrict__ out) {
    extern __shared__ int32_t lds_i[];
    __shared__ int32_t s_wave[kWavesPerBlock];
    for (int p = threadIdx.x; p < P; p += kBlock) lds_i[p] = ids[p];
    grouped_lds_table<NCH>(x, W, lds_i, lds_i + P, lds_i + P + E, s_wave, P, E, N, K8, topk,
                           tiles, out);
}

// Router top-k and routed-expert projection in one launch, for a few tokens
// (T <= kRouteFusedMaxT = kWavesPerBlock): every workgroup ranks the scores
// itself -- wave t ranks token t with the router kernel's wave_topk, so the
// ids are the same bits -- and workgroup 0 also stores them (and the selected
// scores).  Then the fused table and the grouped loop as above.  This drops
// the top-k launch and the round trip of the ids through memory.
//
// With Nsh > 0 the launch also computes the shared expert, shared_out[t, r] =
// x[t] . Wsh[r] ("Hyper Optimizing Kimi K3 in vLLM" deepnotes page, Method
// details §3: the shared expert overlaps the routing).  Its rows are split
// evenly over every wave of the grid; each wave requests its first row right
// behind its scores, so the row streams from HBM while the wave ranks --
// until the ids are known no routed weight can be requested -- and finishes
// its rows (one dot product per token, x from L2) before the table.
template <int NCH, int PER>
__global__ __launch_bounds__(kBlock) void route_grouped_kernel(
    const float* __restrict__ scores, int64_t ld, int T, int E, int k,
    int32_t* __restrict__ ids_out, float* __restrict__ top_out, const uint4* __restrict__ x,
    const uint4* __restrict__ W, int N, int K8, int tiles, float* __restrict__ out,
    const uint4* __restrict__ Wsh, int Nsh, float* __restrict__ shared_out) {
    extern __shared__ int32_t lds_i[];
    __shared__ int32_t s_wave[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = wave_id_in_block();
    const int P = T * k;
    const bool ranks = wv < T;  // wave t ranks token t
    // The scores, then the first shared row, are requested with no branch
    // around them (a wave with no token, or no shared row, reads through a
    // 0-byte descriptor, which gives zeros), and every wave ranks, only the
    // stores depending on the token: behind a branch the compiler cannot
    // count the loads in flight and its waits for the scores drain the row's,
    // and loads used only under a branch are moved into it, behind the row's.
    uint32_t sv[PER];
    wave_topk_fetch<PER>(scores + (ranks ? wv : 0) * ld, ranks ? E : 0, lane, sv);
    __builtin_amdgcn_sched_barrier(0);

    // this wave's shared-expert rows [sr0, sr1); a row past them reads zero
    const int nw = gridDim.x * kWavesPerBlock;
    const int sper = (Nsh + nw - 1) / nw;
    const int sr0 = min(Nsh, (blockIdx.x * kWavesPerBlock + wv) * sper);
    const int sr1 = min(Nsh, sr0 + sper);
    uint4 wsr[NCH];
    auto load_srow = [&](int r) {
        const bool ok = r < sr1;
        const rsrc_t rs = make_rsrc(Wsh + (int64_t)(ok ? r : 0) * K8, ok ? (uint32_t)K8 * 16u : 0u);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            wsr[c] = load16<kStream>(rs, (uint32_t)(c * kWave + lane) * 16u);
    };
    load_srow(sr0);
    __builtin_amdgcn_sched_barrier(0);  // the row's loads stay ahead of the ranking

    {
        __builtin_assume(k >= 1);  // (checked by the caller) else the scores wait behind k > 0
        uint64_t key[PER];
        wave_topk_keys<PER>(sv, E, lane, key);
        const uint64_t mine = wave_topk_rank<PER>(key, k, lane);
        if (ranks && lane < k) {
            const int id = key_id(mine);
            lds_i[wv * k + lane] = id;
            if (blockIdx.x == 0) {
                ids_out[(int64_t)wv * k + lane] = id;
                if (top_out) top_out[(int64_t)wv * k + lane] = scores[wv * ld + id];  // as given
            }
        }
    }
    for (int r = sr0; r < sr1; ++r) {
        if (r > sr0) load_srow(r);
        for (int t = 0; t < T; ++t) {
            const rsrc_t rx = make_rsrc(x + (int64_t)t * K8, (uint32_t)K8 * 16u);
            uint4 xa[NCH];
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                xa[c] = load16<kCached>(rx, (uint32_t)(c * kWave + lane) * 16u);
            const float tot = wave_sum(dot_row<NCH>(xa, wsr));
            if (lane == 0) shared_out[(int64_t)t * Nsh + r] = tot;
        }
    }
    grouped_lds_table<NCH>(x, W, lds_i, lds_i + P, lds_i + P + E, s_wave, P, E, N, K8, k,
                           tiles, out);
}

int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

}  // namespace

size_t grouped_workspace_bytes(int E, int P) {
    const size_t ints = (size_t)E + (E + 1) + P + 1 + E + 1;
    return (ints * sizeof(int32_t) + 255) / 256 * 256;
}

GroupedWorkspace grouped_workspace_layout(void* ws, int E, int P) {
    int32_t* base = static_cast<int32_t*>(ws);
    GroupedWorkspace g;
    g.counts = base;
    g.offsets = g.counts + E;
    g.sorted = g.offsets + E + 1;
    g.invalid = g.sorted + P;
    g.active = g.invalid + 1;
    g.num_active = g.active + E;
    return g;
}

hipError_t launch_moe_table(const int32_t* ids, int T, int topk, int E, int N,
                            const GroupedWorkspace& g, int32_t* user_offsets,
                            int32_t* user_sorted, int32_t* user_invalid, float* out,
                            hipStream_t stream) {
    moe_table_kernel<<<1, kTableThreads, 0, stream>>>(ids, T * topk, E, N, g, user_offsets,
                                                      user_sorted, user_invalid, out);
    return hipGetLastError();
}

hipError_t launch_grouped_fused(const void* x, int T, const void* W, const int32_t* ids, int E,
                                int N, int K, int topk, float* out, hipStream_t stream) {
    const int P = T * topk;
    const int K8 = K / kPiece;
    const int tiles = (N + kGroupedTileN - 1) / kGroupedTileN;
    const int max_active = E < P ? E : P;
    const int64_t max_items = (int64_t)max_active * tiles;
    const int resident = 512;  // 256 CUs x 2 workgroups
    int grid = (int)(max_items < resident ? max_items : resident);
    if (grid < 1) grid = 1;  // still zero-fills the rows of invalid ids
    const size_t lds = (size_t)(P + 2 * E) * sizeof(int32_t);
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const int nch = (K + kLaneSpan - 1) / kLaneSpan;
    switch (next_pow2(nch < 1 ? 1 : nch)) {
#define SG_FUSED(c) \
    case c: \
        grouped_fused_kernel<c><<<grid, kBlock, lds, stream>>>(xp, wp, ids, P, E, N, K8, topk, \
                                                              tiles, out); \
        break;
        SG_FUSED(1) SG_FUSED(2) SG_FUSED(4) SG_FUSED(8) SG_FUSED(16)
#undef SG_FUSED
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int NCH>
static hipError_t launch_route_nch(int per, int grid, size_t lds, hipStream_t stream,
                             const float* scores, int64_t ld, int T, int E, int k, int32_t* ids,
                             float* top, const uint4* xp, const uint4* wp, int N, int K8,
                             int tiles, float* out, const uint4* wsh, int Nsh, float* sout) {
#define SG_ROUTE(pp) \
    if (per <= pp) { \
        route_grouped_kernel<NCH, pp><<<grid, kBlock, lds, stream>>>( \
            scores, ld, T, E, k, ids, top, xp, wp, N, K8, tiles, out, wsh, Nsh, sout); \
        return hipGetLastError(); \
    }
    SG_ROUTE(2) SG_ROUTE(4) SG_ROUTE(6) SG_ROUTE(8)
#undef SG_ROUTE
    return hipErrorInvalidValue;
}

hipError_t launch_route_grouped(const float* scores, int64_t ld, int T, int E, int k,
                                int32_t* ids, float* top, const void* x, const void* W, int N,
                                int K, float* out, const void* W_shared, int N_shared,
                                float* shared_out, hipStream_t stream) {
    const int per = (E + kWave - 1) / kWave;
    if (T < 1 || T > kRouteFusedMaxT || per > kSortedPerLane || N < 1) return hipErrorInvalidValue;
    const int P = T * k;
    const int K8 = K / kPiece;
    const int tiles = (N + kGroupedTileN - 1) / kGroupedTileN;
    const int max_active = E < P ? E : P;
    const int64_t max_items = (int64_t)max_active * tiles;
    const int resident = 512;  // 256 CUs x 2 workgroups
    // enough waves for the shared rows too (about 4 a wave): a workgroup past
    // the routed items only ranks, streams its shared rows and finds no item
    const int64_t want = std::max<int64_t>(max_items, ((int64_t)N_shared + 15) / 16);
    const int grid = (int)(want < resident ? want : resident);
    const size_t lds = (size_t)(P + 2 * E) * sizeof(int32_t);
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const uint4* wsh = static_cast<const uint4*>(W_shared);
    const int nch = (K + kLaneSpan - 1) / kLaneSpan;
    switch (next_pow2(nch < 1 ? 1 : nch)) {
        case 1:
            return launch_route_nch<1>(per, grid, lds, stream, scores, ld, T, E, k, ids, top, xp,
                                        wp, N, K8, tiles, out, wsh, N_shared, shared_out);
        case 2:
            return launch_route_nch<2>(per, grid, lds, stream, scores, ld, T, E, k, ids, top, xp,
                                        wp, N, K8, tiles, out, wsh, N_shared, shared_out);
        case 4:
            return launch_route_nch<4>(per, grid, lds, stream, scores, ld, T, E, k, ids, top, xp,
                                        wp, N, K8, tiles, out, wsh, N_shared, shared_out);
        case 8:
            return launch_route_nch<8>(per, grid, lds, stream, scores, ld, T, E, k, ids, top, xp,
                                        wp, N, K8, tiles, out, wsh, N_shared, shared_out);
        case 16:
            return launch_route_nch<16>(per, grid, lds, stream, scores, ld, T, E, k, ids, top, xp,
                                        wp, N, K8, tiles, out, wsh, N_shared, shared_out);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_grouped(const void* x, int T, const void* W, int E, int N, int K, int topk,
                          const GroupedWorkspace& g, float* out, hipStream_t stream) {
    const int K8 = K / kPiece;
    const int tiles = (N + kGroupedTileN - 1) / kGroupedTileN;
    const int max_active = E < T * topk ? E : T * topk;
    const int64_t max_items = (int64_t)max_active * tiles;
    const int resident = 512;  // 256 CUs x 2 workgroups
    const int grid = (int)(max_items < resident ? max_items : resident);
    if (grid <= 0) return hipSuccess;
    const uint4* xp = static_cast<const uint4*>(x);
    const uint4* wp = static_cast<const uint4*>(W);
    const int nch = (K + kLaneSpan - 1) / kLaneSpan;
    switch (next_pow2(nch < 1 ? 1 : nch)) {
        case 1: grouped_kernel<1><<<grid, kBlock, 0, stream>>>(xp, wp, N, K8, topk, tiles, g, out); break;
        case 2: grouped_kernel<2><<<grid, kBlock, 0, stream>>>(xp, wp, N, K8, topk, tiles, g, out); break;
        case 4: grouped_kernel<4><<<grid, kBlock, 0, stream>>>(xp, wp, N, K8, topk, tiles, g, out); break;
        case 8: grouped_kernel<8><<<grid, kBlock, 0, stream>>>(xp, wp, N, K8, topk, tiles, g, out); break;
        case 16: grouped_kernel<16><<<grid, kBlock, 0, stream>>>(xp, wp, N, K8, topk, tiles, g, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sg
