// host_checks.cpp -- drives the library's host code (planner, argument
// checks, tuned-table parsing) under AddressSanitizer on a host without a
// GPU.  Every call made here returns before any launch; the GPU-side code is
// linked in unchanged (and never runs).  Exit status 0 when every status
// matches what the header promises.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "skinny_gemm.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
    if (!ok) {
        std::fprintf(stderr, "host_checks: line %d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Fake device addresses: never dereferenced, every call below returns first.
template <class T>
T* fake(uintptr_t a) {
    return reinterpret_cast<T*>(a);
}

void plans() {
    const int32_t Ns[] = {0, 1, 7, 16, 33, 300, 384, 1024, 2048, 4096, 6144, 7168, 8192, 8200, 20000};
    const int32_t Ks[] = {0, 8, 64, 1024, 1040, 4096, 7168, 8192, 16384, 30000, 65536};
    for (int32_t M = 0; M <= 66; ++M)
        for (int32_t N : Ns)
            for (int32_t K : Ks) {
                sg_plan p;
                std::memset(&p, 0xAB, sizeof p);
                const sg_status st = skinny_gemm_plan(M, N, K, &p);
                if (M > SG_MAX_M) {
                    EXPECT(st == SG_ERR_UNSUPPORTED);
                    continue;
                }
                EXPECT(st == SG_OK);
                if (st != SG_OK) continue;
                EXPECT(p.M == M && p.N == N && p.K == K);
                if (M == 0 || N == 0) {
                    EXPECT(p.kernel == SG_KERNEL_NONE);
                    continue;
                }
                EXPECT(p.split_k >= 1 && p.grid >= 1 && p.tile_n >= 1);
                EXPECT((p.workspace_bytes > 0) == (p.two_pass != 0));
                // forcing the plan's own choices reproduces it (on matrix cores the
                // tile width names the kernel: 16 the team kernel, reduced inside the
                // workgroup; 128 or 256 the chunk kernel, whose partials take the
                // second pass whenever it splits K)
                const bool mfma = p.kernel == SG_KERNEL_SPLITK_MFMA;
                sg_plan q;
                const sg_status fs = skinny_gemm_plan_force(
                    M, N, K, p.kernel, p.split_k, mfma ? (p.tile_n == 16 ? 0 : 1) : p.two_pass,
                    mfma ? p.tile_n : 0, &q);
                const bool same = fs == SG_OK && q.kernel == p.kernel && q.split_k == p.split_k &&
                                  q.k_chunk == p.k_chunk && q.tile_n == p.tile_n &&
                                  q.grid == p.grid && q.two_pass == p.two_pass &&
                                  q.workspace_bytes == p.workspace_bytes;
                if (!same && failures < 8)
                    std::fprintf(stderr, "M=%d N=%d K=%d plan k%d S=%d t=%d g=%d tp=%d -> %d: k%d S=%d t=%d g=%d tp=%d\n",
                                 M, N, K, p.kernel, p.split_k, p.tile_n, p.grid, p.two_pass, fs,
                                 q.kernel, q.split_k, q.tile_n, q.grid, q.two_pass);
                EXPECT(same);
                // the low-precision workspace queries answer for every shape
                (void)skinny_gemm_fp8_workspace(M, N, K);
                (void)skinny_gemm_mxfp4_workspace(M, N, K);
            }
    sg_plan p;
    EXPECT(skinny_gemm_plan(1, -1, 8, &p) == SG_ERR_SHAPE);
    EXPECT(skinny_gemm_plan(1, 8, 12, &p) == SG_ERR_ALIGN);
    EXPECT(skinny_gemm_plan(1, 8, 8, nullptr) == SG_ERR_NULL);
    EXPECT(skinny_gemm_plan_force(4, 4096, 7168, SG_KERNEL_GEMV, 1, -1, 0, &p) == SG_ERR_PLAN);
    EXPECT(skinny_gemm_plan_force(20, 4096, 7168, 99, 1, -1, 0, &p) == SG_ERR_PLAN);
}

void calls() {
    const uintptr_t A = 0x10000;
    sg_plan p;
    EXPECT(skinny_gemm_plan(16, 4096, 7168, &p) == SG_OK);
    // null plan, stale plan, missing outputs, misaligned pointers, short workspace
    EXPECT(skinny_gemm(nullptr, fake<sg_bf16>(A), fake<sg_bf16>(A), fake<float>(A), nullptr,
                       nullptr, 0, nullptr) == SG_ERR_NULL);
    sg_plan bad = p;
    bad.grid += 1;
    EXPECT(skinny_gemm(&bad, fake<sg_bf16>(A), fake<sg_bf16>(A), fake<float>(A), nullptr,
                       nullptr, 0, nullptr) == SG_ERR_PLAN);
    EXPECT(skinny_gemm(&p, fake<sg_bf16>(A), fake<sg_bf16>(A), nullptr, nullptr, nullptr, 0,
                       nullptr) == SG_ERR_NULL);
    EXPECT(skinny_gemm(&p, fake<sg_bf16>(A + 2), fake<sg_bf16>(A), fake<float>(A), nullptr,
                       fake<void>(A), p.workspace_bytes, nullptr) == SG_ERR_ALIGN);
    sg_plan two;
    EXPECT(skinny_gemm_plan(64, 4096, 7168, &two) == SG_OK && two.workspace_bytes > 0);
    EXPECT(skinny_gemm(&two, fake<sg_bf16>(A), fake<sg_bf16>(A), fake<float>(A), nullptr,
                       fake<void>(A), two.workspace_bytes - 256, nullptr) == SG_ERR_WORKSPACE);
    EXPECT(skinny_gemm_residual(&p, fake<sg_bf16>(A), fake<sg_bf16>(A), nullptr, fake<sg_bf16>(A),
                                nullptr, nullptr, 0, nullptr) == SG_ERR_NULL);
    // the entry point without a workspace argument: argument and size checks
    EXPECT(skinny_gemm_noalloc(nullptr, fake<sg_bf16>(A), fake<sg_bf16>(A), fake<float>(A), nullptr,
                               nullptr) == SG_ERR_NULL);
    EXPECT(skinny_gemm_noalloc(&bad, fake<sg_bf16>(A), fake<sg_bf16>(A), fake<float>(A), nullptr,
                               nullptr) == SG_ERR_PLAN);
    sg_plan huge;
    EXPECT(skinny_gemm_plan_force(64, 4096, 7168, SG_KERNEL_SPLITK_MFMA, 32, 1, 128, &huge) ==
           SG_OK);  // 32 planes of fp32 partials: 33.5 MB
    EXPECT(huge.workspace_bytes > SG_NOALLOC_MAX_WORKSPACE);
    EXPECT(skinny_gemm_noalloc(&huge, fake<sg_bf16>(A), fake<sg_bf16>(A), fake<float>(A), nullptr,
                               nullptr) == SG_ERR_WORKSPACE);
    // grouped: shapes past the limits
    EXPECT(grouped_skinny_gemm(fake<sg_bf16>(A), 257, fake<sg_bf16>(A), 8, 64, 64, fake<int32_t>(A),
                               8, fake<float>(A), nullptr, nullptr, nullptr, fake<void>(A), 1 << 20,
                               nullptr) == SG_ERR_SHAPE);
    EXPECT(grouped_skinny_gemm(fake<sg_bf16>(A), 4, fake<sg_bf16>(A), 8, 64, 8200, fake<int32_t>(A),
                               8, fake<float>(A), nullptr, nullptr, nullptr, fake<void>(A), 1 << 20,
                               nullptr) == SG_ERR_SHAPE);
    // low precision: limits and workspace
    EXPECT(skinny_gemm_fp8(65, 8, 64, fake<sg_bf16>(A), fake<uint8_t>(A), fake<float>(A), nullptr,
                           fake<float>(A), nullptr, nullptr, 0, nullptr) == SG_ERR_UNSUPPORTED);
    EXPECT(skinny_gemm_fp8(4, 8, 24, fake<sg_bf16>(A), fake<uint8_t>(A), fake<float>(A), nullptr,
                           fake<float>(A), nullptr, nullptr, 0, nullptr) == SG_ERR_ALIGN);
    const size_t need = skinny_gemm_fp8_workspace(20, 4096, 7168);
    EXPECT(need > 0);
    EXPECT(skinny_gemm_fp8(20, 4096, 7168, fake<sg_bf16>(A), fake<uint8_t>(A), fake<float>(A),
                           nullptr, fake<float>(A), nullptr, fake<void>(A), need - 256,
                           nullptr) == SG_ERR_WORKSPACE);
    EXPECT(skinny_gemm_mxfp4(65, 8, 64, fake<sg_bf16>(A), fake<uint8_t>(A), fake<uint8_t>(A),
                             nullptr, fake<float>(A), nullptr, nullptr, 0, nullptr) ==
           SG_ERR_UNSUPPORTED);
    EXPECT(skinny_gemm_mxfp4(4, 8, 48, fake<sg_bf16>(A), fake<uint8_t>(A), fake<uint8_t>(A),
                             nullptr, fake<float>(A), nullptr, nullptr, 0, nullptr) == SG_ERR_ALIGN);
    // router, probe, prefetch
    EXPECT(skinny_gemm_router_topk(fake<float>(A), 4, 8, 9, fake<int32_t>(A), nullptr, nullptr) ==
           SG_ERR_SHAPE);
    EXPECT(skinny_gemm_read_probe(fake<void>(A), 8, 8, 2, 512, nullptr) == SG_ERR_SHAPE);
    EXPECT(skinny_gemm_read_probe(fake<void>(A + 8), 8, 14336, 2, 512, nullptr) == SG_ERR_ALIGN);
    EXPECT(skinny_gemm_read_probe(nullptr, 0, 14336, 2, 512, nullptr) == SG_OK);
    EXPECT(skinny_gemm_prefetch(fake<void>(A), 24, nullptr) == SG_ERR_ALIGN);
    EXPECT(skinny_gemm_prefetch(nullptr, 0, nullptr) == SG_OK);
    // every status has text
    for (int s = SG_OK; s <= SG_ERR_HIP + 1; ++s)
        EXPECT(skinny_gemm_status_str(static_cast<sg_status>(s)) != nullptr);
    uint64_t counts[SG_NUM_COUNTERS];
    skinny_gemm_get_counters(counts);
    for (uint64_t c : counts) EXPECT(c == 0);  // nothing above launched
    skinny_gemm_reset_counters();
}

}  // namespace

int main() {
    plans();
    calls();
    if (failures) std::fprintf(stderr, "host_checks: %d failures\n", failures);
    else std::printf("host_checks: ok\n");
    return failures ? 1 : 0;
}
