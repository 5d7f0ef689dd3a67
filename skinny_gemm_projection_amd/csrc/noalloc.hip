// noalloc.hip -- skinny_gemm for callers that cannot allocate device memory
// (code under HIP graph capture that must not call hipMalloc, tight serving
// loops, harnesses that forbid allocation).
//
// The two-pass split-K plans need a workspace for their fp32 partial sums.
// Here it is a file-scope device array of kScratchBytes, which every GPU the
// library runs on holds from the first call until the process ends.  Host
// code never passes the array's name to a kernel (on the host that name is a
// stand-in, not a device address): the first call on a device, with that
// device current, asks the runtime for the array's address on that device
// once and keeps it per device; every later call hands that pointer to the
// same kernels skinny_gemm launches.
//
// All calls on one GPU share its array: two calls that overlap in time on one
// GPU (different streams, or different host threads) race on it.  Nothing in
// it needs clearing between calls: the partial kernels write every partial
// slot before the reduction reads it, in stream order.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "plan_internal.h"
#include "skinny_gemm.h"

namespace {

constexpr size_t kScratchBytes = SG_NOALLOC_MAX_WORKSPACE;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the scratch array on the current device (looked up once
// per device, with that device current).
sg_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SG_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return SG_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SG_OK;
}

}  // namespace

extern "C" sg_status skinny_gemm_noalloc(const sg_plan* plan, const sg_bf16* x, const sg_bf16* W,
                                         float* y_f32, sg_bf16* y_bf16, void* stream) {
    if (!plan) return SG_ERR_NULL;
    if (!sg::plan_matches(plan)) return SG_ERR_PLAN;
    if (plan->workspace_bytes > kScratchBytes) return SG_ERR_WORKSPACE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (plan->workspace_bytes > 0) {
        const sg_status st = scratch_on_current_device(&ws);
        if (st != SG_OK) return st;
        ws_bytes = kScratchBytes;
    }
    return skinny_gemm(plan, x, W, y_f32, y_bf16, ws, ws_bytes, stream);
}
