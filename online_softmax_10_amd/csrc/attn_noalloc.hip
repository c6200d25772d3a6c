// attn_fwd_masked_noalloc: attn_fwd_masked with the split workspace in a
// static device array instead of a stream-ordered allocation, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Same planning and kernels as
// attn_fwd_masked; the contract is in include/attn.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"
#include "kernels.h"

namespace {

// The split partials of every call on one GPU (each GPU the library runs on
// holds its own copy until the process ends).  In host code `scratch` is only
// a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device.
__device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once known

// The current device's address of `scratch` (set up on the first call there).
int scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        osa::set_hip_detail("hipGetDevice", e);
        return ATTN_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        osa::set_hip_detail("device index beyond the scratch table", hipErrorInvalidDevice);
        return ATTN_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            osa::set_hip_detail("hipGetSymbolAddress of the static scratch", e != hipSuccess ? e : hipErrorUnknown);
            return ATTN_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_masked_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                                       int64_t H, int64_t N, int64_t M, int d, float scale, const attn_mask *mask,
                                       int dtype, int num_splits, void *stream) {
    osa::PlannedCall plan;
    bool nothing = false;
    int rc = osa::plan_attn(q, k, v, o, lse, B, H, N, M, d, scale, mask, dtype, num_splits, &plan, &nothing);
    if (rc != ATTN_OK || nothing) return rc;
    // Checked before any HIP call.
    if (plan.split && plan.workspace_bytes > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    void *ws = nullptr;
    if (plan.split) {
        rc = scratch_address(&ws);
        if (rc != ATTN_OK) return rc;
    }
    // The kernels write every partial the merge reads, so nothing in the
    // scratch needs clearing between calls.
    return osa::launch_planned(plan, ws, static_cast<hipStream_t>(stream));
}
