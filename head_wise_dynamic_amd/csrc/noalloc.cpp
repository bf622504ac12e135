// saf_sparse_attention_noalloc: the layer for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The workspace comes from a file-scope
// device array, `scratch`, instead of the caller; every GPU the library runs
// on holds its own copy until the process ends.  In host code the array's
// name is a host-side stand-in, not a device address: kernels and copies only
// ever get the per-device address that hipGetSymbolAddress returns, looked up
// once per device, with that device current, on the entry point's first call
// there.  The contract is in include/saf3r.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// this device's address of `scratch` (looked up on the first call here)
saf_status_t scratch_address(saf_ctx_t *c, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return saf_fail_internal(c, SAF_EHIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return saf_fail_internal(c, SAF_EUNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return saf_fail_internal(c, SAF_EHIP, "hipGetSymbolAddress(scratch) failed");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SAF_OK;
}

}  // namespace

extern "C" saf_status_t saf_sparse_attention_noalloc(saf_ctx_t *c, const saf_head_plan_t *plan, const void *q,
                                                     const void *k, const void *v, void *o, saf_layout_t lay,
                                                     const int32_t *vert_idx, int64_t vert_ld, void *stream) {
    if (!c) return SAF_EINVAL;
    size_t need = 0;
    // the plan and its workspace size first: nothing touches the device when
    // either is rejected
    saf_status_t st = saf_layer_internal(c, plan, q, k, v, o, lay, vert_idx, vert_ld, nullptr, 0, stream,
                                         kScratchBytes, &need);
    if (st != SAF_OK) return st;
    void *ws = nullptr;
    if ((st = scratch_address(c, &ws)) != SAF_OK) return st;
    return saf_layer_internal(c, plan, q, k, v, o, lay, vert_idx, vert_ld, ws, kScratchBytes, stream, kScratchBytes,
                              &need);
}
