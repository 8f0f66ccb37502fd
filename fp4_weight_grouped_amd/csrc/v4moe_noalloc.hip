// v4moe_noalloc.hip -- the layer forward on a workspace the library owns, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace is a file-scope device array, one copy per GPU, held until the
// process ends.  In host code the array's name is only a host-side stand-in:
// its device address is looked up with hipGetSymbolAddress once per device
// (with that device current) during the library's device set-up, and only that
// address is ever handed to kernels.  Every call on a GPU uses the same array,
// so calls that overlap on one GPU (different streams, or a second host
// thread) race; calls in one stream are ordered.  None of the layer's kernels
// needs the workspace zeroed: every piece of it is written before it is read
// in the same call (the m-tile builder clears its own counters).
#include "v4moe.h"
#include "v4moe_internal.h"

#include <hip/hip_runtime.h>

namespace v4moe {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device
}

hipError_t noalloc_setup_device(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
    return hipSuccess;
}

void* noalloc_scratch(int dev) { return dev >= 0 && dev < kMaxDevices ? g_scratch_ptr[dev] : nullptr; }

}  // namespace v4moe

extern "C" {

__attribute__((visibility("default"))) size_t moe_noalloc_max_workspace_bytes(void) { return v4moe::kScratchBytes; }

__attribute__((visibility("default"))) int moe_layer_forward_noalloc(
    const v4moe_dims* d, const uint16_t* x, const float* w_router, const float* bias, int32_t mode,
    const int64_t* token_ids, const v4moe_experts* w, int32_t* topk_ids, float* topk_w,
    int32_t* expert_offsets, uint16_t* out, void* stream)
{
    const size_t need = moe_workspace_bytes(d);
    if (need == 0) return V4MOE_EDIMS;
    if (need > v4moe::kScratchBytes) return V4MOE_EWORKSPACE;
    if (!v4moe::device_ready()) return V4MOE_EDEVICE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return V4MOE_ELAUNCH;
    void* ws = v4moe::noalloc_scratch(dev);
    if (!ws) return V4MOE_ELAUNCH;
    return v4moe::layer_forward_ws(d, x, w_router, bias, mode, token_ids, w, topk_ids, topk_w, expert_offsets, out,
                                   ws, v4moe::kScratchBytes, stream);
}

}  // extern "C"
