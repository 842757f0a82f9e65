// kan_forward_static: the layer forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  Its workspace is a fixed array of device memory
// inside the library instead of a caller's buffer; everything else is
// kan_forward.
#include <atomic>

#include "kan_internal.h"

namespace {

// The static workspace: KAN_STATIC_SCRATCH_BYTES of device memory, held by
// every GPU the library runs on until the process ends.  In host code its
// name is only a stand-in for the device symbol; its device address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[KAN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call on that device (racing first calls look it up alike and store
// the same address).
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KAN_ERR_HIP;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KAN_ERR_HIP;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return KAN_OK;
}

}  // namespace

extern "C" {

int kan_forward_static(const kan_desc_t* desc, const void* x, const void* C, const void* W_base, float* y,
                       void* stream) {
    kan::Plan p;
    int st = kan::make_plan(desc, &p, false);
    if (st != KAN_OK) return st;
    if (desc->flags & KAN_FLAG_PREPARED) return KAN_ERR_UNSUPPORTED;   // the array is shared by every call
    if (p.ws_fwd > (size_t)KAN_STATIC_SCRATCH_BYTES) return KAN_ERR_WORKSPACE;
    if ((st = kan::forward_validate(p, x, C, W_base, y, nullptr, 0, true)) != KAN_OK) return st;
    if (p.N == 0) return KAN_OK;
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != KAN_OK) return st;
    return kan::forward_launch(p, desc->flags, x, C, W_base, y, ws, stream);
}

}  // extern "C"
