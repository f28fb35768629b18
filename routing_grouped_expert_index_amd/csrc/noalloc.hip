// moe_decode_forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// same launches, with the workspace in a file-scope device array of this
// library instead of a caller-supplied buffer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "moe.h"
#include "launch.h"

namespace moe {
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
}

// Each GPU the library runs on holds its own copy until the process ends.  In
// host code this name is only a handle for hipGetSymbolAddress, never an
// address to pass to a kernel.
static __device__ __align__(256) uint8_t scratch[moe::kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current device's copy of `scratch`, looked up once
// per device with that device current.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return moe::set_error(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return moe::set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" int moe_decode_forward_noalloc(const float* logits, const void* x, int T, int E, int k,
                                          moe_routes* routes, const moe_packed_weights* w, const moe_scales* scales,
                                          void* out, int H, int I, int quant, int path, const moe_ep* ep,
                                          void* stream) {
    // anything but a non-empty route-direct call is validated and answered by the
    // regular entry without the scratch (errors, the empty batch)
    if (T == 0 || moe_select_path(T, H, I, E, k, quant, path) != MOE_PATH_ROUTE_DIRECT)
        return moe_decode_forward(logits, x, T, E, k, routes, w, scales, out, H, I, quant, path, ep, nullptr, 0,
                                  stream);
    const size_t need = moe_forward_workspace_size(T, H, I, E, k, quant, path);
    if (need > moe::kNoAllocScratchBytes)
        return moe::set_error(MOE_ERR_UNSUPPORTED,
                              "this call needs %zu bytes of workspace; the static scratch holds %zu", need,
                              moe::kNoAllocScratchBytes);
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != MOE_OK) return rc;
    return moe_decode_forward(logits, x, T, E, k, routes, w, scales, out, H, I, quant, path, ep, ws,
                              moe::kNoAllocScratchBytes, stream);
}
