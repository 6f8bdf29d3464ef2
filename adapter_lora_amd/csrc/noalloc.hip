// Fixed exchange workspace of lora_fused_decode_noalloc, for callers that
// cannot allocate device memory.  One array per GPU, zero when the library's
// code object is loaded, holding the same header and exchange slots as a
// caller's workspace.  Nothing in it has to be cleared between calls: every
// launch tags the slots it writes with a tag of its own and reads only slots
// with that tag, so values left by an earlier call are ignored.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"

namespace mlora {

static __device__ __align__(256) unsigned char scratch[LORA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// Device address of the current GPU's array, looked up on the first call for
// that device (with the device current) and kept.  Host code never passes
// the array's name itself: on the host it is only a stand-in for the symbol.
hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!ptr) return hipErrorInvalidSymbol;
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return hipSuccess;
}

}  // namespace mlora
