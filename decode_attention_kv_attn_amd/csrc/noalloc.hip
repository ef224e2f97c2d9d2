// Fixed device scratch for attn_decode_gqa_noalloc, the entry point for
// callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, from the first use of this code
// object on that GPU until the process ends.  In host code the array's name
// is only a host-side stand-in, never a device address: the address is read
// once per device with hipGetSymbolAddress (that device current) and kept,
// and only that address is handed to kernels.  The array has no initialiser,
// so each copy starts as zeros; its first kArriveBytes serve as the arrival
// counters of the in-kernel split merge, which every call leaves at zero.
#include <atomic>

#include "kernels.h"

namespace attn {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];   // 0 = not looked up yet
}  // namespace

hipError_t noalloc_scratch(void** out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (a == 0) {
        // first call on this device: this device's copy of the array
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        a = (uintptr_t)ptr;
        g_scratch_addr[dev].store(a, std::memory_order_release);   // racing threads store the same value
    }
    *out = (void*)a;
    return hipSuccess;
}

}  // namespace attn
