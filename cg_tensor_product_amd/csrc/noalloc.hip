// Scratch memory of oeq_tp_conv_bwd_noalloc: a file-scope device array, so that the
// entry point needs no allocation call.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol); it uses the device address
// hipGetSymbolAddress returns, which is looked up once per device and kept.  Every call
// on a device shares that device's array, and the array keeps the last call's contents.
#include <mutex>

#include "noalloc.hpp"

namespace oeq {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace oeq
