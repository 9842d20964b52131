// Device scratch of the allocation-free backward entry point (see noalloc.hip).
#pragma once

#include <cstddef>

#include <hip/hip_runtime.h>

namespace oeq {

// Bytes of the file-scope device array behind oeq_tp_conv_bwd_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// Device address of that array on the current device (looked up once per device with
// hipGetSymbolAddress, then cached).  Allocates nothing beyond the array itself, which
// the runtime places when it loads this library's device code on the device.
hipError_t noalloc_scratch(void **ptr);

}  // namespace oeq
