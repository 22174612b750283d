// Declarations shared by every HIP source of the library (not part of the C ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vap.h"

namespace vap {

// Timing events of one launch (both null when the kernel timer is off).  The launchers pass them
// to hipExtLaunchKernelGGL, which stamps the kernel's own start and end, so the interval excludes
// the wait between the previous kernel's end and this kernel's first wave.
struct KTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace vap
