// Host-side helpers shared by the C ABI sources (argument checks and launch
// sizing).  Internal: not part of include/attn.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ea02 {
namespace abi {

// Whether the byte ranges [a, a + na) and [b, b + nb) overlap (an empty or
// NULL range overlaps nothing).
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Compute units of the current device; 256 (MI355X) when the runtime cannot
// say (e.g. no device visible, as in argument-check tests on a CPU host).
inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}

}  // namespace abi
}  // namespace ea02
