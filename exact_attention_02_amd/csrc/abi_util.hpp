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

// A dispatch counts its work-items in 32 bits.  Most workgroups a launch of
// `threads`-thread workgroups may take, leaving room for the spare workgroups
// of work stealing (plan_steal adds at most a tenth plus 8).
inline int64_t max_launch_blocks(int64_t threads) { return (int64_t(UINT32_MAX) / threads - 8) * 8 / 9; }

// Compute units of the current device; 256 (MI355X) when the runtime cannot
// say (e.g. no device visible, as in argument-check tests on a CPU host).
inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}

// Work stealing between the XCDs (work_item in attn_fwd_kernel.hpp).  The
// claim counters of `stream` on the current device (a slot of a static
// device array, zero between launches), or nullptr when the launch must keep
// the static order (graph capture, hipStreamPerThread, no free slot).
int* steal_slot(hipStream_t stream);

// How a launch of `items` workgroups (wg_per_cu of them fit on a CU) runs:
// counters (nullptr: static order), the workgroups that keep their own item,
// and the grid to launch (items plus spare workgroups for the fast XCDs).
struct StealPlan {
  int* counters;
  int n_static;
  int64_t launch_grid;
};
StealPlan plan_steal(hipStream_t stream, int64_t items, int64_t wg_per_cu);

}  // namespace abi
}  // namespace ea02
