// Host-side helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/fp8bs.h"

namespace fp8bs {

// Largest 1-D grid the launchers use (gridDim.x is 32 bits; keep well inside it).
constexpr int64_t kMaxGrid = 0x7FFFFFFFLL;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Status after enqueueing: a launch the runtime rejected is reported here; a
// fault inside a kernel surfaces at the caller's next synchronization.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_LAUNCH;
}

// Inputs above this size are read (and, for weight codes, written) with the
// non-temporal hint: at more than half of the 256 MB last-level cache they
// are not expected to be found there, and the hint keeps them from evicting
// data that is.  Smaller inputs may still be cached from their producer.
constexpr int64_t kStreamBytes = 128LL << 20;

// Compute units of the current device, cached per device ordinal.  Each
// entry is an atomic, so host threads calling the library at once see either
// 0 (and query the attribute themselves) or the device's count; the tile
// shape, the persistent grid and the dgrad contraction split are sized by it.
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fp8bs
