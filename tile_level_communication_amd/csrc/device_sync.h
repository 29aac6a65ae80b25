// Device-side signalling helpers shared by the kernels: the bounded wait on
// per-chunk flags and the status report.  A flag is "ready" when it has reached
// the call's epoch, so flags never need to be reset between calls (the caller
// raises the epoch instead).
#pragma once

#include <hip/hip_runtime.h>

#include "tlc.h"

namespace tlc {

// Waits until flag[c] >= epoch for every bit c of `need` (one thread only),
// flag being one of the flag arrays of `sig` (chunk flags, or the scatter
// mode's per-destination ready flags).  Returns 0 when all are ready (after
// an acquire fence at system scope, so the copy engine's and other kernels'
// writes are visible), 1 if the call was aborted (another workgroup failed,
// or this wait timed out).
__device__ inline int wait_flags(tlc_signals* sig, const uint32_t* flag, uint32_t need, uint32_t epoch,
                                 int64_t timeout_ticks, int64_t tile_index) {
  const uint64_t start = wall_clock64();
  while (need) {
    const int c = __builtin_ctz(need);
    const uint32_t v = __hip_atomic_load(&flag[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (static_cast<int32_t>(v - epoch) >= 0) {
      need &= need - 1;
      continue;
    }
    if (__hip_atomic_load(&sig->status[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0)
      return 1;
    if (static_cast<int64_t>(wall_clock64() - start) > timeout_ticks) {
      int expected = 0;
      if (__hip_atomic_compare_exchange_strong(&sig->status[0], &expected, TLC_ERR_TIMEOUT,
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_SYSTEM)) {
        __hip_atomic_store(&sig->status[1], static_cast<int32_t>(tile_index), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(&sig->status[2], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      return 1;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  return 0;
}

// The chunk flags: flags[c] >= epoch  <=>  chunk c has landed.
__device__ inline int wait_chunks(tlc_signals* sig, uint32_t need, uint32_t epoch, int64_t timeout_ticks,
                                  int64_t tile_index) {
  return wait_flags(sig, sig->flags, need, epoch, timeout_ticks, tile_index);
}

__device__ inline void report(tlc_signals* sig, int32_t code, int64_t tile_index) {
  int expected = 0;
  if (__hip_atomic_compare_exchange_strong(&sig->status[0], &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
    __hip_atomic_store(&sig->status[1], static_cast<int32_t>(tile_index), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace tlc
