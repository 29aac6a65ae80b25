// Co-located landing (AutoOverlap §5.3, backend 5: transfers by load/store
// instructions on the SMs that compute, coordinated through global-memory
// signals), shared by the GEMM kernels and the AG-MoE top-k kernel.
//
// Each thread keeps COPY_UNROLL 16-byte loads in flight (non-temporal: the
// source is read once).  The stores are device-coherent (sc1: written through
// past the XCD's L2), so after waiting for them a workgroup counts itself into
// the chunk's arrival counter with a relaxed atomic and no L2 write-back; the
// share that completes a chunk rewinds the counter and raises the chunk's flag
// with a release store at system scope.
#pragma once

#include <hip/hip_runtime.h>

#include "tlc_internal.h"

namespace tlc {

constexpr int COPY_UNROLL = 16;
constexpr int CPOL_SC1 = 16;  // cache-policy bit of a device-coherent store
typedef unsigned int copy_vec __attribute__((ext_vector_type(4)));

// Store-side buffer resource with wave-uniform fields.
__device__ inline __amdgpu_buffer_rsrc_t copy_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0),
                                           static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           0x00020000);
}

// Copies units [lo, hi) of chunk i (hi - lo < 2^27: 32-bit offsets), waits for the stores and
// counts the workgroup in; `arrivals` shares complete the chunk.
__device__ inline void copy_share(const CopyPlan& cp, int i, int64_t lo, int64_t hi, uint32_t arrivals,
                                  tlc_signals* sig, uint32_t epoch) {
  const int nt = blockDim.x;
  const int cnt = static_cast<int>(hi - lo);
  const copy_vec* src = reinterpret_cast<const copy_vec*>(cp.src[i]) + lo;
  const __amdgpu_buffer_rsrc_t rd = copy_rsrc(cp.dst[i] + lo, static_cast<uint32_t>(cnt) * 16u);
  for (int base = threadIdx.x; base < cnt; base += nt * COPY_UNROLL) {
    copy_vec v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) {
      const int k = base + u * nt;
      if (k < cnt) v[u] = __builtin_nontemporal_load(src + k);
    }
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) {
      const int k = base + u * nt;
      if (k < cnt) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, k * 16, 0, CPOL_SC1);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int c = cp.flag[i];
    const uint32_t prev =
        __hip_atomic_fetch_add(&sig->land_count[c], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == arrivals - 1) {
      __hip_atomic_store(&sig->land_count[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&sig->flags[c], epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// Landing order: workgroup g < cp.wgs copies the g-th of cp.wgs equal shares
// of every chunk, chunk after chunk, so that the chunks land in order while
// the other workgroups compute.
__device__ inline void copy_in_landing_order(const CopyPlan& cp, tlc_signals* sig, uint32_t epoch) {
  const int g = blockIdx.x;
  const int64_t lo = cp.vec * g / cp.wgs, hi = cp.vec * (g + 1) / cp.wgs;
  for (int i = 0; i < cp.chunks; ++i)
    copy_share(cp, i, lo, hi, static_cast<uint32_t>(cp.wgs), sig, epoch);
}

// All chunks at once: cp.wgs = per * cp.chunks copying workgroups, copying
// workgroup g (0 <= g < cp.wgs) copies share g % per of chunk g / per (one
// arrival per workgroup).
__device__ inline void copy_by_chunk(const CopyPlan& cp, int g, tlc_signals* sig, uint32_t epoch) {
  const int per = cp.wgs / cp.chunks;
  const int i = g / per, s = g % per;
  copy_share(cp, i, cp.vec * s / per, cp.vec * (s + 1) / per, static_cast<uint32_t>(per), sig, epoch);
}

}  // namespace tlc
