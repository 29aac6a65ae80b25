// Kernels around the GEMM: the scatter-mode reduce, the CU landing backend
// and the signal helpers.
//
// Reduce (GEMM-ReduceScatter, second half): out = S_0 + S_1 + ... + S_{W-1}
// element-wise in ascending rank order, where S_rank is this rank's own row
// chunk of the partial product and S_s (s != rank) the partial that rank s
// produced for these rows.  It starts once the remote partials' flags reach the
// epoch (Triton-Distributed talk, GEMM-ReduceScatter example: the reduce
// kernel waits on per-tile notifications; here the GEMM precedes the reduce in
// stream order, so only the landed partials are waited for).  float4 loads and
// stores, grid-stride; HBM-bound.
//
// CU landing (AutoOverlap §5.3, backends 4/5: transfers by load/store on SMs,
// signalled through global memory): workgroups copy the chunks in landing
// order; each workgroup publishes its part of a chunk with a release fence and
// an arrival count, and the last arrival raises the chunk's flag.
//
// Sends of the scatter mode (DITRON §3.2 scatter mode; Triton-Distributed
// talk, GEMM-ReduceScatter example: the GEMM notifies per tile, a consumer on
// another stream waits and moves the data): the GEMM raises dest_ready[c] once
// every element of the destination slice P[c] is stored.  Either a
// one-wavefront gate waits for that flag in front of a runtime copy of the
// slice, or a copy kernel's workgroups wait for each slice in send order and
// copy it themselves.
#include <hip/hip_runtime.h>

#include "device_sync.h"
#include "tlc_internal.h"

namespace tlc {
namespace {

constexpr int RED_UNROLL = 4;
typedef float red_vec __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams p) {
  __shared__ int s_abort;
  if (p.wait_mask) {
    if (threadIdx.x == 0) s_abort = wait_chunks(p.sig, p.wait_mask, p.epoch, p.timeout_ticks, -1);
    __syncthreads();
    if (s_abort) return;
  }
  // RED_UNROLL elements per thread per pass, all W sources loaded before the
  // sums, so that W * RED_UNROLL 16-byte loads are in flight; the partials are
  // read once and the output written once (non-temporal both ways: 4 % more
  // bandwidth on the 3 GB slice than plain stores).  The sum runs in ascending
  // source rank.
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * RED_UNROLL;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x * RED_UNROLL + threadIdx.x;
       i0 < p.n_vec4; i0 += stride) {
    red_vec acc[RED_UNROLL];
#pragma unroll
    for (int u = 0; u < RED_UNROLL; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
      if (i < p.n_vec4) acc[u] = __builtin_nontemporal_load(reinterpret_cast<const red_vec*>(p.src[0]) + i);
    }
    for (int s = 1; s < p.world; ++s) {
      red_vec v[RED_UNROLL];
#pragma unroll
      for (int u = 0; u < RED_UNROLL; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
        if (i < p.n_vec4) v[u] = __builtin_nontemporal_load(reinterpret_cast<const red_vec*>(p.src[s]) + i);
      }
#pragma unroll
      for (int u = 0; u < RED_UNROLL; ++u) acc[u] += v[u];
    }
#pragma unroll
    for (int u = 0; u < RED_UNROLL; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
      if (i < p.n_vec4) __builtin_nontemporal_store(acc[u], reinterpret_cast<red_vec*>(p.out) + i);
    }
  }
}

// Each workgroup copies blocks of LAND_THREADS * LAND_UNROLL 16-byte units of a
// chunk: every thread first loads LAND_UNROLL units (consecutive threads read
// consecutive units), then stores them, so each CU keeps 128 KB of reads in
// flight.  The source is read once (non-temporal loads).  The stores are
// device-coherent (sc1: written through past the XCD's L2), so after waiting
// for them a workgroup counts itself in with a relaxed atomic and no L2
// write-back; the last arrival raises the chunk's flag with a release store.
constexpr int LAND_THREADS = 1024;
constexpr int LAND_UNROLL = 8;
constexpr int LAND_CPOL_SC1 = 16;  // cache-policy bit of a device-coherent store
typedef unsigned int land_vec __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t land_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0),
                                           static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           0x00020000);
}

__global__ __launch_bounds__(LAND_THREADS) void land_kernel(LandParams p) {
  const int64_t block = static_cast<int64_t>(LAND_THREADS) * LAND_UNROLL;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * block;
  for (int i = 0; i < p.n_chunks; ++i) {
    const int c = p.order[i];
    const land_vec* src = reinterpret_cast<const land_vec*>(p.src[c]);
    const int64_t n = p.vec_per_chunk;  // a chunk is < 2^32 bytes
    const __amdgpu_buffer_rsrc_t rd = land_rsrc(p.dst[c], static_cast<uint32_t>(n * 16));
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * block + threadIdx.x; base < n;
         base += stride) {
      land_vec v[LAND_UNROLL];
#pragma unroll
      for (int u = 0; u < LAND_UNROLL; ++u) {
        const int64_t k = base + static_cast<int64_t>(u) * LAND_THREADS;
        if (k < n) v[u] = __builtin_nontemporal_load(src + k);
      }
#pragma unroll
      for (int u = 0; u < LAND_UNROLL; ++u) {
        const int64_t k = base + static_cast<int64_t>(u) * LAND_THREADS;
        if (k < n)
          __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, static_cast<int>(k * 16), 0, LAND_CPOL_SC1);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      const int f = p.flag_base + c;
      const uint32_t prev = __hip_atomic_fetch_add(&p.sig->land_count[f], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (prev == gridDim.x - 1) {
        __hip_atomic_store(&p.sig->land_count[f], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.sig->flags[f], p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
}

// Holds the stream until the GEMM has stored every element of slice c.  The
// wait is bounded; after a timeout or another kernel's failure (status[0]
// nonzero) it returns at once and the copy that follows moves stale data.
__global__ __launch_bounds__(64) void send_gate_kernel(tlc_signals* sig, int c, uint32_t epoch,
                                                       int64_t timeout_ticks) {
  if (threadIdx.x == 0) (void)wait_flags(sig, sig->dest_ready, 1u << c, epoch, timeout_ticks, -1);
}

// Every workgroup waits for slice order[i] to be complete, then copies its
// share of it (grid-stride over 16-byte units, LAND_UNROLL loads in flight
// per thread), slice after slice in send order.
__global__ __launch_bounds__(LAND_THREADS) void send_kernel(SendParams p) {
  __shared__ int s_abort;
  const int64_t block = static_cast<int64_t>(LAND_THREADS) * LAND_UNROLL;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * block;
  for (int i = 0; i < p.n; ++i) {
    const int c = p.order[i];
    if (threadIdx.x == 0) s_abort = wait_flags(p.sig, p.sig->dest_ready, 1u << c, p.epoch, p.timeout_ticks, -1);
    __syncthreads();
    if (s_abort) return;
    const land_vec* src = reinterpret_cast<const land_vec*>(p.src[c]);
    land_vec* dst = reinterpret_cast<land_vec*>(p.dst[c]);
    const int64_t n = p.vec_per_slice;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * block + threadIdx.x; base < n;
         base += stride) {
      land_vec v[LAND_UNROLL];
#pragma unroll
      for (int u = 0; u < LAND_UNROLL; ++u) {
        const int64_t k = base + static_cast<int64_t>(u) * LAND_THREADS;
        if (k < n) v[u] = __builtin_nontemporal_load(src + k);
      }
#pragma unroll
      for (int u = 0; u < LAND_UNROLL; ++u) {
        const int64_t k = base + static_cast<int64_t>(u) * LAND_THREADS;
        if (k < n) __builtin_nontemporal_store(v[u], dst + k);
      }
    }
    // the next wait's flag load must not pass this workgroup's reads of s_abort
    __syncthreads();
  }
}

__global__ void signals_set_kernel(tlc_signals* sig, int world, uint32_t value) {
  const int c = threadIdx.x;
  if (c < world) __hip_atomic_store(&sig->flags[c], value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Every flag and ready flag back to 0, before the epochs restart at 1.
__global__ void signals_rewind_kernel(tlc_signals* sig) {
  const int c = threadIdx.x;
  if (c < TLC_MAX_WORLD) {
    __hip_atomic_store(&sig->dest_ready[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&sig->flags[c], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__global__ void status_clear_kernel(tlc_signals* sig) {
  const int i = threadIdx.x;
  if (i < 4) __hip_atomic_store(&sig->status[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (i < TLC_MAX_WORLD)
    __hip_atomic_store(&sig->dest_done[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

tlc_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

tlc_status launch_reduce(const ReduceParams& p, int grid, void* stream) {
  hipLaunchKernelGGL(reduce_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), p);
  return check_launch("reduce");
}

tlc_status launch_land_cu(const LandParams& p, int grid, void* stream) {
  hipLaunchKernelGGL(land_kernel, dim3(grid), dim3(LAND_THREADS), 0, static_cast<hipStream_t>(stream), p);
  return check_launch("land");
}

tlc_status launch_send_gate(tlc_signals* sig, int c, uint32_t epoch, int64_t timeout_ticks,
                            void* stream) {
  hipLaunchKernelGGL(send_gate_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), sig, c,
                     epoch, timeout_ticks);
  return check_launch("send_gate");
}

tlc_status launch_send_cu(const SendParams& p, int grid, void* stream) {
  hipLaunchKernelGGL(send_kernel, dim3(grid), dim3(LAND_THREADS), 0, static_cast<hipStream_t>(stream), p);
  return check_launch("send");
}

tlc_status launch_signals_set(tlc_signals* sig, int world, uint32_t value, void* stream) {
  hipLaunchKernelGGL(signals_set_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), sig,
                     world, value);
  return check_launch("signals_set");
}

tlc_status launch_signals_rewind(tlc_signals* sig, void* stream) {
  hipLaunchKernelGGL(signals_rewind_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), sig);
  return check_launch("signals_rewind");
}

tlc_status launch_status_clear(tlc_signals* sig, void* stream) {
  hipLaunchKernelGGL(status_clear_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), sig);
  return check_launch("status_clear");
}

}  // namespace tlc
