// AG-MoE routing on the device: top-k softmax gate, per-expert row lists in
// chunk-arrival order, and the readiness-sorted grouped-GEMM tile list.
//
// Device-level chunks in the pages have sizes that are only known at run time
// for MoE routing (DITRON paper notes, §3.1 device-level interface); the tile
// order of the grouped GEMM starts from the tiles with the fewest pending
// communication dependencies (Triton-Distributed talk, "MoE dynamic sorting").
// Everything here is integer or order-only work except the gate softmax; it is
// deterministic: no atomics whose order could change a result.
//
//   topk_kernel   one wavefront per token, one expert per lane (E <= 64):
//                 k rounds of a butterfly arg-max (ties -> lower expert),
//                 softmax over the k winners, a 64-bit membership mask.
//   count_kernel  one wavefront per expert: ballots over the membership masks.
//   list_kernel   one wavefront per expert: offsets, then the expert's rows in
//                 (p(chunk), token) order via ballot prefix counts; slot[t][j].
//   pair_kernel   one wavefront per (expert, m-tile): readiness key and chunk
//                 mask over the tile's rows.
//   sort_kernel   one workgroup: stable counting sort of the (expert, m-tile)
//                 pairs by key, expanded over the n-tiles.
#include <hip/hip_runtime.h>

#include "tlc_internal.h"

namespace tlc {

namespace {

__device__ inline bool better(float va, int ia, bool oka, float vb, int ib, bool okb) {
  if (oka != okb) return oka;
  if (va != vb) return va > vb;
  return ia < ib;
}

__global__ __launch_bounds__(256) void topk_kernel(MoeDev d) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= d.T) return;
  const bool mine = lane < d.E;
  const float v = mine ? d.logits[static_cast<int64_t>(t) * d.E + lane] : 0.0f;
  bool taken = !mine;
  float win_v[16];
  int win_i[16];
  unsigned long long member = 0;
  for (int j = 0; j < d.k; ++j) {
    float bv = v;
    int bi = lane;
    bool bok = !taken;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const bool ook = __shfl_xor(static_cast<int>(bok), off) != 0;
      if (better(ov, oi, ook, bv, bi, bok)) {
        bv = ov;
        bi = oi;
        bok = ook;
      }
    }
    win_v[j] = bv;
    win_i[j] = bi;
    member |= 1ull << bi;
    if (lane == bi) taken = true;
  }
  if (lane == 0) {
    const float mx = win_v[0];
    float e[16];
    float sum = 0.0f;
    for (int j = 0; j < d.k; ++j) {
      e[j] = expf(win_v[j] - mx);
      sum += e[j];
    }
    for (int j = 0; j < d.k; ++j) {
      d.topk[static_cast<int64_t>(t) * d.k + j] = win_i[j];
      d.gates[static_cast<int64_t>(t) * d.k + j] = e[j] / sum;
    }
    d.member[t] = member;
  }
}

__global__ __launch_bounds__(64) void count_kernel(MoeDev d) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x;
  int total = 0;
  for (int base = 0; base < d.T; base += 64) {
    const int t = base + lane;
    const bool in = t < d.T && ((d.member[t] >> e) & 1ull);
    total += __popcll(__ballot(in));
  }
  if (lane == 0) d.counts[e] = total;
}

__global__ __launch_bounds__(64) void list_kernel(MoeDev d) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x;
  int off = 0, pst = 0;
  for (int i = 0; i < e; ++i) {
    off += d.counts[i];
    pst += (d.counts[i] + d.bm - 1) / d.bm;
  }
  if (lane == 0) {
    d.offsets[e] = off;
    d.pstart[e] = pst;
    if (e == d.E - 1) {
      d.offsets[d.E] = off + d.counts[e];
      d.pstart[d.E] = pst + (d.counts[e] + d.bm - 1) / d.bm;
    }
  }
  int row = off;
  for (int pos = 0; pos < d.world; ++pos) {
    const int c = (d.rank + pos) % d.world;
    for (int base = c * d.Tc; base < (c + 1) * d.Tc; base += 64) {
      const int t = base + lane;
      const bool in = t < (c + 1) * d.Tc && ((d.member[t] >> e) & 1ull);
      const unsigned long long bal = __ballot(in);
      if (in) {
        const int r = row + __popcll(bal & ((1ull << lane) - 1ull));
        d.row_token[r] = t;
        for (int j = 0; j < d.k; ++j)
          if (d.topk[static_cast<int64_t>(t) * d.k + j] == e) d.slot[static_cast<int64_t>(t) * d.k + j] = r;
      }
      row += __popcll(bal);
    }
  }
}

__global__ __launch_bounds__(256) void pair_kernel(MoeDev d) {
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int P = d.pstart[d.E];
  if (q >= P) return;
  int lo = 0, hi = d.E - 1;  // expert e with pstart[e] <= q < pstart[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (d.pstart[mid] <= q) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int mt = q - d.pstart[e];
  const int first = d.offsets[e] + mt * d.bm;
  const int rows = min(d.bm, d.counts[e] - mt * d.bm);
  uint32_t mask = 0;
  int key = 0;
  for (int i = lane; i < rows; i += 64) {
    const int c = d.row_token[first + i] / d.Tc;
    mask |= 1u << c;
    key = max(key, (c - d.rank + d.world) % d.world);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mask |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(mask), off));
    key = max(key, __shfl_xor(key, off));
  }
  if (lane == 0) {
    d.pair_key[q] = d.order == TLC_ORDER_NATURAL ? 0 : key;
    d.pair_mask[q] = mask;
  }
}

__global__ __launch_bounds__(256) void sort_kernel(MoeDev d) {
  __shared__ int bucket[TLC_MAX_WORLD + 1];
  const int P = d.pstart[d.E];
  const int W = d.world;
  const int tid = threadIdx.x;
  if (tid < W) {
    int n = 0;
    for (int q = 0; q < P; ++q) n += d.pair_key[q] == tid;
    bucket[tid + 1] = n;
  }
  __syncthreads();
  if (tid == 0) {
    bucket[0] = 0;
    for (int w = 0; w < W; ++w) bucket[w + 1] += bucket[w];
    *d.n_tiles = P * d.ntiles_n;
  }
  __syncthreads();
  if (tid < W) {
    int out = bucket[tid] * d.ntiles_n;
    int e = 0;
    for (int q = 0; q < P; ++q) {
      while (d.pstart[e + 1] <= q) ++e;
      if (d.pair_key[q] != tid) continue;
      const int mt = q - d.pstart[e];
      const int m0 = d.offsets[e] + mt * d.bm;
      const int rows = min(d.bm, d.counts[e] - mt * d.bm);
      for (int nt = 0; nt < d.ntiles_n; ++nt) {
        tlc_tile tl;
        tl.m0 = m0;
        tl.n0 = nt * d.bn;
        tl.m_rows = rows;
        tl.n_cols = min(d.bn, d.N - nt * d.bn);
        tl.expert = e;
        tl.chunk_mask = d.pair_mask[q];
        tl.key = tid;
        tl.split = 0;
        d.plan[out++] = tl;
      }
    }
  }
}

}  // namespace

int64_t moe_max_pairs(int32_t T, int32_t topk, int32_t experts, int32_t bm) {
  return static_cast<int64_t>(T) * topk / bm + experts;
}

tlc_status launch_moe_route(const MoeDev& d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(topk_kernel, dim3((d.T + 3) / 4), dim3(256), 0, s, d);
  hipLaunchKernelGGL(count_kernel, dim3(d.E), dim3(64), 0, s, d);
  hipLaunchKernelGGL(list_kernel, dim3(d.E), dim3(64), 0, s, d);
  hipLaunchKernelGGL(pair_kernel, dim3((d.max_pairs + 3) / 4), dim3(256), 0, s, d);
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(256), 0, s, d);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "moe route launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace tlc
