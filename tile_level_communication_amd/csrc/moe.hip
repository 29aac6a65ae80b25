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
// Tokens are visited in arrival order: the local chunk first, then rank+1,
// rank+2, ... (position a = p(c) * Tc + token offset), in blocks of 64.
//
//   topk_kernel     (optionally, its first workgroups also land the peers'
//                   token chunks: the co-located landing beside the routing)
//                   one wavefront per token, one expert per lane (E <= 64):
//                   k rounds of a wavefront maximum of order-preserving keys
//                   and a ballot for the lowest expert holding it (ties ->
//                   lower expert), softmax over the k winners, a 64-bit
//                   membership mask.
//   block_count     one wavefront per block of 64 arrival positions: for each
//                   expert, how many of the block's tokens chose it.
//   scan_kernel     sixteen wavefronts over runs of blocks: per expert, the
//                   prefix of those counts over the blocks; counts, offsets and
//                   m-tile starts over experts.
//   scatter_kernel  one wavefront per (block, 16 experts): each (token, expert)
//                   pair's row = offsets[e] + rows of e in earlier blocks +
//                   earlier lanes of this block; row_token and slot.
//   pair_kernel     one wavefront per (expert, m-tile): readiness key and chunk
//                   mask over the tile's rows.
//   sort_kernel     one workgroup: stable counting sort of the (expert, m-tile)
//                   pairs by key (ballot ranks per wavefront, carried over
//                   batches of pairs), expanded over the n-tiles.
#include <hip/hip_runtime.h>

#include <mutex>

#include "colocated_copy.h"
#include "tlc_internal.h"

namespace tlc {

namespace {

// Order-preserving map of a float to an unsigned key (-0 counts as +0, as in
// a value comparison); 0 is below every finite float's key.
__device__ inline uint32_t ordered_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Maximum over the wavefront, the same in every lane: quad swaps, half-row and
// row mirrors (DPP), then the four rows' maxima through scalar registers.
__device__ inline uint32_t wave_max(uint32_t x) {
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(x), static_cast<int>(x),
                                                               0xB1, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(x), static_cast<int>(x),
                                                               0x4E, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(x), static_cast<int>(x),
                                                               0x141, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(x), static_cast<int>(x),
                                                               0x140, 0xF, 0xF, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Routing of token t by one wavefront (lane = expert): k rounds of the
// largest remaining logit (wave maximum of the ordered keys) and the lowest
// expert holding it (first set bit of the ballot), then the softmax over the k
// winners in lane 0.  Returns the membership mask (the same in every lane).
__device__ inline unsigned long long route_token(const MoeDev& d, int t, int lane) {
  const bool mine = lane < d.E;
  const uint32_t key = mine ? ordered_key(d.logits[static_cast<int64_t>(t) * d.E + lane]) : 0u;
  bool taken = !mine;
  float win_v[16];
  int win_i[16];
  unsigned long long member = 0;
  for (int j = 0; j < d.k; ++j) {
    const uint32_t kk = taken ? 0u : key;
    const uint32_t mx = wave_max(kk);
    int bi = __ffsll(static_cast<unsigned long long>(__ballot(kk == mx))) - 1;
    bi = bi < 0 ? 0 : bi;  // a lane always holds the maximum; keeps the mask shift defined
    win_v[j] = key_value(mx);
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
  return member;
}

// Token at arrival position a (0 <= a < T).
__device__ inline int arrival_token(const MoeDev& d, int a) {
  const int pos = a / d.Tc;
  const int c = (d.rank + pos) % d.world;
  return c * d.Tc + (a - pos * d.Tc);
}

__global__ __launch_bounds__(256) void topk_kernel(MoeDev d) {
  // co-located landing of the token chunks (d.copy.wgs = 0: none); the
  // routing waits for nothing, so the copy overlaps it
  if (static_cast<int>(blockIdx.x) < d.copy.wgs) copy_by_chunk(d.copy, d.sig, d.epoch);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < d.T) route_token(d, t, threadIdx.x & 63);
}

__global__ __launch_bounds__(64) void block_count_kernel(MoeDev d) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int a = b * 64 + lane;
  const unsigned long long m = a < d.T ? d.member[arrival_token(d, a)] : 0ull;
  int mine = 0;
  for (int e = 0; e < d.E; ++e) {
    const int n = __popcll(__ballot((m >> e) & 1ull));
    if (lane == e) mine = n;
  }
  if (lane < d.E) d.blk[static_cast<int64_t>(b) * d.E + lane] = mine;
}

// Sixteen wavefronts: wavefront w takes a contiguous run of blocks, lane =
// expert.  Its per-expert total goes through LDS; each wavefront then rewrites
// its blocks with the exclusive prefix (the totals of the runs before it plus
// its own running sum), and wavefront 0 forms counts, offsets and m-tile starts.
constexpr int SCAN_WAVES = 16;

__global__ __launch_bounds__(64 * SCAN_WAVES) void scan_kernel(MoeDev d) {
  __shared__ int part[SCAN_WAVES][64];
  const int e = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int NB = (d.T + 63) / 64;
  const int per = (NB + SCAN_WAVES - 1) / SCAN_WAVES;
  const int b_lo = min(NB, w * per), b_hi = min(NB, b_lo + per);
  const bool lane_ok = e < d.E;
  int v[16];
  int tot = 0;
  for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = (lane_ok && b0 + i < b_hi) ? d.blk[static_cast<int64_t>(b0 + i) * d.E + e] : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += v[i];
  }
  part[w][e] = tot;
  __syncthreads();
  int run = 0;
  for (int u = 0; u < w; ++u) run += part[u][e];
  // a run of at most 16 blocks is still in v[]; longer runs are read again
  for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
    if (per > 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = (lane_ok && b0 + i < b_hi) ? d.blk[static_cast<int64_t>(b0 + i) * d.E + e] : 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (lane_ok && b0 + i < b_hi) d.blk[static_cast<int64_t>(b0 + i) * d.E + e] = run;
      run += v[i];
    }
  }
  if (w != 0) return;
  run = 0;
  for (int u = 0; u < SCAN_WAVES; ++u) run += part[u][e];
  const int cnt = e < d.E ? run : 0;
  const int tiles = (cnt + d.bm - 1) / d.bm;
  // exclusive scans over the experts (lanes)
  int off = cnt, pst = tiles;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const int o = __shfl_up(off, sh), q = __shfl_up(pst, sh);
    if (e >= sh) {
      off += o;
      pst += q;
    }
  }
  if (e < d.E) {
    d.counts[e] = cnt;
    d.offsets[e] = off - cnt;
    d.pstart[e] = pst - tiles;
    if (e == d.E - 1) {
      d.offsets[d.E] = off;
      d.pstart[d.E] = pst;
    }
  }
}

// One wavefront per (block of 64 arrival positions, group of 16 experts).
constexpr int SCATTER_GROUP = 16;

__global__ __launch_bounds__(64) void scatter_kernel(MoeDev d) {
  const int b = blockIdx.x, g0 = blockIdx.y * SCATTER_GROUP, lane = threadIdx.x;
  const int a = b * 64 + lane;
  const bool valid = a < d.T;
  const int t = valid ? arrival_token(d, a) : 0;
  const unsigned long long m = valid ? d.member[t] : 0ull;
  // lane j < 16 holds the first row of expert g0 + j for this block
  const int ej = g0 + lane;
  const int base = (lane < SCATTER_GROUP && ej < d.E)
                       ? d.offsets[ej] + d.blk[static_cast<int64_t>(b) * d.E + ej]
                       : 0;
  int sel[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    sel[j] = (valid && j < d.k) ? d.topk[static_cast<int64_t>(t) * d.k + j] : -1;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < SCATTER_GROUP; ++j) {
    const int e = g0 + j;
    const bool in = e < d.E && ((m >> e) & 1ull);
    const unsigned long long bal = __ballot(in);
    const int first = __shfl(base, j);
    if (in) {
      const int r = first + __popcll(bal & below);
      d.row_token[r] = t;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (sel[q] == e) d.slot[static_cast<int64_t>(t) * d.k + q] = r;
    }
  }
}

// Pair q = (expert e, m-tile mt) by one wavefront: the readiness key (latest
// consume position of the chunks its rows come from) and the chunk mask.
__device__ inline void pair_one(const MoeDev& d, int q, int lane) {
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

__global__ __launch_bounds__(256) void pair_kernel(MoeDev d) {
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q < d.pstart[d.E]) pair_one(d, q, threadIdx.x & 63);
}

__global__ __launch_bounds__(1024) void sort_kernel(MoeDev d) {
  constexpr int NW = 16;  // wavefronts per workgroup
  __shared__ int bucket[TLC_MAX_WORLD + 1];
  __shared__ int carry[TLC_MAX_WORLD];
  __shared__ int wave_cnt[NW][TLC_MAX_WORLD];
  const int P = d.pstart[d.E];
  const int W = d.world;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid <= TLC_MAX_WORLD) bucket[tid] = 0;
  if (tid < TLC_MAX_WORLD) carry[tid] = 0;
  __syncthreads();
  for (int q = tid; q < P; q += blockDim.x) atomicAdd(&bucket[d.pair_key[q] + 1], 1);
  __syncthreads();
  if (tid == 0) {
    for (int w = 0; w < W; ++w) bucket[w + 1] += bucket[w];
    *d.n_tiles = P * d.ntiles_n;
  }
  __syncthreads();
  // stable ranks: pairs in q order, a batch of blockDim.x pairs at a time
  for (int q0 = 0; q0 < P; q0 += blockDim.x) {
    const int q = q0 + tid;
    const bool valid = q < P;
    const int key = valid ? d.pair_key[q] : -1;
    int local = 0;
    for (int w = 0; w < W; ++w) {
      const unsigned long long bal = __ballot(key == w);
      if (key == w) local = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_cnt[wave][w] = __popcll(bal);
    }
    __syncthreads();
    if (valid) {
      int rank = carry[key] + local;
      for (int v = 0; v < wave; ++v) rank += wave_cnt[v][key];
      int lo = 0, hi = d.E - 1;  // expert e with pstart[e] <= q < pstart[e+1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (d.pstart[mid] <= q) lo = mid; else hi = mid - 1;
      }
      const int e = lo;
      const int mt = q - d.pstart[e];
      const int m0 = d.offsets[e] + mt * d.bm;
      const int rows = min(d.bm, d.counts[e] - mt * d.bm);
      const int out = (bucket[key] + rank) * d.ntiles_n;
      for (int nt = 0; nt < d.ntiles_n; ++nt) {
        tlc_tile tl;
        tl.m0 = m0;
        tl.n0 = nt * d.bn;
        tl.m_rows = rows;
        tl.n_cols = min(d.bn, d.N - nt * d.bn);
        tl.expert = e;
        tl.chunk_mask = d.pair_mask[q];
        tl.key = key;
        tl.split = 0;
        d.plan[out + nt] = tl;
      }
    }
    __syncthreads();
    if (tid < W) {
      int add = 0;
      for (int v = 0; v < NW; ++v) add += wave_cnt[v][tid];
      carry[tid] += add;
    }
    __syncthreads();
  }
}

}  // namespace

int64_t moe_max_pairs(int32_t T, int32_t topk, int32_t experts, int32_t bm) {
  return static_cast<int64_t>(T) * topk / bm + experts;
}

tlc_status launch_moe_route(const MoeDev& d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = (d.T + 63) / 64;
  const int topk_grid = (d.T + 3) / 4;
  hipLaunchKernelGGL(topk_kernel, dim3(topk_grid > d.copy.wgs ? topk_grid : d.copy.wgs), dim3(256), 0,
                     s, d);
  hipLaunchKernelGGL(block_count_kernel, dim3(nb), dim3(64), 0, s, d);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(64 * SCAN_WAVES), 0, s, d);
  hipLaunchKernelGGL(scatter_kernel, dim3(nb, (d.E + SCATTER_GROUP - 1) / SCATTER_GROUP), dim3(64),
                     0, s, d);
  hipLaunchKernelGGL(pair_kernel, dim3((d.max_pairs + 3) / 4), dim3(256), 0, s, d);
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(1024), 0, s, d);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "moe route launch: %s", hipGetErrorString(e));
  return ok();
}

// Workspace of the routing variant that allocates nothing (tlc_moe_route_static):
// one array in every device's memory, kept until the process ends.  In host
// code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) char scratch[kMoeStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

tlc_status moe_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TLC_ERR_UNSUPPORTED, "device id %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TLC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TLC_OK;
}

}  // namespace tlc
