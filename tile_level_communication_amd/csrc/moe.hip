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
// rank+2, ... (the chunk consumed p-th is c = (rank + p) mod world).  Each
// chunk's tokens split into blocks of up to 16 consecutive tokens (a block
// never spans two chunks), numbered in arrival order.  Three kernels:
//
//   route_kernel    one workgroup per block, one wavefront per token, one
//                   expert per lane (E <= 64), k rounds of a wavefront
//                   maximum of order-preserving keys and a ballot for the
//                   lowest expert holding it (ties -> lower expert); lane j
//                   keeps winner j, so the softmax over the k winners and the
//                   stores are lane-parallel; a 64-bit membership mask per
//                   token; then the block's token count per expert.
//                   Optionally, workgroups after the blocks' land the peers'
//                   token chunks (the co-located landing beside the routing).
//   plan_kernel     one workgroup of sixteen wavefronts, lane = expert: the
//                   exclusive prefix of the block counts over the blocks (each
//                   wavefront a contiguous run), the rows of every expert that
//                   come before each chunk position, counts, offsets and
//                   m-tile starts; then every (expert, m-tile) pair's
//                   readiness key and chunk mask, read off those per-position
//                   row ranges, and a stable counting sort of the pairs by key
//                   (ballot ranks per wavefront, carried over batches),
//                   expanded over the n-tiles.
//   scatter_kernel  one wavefront per (four blocks, sixteen experts): each
//                   (token, expert) pair's row = offsets[e] + rows of e in
//                   earlier blocks + earlier tokens of its block; row_token and
//                   slot.
#include <hip/hip_runtime.h>

#include <mutex>

#include "colocated_copy.h"
#include "tlc_internal.h"

namespace tlc {

namespace {

constexpr int BLK = 16;  // tokens per arrival block

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

// Sum over the wavefront, the same in every lane: the steps of wave_max with
// an addition (every step adds two disjoint sets of lanes), then the four
// rows' sums.
template <int CTRL>
__device__ inline float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x),
                                                                   __builtin_bit_cast(int, x), CTRL,
                                                                   0xF, 0xF, false));
}

__device__ inline float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

__device__ inline float wave_sum(float x) {
  x = dpp_add<0xB1>(x);
  x = dpp_add<0x4E>(x);
  x = dpp_add<0x141>(x);
  x = dpp_add<0x140>(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}

// Blocks per chunk position, and the token in slot i of block b (-1 past the
// chunk's end).
__device__ inline int blocks_per_chunk(const MoeDev& d) { return (d.Tc + BLK - 1) / BLK; }

__device__ inline int block_token(const MoeDev& d, int bpc, int b, int i) {
  const int p = b / bpc;
  const int off = (b - p * bpc) * BLK + i;
  if (off >= d.Tc) return -1;
  return ((d.rank + p) % d.world) * d.Tc + off;
}

// Routing of token t by one wavefront (lane = expert, `key` the lane's
// ordered logit key): k rounds of the largest remaining key (wave maximum)
// and the lowest expert holding it (first set bit of the ballot); lane j keeps
// winner j, then the softmax over the k winners.  Returns the membership mask
// (the same in every lane).
__device__ inline unsigned long long route_token(const MoeDev& d, int t, uint32_t key, int lane) {
  bool taken = lane >= d.E;
  uint32_t top = 0, my_key = 0;
  int my_e = 0;
  unsigned long long member = 0;
  for (int j = 0; j < d.k; ++j) {
    const uint32_t kk = taken ? 0u : key;
    const uint32_t mx = wave_max(kk);
    int bi = __ffsll(static_cast<unsigned long long>(__ballot(kk == mx))) - 1;
    bi = bi < 0 ? 0 : bi;  // a lane always holds the maximum; keeps the mask shift defined
    if (j == 0) top = mx;
    if (lane == j) {
      my_key = mx;
      my_e = bi;
    }
    member |= 1ull << bi;
    if (lane == bi) taken = true;
  }
  const bool win = lane < d.k;
  const float ex = win ? expf(key_value(my_key) - key_value(top)) : 0.0f;
  const float sum = wave_sum(ex);
  if (win) {
    d.topk[static_cast<int64_t>(t) * d.k + lane] = my_e;
    d.gates[static_cast<int64_t>(t) * d.k + lane] = ex / sum;
  }
  return member;
}

__global__ __launch_bounds__(64 * BLK) void route_kernel(MoeDev d, int nb) {
  const int g = blockIdx.x;
  if (g >= nb) {
    // co-located landing of the token chunks, after the blocks' workgroups;
    // the routing waits for nothing, so the copy overlaps it
    copy_by_chunk(d.copy, g - nb, d.sig, d.epoch);
    return;
  }
  __shared__ unsigned long long s_member[BLK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wavefront w routes the block's token w
  const int t = block_token(d, blocks_per_chunk(d), g, wave);
  unsigned long long m = 0;
  if (t >= 0) {
    const uint32_t key = lane < d.E ? ordered_key(d.logits[static_cast<int64_t>(t) * d.E + lane]) : 0u;
    m = route_token(d, t, key, lane);
    if (lane == 0) d.member[t] = m;
  }
  if (lane == 0) s_member[wave] = m;
  __syncthreads();
  if (wave == 0 && lane < d.E) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < BLK; ++i) n += static_cast<int>((s_member[i] >> lane) & 1ull);
    d.blk[static_cast<int64_t>(g) * d.E + lane] = n;
  }
}

constexpr int PLAN_WAVES = 16;

__global__ __launch_bounds__(64 * PLAN_WAVES) void plan_kernel(MoeDev d, int nb) {
  __shared__ int part[PLAN_WAVES][64];
  __shared__ int pos_pre[TLC_MAX_WORLD + 1][64];  // rows of expert e before chunk position p
  __shared__ int s_cnt[64], s_off[65], s_pst[65];
  __shared__ int key_cnt[TLC_MAX_WORLD];  // pairs per readiness key, then the first slot of each
  __shared__ int carry[TLC_MAX_WORLD];
  __shared__ int wave_cnt[PLAN_WAVES][TLC_MAX_WORLD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int e = lane;
  const int bpc = blocks_per_chunk(d);
  const int W = d.world;
  const bool lane_ok = e < d.E;
  // per-expert totals of each wavefront's run of blocks
  const int per = (nb + PLAN_WAVES - 1) / PLAN_WAVES;
  const int b_lo = min(nb, w * per), b_hi = min(nb, b_lo + per);
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
  if (tid < TLC_MAX_WORLD) {
    key_cnt[tid] = 0;
    carry[tid] = 0;
  }
  __syncthreads();
  // each block's counts become their exclusive prefix; the first block of a
  // chunk position gives the rows before that position
  int run = 0;
  for (int u = 0; u < w; ++u) run += part[u][e];
  int pos = (b_lo + bpc - 1) / bpc, pos_b = pos * bpc;  // next position's first block
  for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
    if (per > 16) {  // a run of at most 16 blocks is still in v[]
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = (lane_ok && b0 + i < b_hi) ? d.blk[static_cast<int64_t>(b0 + i) * d.E + e] : 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int b = b0 + i;
      if (lane_ok && b < b_hi) {
        d.blk[static_cast<int64_t>(b) * d.E + e] = run;
        if (b == pos_b) {
          pos_pre[pos][e] = run;
          ++pos;
          pos_b += bpc;
        }
      }
      run += v[i];
    }
  }
  if (w == 0) {
    run = 0;
    for (int u = 0; u < PLAN_WAVES; ++u) run += part[u][e];
    const int cnt = lane_ok ? run : 0;
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
    if (lane_ok) {
      pos_pre[W][e] = cnt;
      s_cnt[e] = cnt;
      s_off[e] = off - cnt;
      s_pst[e] = pst - tiles;
      d.counts[e] = cnt;
      d.offsets[e] = off - cnt;
      if (e == d.E - 1) {
        s_off[d.E] = off;
        s_pst[d.E] = pst;
        d.offsets[d.E] = off;
      }
    }
  }
  __syncthreads();
  const int P = s_pst[d.E];
  // pair q = (expert e, m-tile mt): its expert, readiness key (the latest
  // chunk position among its rows; 0 in natural order) and chunk mask, read
  // off the expert's rows per position (rows pos_pre[p][e] .. pos_pre[p+1][e]
  // - 1 come from the chunk consumed p-th)
  auto pair_info = [&](int q, int* pe, uint32_t* pmask) __attribute__((always_inline)) {
    int lo = 0, hi = d.E - 1;  // expert with s_pst[e] <= q < s_pst[e+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pst[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int ex = lo;
    const int r0 = (q - s_pst[ex]) * d.bm, r1 = min(r0 + d.bm, s_cnt[ex]);
    uint32_t mask = 0;
    int key = 0;
    int c = d.rank;  // chunk consumed p-th
    for (int p = 0; p < W; ++p) {
      if (max(pos_pre[p][ex], r0) < min(pos_pre[p + 1][ex], r1)) {
        mask |= 1u << c;
        key = p;
      }
      c = c + 1 == W ? 0 : c + 1;
    }
    *pe = ex;
    *pmask = mask;
    return d.order == TLC_ORDER_NATURAL ? 0 : key;
  };
  // the first batch of pairs keeps its information in registers
  int ex0 = 0;
  uint32_t mask0 = 0;
  const int key0 = tid < P ? pair_info(tid, &ex0, &mask0) : -1;
  if (key0 >= 0) atomicAdd(&key_cnt[key0], 1);
  for (int q = tid + blockDim.x; q < P; q += blockDim.x) {
    int ex;
    uint32_t mask;
    atomicAdd(&key_cnt[pair_info(q, &ex, &mask)], 1);
  }
  __syncthreads();
  if (w == 0) {
    // exclusive scan of the key counts: the first pair slot of each key
    const int kc = lane < W ? key_cnt[lane] : 0;
    int incl = kc;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int o = __shfl_up(incl, sh);
      if (lane >= sh) incl += o;
    }
    if (lane < W) key_cnt[lane] = incl - kc;
    if (lane == 0) *d.n_tiles = P * d.ntiles_n;
  }
  __syncthreads();
  // stable ranks: pairs in q order, a batch of blockDim.x pairs at a time
  for (int q0 = 0; q0 < P; q0 += blockDim.x) {
    const int q = q0 + tid;
    int ex = ex0;
    uint32_t mask = mask0;
    const int key = q0 == 0 ? key0 : (q < P ? pair_info(q, &ex, &mask) : -1);
    int local = 0;
    for (int u = 0; u < W; ++u) {
      const unsigned long long bal = __ballot(key == u);
      if (key == u) local = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_cnt[w][u] = __popcll(bal);
    }
    __syncthreads();
    if (key >= 0) {
      int rank = carry[key] + local;
      for (int u = 0; u < w; ++u) rank += wave_cnt[u][key];
      const int mt = q - s_pst[ex];
      const int m0 = s_off[ex] + mt * d.bm;
      const int rows = min(d.bm, s_cnt[ex] - mt * d.bm);
      const int out = (key_cnt[key] + rank) * d.ntiles_n;
      for (int nt = 0; nt < d.ntiles_n; ++nt) {
        tlc_tile tl;
        tl.m0 = m0;
        tl.n0 = nt * d.bn;
        tl.m_rows = rows;
        tl.n_cols = min(d.bn, d.N - nt * d.bn);
        tl.expert = ex;
        tl.chunk_mask = mask;
        tl.key = key;
        tl.split = 0;
        d.plan[out + nt] = tl;
      }
    }
    __syncthreads();
    if (tid < W) {
      int add = 0;
      for (int u = 0; u < PLAN_WAVES; ++u) add += wave_cnt[u][tid];
      carry[tid] += add;
    }
    __syncthreads();
  }
}

// One wavefront per (four blocks, group of 16 experts): lanes 16 s .. 16 s + 15
// hold the tokens of block 4 x + s.
constexpr int SCATTER_GROUP = 16;

__global__ __launch_bounds__(64) void scatter_kernel(MoeDev d, int nb) {
  const int lane = threadIdx.x, g0 = blockIdx.y * SCATTER_GROUP;
  const int seg = lane >> 4, i = lane & 15;
  const int b = blockIdx.x * 4 + seg;
  const int t = b < nb ? block_token(d, blocks_per_chunk(d), b, i) : -1;
  const bool valid = t >= 0;
  const unsigned long long m = valid ? d.member[t] : 0ull;
  // lane (seg, j) holds the first row of expert g0 + j for block b
  const int ej = g0 + i;
  const int base = (b < nb && ej < d.E) ? d.offsets[ej] + d.blk[static_cast<int64_t>(b) * d.E + ej] : 0;
  int sel[16], row[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    sel[q] = (valid && q < d.k) ? d.topk[static_cast<int64_t>(t) * d.k + q] : -1;
    row[q] = 0;
  }
  const unsigned long long before = ((1ull << lane) - 1ull) & (0xFFFFull << (16 * seg));
#pragma unroll
  for (int j = 0; j < SCATTER_GROUP; ++j) {
    const int e = g0 + j;
    const bool in = e < d.E && ((m >> e) & 1ull);
    const unsigned long long bal = __ballot(in);
    const int first = __shfl(base, 16 * seg + j);
    if (in) {
      const int r = first + __popcll(bal & before);
      d.row_token[r] = t;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (sel[q] == e) row[q] = r;
    }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (sel[q] >= g0 && sel[q] < g0 + SCATTER_GROUP) d.slot[static_cast<int64_t>(t) * d.k + q] = row[q];
}

}  // namespace

int64_t moe_max_pairs(int32_t T, int32_t topk, int32_t experts, int32_t bm) {
  return static_cast<int64_t>(T) * topk / bm + experts;
}

int64_t moe_max_blocks(int64_t T) { return (T + BLK - 1) / BLK + TLC_MAX_WORLD; }

tlc_status launch_moe_route(const MoeDev& d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = d.world * ((d.Tc + BLK - 1) / BLK);
  hipLaunchKernelGGL(route_kernel, dim3(nb + d.copy.wgs), dim3(64 * BLK), 0, s, d, nb);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64 * PLAN_WAVES), 0, s, d, nb);
  hipLaunchKernelGGL(scatter_kernel, dim3((nb + 3) / 4, (d.E + SCATTER_GROUP - 1) / SCATTER_GROUP), dim3(64),
                     0, s, d, nb);
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
