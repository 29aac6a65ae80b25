// Persistent, plan-driven bf16 GEMM for gfx950 (MFMA 32x32x16 bf16 -> fp32).
//
// A workgroup owns one work unit at a time -- an output tile, or one K range
// of a tile split along K -- and walks the unit list in plan order.  With the
// dynamic schedule it takes the next unit from a counter as soon as it is
// free; with the static one slot s takes units s, s + G, s + 2G, ... (G = grid
// size), the slots spread so that each XCD (8 per MI355X; workgroups are dealt
// to XCDs round-robin) gets a contiguous run of the plan.
//
// A unit of a split tile writes its fp32 partial to a workspace slot and counts
// itself in; the last unit of the tile adds the partials in ascending split
// index and stores the tile, so results do not depend on the schedule.
//
// Before touching a tile's A rows, the workgroup waits until every chunk the
// tile reads has landed (flag >= epoch), with a bounded spin that reports a
// timeout instead of hanging.  This is the tile-granular consumer wait of the
// pages (Triton-Distributed talk: consumer_tile_wait keyed by tile id, and the
// low-level signal wait with scope, memory semantics and expected value;
// AutoOverlap §5.2: only the tiles that consume a chunk wait for it).
//
// Tile cores:
//  * 256 x 256, 4 wavefronts (2 x 2), 128 x 128 per wavefront, one per SIMD,
//    accumulators in the accumulation registers (whole-matrix GEMMs).  Its
//    K loop for whole tiles fixes the place of every instruction: fragment
//    reads and loads are threaded one by one between the MFMAs, since no
//    second wavefront on the SIMD fills the gaps, and the loads that refill
//    a stage go one every two MFMAs from the barrier that frees it.
//  * 256 x 256, 8 wavefronts (2 x 4), 128 x 64 per wavefront, two per SIMD
//    so that one wave's MFMAs cover the other's LDS reads (grouped MoE GEMM,
//    whose ragged tiles it runs as fast as whole ones).
//  Both: operands go global -> LDS with buffer loads that write LDS directly
//  (no register staging), BK = 64, two stages of 64 KB.  A rows (and N x K
//  weight rows) are 64 bf16 = eight 16-byte chunks per LDS row, chunk c of
//  row r stored at c ^ ((r >> 1) & 7): the 16 lanes that one LDS cycle
//  serves read 16 different bank groups.  A K x N weight is kept K-major in
//  LDS (512-byte rows, chunk c of row k at c ^ 2(k & 15)) and transposed on
//  the way to the registers with ds_read_b64_tr_b16.
//  * 128 x 128 (small problems): 4 wavefronts, register-staged loads.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "colocated_copy.h"
#include "device_sync.h"
#include "tlc_internal.h"

namespace tlc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int THREADS = 256;

// 8 x 8 transpose of bf16 pairs: in[kk] holds 8 consecutive n at row k = kk;
// out[nn] receives 8 consecutive k at column n = nn.
__device__ inline void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) {
    const int w = nn >> 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = in[2 * j][w], hi = in[2 * j + 1][w];
      out[nn][j] = (nn & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
  }
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): loop
// bodies whose indices are compile-time constants, so that register arrays
// indexed by them stay in registers.
template <int N, int I = 0, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// K steps [kt0, kt1) of a unit (all KT steps for a whole tile).
__device__ inline void unit_k_range(uint32_t split, int KT, int* kt0, int* kt1) {
  const int S = static_cast<int>(split & 0xFFu);
  if (S < 2) {
    *kt0 = 0;
    *kt1 = KT;
    return;
  }
  const int s = static_cast<int>((split >> 8) & 0xFFu);
  *kt0 = s * KT / S;
  *kt1 = (s + 1) * KT / S;
}

// Split-tile epilogue, first half.  Returns true when the caller is to store
// the tile: always for a whole tile; for a split tile only in the workgroup
// that counted itself in last, which then stores the sum of the S partials
// (split_sum_store).  Partial slots hold each thread's accumulators at index
// (element * NT + thread), so every store and load instruction of a
// wavefront covers 256 consecutive bytes.
//
// The units of one tile may run on different XCDs, whose L2 caches are not
// coherent with each other.  Partials are therefore written and read with
// device-scope atomic stores and loads, which the hardware keeps coherent
// across XCDs without a full L2 write-back, and each wave waits for its stores
// to complete before the workgroup counts itself in.
template <int NT, int FM, int FN>
__device__ inline bool split_epilogue(const GemmParams& p, const tlc_tile& tl,
                                      f32x16 (&acc)[FM][FN], int* s_flag) {
  const uint32_t S = tl.split & 0xFFu;
  if (S < 2) return true;
  const uint32_t s = (tl.split >> 8) & 0xFFu, f = tl.split >> 16;
  // an opaque copy of the thread index: keeps the compiler from computing the
  // partial-slot addresses before the K loop and holding them across it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  constexpr int PER = FM * FN * 16;  // floats per thread = tile floats / NT
  char* block = p.split_ws + static_cast<int64_t>(f) * (256 + static_cast<int64_t>(S) * NT * PER * 4);
  uint32_t* counter = reinterpret_cast<uint32_t*>(block);
  float* slots = reinterpret_cast<float*>(block + 256);
  float* mine = slots + static_cast<int64_t>(s) * NT * PER + tid;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        __hip_atomic_store(mine + ((i * FN + j) * 16 + e) * NT, acc[i][j][e], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial has landed
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == S - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// One piece of a tile of the stream-K tail: K steps [kt0, kt1) of the tile,
// piece `self` in K order of `count` (count = 0: a unit of the plan, its K
// range given by its split field).  `block`: the tile's workspace block, its
// arrival counter at the start and piece u's partial at 256 + u * 256 KB.
struct SkPiece {
  int kt0, kt1;
  int count, self;
  char* block;
};

typedef float f32x4_st __attribute__((ext_vector_type(4)));

// Tail epilogue of the whole-tile core (256 threads, 4 x 4 blocks of 32 x 32
// per thread).  Every piece writes its fp32 partial (16-byte device-coherent
// stores, written through past this XCD's L2: the pieces of a tile may run on
// different XCDs), waits for the stores and counts itself in.  The piece that
// counts itself in last rewinds the counter and returns true: it stores the
// tile, adding the other pieces to its own while it stages them (SkAddPieces).
__device__ inline bool sk_epilogue(const SkPiece& pc, f32x16 (&acc)[4][4], int* s_flag) {
  // an opaque copy of the thread index: keeps the compiler from forming the
  // addresses before the K loop and holding them across it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const uint32_t voff = static_cast<uint32_t>(tid) * 16u;
  // vector V (0..63) of the thread: block (V / 16, V / 4 % 4), elements 4 (V % 4) ..
  {
    const __amdgpu_buffer_rsrc_t rs =
        copy_rsrc(pc.block + 256 + pc.self * kSkTileBytes, static_cast<uint32_t>(kSkTileBytes));
    static_for<64>([&](auto v_c) __attribute__((always_inline)) {
      constexpr int V = decltype(v_c)::value, I = V / 16, J = (V / 4) % 4, Q = V % 4;
      const f32x4_st x = {acc[I][J][4 * Q], acc[I][J][4 * Q + 1], acc[I][J][4 * Q + 2],
                          acc[I][J][4 * Q + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(copy_vec, x), rs, voff + V * 4096u,
                                             0, CPOL_SC1);
    });
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial (and loads) are in
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* counter = reinterpret_cast<uint32_t*>(pc.block);
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == static_cast<uint32_t>(pc.count) - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// One element of C.  Scatter mode with sends: a device-coherent store (written
// through past this XCD's L2), so that the slice is complete in memory when
// the notification below is raised and a copy on another engine or XCD reads
// it whole.
template <int KIND>
__device__ inline void store_c(float* dst, float v) {
  if constexpr (KIND == KIND_RS_NOTIFY)
    __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *dst = v;
}

// Split-tile epilogue, second half, in the workgroup that counted itself in
// last: each 32 x 32 block of the tile is the sum of the S partials in
// ascending split index (its own partial read back like the others, so the
// sum does not depend on which unit came last), stored through the
// accumulators' element map (element e of block (i, j): row i*32 + 8*(e/4) +
// 4*(lane/32) + e%4, column j*32 + lane%32 of the wavefront's sub-tile) and
// masked at the tile's edges.  Two blocks are summed per batch of independent
// loads, so that each batch costs one round trip; the sums live in vector
// registers and the accumulators are not written, which keeps them in the
// accumulation registers.
template <int KIND, int NT, int WM, int WN, int FM, int FN>
__device__ inline void split_sum_store(const GemmParams& p, const tlc_tile& tl, int wm, int wn,
                                       int lane) {
  static_assert((FM * FN) % 2 == 0, "blocks are summed in pairs");
  const uint32_t S = tl.split & 0xFFu, f = tl.split >> 16;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  constexpr int PER = FM * FN * 16;
  const float* all = reinterpret_cast<const float*>(
      p.split_ws + static_cast<int64_t>(f) * (256 + static_cast<int64_t>(S) * NT * PER * 4) + 256) + tid;
  float* cbase = p.c + static_cast<int64_t>(tl.m0) * p.ldc + tl.n0;
  for (int b = 0; b < FM * FN; b += 2) {
    const float* p0 = all + static_cast<int64_t>(b) * 16 * NT;
    float x0[16], x1[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x0[e] = __hip_atomic_load(p0 + e * NT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      x1[e] = __hip_atomic_load(p0 + (16 + e) * NT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (uint32_t u = 1; u < S; ++u) {
      const float* pu = p0 + static_cast<int64_t>(u) * NT * PER;
      float t0[16], t1[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        t0[e] = __hip_atomic_load(pu + e * NT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t1[e] = __hip_atomic_load(pu + (16 + e) * NT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x0[e] += t0[e];
        x1[e] += t1[e];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = (b + h) / FN, j = (b + h) % FN;
      const int col = wn * WN + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * WM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row < tl.m_rows && col < tl.n_cols)
          store_c<KIND>(cbase + static_cast<int64_t>(row) * p.ldc + col, h ? x1[e] : x0[e]);
      }
    }
  }
}

// Per-destination notification after a tile is stored (scatter mode with
// sends): once every wave's stores have completed, one thread adds the
// tile's element count in each destination slice it wrote; the addition that
// completes a slice (R * N elements) rewinds the count and raises the slice's
// ready flag with a release store.
template <int KIND>
__device__ inline void notify_dests(const GemmParams& p, const tlc_tile& tl) {
  if constexpr (KIND != KIND_RS_NOTIFY) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint32_t m = tl.chunk_mask & p.notify_mask;
  const int64_t R = p.rows_per_chunk;
  while (m) {
    const int c = __builtin_ctz(m);
    m &= m - 1;
    const int64_t lo = tl.m0 > c * R ? tl.m0 : c * R;
    const int64_t hi = tl.m0 + tl.m_rows < (c + 1) * R ? tl.m0 + tl.m_rows : (c + 1) * R;
    if (hi <= lo) continue;
    const uint32_t add = static_cast<uint32_t>((hi - lo) * tl.n_cols);
    const uint32_t prev =
        __hip_atomic_fetch_add(&p.sig->dest_done[c], add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + add == p.dest_total) {
      __hip_atomic_store(&p.sig->dest_done[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.sig->dest_ready[c], p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// Epilogue of the 256 x 256 cores: the wave's fp32 accumulators to C, edge
// tiles masked.  Element e of block (i, j) belongs to row i*32 + 8*(e/4) +
// 4*(lane/32) + e%4 and column j*32 + lane%32 of the wave's sub-tile.  The
// row offset is advanced row by row in one register (opaque to the compiler,
// so that it does not form all 4*FM row offsets ahead and keep them), and
// the column block is the store's immediate offset.
template <int KIND, int WM, int WN, int FM, int FN>
__device__ inline void store_tile(const GemmParams& p, const tlc_tile& tl, f32x16 (&acc)[FM][FN],
                                  int wm, int wn, int lane) {
  const int ldc = static_cast<int>(p.ldc);
  float* cbase = p.c + static_cast<int64_t>(tl.m0) * p.ldc + tl.n0;
  const bool full = tl.m_rows == 256 && tl.n_cols == 256;
  const int lrow = wm * WM + 4 * (lane >> 5), lcol = wn * WN + (lane & 31);
  int off = lrow * ldc + lcol;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = i * 32 + 8 * (e >> 2) + (e & 3);
      asm volatile("" : "+v"(off));
      float* row = cbase + off;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (full || (lrow + rr < tl.m_rows && lcol + j * 32 < tl.n_cols))
          store_c<KIND>(row + j * 32, acc[i][j][e]);
      off += ((e & 3) == 3 ? 5 : 1) * ldc;
    }
}

template <int BM, int BN, int B_NK, int KIND>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;  // per-wave sub-tile
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_PT = BM * (BK / 8) / THREADS;   // 16-byte loads per thread, A
  static constexpr int B_ROWS_PT = BN * (BK / 8) / THREADS;  // N x K weight
  static constexpr int B_BLOCKS = (BK / 8) * (BN / 8);       // K x N weight: 8x8 blocks
  static constexpr int LDS_A = BM * 8, LDS_B = BN * 8;       // 16-byte units per stage
  static_assert(A_PT >= 1 && B_ROWS_PT >= 1, "tile too small");
  static_assert(B_BLOCKS <= THREADS, "one 8x8 block per thread at most");

  __device__ static void run(const GemmParams& p, const tlc_tile& tl, u32x4* lds, int* s_flag) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    u32x4* As = lds;
    u32x4* Bs = lds + 2 * LDS_A;

    // ---- per-thread source offsets (elements, 32-bit; rows clamped into the
    // tile so edge tiles never read outside the operands) ----
    const uint16_t* abase = KIND == KIND_MOE ? p.a : p.a + static_cast<int64_t>(tl.m0) * p.lda;
    int32_t a_off[A_PT];
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int id = i * THREADS + tid;
      int row = id >> 3;
      row = row < tl.m_rows ? row : tl.m_rows - 1;
      const int32_t src_row = KIND == KIND_MOE ? p.row_token[tl.m0 + row] : row;
      a_off[i] = src_row * static_cast<int32_t>(p.lda) + (id & 7) * 8;
    }
    const uint16_t* bbase = p.b + (KIND == KIND_MOE ? tl.expert * p.b_expert_stride : 0);
    int32_t b_off[B_NK ? B_ROWS_PT : 1];
    int b_kb = 0, b_nb = 0;
    bool b_active = true;
    if (B_NK) {
      bbase += static_cast<int64_t>(tl.n0) * p.ldb;
#pragma unroll
      for (int i = 0; i < B_ROWS_PT; ++i) {
        const int id = i * THREADS + tid;
        int row = id >> 3;
        row = row < tl.n_cols ? row : tl.n_cols - 1;
        b_off[i] = row * static_cast<int32_t>(p.ldb) + (id & 7) * 8;
      }
    } else {
      b_active = tid < B_BLOCKS;
      b_kb = tid & 7;          // which 8 k-rows
      b_nb = tid >> 3;         // which 8 columns
      int ncol = b_nb * 8;
      ncol = ncol < tl.n_cols ? ncol : tl.n_cols - 8;
      bbase += tl.n0;
      b_off[0] = b_kb * 8 * static_cast<int32_t>(p.ldb) + ncol;
    }

    u32x4 ra[A_PT];
    u32x4 rb[8];

    auto gload = [&](int kt) {
      const uint16_t* ak = abase + kt * BK;
#pragma unroll
      for (int i = 0; i < A_PT; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ak + a_off[i]);
      if (B_NK) {
        const uint16_t* bk = bbase + kt * BK;
#pragma unroll
        for (int i = 0; i < B_ROWS_PT; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bk + b_off[i]);
      } else if (b_active) {
        const uint16_t* bk = bbase + static_cast<int64_t>(kt) * BK * p.ldb + b_off[0];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          rb[kk] = *reinterpret_cast<const u32x4*>(bk + kk * p.ldb);
      }
    };
    auto swrite = [&](int buf) {
      u32x4* as = As + buf * LDS_A;
      u32x4* bs = Bs + buf * LDS_B;
#pragma unroll
      for (int i = 0; i < A_PT; ++i) {
        const int id = i * THREADS + tid;
        const int row = id >> 3, kc = id & 7;
        as[row * 8 + (kc ^ (row & 7))] = ra[i];
      }
      if (B_NK) {
#pragma unroll
        for (int i = 0; i < B_ROWS_PT; ++i) {
          const int id = i * THREADS + tid;
          const int row = id >> 3, kc = id & 7;
          bs[row * 8 + (kc ^ (row & 7))] = rb[i];
        }
      } else if (b_active) {
        u32x4 t[8];
        transpose8x8(rb, t);
#pragma unroll
        for (int nn = 0; nn < 8; ++nn) {
          const int n = b_nb * 8 + nn;
          bs[n * 8 + (b_kb ^ (n & 7))] = t[nn];
        }
      }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    int kt0, kt1;
    unit_k_range(tl.split, p.K / BK, &kt0, &kt1);
    if (kt0 < kt1) {
      gload(kt0);
      swrite(0);
    }
    __syncthreads();
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      if (kt + 1 < kt1) gload(kt + 1);
      const u32x4* as = As + cur * LDS_A;
      const u32x4* bs = Bs + cur * LDS_B;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int kc = ks * 2 + (lane >> 5);
        const int sw = kc ^ (lane & 7);
        bf16x8 af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * WM + i * 32 + (lane & 31);
          u32x4 v = as[row * 8 + sw];
          af[i] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = wn * WN + j * 32 + (lane & 31);
          u32x4 v = bs[col * 8 + sw];
          bfr[j] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < kt1) swrite(cur ^ 1);
      __syncthreads();
    }
    if (!split_epilogue<THREADS>(p, tl, acc, s_flag)) return;
    if ((tl.split & 0xFFu) >= 2) {
      split_sum_store<KIND, THREADS, WM, WN, FM, FN>(p, tl, wm, wn, lane);
      notify_dests<KIND>(p, tl);
      return;
    }

    // ---- epilogue: fp32 tile to C, masked at the tile's edges ----
    float* cbase = p.c + static_cast<int64_t>(tl.m0) * p.ldc + tl.n0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = wn * WN + j * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * WM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (row < tl.m_rows && col < tl.n_cols)
            store_c<KIND>(cbase + static_cast<int64_t>(row) * p.ldc + col, acc[i][j][e]);
        }
      }
    notify_dests<KIND>(p, tl);
  }
};

// ---------------------------------------------------------------------------
// 256 x 256 core, 8 wavefronts, direct-to-LDS operand loads.
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define TLC_LDS __attribute__((address_space(3)))

// Buffer descriptor as four wave-uniform words (base, 0 stride, byte size,
// format flags) for the LDS-writing loads below.
typedef unsigned int rsrc_words __attribute__((ext_vector_type(4)));

// Epilogue of the whole-tile kernel: the wavefront's 128 x 128 fp32 sub-tile
// to C through LDS, so that each store instruction writes 16 bytes per lane
// and two 512-byte row pieces.  All CUs store their tiles at once at the end
// of a round; stores of long row pieces drain faster than stores in the
// accumulator layout, whose instructions write 128-byte pieces of two rows
// (a store-only probe of the same 208 tiles: 9.4 against 11.7 us).
//   Half the sub-tile (64 rows) at a time goes into the wavefront's own 32 KB
// of the stage buffers, which the K loop no longer uses: written in the
// accumulator layout (element e of block (i, j) is row i*32 + 8*(e/4) +
// 4*(lane/32) + e%4, column j*32 + lane%32), read back a row piece per half
// wavefront.  Its 16-byte column groups are XORed with bit 2 of the row times
// 8, so that the two halves of a wavefront, four rows apart, write different
// banks.  The caller makes the stages idle first (every wavefront's loads in,
// a workgroup barrier) and keeps the next unit's loads out until every
// wavefront has read its staging area back (a barrier after).  In scatter
// mode with sends the stores are device-coherent (write-through) 16-byte
// buffer stores.
__device__ inline int stage_index(int r, int c) {
  return r * 128 + ((((c >> 2) ^ (((r >> 2) & 1) << 3))) << 2) + (c & 3);
}

template <int KIND, typename Adjust>
__device__ inline void store_tile_rows(const GemmParams& p, const tlc_tile& tl, f32x16 (&acc)[4][4],
                                       Adjust adjust, int wm, int wn, int lane, TLC_LDS float* st) {
  const int64_t ldc = p.ldc;
  float* cbase = p.c + static_cast<int64_t>(tl.m0 + wm * 128) * ldc + tl.n0 + wn * 128;
  const int rows_left = tl.m_rows - wm * 128, cols_left = tl.n_cols - wn * 128;

  static_for<2>([&](auto h_c) __attribute__((always_inline)) {
    constexpr int h = decltype(h_c)::value;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int e = 0; e < 16; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st[stage_index(ii * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), j * 32 + (lane & 31))] =
              acc[2 * h + ii][j][e];
    // a stream-K tail tile adds the other pieces to the staged half here
    adjust(h_c, st);
#pragma unroll
    for (int rr = 0; rr < 32; ++rr) {
      const int r = 2 * rr + (lane >> 5), c = (lane & 31) * 4;
      const f32x4_st v = *reinterpret_cast<const TLC_LDS f32x4_st*>(st + stage_index(r, c));
      if constexpr (KIND == KIND_RS_NOTIFY) {
        // scatter mode with sends: device-coherent stores (written through past
        // this XCD's L2), through a buffer resource over the instruction's two rows
        const __amdgpu_buffer_rsrc_t rc =
            copy_rsrc(cbase + static_cast<int64_t>(h * 64 + 2 * rr) * ldc, static_cast<uint32_t>(2 * ldc * 4));
        if (h * 64 + r < rows_left && c < cols_left)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(copy_vec, v), rc,
                                                 static_cast<int>(((lane >> 5) * ldc + c) * 4), 0, CPOL_SC1);
      } else if (h * 64 + r < rows_left && c < cols_left) {
        *reinterpret_cast<f32x4_st*>(cbase + static_cast<int64_t>(h * 64 + r) * ldc + c) = v;
      }
    }
  });
}

// store_tile_rows as it is: a whole tile.
struct NoAdjust {
  template <int H>
  __device__ void operator()(std::integral_constant<int, H>, TLC_LDS float*) const {}
};

// Half H (row blocks 2H and 2H + 1) of a tail tile for store_tile_rows,
// staged in LDS with this piece's own partial: replaced by the pieces summed
// in K order, ((x0 + x1) + x2) + ..., whichever piece completed the tile.  So
// the result depends on the grid (where the pieces start) but not on which
// workgroup finishes when.  The pieces before this one are summed in
// registers and added to the staged value (t + own == own + t); the later
// ones are added to the staged value one by one.  Element k of vector
// w = 4 j + q of row block i is element e = 4 q + k of block (i, j).
struct SkAddPieces {
  const GemmParams& p;
  const SkPiece& pc;
  int lane;
  template <int H>
  __device__ void operator()(std::integral_constant<int, H>, TLC_LDS float* st) const {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const uint32_t voff = static_cast<uint32_t>(tid) * 16u;
    // eight vectors (half a row block) at a time
    auto load = [&](int u, int v0, f32x4_st (&x)[8]) __attribute__((always_inline)) {
      const __amdgpu_buffer_rsrc_t rs =
          copy_rsrc(pc.block + 256 + u * kSkTileBytes, static_cast<uint32_t>(kSkTileBytes));
#pragma unroll
      for (int w = 0; w < 8; ++w)
        x[w] = __builtin_bit_cast(
            f32x4_st, __builtin_amdgcn_raw_buffer_load_b128(
                          rs, voff + static_cast<uint32_t>(v0 + w) * 4096u, 0, CPOL_SC1));
    };
    auto add_staged = [&](int ii, int w0, const f32x4_st (&x)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int w = 0; w < 8; ++w)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int ww = w0 + w;
          const int idx = stage_index(ii * 32 + 8 * (ww % 4) + 4 * (lane >> 5) + k, (ww / 4) * 32 + (lane & 31));
          st[idx] = x[w][k] + st[idx];
        }
    };
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
      for (int w0 = 0; w0 < 16; w0 += 8) {
        const int v0 = (2 * H + ii) * 16 + w0;
        if (pc.self > 0) {
          f32x4_st t[8];
          load(0, v0, t);
          for (int u = 1; u < pc.self; ++u) {
            f32x4_st x[8];
            load(u, v0, x);
#pragma unroll
            for (int w = 0; w < 8; ++w) t[w] += x[w];
          }
          add_staged(ii, w0, t);
        }
        for (int u = pc.self + 1; u < pc.count; ++u) {
          f32x4_st x[8];
          load(u, v0, x);
          add_staged(ii, w0, x);
        }
      }
    }
  }
};

__device__ inline rsrc_words rsrc_raw(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  rsrc_words d;
  d.x = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  d.y = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)) & 0xFFFFu;
  d.z = __builtin_amdgcn_readfirstlane(bytes);
  d.w = 0x00020000u;
  return d;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Every scalar operand goes through readfirstlane: under register pressure the
// compiler may hold a uniform value in a vector register, and the instruction
// takes scalar registers only (and no literal offset).
__device__ inline void load_lds16_m0(rsrc_words r, uint32_t m0, uint32_t voff, uint32_t soff) {
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t ms = __builtin_amdgcn_readfirstlane(m0);
  rsrc_words rs;
  rs.x = __builtin_amdgcn_readfirstlane(r.x);
  rs.y = __builtin_amdgcn_readfirstlane(r.y);
  rs.z = __builtin_amdgcn_readfirstlane(r.z);
  rs.w = __builtin_amdgcn_readfirstlane(r.w);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(ms), "v"(voff), "s"(rs), "s"(so) : "memory", "m0");
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (the LDS base goes in M0).  Written as an instruction rather than the
// compiler builtin: the compiler cannot tell which LDS stage such a load
// writes, and would otherwise wait for every outstanding one before each LDS
// read of the other stage.  Completion is awaited explicitly (vmcnt) before
// the workgroup barrier that precedes any read of the stage.
__device__ inline void load_lds16(rsrc_words r, const TLC_LDS void* lds, uint32_t voff,
                                  uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  load_lds16_m0(r, m0, voff, soff);
}

template <int B_NK, int KIND>
struct Tile8w {
  static constexpr int BM = 256, BN = 256, WM = 128, WN = 64, FM = 4, FN = 2, NT = 512;
  __device__ static int swz(int row) { return (row >> 1) & 7; }

  __device__ static void run(const GemmParams& p, const tlc_tile& tl, TLC_LDS u32x4* A0,
                             TLC_LDS u32x4* A1, TLC_LDS u32x4* B0, TLC_LDS u32x4* B1,
                             int* s_flag) {
    // the thread index is made opaque per tile, so that the lane-dependent
    // offsets below are formed per tile instead of being kept (and spilled)
    // across the whole persistent loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const uint32_t lda2 = static_cast<uint32_t>(p.lda) * 2, ldb2 = static_cast<uint32_t>(p.ldb) * 2;

    // ---- global sources of the 4 A blocks and 4 B blocks (1 KB each) this
    // wave fills per stage; rows outside the tile are clamped into it ----
    rsrc_words ra;
    uint32_t a_off[4];
    if (KIND == KIND_MOE) {
      ra = rsrc_raw(p.a, static_cast<uint32_t>(p.a_rows) * lda2);
    } else {
      ra = rsrc_raw(p.a + static_cast<int64_t>(tl.m0) * p.lda, static_cast<uint32_t>(tl.m_rows) * lda2);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int row = (wave * 4 + q) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(row);
      row = row < tl.m_rows ? row : tl.m_rows - 1;
      const uint32_t src_row = KIND == KIND_MOE ? static_cast<uint32_t>(p.row_token[tl.m0 + row])
                                                 : static_cast<uint32_t>(row);
      a_off[q] = src_row * lda2 + kc * 16;
    }
    const uint16_t* bexp = p.b + (KIND == KIND_MOE ? tl.expert * p.b_expert_stride : 0);
    rsrc_words rb;
    uint32_t b_off[4];
    if constexpr (B_NK) {
      rb = rsrc_raw(bexp + static_cast<int64_t>(tl.n0) * p.ldb, static_cast<uint32_t>(tl.n_cols) * ldb2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int row = (wave * 4 + q) * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ swz(row);
        row = row < tl.n_cols ? row : tl.n_cols - 1;
        b_off[q] = row * ldb2 + kc * 16;
      }
    } else {
      rb = rsrc_raw(bexp + tl.n0, static_cast<uint32_t>(p.K) * ldb2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = (wave * 4 + q) * 2 + (lane >> 5);
        int n = ((lane & 31) ^ (2 * (k & 15))) * 8;
        n = n < tl.n_cols ? n : tl.n_cols - 8;
        b_off[q] = k * ldb2 + n * 2;
      }
    }
    const uint32_t b_step = B_NK ? 128u : 64u * ldb2;
    auto issue = [&](int kt, TLC_LDS u32x4* As, TLC_LDS u32x4* Bs) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        load_lds16(ra, (const TLC_LDS void*)(As + (wave * 4 + q) * 64), a_off[q], kt * 128u);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        load_lds16(rb, (const TLC_LDS void*)(Bs + (wave * 4 + q) * 64), b_off[q], kt * b_step);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
    const int h = lane >> 5;
    const int s_lane = swz(lane & 31);
    bf16x8 fa[2][FM], fb[2][FN];
    // Rows of the unit this wave computes: 32-row blocks i < fm_act hold rows
    // below m_rows.  In a tile with fewer rows (the ragged last m-tile of an
    // expert, or of M) a wave skips the fragment reads and MFMAs of its empty
    // blocks -- a wave with no rows only loads and meets the barriers -- in a
    // second copy of the K loop, so the loop of a full tile is unchanged.  The
    // stored rows' results do not change.
    int kt0, kt1;
    unit_k_range(tl.split, p.K / 64, &kt0, &kt1);
    const int nk = kt1 - kt0;
    const int rows_left = tl.m_rows - __builtin_amdgcn_readfirstlane(wm) * WM;
    const int fm_act = rows_left <= 0 ? 0 : (rows_left >= FM * 32 ? FM : (rows_left + 31) >> 5);
    // One BK = 64 step on stage (Ac, Bc), whose first fragments are already in
    // registers: the fragments of sub-step ks+1 are requested before the MFMAs
    // of sub-step ks (the scheduling barriers keep that order).  Before the
    // last sub-step's MFMAs -- their fragments are in registers -- the wave
    // waits for its LDS reads and its loads of the next stage, and the
    // workgroup barrier makes the next stage whole and this one free; under
    // those MFMAs go the next stage's first fragment reads and the loads of
    // the step after next into this stage.
    auto kloop = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      auto fread = [&](const TLC_LDS u32x4* As, const TLC_LDS u32x4* Bs, int ks, int slot) {
        const int phys = (ks * 2 + h) ^ s_lane;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (!FULL && i >= fm_act) continue;
          fa[slot][i] = __builtin_bit_cast(
              bf16x8, *(const TLC_LDS u32x4*)((const TLC_LDS char*)As +
                                              (wm * WM + i * 32 + (lane & 31)) * 128 + phys * 16));
        }
        if (!FULL && fm_act == 0) return;
        if constexpr (B_NK) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            fb[slot][j] = __builtin_bit_cast(
                bf16x8, *(const TLC_LDS u32x4*)((const TLC_LDS char*)Bs +
                                                (wn * WN + j * 32 + (lane & 31)) * 128 + phys * 16));
        } else {
          // Lane l needs B[k = 16 ks + 8 (l / 32) + t][n] for t = 0..7 (n = l % 32 of the block):
          // two transposing reads, each giving 4 consecutive k of one column.
          const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            v4i16 hv[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int k = ks * 16 + 8 * (g >> 1) + 4 * hh + (i16 >> 2);
              const int n = wn * WN + j * 32 + 16 * (g & 1) + 4 * (i16 & 3);
              const int pc = (n >> 3) ^ (2 * (k & 15));
              hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (TLC_LDS v4i16*)((const TLC_LDS char*)Bs + k * 512 + pc * 16 + (n & 7) * 2));
            }
            const v8i16 v = {hv[0][0], hv[0][1], hv[0][2], hv[0][3], hv[1][0], hv[1][1], hv[1][2], hv[1][3]};
            fb[slot][j] = __builtin_bit_cast(bf16x8, v);
          }
        }
      };
      auto mfmas = [&](int sl) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (!FULL && i >= fm_act) continue;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][i], fb[sl][j], acc[i][j], 0, 0, 0);
        }
      };
      auto step = [&](int i, const TLC_LDS u32x4* Ac, const TLC_LDS u32x4* Bc, TLC_LDS u32x4* Aw,
                      TLC_LDS u32x4* Bw, const TLC_LDS u32x4* An, const TLC_LDS u32x4* Bn) {
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
          fread(Ac, Bc, ks + 1, (ks + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
          mfmas(ks & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < nk) fread(An, Bn, 0, 0);
        if (i + 2 < nk) issue(kt0 + i + 2, Aw, Bw);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1);
        __builtin_amdgcn_sched_barrier(0);
      };
      if (nk > 0) {
        issue(kt0, A0, B0);
        if (nk > 1) {
          issue(kt0 + 1, A1, B1);
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // stage 0's eight loads done
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        fread(A0, B0, 0, 0);
        for (int i = 0; i < nk; i += 2) {
          step(i, A0, B0, A0, B0, A1, B1);
          if (i + 1 < nk) step(i + 1, A1, B1, A1, B1, A0, B0);
        }
      } else {
        __syncthreads();
      }
    };
    if (fm_act == FM)
      kloop(std::true_type{});
    else
      kloop(std::false_type{});
    if (!split_epilogue<NT>(p, tl, acc, s_flag)) return;

    if ((tl.split & 0xFFu) >= 2)
      split_sum_store<KIND, NT, WM, WN, FM, FN>(p, tl, wm, wn, lane);
    else
      store_tile<KIND, WM, WN, FM, FN>(p, tl, acc, wm, wn, lane);
    notify_dests<KIND>(p, tl);
  }
};

// ---------------------------------------------------------------------------
// 256 x 256 core, 4 wavefronts (2 x 2), 128 x 128 per wavefront: one
// wavefront per SIMD with its 256 accumulators in the accumulation registers.
// Against the 8-wavefront core it reads a third fewer LDS bytes per MFMA
// (each fragment read feeds four MFMAs instead of two or four) and leaves
// part of every SIMD's register file free, so that a copy kernel on another
// stream can run beside it on the same compute unit.  Same LDS layout, same
// loads, same K-step pipeline.
// ---------------------------------------------------------------------------
template <int B_NK, int KIND, int FAST, int SK>
struct Tile4w {
  static constexpr int BM = 256, BN = 256, WM = 128, WN = 128, FM = 4, FN = 4, NT = 256;
  __device__ static int swz(int row) { return (row >> 1) & 7; }
  // one load of the next stage every LSTRIDE MFMAs (see the fast loop)
  static constexpr int LSTRIDE = 2;

  __device__ static void run(const GemmParams& p, const tlc_tile& tl, const SkPiece& pc,
                             TLC_LDS u32x4* A0, TLC_LDS u32x4* A1, TLC_LDS u32x4* B0,
                             TLC_LDS u32x4* B1, int* s_flag) {
    // the thread index is made opaque per tile, so that the lane-dependent
    // offsets below are formed per tile instead of being kept (and spilled)
    // across the whole persistent loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t lda2 = static_cast<uint32_t>(p.lda) * 2, ldb2 = static_cast<uint32_t>(p.ldb) * 2;

    // ---- global sources of the 8 A blocks and 8 B blocks (1 KB each) this
    // wave fills per stage; rows outside the tile are clamped into it ----
    rsrc_words ra;
    uint32_t a_off[8];
    if (KIND == KIND_MOE) {
      ra = rsrc_raw(p.a, static_cast<uint32_t>(p.a_rows) * lda2);
    } else {
      ra = rsrc_raw(p.a + static_cast<int64_t>(tl.m0) * p.lda, static_cast<uint32_t>(tl.m_rows) * lda2);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      int row = (wave * 8 + q) * 8 + (lane >> 3);
      const int kc = (lane & 7) ^ swz(row);
      row = row < tl.m_rows ? row : tl.m_rows - 1;
      const uint32_t src_row = KIND == KIND_MOE ? static_cast<uint32_t>(p.row_token[tl.m0 + row])
                                                 : static_cast<uint32_t>(row);
      a_off[q] = src_row * lda2 + kc * 16;
    }
    const uint16_t* bexp = p.b + (KIND == KIND_MOE ? tl.expert * p.b_expert_stride : 0);
    rsrc_words rb;
    uint32_t b_off[8];
    if constexpr (B_NK) {
      rb = rsrc_raw(bexp + static_cast<int64_t>(tl.n0) * p.ldb, static_cast<uint32_t>(tl.n_cols) * ldb2);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        int row = (wave * 8 + q) * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ swz(row);
        row = row < tl.n_cols ? row : tl.n_cols - 1;
        b_off[q] = row * ldb2 + kc * 16;
      }
    } else {
      rb = rsrc_raw(bexp + tl.n0, static_cast<uint32_t>(p.K) * ldb2);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int k = (wave * 8 + q) * 2 + (lane >> 5);
        int n = ((lane & 31) ^ (2 * (k & 15))) * 8;
        n = n < tl.n_cols ? n : tl.n_cols - 8;
        b_off[q] = k * ldb2 + n * 2;
      }
    }
    const uint32_t b_step = B_NK ? 128u : 64u * ldb2;
    auto issue = [&](int kt, TLC_LDS u32x4* As, TLC_LDS u32x4* Bs) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        load_lds16(ra, (const TLC_LDS void*)(As + (wave * 8 + q) * 64), a_off[q], kt * 128u);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        load_lds16(rb, (const TLC_LDS void*)(Bs + (wave * 8 + q) * 64), b_off[q], kt * b_step);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
    const int h = lane >> 5;
    const int s_lane = swz(lane & 31);
    bf16x8 fa[2][FM], fb[2][FN];
    // Rows of the unit this wave computes: 32-row blocks i < fm_act hold rows
    // below m_rows.  In a tile with fewer rows (the ragged last m-tile of an
    // expert, or of M) a wave skips the fragment reads and MFMAs of its empty
    // blocks -- a wave with no rows only loads and meets the barriers -- in a
    // second copy of the K loop, so the loop of a full tile is unchanged.  The
    // stored rows' results do not change.
    // a piece of a stream-K tail tile runs its own K steps (the whole-tile
    // kernel only); a unit of the plan runs the range of its split field
    int kt0, kt1;
    if (SK && pc.count > 0) {
      kt0 = pc.kt0;
      kt1 = pc.kt1;
    } else {
      unit_k_range(tl.split, p.K / 64, &kt0, &kt1);
    }
    const int nk = kt1 - kt0;
    const int rows_left = tl.m_rows - __builtin_amdgcn_readfirstlane(wm) * WM;
    const int fm_act = rows_left <= 0 ? 0 : (rows_left >= FM * 32 ? FM : (rows_left + 31) >> 5);
    // One BK = 64 step on stage (Ac, Bc), whose first fragments are already in
    // registers: the fragments of sub-step ks+1 are requested before the MFMAs
    // of sub-step ks (the scheduling barriers keep that order).  Before the
    // last sub-step's MFMAs -- their fragments are in registers -- the wave
    // waits for its LDS reads and its loads of the next stage, and the
    // workgroup barrier makes the next stage whole and this one free; under
    // those MFMAs go the next stage's first fragment reads and the loads of
    // the step after next into this stage.
    auto kloop = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      auto fread = [&](const TLC_LDS u32x4* As, const TLC_LDS u32x4* Bs, int ks, int slot) {
        const int phys = (ks * 2 + h) ^ s_lane;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (!FULL && i >= fm_act) continue;
          fa[slot][i] = __builtin_bit_cast(
              bf16x8, *(const TLC_LDS u32x4*)((const TLC_LDS char*)As +
                                              (wm * WM + i * 32 + (lane & 31)) * 128 + phys * 16));
        }
        if (!FULL && fm_act == 0) return;
        if constexpr (B_NK) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            fb[slot][j] = __builtin_bit_cast(
                bf16x8, *(const TLC_LDS u32x4*)((const TLC_LDS char*)Bs +
                                                (wn * WN + j * 32 + (lane & 31)) * 128 + phys * 16));
        } else {
          // Lane l needs B[k = 16 ks + 8 (l / 32) + t][n] for t = 0..7 (n = l % 32 of the block):
          // two transposing reads, each giving 4 consecutive k of one column.
          const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            v4i16 hv[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int k = ks * 16 + 8 * (g >> 1) + 4 * hh + (i16 >> 2);
              const int n = wn * WN + j * 32 + 16 * (g & 1) + 4 * (i16 & 3);
              const int pc = (n >> 3) ^ (2 * (k & 15));
              hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (TLC_LDS v4i16*)((const TLC_LDS char*)Bs + k * 512 + pc * 16 + (n & 7) * 2));
            }
            const v8i16 v = {hv[0][0], hv[0][1], hv[0][2], hv[0][3], hv[1][0], hv[1][1], hv[1][2], hv[1][3]};
            fb[slot][j] = __builtin_bit_cast(bf16x8, v);
          }
        }
      };
      auto mfmas = [&](int sl) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (!FULL && i >= fm_act) continue;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sl][i], fb[sl][j], acc[i][j], 0, 0, 0);
        }
      };
      auto step = [&](int i, const TLC_LDS u32x4* Ac, const TLC_LDS u32x4* Bc, TLC_LDS u32x4* Aw,
                      TLC_LDS u32x4* Bw, const TLC_LDS u32x4* An, const TLC_LDS u32x4* Bn) {
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
          fread(Ac, Bc, ks + 1, (ks + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
          mfmas(ks & 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < nk) fread(An, Bn, 0, 0);
        if (i + 2 < nk) issue(kt0 + i + 2, Aw, Bw);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1);
        __builtin_amdgcn_sched_barrier(0);
      };
      if (nk > 0) {
        issue(kt0, A0, B0);
        if (nk > 1) {
          issue(kt0 + 1, A1, B1);
          asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // stage 0's sixteen loads done
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        fread(A0, B0, 0, 0);
        for (int i = 0; i < nk; i += 2) {
          step(i, A0, B0, A0, B0, A1, B1);
          if (i + 1 < nk) step(i + 1, A1, B1, A1, B1, A0, B0);
        }
      } else {
        __syncthreads();
      }
    };
    // Full tiles: the K loop with the place of every instruction fixed.  One
    // wavefront per SIMD has no second wavefront to fill its gaps, so the
    // other instructions are threaded between the MFMAs (each keeps the MFMA
    // pipe busy for 32 cycles): during sub-step ks the fragment reads of
    // sub-step ks+1 follow the first MFMAs one by one, in the order their
    // MFMAs need them.  Before the last sub-step the wave waits for its reads
    // and for its loads of the next stage and meets the barrier; the first
    // instruction after it is an MFMA, and the next stage's first fragment
    // reads are threaded through the last sub-step's MFMAs.
    //   The sixteen loads that refill a stage go one every LSTRIDE MFMAs from
    // the moment the stage is free (the barrier) on: the first 16 / LSTRIDE
    // under the last sub-step of the step that frees it, the rest under the
    // first sub-steps of the next step, which waits for all of them at its
    // own barrier.  A CU's loads then reach the texture path at an even rate
    // (64 per step from its four wavefronts) instead of in one burst behind
    // which each wavefront's MFMAs stall: the whole-tile step took 3450
    // cycles with the sixteen loads in the last sub-step, 2950 with them
    // spread over three (the MFMAs alone take 2048).  LSTRIDE 2 leaves the
    // last load about a thousand cycles before its wait.
    constexpr int NRB = B_NK ? FN : 2 * FN;  // B reads per sub-step
    constexpr int NR = FM + NRB;             // fragment reads per sub-step
    v4i16 fbh[2][FN][2];                     // K x N weight: fragment halves
    const uint32_t wave_s = __builtin_amdgcn_readfirstlane(wave);
    // read R of sub-step ks from stage (As, Bs) into slot SL; reads in the
    // order of first use: A block 0, the B fragments, then A blocks 1..3
    auto read_one = [&](const TLC_LDS u32x4* As, const TLC_LDS u32x4* Bs, int ks, auto sl_c,
                        auto r_c) __attribute__((always_inline)) {
      constexpr int SL = decltype(sl_c)::value, R = decltype(r_c)::value;
      constexpr int AI = R == 0 ? 0 : (R <= NRB ? -1 : R - NRB);
      constexpr int BJ = R == 0 || R > NRB ? -1 : (B_NK ? R - 1 : (R - 1) >> 1);
      constexpr int HH = B_NK ? 0 : (R - 1) & 1;
      const int phys = (ks * 2 + h) ^ s_lane;
      if constexpr (AI >= 0) {
        fa[SL][AI] = __builtin_bit_cast(
            bf16x8, *(const TLC_LDS u32x4*)((const TLC_LDS char*)As +
                                            (wm * WM + AI * 32 + (lane & 31)) * 128 + phys * 16));
      } else if constexpr (B_NK) {
        fb[SL][BJ] = __builtin_bit_cast(
            bf16x8, *(const TLC_LDS u32x4*)((const TLC_LDS char*)Bs +
                                            (wn * WN + BJ * 32 + (lane & 31)) * 128 + phys * 16));
      } else {
        const int g = lane >> 4, i16 = lane & 15;
        const int k = ks * 16 + 8 * (g >> 1) + 4 * HH + (i16 >> 2);
        const int n = wn * WN + BJ * 32 + 16 * (g & 1) + 4 * (i16 & 3);
        const int pc = (n >> 3) ^ (2 * (k & 15));
        fbh[SL][BJ][HH] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (TLC_LDS v4i16*)((const TLC_LDS char*)Bs + k * 512 + pc * 16 + (n & 7) * 2));
      }
    };
    // MFMA M of a sub-step on slot SL: row block M / FN, column block M % FN
    auto mfma_one = [&](auto sl_c, auto m_c) __attribute__((always_inline)) {
      constexpr int SL = decltype(sl_c)::value, M = decltype(m_c)::value;
      constexpr int I = M / FN, J = M % FN;
      bf16x8 bv;
      if constexpr (B_NK) {
        bv = fb[SL][J];
      } else {
        const v8i16 v = {fbh[SL][J][0][0], fbh[SL][J][0][1], fbh[SL][J][0][2], fbh[SL][J][0][3],
                         fbh[SL][J][1][0], fbh[SL][J][1][1], fbh[SL][J][1][2], fbh[SL][J][1][3]};
        bv = __builtin_bit_cast(bf16x8, v);
      }
      acc[I][J] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SL][I], bv, acc[I][J], 0, 0, 0);
    };
    // load Q of the sixteen that fill stage (As, Bs) with K step kt
    auto load_one = [&](int kt, TLC_LDS u32x4* As, TLC_LDS u32x4* Bs, auto q_c)
        __attribute__((always_inline)) {
      constexpr int Q = decltype(q_c)::value;
      if constexpr (Q < 8)
        load_lds16_m0(ra, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(As)) + (wave_s * 8 + Q) * 1024,
                      a_off[Q], kt * 128u);
      else
        load_lds16_m0(rb, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(Bs)) + (wave_s * 8 + Q - 8) * 1024,
                      b_off[Q - 8], kt * b_step);
    };
    // one K step on stage (Ac, Bc): finishes the loads of the next step into
    // (An, Bn), reads that stage's first fragments at its end, and starts the
    // loads of the step after next into this stage once it is free
    // C (compute): false for a wavefront whose 128 x 128 share of the unit
    // lies wholly outside its rows or columns (the empty half of a 128-wide
    // last column tile, or of an expert's unit of 128 rows or fewer): it
    // issues its share of the stage loads and meets the barriers, but makes
    // no fragment reads and no MFMAs, which saves their power on a part whose
    // clock the power limit sets.
    auto fstep = [&](int i, TLC_LDS u32x4* Ac, TLC_LDS u32x4* Bc, TLC_LDS u32x4* An,
                     TLC_LDS u32x4* Bn, auto c_c) __attribute__((always_inline)) {
      constexpr bool C = decltype(c_c)::value;
      static_for<3>([&](auto ks_c) __attribute__((always_inline)) {
        constexpr int KS = decltype(ks_c)::value;
        static_for<FM * FN>([&](auto m_c) __attribute__((always_inline)) {
          constexpr int M = decltype(m_c)::value;
          if constexpr (C) {
            mfma_one(std::integral_constant<int, KS & 1>{}, m_c);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (C && M < NR) {
            read_one(Ac, Bc, KS + 1, std::integral_constant<int, (KS + 1) & 1>{}, m_c);
            __builtin_amdgcn_sched_barrier(0);
          }
          constexpr int G = 16 + KS * 16 + M;
          if constexpr (G % LSTRIDE == 0 && G / LSTRIDE < 16) {
            load_one(kt0 + i + 1, An, Bn, std::integral_constant<int, G / LSTRIDE>{});
            __builtin_amdgcn_sched_barrier(0);
          }
        });
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      static_for<FM * FN>([&](auto m_c) __attribute__((always_inline)) {
        constexpr int M = decltype(m_c)::value;
        if constexpr (C) {
          mfma_one(std::integral_constant<int, 1>{}, m_c);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (C && M < NR) {
          read_one(An, Bn, 0, std::integral_constant<int, 0>{}, m_c);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (M % LSTRIDE == 0) {
          load_one(kt0 + i + 2, Ac, Bc, std::integral_constant<int, M / LSTRIDE>{});
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    };
    // Every step reads the next stage and loads the step after next, also the
    // last two: their loads fall past the unit's K range (the next row, or
    // zeros past the end of the operand, which a buffer load returns) into a
    // stage nobody reads any more, and they complete before the next unit's
    // loads, vector memory operations completing in order.  An even number of
    // steps keeps the loop body one pair of steps.
    auto fast_loop = [&](auto c_c) __attribute__((always_inline)) {
      constexpr bool C = decltype(c_c)::value;
      static_assert(FM * FN == 16, "sixteen MFMAs and sixteen loads per sub-step");
      static_for<16>([&](auto q_c) __attribute__((always_inline)) { load_one(kt0, A0, B0, q_c); });
      // step 1's loads that the steady state issues before the first step
      static_assert(LSTRIDE == 2, "the wait below counts 16 / LSTRIDE loads");
      static_for<16 / LSTRIDE>([&](auto q_c) __attribute__((always_inline)) {
        load_one(kt0 + 1, A1, B1, q_c);
      });
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // stage 0's sixteen loads done
      __syncthreads();
      if constexpr (C) {
        static_for<NR>([&](auto r_c) __attribute__((always_inline)) {
          read_one(A0, B0, 0, std::integral_constant<int, 0>{}, r_c);
        });
      }
      for (int i = 0; i < nk; i += 2) {
        fstep(i, A0, B0, A1, B1, c_c);
        fstep(i + 1, A1, B1, A0, B0, c_c);
      }
    };
    // a wavefront with nothing to compute in this unit (wave-uniform)
    const bool idle = __builtin_amdgcn_readfirstlane(
                          static_cast<int>(wm * WM >= tl.m_rows || wn * WN >= tl.n_cols)) != 0;
    auto fast_loop_any = [&]() __attribute__((always_inline)) {
      if (idle)
        fast_loop(std::false_type{});
      else
        fast_loop(std::true_type{});
    };
    // the same loop for every wavefront of the workgroup: the fast loop's
    // barriers and LDS layout differ from the other loop's.  The FAST kernel
    // has only the fast loop: the host picks it when every unit is a whole
    // tile with an even number of K steps and no unit is split.
    if constexpr (FAST) {
      fast_loop_any();
    } else {
      if (tl.m_rows >= BM && nk > 0 && (nk & 1) == 0)
        fast_loop_any();
      else if (fm_act == FM)
        kloop(std::true_type{});
      else
        kloop(std::false_type{});
    }
    if constexpr (!FAST) {
      if (!split_epilogue<NT>(p, tl, acc, s_flag)) return;
    } else {
      (void)s_flag;
    }

    if constexpr (FAST) {
      // a piece of a shared tile: its partial out, and the tile stored only by
      // the piece that completes it
      const bool shared = SK && pc.count > 1;
      if constexpr (SK) {
        if (shared && !sk_epilogue(pc, acc, s_flag)) return;
      }
      // every wavefront's loads (also those past the K range) are in and
      // every wavefront is done with the stages: they hold the staging areas
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      TLC_LDS u32x4* mine = wave == 0 ? A0 : (wave == 1 ? A1 : (wave == 2 ? B0 : B1));
      TLC_LDS float* st = reinterpret_cast<TLC_LDS float*>(mine);
      if constexpr (SK) {
        if (shared)
          store_tile_rows<KIND>(p, tl, acc, SkAddPieces{p, pc, lane}, wm, wn, lane, st);
        else
          store_tile_rows<KIND>(p, tl, acc, NoAdjust{}, wm, wn, lane, st);
      } else {
        store_tile_rows<KIND>(p, tl, acc, NoAdjust{}, wm, wn, lane, st);
      }
      __syncthreads();  // the next unit's loads refill the stages
    } else if ((tl.split & 0xFFu) >= 2) {
      split_sum_store<KIND, NT, WM, WN, FM, FN>(p, tl, wm, wn, lane);
    } else {
      store_tile<KIND, WM, WN, FM, FN>(p, tl, acc, wm, wn, lane);
    }
    notify_dests<KIND>(p, tl);
  }
};

// Walks the plan: takes units (dynamic counter or static slots), validates
// them, waits for their chunks, then `run_tile(unit)`.
struct LoopShared {
  int abort;
  int split_last;
  int64_t next[2];
};

template <int BM, int BN, int KIND, int WAIT, int SK, typename RunTile>
__device__ inline void tile_loop(const GemmParams& p, LoopShared* sh, RunTile run_tile) {
  const int G = gridDim.x;
  // co-located landing: the first copy.wgs workgroups copy every chunk's
  // share before their first unit; no wait precedes the copy, so the flags it
  // raises cannot depend on the units behind it
  if (WAIT && static_cast<int>(blockIdx.x) < p.copy.wgs) copy_in_landing_order(p.copy, p.sig, p.epoch);
  // MoE: the unit count the routing wrote on the device, bounded by the plan's
  // capacity (a count beyond it is reported and nothing is run)
  int64_t n_tiles = p.n_tiles;
  if (KIND == KIND_MOE) {
    const int64_t nd = *p.n_tiles_dev;
    if (nd < 0 || nd > p.n_tiles) {
      if (threadIdx.x == 0) report(p.sig, TLC_ERR_BAD_PLAN, nd);
      n_tiles = 0;
    } else {
      n_tiles = nd;
    }
  }
  // stream-K tail: the work items past sk_from are pieces of the last tiles
  const bool tail = SK && p.sk_split > 0;
  const int64_t n_work = tail ? p.sk_from + static_cast<int64_t>(p.sk_split) * p.sk_tiles : n_tiles;
  uint32_t seen = p.no_wait_mask;
  // A unit's checks and chunk wait; false: stop (a bad unit was reported, or
  // a wait was aborted).
  auto admit = [&](int64_t t, const tlc_tile& tl) -> bool {
    const uint32_t S = tl.split & 0xFFu;
    const bool bad_split =
        tl.split != 0 &&
        (S < 2 || ((tl.split >> 8) & 0xFFu) >= S ||
         static_cast<int64_t>((tl.split >> 16) + 1) * (256 + static_cast<int64_t>(S) * BM * BN * 4) >
             p.split_bytes);
    const bool bad = tl.m_rows < 1 || tl.n_cols < 1 || tl.m0 < 0 || tl.n0 < 0 ||
                     tl.m0 + tl.m_rows > p.M || tl.n0 + tl.n_cols > p.N || tl.m_rows > BM ||
                     tl.n_cols > BN || (tl.n_cols & 7) != 0 || (KIND == KIND_MOE && tl.expert < 0) ||
                     bad_split;
    if (bad) {
      if (threadIdx.x == 0) report(p.sig, TLC_ERR_BAD_PLAN, t);
      return false;
    }
    // trace stamps go to memory as they are taken, so that nothing is kept
    // in registers across the unit
    if (p.trace && threadIdx.x == 0) p.trace[6 * t + 1] = static_cast<int64_t>(wall_clock64());
    if (WAIT) {
      const uint32_t need = tl.chunk_mask & ~seen;
      if (need) {
        if (threadIdx.x == 0) sh->abort = wait_chunks(p.sig, need, p.epoch, p.timeout_ticks, t);
        __syncthreads();
        if (sh->abort) return false;
        seen |= need;
      }
    }
    return true;
  };
  auto stamp_start = [&](int64_t t) {
    if (p.trace && threadIdx.x == 0) {
      int64_t* e = p.trace + 6 * t;
      e[2] = static_cast<int64_t>(wall_clock64());
      e[4] = static_cast<int64_t>(__builtin_amdgcn_s_memtime());
    }
  };
  auto stamp_end = [&](int64_t t) {
    if (p.trace && threadIdx.x == 0) {
      int64_t* e = p.trace + 6 * t;
      e[0] = blockIdx.x;
      e[3] = static_cast<int64_t>(wall_clock64());
      e[5] = static_cast<int64_t>(__builtin_amdgcn_s_memtime());
    }
  };
  // The first unit of every workgroup is its slot (no counter traffic while all
  // workgroups start at once); the dynamic schedule then hands out units
  // G, G+1, ... from the counter as workgroups become free.  Slots are spread
  // so that each XCD takes a contiguous run of the plan.  With co-located
  // copying, the copying workgroups -- busy first -- take the last slots of
  // the round, the units of the latest chunks, and the others the rest.
  const int g = blockIdx.x;
  int64_t t;
  const int cw = WAIT ? p.copy.wgs : 0;
  if (cw > 0 && cw < G) {
    const int Gr = G - cw, r = g - cw;
    t = g < cw ? Gr + g : ((p.xcd_remap && Gr % 8 == 0 && cw % 8 == 0) ? (r & 7) * (Gr >> 3) + (r >> 3) : r);
  } else {
    t = p.xcd_remap ? (g & 7) * (G >> 3) + (g >> 3) : g;
  }
  for (int it = 1; t < n_work; ++it) {
    if (tail && t >= p.sk_from) {
      // Piece s of tail tile j (static slots only): pieces s of consecutive
      // tiles go to consecutive slots, so the workgroups of an XCD run one K
      // range of a run of neighbouring tiles at the same time.
      const int KT = p.K / 64, S = p.sk_split;
      const int64_t q = t - p.sk_from;
      const int s = static_cast<int>(q / p.sk_tiles);
      const int64_t j = q - static_cast<int64_t>(s) * p.sk_tiles;
      const int64_t tt = p.sk_from + j;
      const tlc_tile tl = p.plan[tt];
      if (!admit(tt, tl)) break;
      SkPiece pc;
      pc.kt0 = (s * KT / S) & ~1;
      pc.kt1 = ((s + 1) * KT / S) & ~1;
      pc.count = S;
      pc.self = s;
      pc.block = p.sk_ws + j * kSkBlockBytes;
      stamp_start(tt);
      run_tile(tl, pc, &sh->split_last);
      stamp_end(tt);
      t += G;
      continue;
    }
    const tlc_tile tl = p.plan[t];
    if (!admit(t, tl)) break;
    // claim the next unit now: the counter's round trip overlaps this unit
    if (p.dynamic && threadIdx.x == 0)
      sh->next[it & 1] = G + static_cast<int64_t>(__hip_atomic_fetch_add(
                                 &p.sig->work_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    stamp_start(t);
    SkPiece whole;
    whole.count = 0;
    run_tile(tl, whole, &sh->split_last);  // has workgroup barriers: next[] is visible after it
    stamp_end(t);
    t = p.dynamic ? sh->next[it & 1] : t + G;
  }
  if (p.dynamic) {
    // the last workgroup out rewinds the counters for the next launch.  Relaxed
    // order suffices: each workgroup's last claim has returned before it counts
    // itself out, and the next launch sees the rewound values at the kernel
    // boundary.  (An acquire-release here would write back the L2 once per
    // workgroup.)
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(&p.sig->work_done, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (prev == static_cast<uint32_t>(G) - 1) {
        __hip_atomic_store(&p.sig->work_next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.sig->work_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int B_NK, int KIND, int WAIT>
__global__ __launch_bounds__(512) void gemm_kernel_8w(GemmParams p) {
  __shared__ u32x4 A0[2048], A1[2048], B0[2048], B1[2048];
  __shared__ LoopShared sh;
  tile_loop<256, 256, KIND, WAIT, 0>(p, &sh, [&](const tlc_tile& tl, const SkPiece&, int* s_flag) {
    Tile8w<B_NK, KIND>::run(p, tl, (TLC_LDS u32x4*)A0, (TLC_LDS u32x4*)A1, (TLC_LDS u32x4*)B0,
                            (TLC_LDS u32x4*)B1, s_flag);
  });
}

// SK: the variant with the stream-K tail (more vector registers in its
// epilogue, so it is launched only when the plan has a tail).
template <int B_NK, int KIND, int WAIT, int FAST, int SK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel_4w(
    GemmParams p) {
  __shared__ u32x4 A0[2048], A1[2048], B0[2048], B1[2048];
  __shared__ LoopShared sh;
  tile_loop<256, 256, KIND, WAIT, SK>(p, &sh, [&](const tlc_tile& tl, const SkPiece& pc, int* s_flag) {
    Tile4w<B_NK, KIND, FAST, SK>::run(p, tl, pc, (TLC_LDS u32x4*)A0, (TLC_LDS u32x4*)A1,
                                      (TLC_LDS u32x4*)B0, (TLC_LDS u32x4*)B1, s_flag);
  });
  // the last unit's loads past its K range land before the wave ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int BM, int BN, int B_NK, int KIND, int WAIT>
__global__ __launch_bounds__(THREADS) void gemm_kernel(GemmParams p) {
  __shared__ u32x4 lds[2 * (BM + BN) * 8];
  __shared__ LoopShared sh;
  tile_loop<BM, BN, KIND, WAIT, 0>(p, &sh, [&](const tlc_tile& tl, const SkPiece&, int* s_flag) {
    Tile<BM, BN, B_NK, KIND>::run(p, tl, lds, s_flag);
  });
}

template <int BM, int BN, int B_NK, int KIND, int WAIT>
void launch_kernel(const GemmParams& p, int grid, void* stream) {
  // 256 x 256 tiles: the 4-wavefront core (3-5 % faster than the 8-wavefront
  // one on the whole-matrix shapes, and its whole-tile kernel 5 % faster on the
  // grouped GEMM); the grouped GEMM falls back to the 8-wavefront core when it
  // cannot run the whole-tile kernel, since the 4-wavefront core's general
  // loop is slower on its ragged tiles
  if constexpr (BM == 256 && BN == 256) {
    if constexpr (KIND == KIND_MOE) {
      if (p.fast)
        hipLaunchKernelGGL((gemm_kernel_4w<B_NK, KIND, WAIT, 1, 0>), dim3(grid), dim3(256), 0,
                           static_cast<hipStream_t>(stream), p);
      else
        hipLaunchKernelGGL((gemm_kernel_8w<B_NK, KIND, WAIT>), dim3(grid), dim3(512), 0,
                           static_cast<hipStream_t>(stream), p);
    } else if (p.fast && p.sk_split > 0)
      hipLaunchKernelGGL((gemm_kernel_4w<B_NK, KIND, WAIT, 1, 1>), dim3(grid), dim3(256), 0,
                         static_cast<hipStream_t>(stream), p);
    else if (p.fast)
      hipLaunchKernelGGL((gemm_kernel_4w<B_NK, KIND, WAIT, 1, 0>), dim3(grid), dim3(256), 0,
                         static_cast<hipStream_t>(stream), p);
    else
      hipLaunchKernelGGL((gemm_kernel_4w<B_NK, KIND, WAIT, 0, 0>), dim3(grid), dim3(256), 0,
                         static_cast<hipStream_t>(stream), p);
  }
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, B_NK, KIND, WAIT>), dim3(grid), dim3(THREADS), 0,
                       static_cast<hipStream_t>(stream), p);
}

template <int BM, int BN, int B_NK, int KIND>
tlc_status launch_one(const GemmParams& p, int grid, void* stream) {
  if (p.do_wait)
    launch_kernel<BM, BN, B_NK, KIND, 1>(p, grid, stream);
  else
    launch_kernel<BM, BN, B_NK, KIND, 0>(p, grid, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "gemm launch: %s", hipGetErrorString(e));
  return ok();
}

template <int BM, int BN>
tlc_status launch_shape(const GemmParams& p, int b_layout, int kind, int grid, void* stream) {
  if (kind == KIND_RS_NOTIFY) {
    // the scatter-mode GEMM never waits for chunks
    if (p.do_wait) return fail(TLC_ERR_UNSUPPORTED, "notifying GEMM with chunk waits");
    if (b_layout == TLC_B_NK) launch_kernel<BM, BN, 1, KIND_RS_NOTIFY, 0>(p, grid, stream);
    else launch_kernel<BM, BN, 0, KIND_RS_NOTIFY, 0>(p, grid, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TLC_ERR_HIP, "gemm launch: %s", hipGetErrorString(e));
    return ok();
  }
  if (kind == KIND_MOE)
    return b_layout == TLC_B_NK ? launch_one<BM, BN, 1, KIND_MOE>(p, grid, stream)
                                : launch_one<BM, BN, 0, KIND_MOE>(p, grid, stream);
  return b_layout == TLC_B_NK ? launch_one<BM, BN, 1, KIND_DENSE>(p, grid, stream)
                              : launch_one<BM, BN, 0, KIND_DENSE>(p, grid, stream);
}

}  // namespace

tlc_status launch_gemm(const GemmParams& p_in, int bm, int bn, int b_layout, int kind, int grid,
                       void* stream) {
  GemmParams p = p_in;
  // The kernel with only the fixed-order loop (and no split epilogue), for
  // plans whose units are all whole 256-row tiles with an even number of
  // K steps: M a multiple of 256, K / 64 even, no split workspace (a split
  // unit without one is reported as a bad plan).  It keeps a fifth of the
  // register file free or more (405 of 512 registers per lane with a K x N
  // weight), so that other kernels' wavefronts (a side stream's copies) can
  // run beside it on the same compute units.  The grouped GEMM
  // runs it on its ragged tiles too (never split): the rows past an expert's
  // end load that expert's last row again and are not stored, and the fixed
  // loop over all 256 rows still beats the general loop that skips them.
  p.fast = (kind == KIND_MOE || p.M % 256 == 0) && (p.K / 64) % 2 == 0 && p.split_bytes == 0;
  if (bm == 256 && bn == 256) return launch_shape<256, 256>(p, b_layout, kind, grid, stream);
  if (bm == 128 && bn == 128) return launch_shape<128, 128>(p, b_layout, kind, grid, stream);
  return fail(TLC_ERR_UNSUPPORTED, "tile %dx%d not built (256x256, 128x128)", bm, bn);
}

}  // namespace tlc
