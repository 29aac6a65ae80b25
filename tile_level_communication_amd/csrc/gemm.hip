// Persistent, plan-driven bf16 GEMM for gfx950 (MFMA 32x32x16 bf16 -> fp32).
//
// One workgroup (4 wavefronts, 2 x 2) owns one BM x BN output tile at a time
// and walks the tile list in plan order: slot s takes tiles s, s + G, s + 2G,
// ... where G is the grid size.  Slots are spread so that each XCD (8 per
// MI355X; workgroups are dealt to XCDs round-robin) gets a contiguous run of
// the plan, keeping the operands that neighbouring tiles share in the same L2.
//
// Before touching a tile's A rows, the workgroup waits until every chunk the
// tile reads has landed (flag >= epoch), with a bounded spin that reports a
// timeout instead of hanging.  This is the tile-granular consumer wait of the
// pages (Triton-Distributed talk: consumer_tile_wait keyed by tile id, and the
// low-level signal wait with scope, memory semantics and expected value;
// AutoOverlap §5.2: only the tiles that consume a chunk wait for it).
//
// K loop: BK = 64, two LDS stages.  Each stage is filled with 128-bit global
// loads (A rows and, for an N x K weight, B rows are K-contiguous; a K x N
// weight is transposed 8 x 8 in registers on its way to LDS) and read back as
// 128-bit MFMA fragments.  LDS rows are 64 bf16 = eight 16-byte chunks stored
// at chunk ^ (row & 7), so the eight lanes of a fragment read or a row write
// always hit eight different 16-byte bank groups.
#include <hip/hip_runtime.h>

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

  __device__ static void run(const GemmParams& p, const tlc_tile& tl, u32x4* lds) {
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

    const int KT = p.K / BK;
    gload(0);
    swrite(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) gload(kt + 1);
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
      if (kt + 1 < KT) swrite(cur ^ 1);
      __syncthreads();
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
          if (row < tl.m_rows && col < tl.n_cols) cbase[static_cast<int64_t>(row) * p.ldc + col] = acc[i][j][e];
        }
      }
  }
};

template <int BM, int BN, int B_NK, int KIND>
__global__ __launch_bounds__(THREADS) void gemm_kernel(GemmParams p) {
  __shared__ u32x4 lds[2 * (BM + BN) * 8];
  __shared__ int s_abort;
  const int G = gridDim.x;
  int slot = blockIdx.x;
  if (p.xcd_remap) slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int64_t n_tiles = KIND == KIND_MOE ? static_cast<int64_t>(*p.n_tiles_dev) : p.n_tiles;
  uint32_t seen = p.no_wait_mask;
  for (int64_t t = slot; t < n_tiles; t += G) {
    const tlc_tile tl = p.plan[t];
    const bool bad = tl.m_rows < 1 || tl.n_cols < 1 || tl.m0 < 0 || tl.n0 < 0 ||
                     tl.m0 + tl.m_rows > p.M || tl.n0 + tl.n_cols > p.N || tl.m_rows > BM ||
                     tl.n_cols > BN || (tl.n_cols & 7) != 0 ||
                     (KIND == KIND_MOE && tl.expert < 0);
    if (bad) {
      if (threadIdx.x == 0) report(p.sig, TLC_ERR_BAD_PLAN, t);
      break;
    }
    if (p.do_wait) {
      const uint32_t need = tl.chunk_mask & ~seen;
      if (need) {
        if (threadIdx.x == 0) s_abort = wait_chunks(p.sig, need, p.epoch, p.timeout_ticks, t);
        __syncthreads();
        const int abort = s_abort;
        if (abort) break;
        seen |= need;
      }
    }
    Tile<BM, BN, B_NK, KIND>::run(p, tl, lds);
  }
}

template <int BM, int BN, int B_NK, int KIND>
tlc_status launch_one(const GemmParams& p, int grid, void* stream) {
  hipLaunchKernelGGL((gemm_kernel<BM, BN, B_NK, KIND>), dim3(grid), dim3(THREADS), 0,
                     static_cast<hipStream_t>(stream), p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "gemm launch: %s", hipGetErrorString(e));
  return ok();
}

template <int BM, int BN>
tlc_status launch_shape(const GemmParams& p, int b_layout, int kind, int grid, void* stream) {
  if (kind == KIND_MOE)
    return b_layout == TLC_B_NK ? launch_one<BM, BN, 1, KIND_MOE>(p, grid, stream)
                                : launch_one<BM, BN, 0, KIND_MOE>(p, grid, stream);
  return b_layout == TLC_B_NK ? launch_one<BM, BN, 1, KIND_DENSE>(p, grid, stream)
                              : launch_one<BM, BN, 0, KIND_DENSE>(p, grid, stream);
}

}  // namespace

tlc_status launch_gemm(const GemmParams& p, int bm, int bn, int b_layout, int kind, int grid,
                       void* stream) {
  if (bm == 256 && bn == 256) return launch_shape<256, 256>(p, b_layout, kind, grid, stream);
  if (bm == 128 && bn == 128) return launch_shape<128, 128>(p, b_layout, kind, grid, stream);
  return fail(TLC_ERR_UNSUPPORTED, "tile %dx%d not built (256x256, 128x128)", bm, bn);
}

}  // namespace tlc
