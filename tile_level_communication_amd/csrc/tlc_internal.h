// Internal declarations shared by the library's translation units (not part of
// the public ABI; see include/tlc.h for the entry points).
#pragma once

#include <stdint.h>

#include <string>

#include <hip/hip_runtime.h>

#include "tlc.h"

namespace tlc {

// Sets the thread's last-error text and returns `s` (for `return fail(...)`).
tlc_status fail(tlc_status s, const char* fmt, ...);
tlc_status ok();

// Device facts cached per device id (compute units, wall-clock rate).
struct DeviceInfo {
  int cus = 0;
  int64_t wall_khz = 0;
  int arch_ok = 0;  // gfx950
};
tlc_status device_info(DeviceInfo* out);

// Co-located landing: the first `wgs` workgroups of a launch copy the peers'
// chunks (landing order i = 0 .. chunks-1, chunk i from src[i] to dst[i]) with
// load/store instructions and count themselves in; the last share of chunk i
// raises flags[flag[i]] to the epoch.
struct CopyPlan {
  int32_t wgs;
  int32_t chunks;
  int64_t vec;  // 16-byte units per chunk
  const uint4* src[TLC_MAX_WORLD];
  uint4* dst[TLC_MAX_WORLD];
  int32_t flag[TLC_MAX_WORLD];
};

// Parameters of the tiled GEMM kernels (one struct for all modes).
struct GemmParams {
  const tlc_tile* plan;
  const int32_t* n_tiles_dev;  // MoE: tile count written by the routing kernels
  int64_t n_tiles;             // dense: tile count; MoE: plan capacity
  const uint16_t* a;           // gathered A (AG), local A (RS), tokens X (MoE)
  const uint16_t* b;           // weight, or stacked expert weights (MoE)
  float* c;                    // output
  const int32_t* row_token;    // MoE only
  int64_t a_rows;              // MoE: rows of the token matrix (bounds of the gathered loads)
  int32_t M, N, K;
  int64_t lda, ldb, ldc;
  int64_t b_expert_stride;     // MoE: elements between experts' weights
  uint32_t no_wait_mask;       // chunks that are never waited for (the local one)
  int32_t do_wait;
  tlc_signals* sig;
  uint32_t epoch;
  int64_t timeout_ticks;
  int32_t xcd_remap;
  int64_t* trace;              // optional: n_tiles x {wg, wait start, wait end, done}
  int32_t dynamic;             // 1: units from the work counter in sig; 0: slot-strided
  char* split_ws;              // split tiles' blocks: 256-byte counter header + S partials
  int64_t split_bytes;         // bytes of split_ws
  // Co-located landing: workgroups [0, copy.wgs) each copy a share of every
  // chunk, in landing order, before their first unit.
  CopyPlan copy;
  // Scatter mode with sends (KIND_RS_NOTIFY): stores are device-coherent and
  // every stored tile counts its elements into sig->dest_done[c] for each
  // destination c in notify_mask it writes; the store completing dest_total
  // elements rewinds the count and raises sig->dest_ready[c] to epoch.
  int32_t rows_per_chunk;
  uint32_t notify_mask;
  uint32_t dest_total;
  // set by launch_gemm: every unit is a whole tile with an even number of K
  // steps and none is split (the kernel with only the fast loop)
  int32_t fast;
  // Stream-K tail (the whole-tile kernel, static slots): work items
  // [0, sk_from) are the plan's first units, run whole; the sk_tiles tiles
  // from sk_from on are each split into sk_split pieces along K, piece s of
  // a tile covering the 64-wide K steps [b(s), b(s + 1)), b(s) = s * KT /
  // sk_split rounded down to even (KT = K / 64, even), and item
  // sk_from + s * sk_tiles + j is piece s of tile sk_from + j: pieces with
  // the same K range of neighbouring tiles run side by side, as whole tiles
  // do.  sk_split = 0: no tail.
  int64_t sk_from;
  int32_t sk_tiles;
  int32_t sk_split;
  // per tail tile a block of kSkBlockBytes: a 256-byte header (the tile's
  // arrival counter) and one fp32 partial tile per piece
  char* sk_ws;
};

// Stream-K tail workspace: pieces per tile at most, bytes per tile.
constexpr int kSkMaxSplit = 4;
constexpr int64_t kSkTileBytes = int64_t{256} * 256 * 4;
constexpr int64_t kSkBlockBytes = 256 + kSkMaxSplit * kSkTileBytes;

// Bytes of one split tile's workspace block (counter header + split_k partials).
int64_t split_block_bytes(int32_t split_k, int32_t bm, int32_t bn);

enum GemmKind { KIND_DENSE = 0, KIND_MOE = 1, KIND_RS_NOTIFY = 2 };

// Launch the persistent tiled GEMM: bm x bn in {256x256, 128x128}.
tlc_status launch_gemm(const GemmParams& p, int bm, int bn, int b_layout, int kind, int grid,
                       void* stream);

struct ReduceParams {
  const float* src[TLC_MAX_WORLD];  // S_0 .. S_{W-1}
  float* out;
  int64_t n_vec4;                   // elements / 4
  int32_t world;
  uint32_t wait_mask;               // chunks whose flags must reach epoch first
  tlc_signals* sig;
  uint32_t epoch;
  int64_t timeout_ticks;
};
tlc_status launch_reduce(const ReduceParams& p, int grid, void* stream);

struct LandParams {
  const uint4* src[TLC_MAX_WORLD];
  uint4* dst[TLC_MAX_WORLD];
  int32_t order[TLC_MAX_WORLD];
  int32_t n_chunks;
  int64_t vec_per_chunk;  // 16-byte units per chunk
  tlc_signals* sig;
  uint32_t epoch;
  int32_t flag_base;      // chunk c raises flags[flag_base + c]
};
tlc_status launch_land_cu(const LandParams& p, int grid, void* stream);

// Sends of the scatter mode: the slices order[0..n) of the partial product,
// each once sig->dest_ready[c] has reached epoch.
struct SendParams {
  const uint4* src[TLC_MAX_WORLD];
  uint4* dst[TLC_MAX_WORLD];
  int32_t order[TLC_MAX_WORLD];
  int32_t n;
  int64_t vec_per_slice;  // 16-byte units per slice (< 2^28)
  tlc_signals* sig;
  uint32_t epoch;
  int64_t timeout_ticks;
};
// One wavefront that waits (bounded) for sig->dest_ready[c] >= epoch.
tlc_status launch_send_gate(tlc_signals* sig, int c, uint32_t epoch, int64_t timeout_ticks,
                            void* stream);
// Copy kernel: its workgroups wait for each slice in order, then copy it.
tlc_status launch_send_cu(const SendParams& p, int grid, void* stream);

tlc_status launch_signals_set(tlc_signals* sig, int world, uint32_t value, void* stream);
tlc_status launch_status_clear(tlc_signals* sig, void* stream);
tlc_status launch_signals_rewind(tlc_signals* sig, void* stream);

struct MoeDev {
  const float* logits;
  int32_t T, E, k, Tc, world, rank, N, bm, bn, order, ntiles_n;
  int32_t* topk;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* slot;
  tlc_tile* plan;
  int32_t* n_tiles;
  unsigned long long* member;  // workspace: T masks
  int32_t* blk;                // workspace: blocks x E block counts, then their prefixes
  // Optional landing of the peers' token chunks by copy.wgs workgroups of the
  // top-k kernel after the routing's own (copy.wgs = 0: none), flags raised to
  // `epoch` in sig.
  CopyPlan copy;
  tlc_signals* sig;
  uint32_t epoch;
};

int64_t moe_max_pairs(int32_t T, int32_t topk, int32_t experts, int32_t bm);
// Arrival blocks of the routing for T tokens, at most (any world and chunk size).
int64_t moe_max_blocks(int64_t T);
tlc_status launch_moe_route(const MoeDev& d, void* stream);

// The static routing workspace (tlc_moe_route_static): its size, and its
// device address on the current device (looked up once per device).
constexpr int64_t kMoeStaticScratchBytes = int64_t{4} << 20;
tlc_status moe_static_scratch(void** out);

// Default persistent grid: the fewest rounds of tiles over the CUs, with the
// tiles spread evenly over that many rounds (rounded up to a multiple of 8).
int default_grid(int64_t n_tiles, int cus);
// CUs left free by the persistent GEMM for the given landing mode.
int reserve_for(int land);

}  // namespace tlc
