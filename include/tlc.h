/*
 * tlc.h -- C ABI of libtlc: chunk-swizzled AllGather-GEMM, GEMM-ReduceScatter
 * and AllGather-MoE on one AMD Instinct MI355X (gfx950).
 *
 * The method (tile-level computation/communication overlap) runs ONE persistent
 * tiled GEMM whose tile order follows communication chunks:
 *   - gather mode (AllGather-GEMM, AG-MoE): every rank computes the tiles of the
 *     chunk it already holds first, then the other chunks in rank-offset order as
 *     per-chunk ready flags flip (DITRON paper notes, §3.2 "distributed
 *     swizzling", gather mode and the rank_id mod local_world_size start;
 *     Triton-Distributed talk, swizzling section);
 *   - scatter mode (GEMM-ReduceScatter): tiles bound for remote ranks are produced
 *     first, the rank's own slice last, into per-destination row slices of the
 *     partial product, which a reduce kernel then sums into the local slice
 *     (DITRON §3.2 scatter mode; talk, GEMM-ReduceScatter example: the GEMM
 *     notifies, a separate reduce kernel waits, two streams).
 * The other ranks are emulated on one GPU: their chunks are device buffers that
 * a side stream lands into the local buffers chunk by chunk, then flags a
 * per-chunk signal (AutoOverlap §5.3, backends 1 "copy engine" and 4/5
 * "load/store on SMs"; global-memory signals for both).
 *
 * Conventions (all entry points)
 *   - Every call returns tlc_status: 0 = OK, negative = error.  Argument errors
 *     are detected on the host and returned synchronously; nothing is enqueued
 *     then.  tlc_last_error() gives a human-readable detail for the calling
 *     thread.
 *   - Calls are asynchronous in stream order; no call synchronizes the host,
 *     except tlc_signals_alloc/free and tlc_read_status.
 *   - Ownership: the caller owns every buffer.  The library allocates no device
 *     memory on these paths and keeps no per-call state.
 *   - Pointers named "device" must point to device-accessible memory of the
 *     current HIP device; "host" pointers are read during the call only.
 *   - Streams are hipStream_t values passed as void* (NULL = default stream).
 *     The landing side takes a host array of n_copy_streams >= 1 streams:
 *     with the copy engine, the i-th chunk in landing order is copied on
 *     copy_streams[i % n] (several streams let several copy engines work at
 *     once, as several links would); the CU landing kernel runs on
 *     copy_streams[0].  The caller orders the copy streams after earlier
 *     readers of the landing buffers, and later readers after them.  The
 *     landing is always enqueued before the kernels that wait for it: when
 *     two streams share one hardware queue the work then runs one after the
 *     other instead of waiting forever.
 *   - Device-side failures (a wait that exceeded its time limit, a plan entry
 *     outside the output) are written to tlc_signals.status and read after the
 *     stream is synchronized (tlc_read_status).  The kernels then stop early;
 *     outputs are undefined.
 *   - Element types: "bf16" = bfloat16 (raw 16-bit), "f32" = IEEE binary32.
 *     All matrices are row-major with the stated leading dimension.
 */
#ifndef TLC_H
#define TLC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t tlc_status;

enum {
  TLC_OK = 0,
  TLC_ERR_INVALID_ARG = -1, /* NULL pointer, size out of range, inconsistent sizes */
  TLC_ERR_UNSUPPORTED = -2, /* tile shape / layout / device not supported */
  TLC_ERR_MISALIGNED = -3,  /* a pointer or row stride not 16-byte aligned */
  TLC_ERR_CAPACITY = -4,    /* output array too small (tlc_chunk_plan) */
  TLC_ERR_HIP = -5,         /* a HIP runtime call failed (text in tlc_last_error) */
  TLC_ERR_TIMEOUT = -6,     /* device: a chunk flag did not reach the epoch in time */
  TLC_ERR_BAD_PLAN = -7     /* device: a plan entry lies outside the output */
};

enum { TLC_MODE_AG = 0, TLC_MODE_RS = 1, TLC_MODE_MOE = 2 };
/* NATURAL: every rank walks tiles from tile 0 (no swizzle).  RANK_OFFSET: the
 * chunk-following order described above. */
enum { TLC_ORDER_NATURAL = 0, TLC_ORDER_RANK_OFFSET = 1 };
/* Layout of a weight operand B of logical shape K x N:
 * KN = K rows of N contiguous elements; NK = N rows of K contiguous elements. */
enum { TLC_B_KN = 0, TLC_B_NK = 1 };
/* How the emulated peers' chunks arrive:
 *   NONE        -- already in place; the caller has set the flags (compute-only)
 *   COPY_ENGINE -- one hipMemcpyAsync(DeviceToDeviceNoCU) per chunk on a copy
 *                  stream, then a 4-byte copy-engine transfer of the epoch into
 *                  the chunk's flag (epoch in 1..TLC_EPOCH_MAX)
 *   CU          -- one copy kernel on the copy stream; its workgroups copy the
 *                  chunks in landing order and the last one to finish a chunk
 *                  publishes its flag with a release store
 *   MEMCPY      -- as COPY_ENGINE but with the default hipMemcpyDeviceToDevice
 *                  kind, which the runtime carries out with its own copy kernels
 *                  on CUs (epoch in 1..TLC_EPOCH_MAX)
 *   COLOCATED   -- no separate landing: the GEMM's own workgroups move the data
 *                  (AutoOverlap §5.3, backend 5: load/store on the SMs that
 *                  compute).  AG-GEMM / AG-MoE: before its first unit, each of
 *                  the first copy_wgs workgroups copies an equal share of every
 *                  peer chunk in landing order; the last workgroup to finish a
 *                  chunk's shares raises its flag with a release store, and the
 *                  GEMM's units wait on the flags as in the other modes.
 *                  A share of 2 GiB or more (chunk bytes / copy_wgs) returns
 *                  TLC_ERR_UNSUPPORTED.  Deadlock freedom rests on the copying
 *                  workgroups having the lowest ids: the dispatcher makes them
 *                  resident first and they wait for nothing before copying.
 *                  So all of them must fit the device at once: more copying
 *                  workgroups than compute units (one GEMM workgroup per
 *                  compute unit) is refused with TLC_ERR_INVALID_ARG.
 *                  GEMM-RS: the reduce loads the peers' partials from
 *                  remote_src itself (no landing buffers, no flags).  The copy
 *                  streams are not used (they may be NULL / 0).            */
enum {
  TLC_LAND_NONE = 0,
  TLC_LAND_COPY_ENGINE = 1,
  TLC_LAND_CU = 2,
  TLC_LAND_MEMCPY = 3,
  TLC_LAND_COLOCATED = 4
};

#define TLC_MAX_WORLD 32

/* One work unit of the plan, 32 bytes: an output tile, or one K range of a
 * tile that is split along K.  Rows [m0, m0+m_rows) and columns
 * [n0, n0+n_cols) of the output.  expert = -1 for dense GEMMs.  chunk_mask bit
 * c = the tile reads rows of chunk c (gather, MoE) or writes rows of
 * destination chunk c (scatter).  key = the primary sort key: wait position
 * (gather), send position (scatter) or readiness (MoE); 0 in natural order.
 * split = 0 for a whole tile; for a tile split into S K ranges (2 <= S <= 255)
 * unit s (0 <= s < S) has split = S | s << 8 | f << 16, where f numbers the
 * split tiles 0, 1, ... in plan order.  Unit s covers the 64-wide K steps
 * [s*KT/S, (s+1)*KT/S) (integer division, KT = K/64); the S units of a tile
 * are adjacent in the plan.  Each unit writes its fp32 partial tile to a
 * workspace slot; the last of the S units to finish adds the S partials in
 * ascending s and stores the tile, so the result does not depend on which
 * workgroup ran which unit or in which order they finished. */
typedef struct {
  int32_t m0, n0, m_rows, n_cols;
  int32_t expert;
  uint32_t chunk_mask;
  int32_t key;
  uint32_t split; /* 0, or S | s << 8 | f << 16 (see above) */
} tlc_tile;

/* Copy-engine landings raise a chunk's flag with a second copy-engine transfer
 * of 4 bytes from a table of epoch values held in the signals block, so no
 * compute unit is involved; epochs are therefore limited to 1..TLC_EPOCH_MAX
 * in that mode (rewind the flags to 0 with tlc_signals_set, then restart at 1). */
#define TLC_EPOCH_MAX 4096

/* Signals shared by the copy side and the kernels (device memory; allocate
 * with tlc_signals_alloc so that it is fine-grained and coherent with the copy
 * engines).  flags[c] >= epoch  <=>  chunk c has landed for this call.
 * status[0] = 0 or a negative tlc_status, status[1] = plan index of the tile
 * that failed, status[2] = chunk it waited for.  land_count is internal to the
 * CU and co-located landings, work_next / work_done to the GEMM's dynamic work queue
 * (all zero between calls; the last workgroup of a launch resets them).
 * Scatter mode with sends (tlc_rs_args.send_dst): dest_done[c] counts the
 * output elements of destination slice P[c] stored so far in this call (zero
 * between calls: the store that completes the slice rewinds it), and
 * dest_ready[c] >= epoch  <=>  P[c] is complete for this call (the GEMM's
 * per-destination notification; Triton-Distributed talk, GEMM-ReduceScatter
 * example: the GEMM notifies, the consumer waits).
 * epoch_table[i] = i + 1, written once by tlc_signals_alloc.  One GEMM call
 * at a time per signals block.  After a device error (status[0] != 0)
 * tlc_signals_clear_status also rewinds dest_done. */
typedef struct {
  uint32_t flags[TLC_MAX_WORLD];
  uint32_t land_count[TLC_MAX_WORLD];
  int32_t status[4];
  uint32_t work_next, work_done;
  uint32_t dest_done[TLC_MAX_WORLD];
  uint32_t dest_ready[TLC_MAX_WORLD];
  uint32_t reserved[122];
  uint32_t epoch_table[TLC_EPOCH_MAX];
} tlc_signals;

/* ---------------------------------------------------------------- plan ---- */

/* tlc_plan_desc: a dense gather or scatter GEMM whose M rows are `world`
 * chunks of `rows_per_chunk` rows (M = world * rows_per_chunk). */
typedef struct {
  int32_t mode;           /* TLC_MODE_AG or TLC_MODE_RS */
  int32_t world;          /* 1 .. TLC_MAX_WORLD */
  int32_t rank;           /* 0 .. world-1 */
  int32_t M, N;           /* output size, >= 1 */
  int32_t rows_per_chunk; /* R >= 1, M == world * R */
  int32_t bm, bn;         /* tile size, >= 1 */
  int32_t order;          /* TLC_ORDER_* */
  int32_t group_m;        /* >= 1: m-tiles per locality band inside a key */
  int32_t split_k;        /* 0 or 1: no split; 2..255: tiles with key >= split_from
                             are split into split_k K ranges */
  int32_t split_from;     /* first key whose tiles are split (>= 0) */
  int32_t sub_chunks;     /* gather mode: 0 or 1, or S >= 2 sub-chunks per rank (see below) */
} tlc_plan_desc;

/* Tile order of the communication-aware scheduler (host code, integers only).
 *   Gather: chunk c is consumed at position p(c) = (c - rank) mod W; a tile is
 *   keyed by the largest p of the chunks it reads, so tiles that straddle
 *   chunks run once their last chunk has landed (Triton-Distributed talk,
 *   non-perfect tile scheduling).  Scatter: destination c is sent at position
 *   q(c) = (c - rank - 1) mod W; a tile is keyed by the smallest q of the
 *   destinations it writes, so the rank's own slice goes last and straddling
 *   tiles go early.  Ties: (m-tile / group_m, n-tile, m-tile) -- bands of
 *   group_m m-tiles walked column by column (AutoOverlap §5.4, Fig. 6: intra-
 *   chunk swizzle for locality).  Natural order: all keys 0.
 *   A tile with key >= split_from (split_k >= 2) becomes split_k adjacent
 *   units, one per K range, so that the work that depends on the last chunks
 *   can spread over every compute unit.
 *   Sub-chunks (gather mode, S = sub_chunks >= 2, R % S == 0, world * S <= 32):
 *   every rank's chunk lands as S pieces of R/S rows, each with its own flag
 *   (AutoOverlap §6.1 and Fig. 11(b): the split factor of a chunk).  The plan is then the one of
 *   world * S chunks of R/S rows with rank * S as the local one: chunk_mask
 *   and key refer to sub-chunks c' = row / (R/S), consumed at position
 *   (c' - rank * S) mod (world * S).
 * tiles:   host array of `cap` entries, or NULL to query the count only.
 * n_tiles: host, receives the number of units: ceil(M/bm) * ceil(N/bn) plus
 *   (split_k - 1) per split tile.
 * landing_order: host array of (world-1) * S entries (S = 1 without sub-chunks)
 *   or NULL; receives the order in which peers' (sub-)chunks land:
 *   rank+1, rank+2, ..., rank-1 (mod W), each as its S sub-chunks in order.
 * Errors: INVALID_ARG (bad desc), CAPACITY (cap < count; *n_tiles is set). */
tlc_status tlc_chunk_plan(const tlc_plan_desc* desc, tlc_tile* tiles, int64_t cap,
                          int64_t* n_tiles, int32_t* landing_order);

/* Bytes of the workspace a plan with `n_split_tiles` split tiles of split_k
 * units needs: one block per split tile, a 256-byte header (its arrival
 * counter) followed by split_k fp32 partial tiles of bm x bn, so
 * n_split_tiles * (256 + split_k * bm * bn * 4).  0 if there is no split tile.
 * The caller allocates it in device memory (256-byte aligned) and zero-fills it
 * once; each call leaves the counters at zero again, except after a device
 * error (TIMEOUT, BAD_PLAN), after which it must be zero-filled before reuse. */
int64_t tlc_split_workspace_bytes(int64_t n_split_tiles, int32_t split_k, int32_t bm, int32_t bn);

/* Bytes of the workspace the stream-K tail (TLC_SCHED_STREAMK) needs on a
 * grid of `grid` workgroups (0: 256, the largest gfx950 part's compute units,
 * enough for the default grid and any grid of at most 256): grid blocks of
 * 256 + 4 * 256 * 256 * 4 bytes, an arrival counter and up to four fp32
 * partial tiles per tail tile (a tail has fewer tiles than the grid has
 * workgroups).  A call whose tail needs more blocks than the workspace holds
 * is refused with INVALID_ARG.  Negative grid: -1.
 * The caller allocates it in device memory (256-byte aligned) and zero-fills it
 * once; each call leaves the counters at zero again, except after a device
 * error, after which it must be zero-filled before reuse.  Not from the
 * pages: a work-sharing device of this library (see TLC_SCHED_STREAMK). */
int64_t tlc_streamk_workspace_bytes(int32_t grid);

/* ------------------------------------------------------------- signals ---- */

/* Allocate / free one zeroed tlc_signals block in fine-grained device memory
 * (synchronous).  *out receives a device pointer.  The block holds the pages'
 * per-chunk signals (talk, signal wait/notify between producer and consumer;
 * DITRON §3.2, per-tile synchronisation of the communication and the GEMM) as
 * device flags; allocating and freeing it is not from the pages. */
tlc_status tlc_signals_alloc(tlc_signals** out);
tlc_status tlc_signals_free(tlc_signals* sig);
/* Enqueue on `stream`: flags[0..world-1] = value (a one-workgroup kernel; no
 * memset, so it may be captured in a graph).  Used to mark every chunk as
 * landed for compute-only runs (not from the pages: epochs are this library's
 * way of never resetting a flag). */
tlc_status tlc_signals_set(tlc_signals* sig, int32_t world, uint32_t value, void* stream);
/* Enqueue on `stream`: every flags[] and dest_ready[] entry = 0, so that the
 * epochs can restart at 1 (after TLC_EPOCH_MAX in copy-engine mode; not from
 * the pages). */
tlc_status tlc_signals_rewind(tlc_signals* sig, void* stream);
/* Enqueue on `stream`: status[0..3] = 0 and dest_done[0..31] = 0 (not from
 * the pages: the status word is this library's error report). */
tlc_status tlc_signals_clear_status(tlc_signals* sig, void* stream);
/* Synchronize `stream`, then copy status[0..3] to the host array out[4] (not
 * from the pages). */
tlc_status tlc_read_status(const tlc_signals* sig, void* stream, int32_t* out);
/* Synchronize `stream`, then copy the whole block to the host struct *out
 * (not from the pages: an aid for tests and debugging, e.g. to check that
 * every counter is back at zero after a call). */
tlc_status tlc_read_signals(const tlc_signals* sig, void* stream, tlc_signals* out);

/* ---------------------------------------------------------- AG-GEMM ------- */

/* C[M x N] (f32) = concat_{c=0..W-1}(A_c) [M x K] (bf16) @ B [K x N] (bf16),
 * fp32 accumulation (DITRON §4.1 AG-GEMM; the pages' core-level tile GEMM).
 * Tile shapes: (bm, bn) in {(256,256), (128,128)}; BK = 64.
 * Requirements: K % 64 == 0, N % 8 == 0, M == world * rows_per_chunk, all
 * pointers 16-byte aligned.  `plan` is a device copy of tlc_chunk_plan(...)
 * output for the same (M, N, rows_per_chunk, bm, bn, world, rank), mode AG.
 * Buffers:
 *   a      device bf16 M x K, the gathered activations; rows of chunk `rank`
 *          must be in place before the call; the other chunks' rows are
 *          written by the landing (or already in place if land == NONE).
 *          The caller must stream-order the copy stream after earlier readers
 *          of `a` (the landing overwrites it).
 *   a_src  host array of `world` device pointers, chunk c's source (R x K
 *          bf16); entry `rank` is ignored; may be NULL if land == NONE.
 *   b      device bf16, layout b_layout (KN: ldb = N; NK: ldb = K).
 *   c      device f32 M x N, ldc = N.
 *   sig    device tlc_signals; status must be 0 on entry; flags < epoch for the
 *          chunks that still have to land.  With land == TLC_LAND_NONE and
 *          epoch == 0 the kernel does not look at the flags at all (every
 *          chunk must already be in place): the plain compute-only GEMM.
 *   workspace  device, tlc_split_workspace_bytes(...) bytes for the plan's
 *          split tiles (zero-filled before first use), or NULL / 0 bytes if the
 *          plan splits no tile.  A split tile whose slot lies beyond
 *          workspace_bytes is reported as BAD_PLAN.  With TLC_SCHED_STREAMK:
 *          the tail's workspace (tlc_streamk_workspace_bytes) instead.
 * Streams: the GEMM runs on `compute_stream`, the landing on the copy streams.
 * grid: persistent workgroups (0 = every compute unit the landing leaves free).
 *   With a COPY_ENGINE, CU or MEMCPY landing a grid above (compute units - 32)
 *   is refused with INVALID_ARG: the landing's kernels (the CU copy kernel, or
 *   the runtime's kernels for the copies and the 4-byte flag transfers) need
 *   CUs that no GEMM workgroup holds while those workgroups wait on flags.
 * schedule: TLC_SCHED_DYNAMIC -- workgroups take the next unit in plan order
 *   from a counter in `sig` as they become free (units that wait for a late
 *   chunk then do not hold back the ones behind them); TLC_SCHED_STATIC --
 *   workgroup slot g runs units g, g + grid, g + 2 grid, ...; TLC_SCHED_STREAMK
 *   -- static slots for the first floor(n_tiles / grid) * grid units, then the
 *   remaining tiles (the last chunks' tiles, in plan order) split along K into
 *   S pieces each (2 <= S <= 4; piece s covers the 64-wide K steps from
 *   s * KT / S to (s + 1) * KT / S, each rounded down to even, KT = K / 64),
 *   piece s of the j-th such tile being item s * (tiles in the tail) + j of the
 *   slots' walk: pieces over the same K steps of neighbouring tiles run side
 *   by side, so that they share their operands in the caches as whole tiles
 *   do.  S is chosen on the host so that the slot with the most tail steps
 *   has the fewest; without a gain over one more round of whole tiles there is
 *   no tail.  A tile's pieces are summed in the workspace
 *   (tlc_streamk_workspace_bytes(grid) bytes) by the piece that completes it,
 *   in K order, so the result does not depend on which workgroup finishes
 *   first (it may differ from the other schedules' in rounding, since the K
 *   sums are grouped differently).  The last round then ends together on every
 *   compute unit instead of leaving units idle (wave quantization: AutoOverlap
 *   §2.1 and Fig. 2(a); the split into K pieces is this library's, not the
 *   pages').  Default grid: every compute unit the landing leaves free.  The
 *   tail is used when the kernel that runs only whole 256 x 256 tiles applies
 *   (M % 256 == 0, K / 64 even, bm = bn = 256) and the tiles do not fill the
 *   grid evenly; otherwise the schedule is TLC_SCHED_STATIC and the workspace
 *   is not touched.  The plan must not split tiles (split_k 0): the workspace
 *   serves the tail alone.  A workspace smaller than needed is refused with
 *   INVALID_ARG.
 * timeout_ns: per-wait limit (0 = 2 s). */
enum { TLC_SCHED_DYNAMIC = 0, TLC_SCHED_STATIC = 1, TLC_SCHED_STREAMK = 2 };
typedef struct {
  const tlc_tile* plan; /* device, n_tiles entries, execution order */
  int64_t n_tiles;
  int32_t M, N, K;
  int32_t world, rank, rows_per_chunk;
  int32_t bm, bn;
  void* a;
  const void* const* a_src;
  const void* b;
  int32_t b_layout;
  float* c;
  tlc_signals* sig;
  uint32_t epoch;
  int32_t land;
  int32_t grid;
  int64_t timeout_ns;
  void* workspace;
  int64_t workspace_bytes;
  int32_t schedule;
  /* 0 or 1, or S >= 2: the landing moves every peer chunk as S pieces of
   * rows_per_chunk / S rows, each raising its own flag (flags[c * S + j]); the
   * plan must be built with the same sub_chunks.  world * S <= 32. */
  int32_t sub_chunks;
  /* TLC_LAND_COLOCATED only: workgroups that copy before computing (1..grid;
   * 0 = those the last round of units leaves idle, grid rounds minus the unit
   * count rounded down to a multiple of 8, or the whole grid when that is
   * under 32; for AG-MoE, whose unit count is known only on the device, a
   * quarter of the grid).  They take the last units of the first round. */
  int32_t copy_wgs;
  /* Optional debug trace (NULL = off): device int64 array of n_tiles x 6,
   * entry t = {workgroup, wall clock at wait start, at wait end, at unit end,
   * shader clock at wait end, at unit end} for the unit at plan index t; wall
   * clock = the device's constant-rate counter (hipDeviceAttributeWallClockRate),
   * shader clock = the compute unit's cycle counter (its ratio to the wall
   * clock gives the clock frequency the unit ran at).  Entries of units not run
   * keep their previous contents. */
  int64_t* trace;
} tlc_ag_args;

tlc_status tlc_ag_gemm(const tlc_ag_args* args, void* compute_stream, void* const* copy_streams,
                       int32_t n_copy_streams);

/* ---------------------------------------------------------- GEMM-RS ------- */

/* Scatter-mode GEMM then reduce (DITRON §4.1 GEMM-RS; talk, GEMM-ReduceScatter
 * example).  P[M x N] (f32) = A [M x K] (bf16, local K shard) @ B [K x N];
 * the row chunk P[c] = rows [c R, (c+1) R) is the partial bound for rank c.
 * out[R x N] (f32) = sum over s = 0..W-1 in ascending s of S_s, S_rank = P[rank]
 * and S_s = landing[s] (the partial rank s computed for this rank's rows).
 * Requirements as tlc_ag_gemm plus N % 4 == 0.  plan: mode RS.
 *   remote_src / landing: host arrays of `world` device pointers (R x N f32);
 *   entries `rank` are ignored; remote_src may be NULL if land == NONE (then
 *   landing[s] must already hold the data and flags be >= epoch); landing may
 *   be NULL if land == COLOCATED (the reduce reads remote_src directly).
 * The GEMM and then the reduce run on `compute`; the reduce waits in-kernel for
 * the remote partials' flags.
 * Sends (send_dst != NULL; DITRON §3.2 scatter mode, the partial results are
 * sent to the other ranks while the rest is computed; talk, GEMM-ReduceScatter
 * example, a producer GEMM that notifies per tile and a consumer that waits on
 * a second stream): the GEMM stores P with device-coherent stores and, for
 * every destination c != rank, counts the elements of P[c] it has stored; the
 * store that completes P[c] raises sig->dest_ready[c] to epoch.  On
 * send_stream, for c in send order (rank+1, rank+2, ..., rank-1 mod W), the
 * slice is then copied to send_dst[c] (the emulated peer's receive buffer,
 * R x N f32, 16-byte aligned; entry rank ignored) as soon as it is complete:
 *   send_land = TLC_LAND_MEMCPY or TLC_LAND_COPY_ENGINE: a one-wavefront gate
 *     kernel waits (bounded by timeout_ns; reports TIMEOUT) for dest_ready[c],
 *     then hipMemcpyAsync(send_dst[c], P[c]) of that kind;
 *   send_land = TLC_LAND_CU: one copy kernel whose workgroups wait for each
 *     slice in send order and copy it with load/store instructions.
 * Requirements for sends: R * N < 2^32, R * N * 4 < 2^32 for TLC_LAND_CU,
 * the GEMM leaves the CUs of a copy-stream landing free (grid limit below),
 * and the caller orders send_stream after earlier readers of send_dst and
 * later readers after it.  The GEMM is always enqueued before the gates.
 * Grid: the GEMM never waits, so by default it takes every compute unit and
 * the runtime's copies (MEMCPY and COPY_ENGINE landings and sends) share them.
 * A caller grid greater than (compute units - 32) is refused with INVALID_ARG
 * only with the CU landing or CU sends, whose copy kernels are sized for
 * compute units no GEMM workgroup holds. */
typedef struct {
  const tlc_tile* plan;
  int64_t n_tiles;
  int32_t M, N, K;
  int32_t world, rank, rows_per_chunk;
  int32_t bm, bn;
  const void* a;
  const void* b;
  int32_t b_layout;
  float* partials;
  const float* const* remote_src;
  float* const* landing;
  float* out;
  tlc_signals* sig;
  uint32_t epoch;
  int32_t land;
  int32_t grid;
  int64_t timeout_ns;
  void* workspace;         /* as in tlc_ag_args */
  int64_t workspace_bytes;
  int32_t schedule;
  float* const* send_dst;  /* host array of `world` device pointers, or NULL: no sends */
  int32_t send_land;       /* TLC_LAND_MEMCPY, TLC_LAND_COPY_ENGINE or TLC_LAND_CU */
  void* send_stream;       /* stream of the sends (NULL = the default stream) */
} tlc_rs_args;

tlc_status tlc_gemm_rs(const tlc_rs_args* args, void* compute_stream, void* const* copy_streams,
                       int32_t n_copy_streams);

/* The reduce step alone, on `compute_stream` (same arguments; neither the GEMM
 * nor the landing is run: landing[s] must hold the data, flags >= epoch). */
tlc_status tlc_rs_reduce(const tlc_rs_args* args, void* compute_stream);

/* --------------------------------------------------- GEMM-AllReduce ------ */

/* GEMM then all-reduce, one rank's share (DITRON §4: GEMM-AllReduce is one of
 * the tensor-parallel overlap kernels next to AG-GEMM and GEMM-RS), taken as
 * tlc_gemm_rs followed by an all-gather of the reduced slices:
 *   P = A @ B in scatter order (rs.plan: mode RS), as tlc_gemm_rs;
 *   C[rows of chunk rank] = sum over s in ascending s of S_s (tlc_gemm_rs's out);
 *   C[rows of chunk c], c != rank = gathered_src[c], the slice rank c reduced.
 * rs: the GEMM-RS arguments; rs.out is ignored (the reduce writes C's row
 *     chunk `rank`).
 * gathered_src: host array of `world` device pointers (R x N f32, 16-byte
 *     aligned); entry `rank` is ignored; may be NULL if rs.land == NONE (then C's
 *     other row chunks must already hold the slices).
 * c: device f32 M x N, ldc = N.
 * Requirements: those of tlc_gemm_rs, and 2 * world <= 32.  The peers' slices
 * land after the remote partials on the same copy streams and raise
 * flags[world + c].  With TLC_LAND_COLOCATED the reduce reads the remote
 * partials in place and the GEMM's first copy_wgs workgroups copy the slices
 * into C before their first unit.  Nothing inside the call waits for the
 * slices' flags: C is complete once the compute stream and the copy streams
 * have finished. */
typedef struct {
  tlc_rs_args rs;
  const float* const* gathered_src;
  float* c;
  int32_t copy_wgs; /* as in tlc_ag_args */
} tlc_ar_args;

tlc_status tlc_gemm_ar(const tlc_ar_args* args, void* compute_stream, void* const* copy_streams,
                       int32_t n_copy_streams);

/* ------------------------------------------------------------ AG-MoE ------ */

/* Routing for AG-MoE, on the device (DITRON §3.1 device level: chunk sizes
 * computed at run time for MoE routing; talk, "MoE dynamic sorting").
 * This is also the MoE mode of the tile planner: the readiness-ordered tile
 * list that tlc_chunk_plan gives on the host for dense GEMMs is built here on
 * the device, where the experts' row counts are known.
 * For T = world * tokens_per_chunk tokens and E experts:
 *   topk[T x k]  experts with the largest logits, largest first, equal logits
 *                -> lower expert index first;
 *   gates[T x k] softmax over the selected logits (f32);
 *   counts[E], offsets[E+1] (exclusive prefix sum);
 *   row_token[T*k]  token of every grouped-GEMM row, expert-major, inside an
 *                   expert ordered by (p(chunk of token), token) with
 *                   p(c) = (c - rank) mod world;
 *   slot[T x k]  the grouped-GEMM row of (token, j-th expert);
 *   plan, *n_tiles_dev: grouped-GEMM tiles (bm x bn over each expert's rows and
 *                N columns), ordered by (readiness, expert, m-tile, n-tile), with
 *                readiness = largest p of the tiles' tokens (0 in natural
 *                order); chunk_mask = chunks of the tile's tokens.
 * Limits: E <= 64 (one expert per lane of a wavefront), k <= E, k <= 16,
 * T <= 2^20, bm in {128, 256}.  plan_cap >= tlc_moe_plan_capacity(...).
 * All arrays are device memory; `workspace` is device memory of at least
 * tlc_moe_workspace_bytes(T, k, E, bm) bytes (contents need not be initialised;
 * the size depends on T and E only: T token masks and the per-expert counts of
 * the blocks of up to 16 tokens that each chunk is cut into).
 *
 * Optional co-located landing of the peers' token chunks (x_src != NULL):
 * extra workgroups of the routing's first (top-k) kernel, beside the routing's
 * own, copy chunk c (c != rank, tokens_per_chunk
 * x H bf16) from x_src[c] into rows [c Tc, (c+1) Tc) of x with load/store
 * instructions, a fixed number of workgroups per chunk, and the last of them
 * raises sig->flags[c] to `epoch` (AutoOverlap §5.3, backend 5, here beside
 * the routing rather than inside the GEMM).  The transfer then overlaps the
 * routing, which waits for nothing; the grouped GEMM that follows consumes the
 * chunks with land = TLC_LAND_NONE and the same epoch (tlc_ag_moe waits for
 * the raised flags).  x: device T x H bf16, 16-byte aligned; x_src: host array
 * of `world` device pointers, 16-byte aligned (entry `rank` unused); H >= 8,
 * H % 8 == 0, tokens_per_chunk * H * 2 < 2^32; sig non-NULL; epoch >= 1.  The
 * other landing fields are ignored when x_src is NULL. */
typedef struct {
  const float* logits; /* device f32 T x E */
  int32_t tokens_per_chunk, world, rank, experts, topk;
  int32_t N, bm, bn, order;
  int32_t* topk_idx;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* slot;
  tlc_tile* plan;
  int64_t plan_cap;
  int32_t* n_tiles_dev;
  void* workspace;
  void* x;                  /* co-located landing: gathered tokens (device) */
  const void* const* x_src; /* co-located landing: peers' chunks, or NULL */
  int32_t H;
  tlc_signals* sig;
  uint32_t epoch;
} tlc_moe_route_args;

int64_t tlc_moe_plan_capacity(int32_t T, int32_t topk, int32_t experts, int32_t N, int32_t bm,
                              int32_t bn);
int64_t tlc_moe_workspace_bytes(int32_t T, int32_t topk, int32_t experts, int32_t bm);
tlc_status tlc_moe_route(const tlc_moe_route_args* args, void* stream);

/* tlc_moe_route for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Identical
 * results; args->workspace is ignored (may be NULL) and the routing's
 * workspace is instead a static array in each device's memory, of
 * tlc_moe_static_workspace_bytes() bytes (4 MiB), which every call on that
 * device shares and which stays allocated until the process ends.  Nothing
 * is allocated: no hipMalloc, hipFree or allocating library call.  A problem
 * whose tlc_moe_workspace_bytes(...) exceeds the array is refused with
 * TLC_ERR_CAPACITY before anything is enqueued (e.g. T = 4096, k = 8,
 * E = 64, bm = 256 needs 104 KB).  The workspace needs no
 * initialisation, and each call leaves the last call's contents in it.
 * Calls that overlap in time on one device (on different streams, or from
 * different threads) race on the array; the caller orders them. */
tlc_status tlc_moe_route_static(const tlc_moe_route_args* args, void* stream);
int64_t tlc_moe_static_workspace_bytes(void);

/* Grouped GEMM of AG-MoE (DITRON §4.1 AG-MoE; Triton-Distributed talk, MoE
 * dynamic sorting: tiles in the order their tokens become ready; DITRON §3.1,
 * shapes known only on the device).
 * Y[(T*k) x N] (f32): Y[i] = X[row_token[i]] (bf16, 1 x H) @ W_e (bf16, H x N)
 * for the expert e whose row segment holds i.  X is the gathered token matrix
 * (T x H, chunk c = rows [c Tc, (c+1) Tc)); chunks land as in tlc_ag_gemm.
 * w: device bf16, E stacked matrices, layout w_layout (KN: E x H x N; NK:
 * E x N x H).  Tiles come from tlc_moe_route (plan, n_tiles_dev).  With
 * land = TLC_LAND_NONE and epoch >= 1 nothing is landed here but the tiles
 * still wait for their chunks' flags: chunks landed by tlc_moe_route's
 * co-located landing (or by the caller), with that epoch.
 * Requirements: H % 64 == 0, N % 8 == 0, 16-byte aligned pointers.
 * grid (0 = every compute unit the landing leaves free): with H / 64 even the
 * GEMM's workgroups leave room on their CUs for the runtime's copy and
 * flag-transfer kernels, so beside a MEMCPY or COPY_ENGINE landing they take
 * every CU; a grid above (compute units - 32) is refused with INVALID_ARG with
 * the CU landing, and with any copy-stream landing when H / 64 is odd (that
 * GEMM kernel fills its CUs while it waits on flags). */
typedef struct {
  const tlc_tile* plan;
  const int32_t* n_tiles_dev;
  int64_t plan_cap;
  const int32_t* row_token;
  int32_t tokens_per_chunk, world, rank, experts, topk;
  int32_t H, N;
  int32_t bm, bn;
  void* x;
  const void* const* x_src;
  const void* w;
  int32_t w_layout;
  float* y;
  tlc_signals* sig;
  uint32_t epoch;
  int32_t land;
  int32_t grid;
  int64_t timeout_ns;
  int32_t schedule; /* TLC_SCHED_* as in tlc_ag_args (MoE tiles are never split;
                       TLC_SCHED_STREAMK runs as TLC_SCHED_STATIC: the unit count
                       is known only on the device) */
  int32_t copy_wgs; /* as in tlc_ag_args */
} tlc_moe_args;

tlc_status tlc_ag_moe(const tlc_moe_args* args, void* compute_stream, void* const* copy_streams,
                      int32_t n_copy_streams);

/* ------------------------------------------------------------ misc -------- */

/* Land the peers' chunks only (the copy side of tlc_ag_gemm / tlc_gemm_rs,
 * no GEMM; the landing order is DITRON §3.2's rank-offset order; the call by
 * itself is not a page operation but the copy-only leg of the overlap
 * measurement): for c in landing order (rank+1, ..., rank-1 mod W) copies
 * `bytes_per_chunk` bytes from src[c] to dst[c] and then raises
 * sig->flags[c] to epoch.  dst, src: host arrays of `world` device pointers,
 * 16-byte aligned; entries `rank` are ignored.  bytes_per_chunk % 16 == 0.
 * land: TLC_LAND_COPY_ENGINE, TLC_LAND_CU, TLC_LAND_MEMCPY, or TLC_LAND_COLOCATED
 * (the co-located copy work alone: the GEMM kernel with no units, its default
 * number of copying workgroups, on copy_streams[0]).  Used for copy-only
 * timings. */
tlc_status tlc_land(void* const* dst, const void* const* src, int64_t bytes_per_chunk,
                    int32_t world, int32_t rank, tlc_signals* sig, uint32_t epoch, int32_t land,
                    void* const* copy_streams, int32_t n_copy_streams);

/* Rate in kHz of the device clock that timeouts and the debug traces count in
 * (hipDeviceAttributeWallClockRate of the current device); 0 if it cannot be
 * queried.  Not from the pages; neither are the three calls below. */
int64_t tlc_wall_clock_khz(void);

const char* tlc_status_string(tlc_status s);
const char* tlc_last_error(void);
/* Library version, e.g. 132 = 0.1.32. */
int32_t tlc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TLC_H */
