// libtlc entry points: argument validation, landing enqueue, kernel launches.
// See include/tlc.h for the contract of every function.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "tlc_internal.h"

namespace tlc {

namespace {
thread_local char g_err[512] = "";
std::mutex g_info_mu;
DeviceInfo g_info[64];
bool g_info_ok[64] = {};
// CUs the persistent GEMM leaves free while it may wait for landings.  The
// landing's kernels -- the CU copy kernel, or on the copy-engine path the
// runtime's kernel for each 4-byte flag transfer (1024-thread workgroups) --
// have to find CUs that no GEMM workgroup holds while those workgroups spin
// (a workgroup of the 8-wavefront core takes all the registers of its CU).
// With fewer than one free CU per shader engine (8 XCDs x 4) their placement
// stalled now and then until the wait timed out, even when the landing kernel
// was dispatched first.  A GEMM that never waits (scatter mode) needs no such
// reserve for the runtime's copies.
constexpr int kReserveCUsLandCU = 32;
constexpr int kReserveCUsCopyEngine = 32;
// The compute units of the largest gfx950 part: a caller grid is checked
// against it on the host before any device query, then against the device's
// own count.
constexpr int kMaxCUs = 256;
// Workgroups of the CU send kernel (scatter mode): they hold their CUs while
// they wait for the slices, so they stay within the reserved ones.
constexpr int kSendCUWorkgroups = 16;
constexpr int64_t kDefaultTimeoutNs = 2000000000LL;
}  // namespace

tlc_status fail(tlc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

tlc_status ok() {
  g_err[0] = '\0';
  return TLC_OK;
}

tlc_status device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(TLC_ERR_UNSUPPORTED, "device id %d", dev);
  std::lock_guard<std::mutex> lk(g_info_mu);
  if (!g_info_ok[dev]) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(TLC_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    DeviceInfo info;
    info.cus = prop.multiProcessorCount;
    int khz = 0;
    e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    info.wall_khz = (e == hipSuccess && khz > 0) ? khz : 100000;
    info.arch_ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_info[dev] = info;
    g_info_ok[dev] = true;
  }
  *out = g_info[dev];
  if (!out->arch_ok) return fail(TLC_ERR_UNSUPPORTED, "libtlc kernels are built for gfx950 only");
  return TLC_OK;
}

int reserve_for(int land) {
  return (land == TLC_LAND_COPY_ENGINE || land == TLC_LAND_MEMCPY) ? kReserveCUsCopyEngine
                                      : (land == TLC_LAND_CU ? kReserveCUsLandCU : 0);
}

int default_grid(int64_t n_tiles, int avail) {
  if (n_tiles <= 0 || avail <= 0) return 1;
  const int64_t rounds = (n_tiles + avail - 1) / avail;
  int64_t g = (n_tiles + rounds - 1) / rounds;
  g = ((g + 7) / 8) * 8;
  if (g > avail) g = avail;
  return static_cast<int>(g);
}

}  // namespace tlc

using namespace tlc;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ticks_for(int64_t ns, const DeviceInfo& info) {
  if (ns <= 0) ns = kDefaultTimeoutNs;
  return ns / 1000 * info.wall_khz / 1000 + 1;
}

tlc_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TLC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return TLC_OK;
}

// Enqueue the emulated peers' chunk transfers on `copy` in landing order
// (rank+n_local, rank+n_local+1, ... mod W: the n_local chunks from `rank` on
// are already in place) and raise each chunk's flag to `epoch` after its bytes.
tlc_status enqueue_landing(int land, void* const* dst, const void* const* src, int64_t bytes,
                           int world, int rank, int n_local, tlc_signals* sig, uint32_t epoch,
                           void* const* copy_streams, int n_copy_streams, const DeviceInfo& info,
                           int flag_base = 0) {
  // the co-located landing is carried out by the GEMM kernel itself
  if (land == TLC_LAND_NONE || land == TLC_LAND_COLOCATED || world <= n_local) return TLC_OK;
  if (land == TLC_LAND_COPY_ENGINE || land == TLC_LAND_MEMCPY) {
    const hipMemcpyKind kind =
        land == TLC_LAND_COPY_ENGINE ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
    for (int i = n_local; i < world; ++i) {
      const int c = (rank + i) % world;
      hipStream_t s = static_cast<hipStream_t>(copy_streams[(i - n_local) % n_copy_streams]);
      tlc_status st = hip_check(hipMemcpyAsync(dst[c], src[c], static_cast<size_t>(bytes), kind, s),
                                "hipMemcpyAsync(landing)");
      if (st) return st;
      // the flag follows the data on the same copy engine queue
      st = hip_check(hipMemcpyAsync(&sig->flags[flag_base + c], &sig->epoch_table[epoch - 1],
                                    sizeof(uint32_t), kind, s),
                     "hipMemcpyAsync(flag)");
      if (st) return st;
    }
    return TLC_OK;
  }
  LandParams p;
  memset(&p, 0, sizeof(p));
  p.n_chunks = world - n_local;
  for (int i = n_local; i < world; ++i) {
    const int c = (rank + i) % world;
    p.order[i - n_local] = c;
    p.src[c] = static_cast<const uint4*>(src[c]);
    p.dst[c] = static_cast<uint4*>(dst[c]);
  }
  p.vec_per_chunk = bytes / 16;
  p.sig = sig;
  p.epoch = epoch;
  p.flag_base = flag_base;
  // one 1024-thread workgroup per CU the GEMM leaves free (a CU that holds a
  // landing workgroup cannot also hold a GEMM workgroup: those take all of a
  // CU's registers)
  const int grid = kReserveCUsLandCU;
  return launch_land_cu(p, grid, copy_streams[0]);
}

tlc_status check_land_args(int land, const void* const* src, const void* const* dst, int world,
                           int rank, int64_t bytes, const char* who, void* const* copy_streams,
                           int n_copy_streams, uint32_t epoch, int n_local = 1) {
  if (land != TLC_LAND_NONE && land != TLC_LAND_COPY_ENGINE && land != TLC_LAND_CU &&
      land != TLC_LAND_MEMCPY && land != TLC_LAND_COLOCATED)
    return fail(TLC_ERR_INVALID_ARG, "%s: land %d unknown", who, land);
  if (land == TLC_LAND_NONE) return TLC_OK;
  if (land == TLC_LAND_COLOCATED) {
    if (epoch < 1) return fail(TLC_ERR_INVALID_ARG, "%s: co-located landing needs epoch >= 1", who);
  } else if (!copy_streams || n_copy_streams < 1) {
    return fail(TLC_ERR_INVALID_ARG, "%s: landing needs n_copy_streams >= 1 streams", who);
  }
  if ((land == TLC_LAND_COPY_ENGINE || land == TLC_LAND_MEMCPY) && (epoch < 1 || epoch > TLC_EPOCH_MAX))
    return fail(TLC_ERR_INVALID_ARG, "%s: copy-engine landing needs 1 <= epoch <= %d (got %u)", who,
                TLC_EPOCH_MAX, epoch);
  if (!src || !dst) return fail(TLC_ERR_INVALID_ARG, "%s: landing needs source and destination arrays", who);
  if (bytes % 16 != 0) return fail(TLC_ERR_MISALIGNED, "%s: chunk bytes %lld not a multiple of 16", who,
                                   static_cast<long long>(bytes));
  // the CU and co-located copies address a chunk with 32-bit buffer offsets
  if ((land == TLC_LAND_CU || land == TLC_LAND_COLOCATED) && bytes >= (1LL << 32))
    return fail(TLC_ERR_UNSUPPORTED, "%s: chunk of %lld bytes (the CU copies take < 4 GiB)", who,
                static_cast<long long>(bytes));
  for (int c = 0; c < world; ++c) {
    if ((c - rank + world) % world < n_local) continue;
    if (!src[c] || !dst[c]) return fail(TLC_ERR_INVALID_ARG, "%s: chunk %d pointer is NULL", who, c);
    if (!aligned16(src[c]) || !aligned16(dst[c]))
      return fail(TLC_ERR_MISALIGNED, "%s: chunk %d pointer not 16-byte aligned", who, c);
  }
  return TLC_OK;
}

tlc_status check_dense(const char* who, int32_t M, int32_t N, int32_t K, int32_t world, int32_t rank,
                       int32_t R, int32_t bm, int32_t bn, int32_t b_layout, const tlc_tile* plan,
                       int64_t n_tiles, const void* a, const void* b, const void* c,
                       const tlc_signals* sig) {
  if (world < 1 || world > TLC_MAX_WORLD) return fail(TLC_ERR_INVALID_ARG, "%s: world %d", who, world);
  if (rank < 0 || rank >= world) return fail(TLC_ERR_INVALID_ARG, "%s: rank %d", who, rank);
  if (M < 1 || N < 1 || K < 1 || R < 1) return fail(TLC_ERR_INVALID_ARG, "%s: sizes must be >= 1", who);
  if (static_cast<int64_t>(world) * R != M)
    return fail(TLC_ERR_INVALID_ARG, "%s: M %d != world %d * rows_per_chunk %d", who, M, world, R);
  if (K % 64 != 0) return fail(TLC_ERR_UNSUPPORTED, "%s: K %d is not a multiple of 64", who, K);
  if (N % 8 != 0) return fail(TLC_ERR_UNSUPPORTED, "%s: N %d is not a multiple of 8", who, N);
  if (!((bm == 256 && bn == 256) || (bm == 128 && bn == 128)))
    return fail(TLC_ERR_UNSUPPORTED, "%s: tile %dx%d not built (256x256, 128x128)", who, bm, bn);
  if (b_layout != TLC_B_KN && b_layout != TLC_B_NK)
    return fail(TLC_ERR_INVALID_ARG, "%s: b_layout %d", who, b_layout);
  if (static_cast<int64_t>(M) * K >= (1LL << 31) || static_cast<int64_t>(K) * N >= (1LL << 31))
    return fail(TLC_ERR_UNSUPPORTED, "%s: operand with >= 2^31 elements", who);
  if (n_tiles < 0) return fail(TLC_ERR_INVALID_ARG, "%s: n_tiles < 0", who);
  if ((n_tiles > 0 && !plan) || !a || !b || !c || !sig)
    return fail(TLC_ERR_INVALID_ARG, "%s: NULL plan, operand, output or signals", who);
  if (!aligned16(a) || !aligned16(b) || !aligned16(c))
    return fail(TLC_ERR_MISALIGNED, "%s: operands must be 16-byte aligned", who);
  return TLC_OK;
}

// Work distribution and split-tile workspace of one GEMM launch: checked with
// the other arguments, applied when the launch parameters are filled in.
tlc_status check_schedule(int32_t schedule, const void* ws, int64_t ws_bytes, const char* who) {
  if (schedule != TLC_SCHED_DYNAMIC && schedule != TLC_SCHED_STATIC && schedule != TLC_SCHED_STREAMK)
    return fail(TLC_ERR_INVALID_ARG, "%s: schedule %d unknown", who, schedule);
  if (ws_bytes < 0 || (ws_bytes > 0 && !ws))
    return fail(TLC_ERR_INVALID_ARG, "%s: workspace NULL with %lld bytes", who,
                static_cast<long long>(ws_bytes));
  if (ws && reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(TLC_ERR_MISALIGNED, "%s: workspace not 256-byte aligned", who);
  return TLC_OK;
}

void set_schedule(GemmParams* p, int32_t schedule, void* ws, int64_t ws_bytes) {
  p->dynamic = schedule == TLC_SCHED_DYNAMIC;
  // stream-K: the workspace serves the tail (configure_tail), not split tiles
  const bool sk = schedule == TLC_SCHED_STREAMK;
  p->split_ws = sk ? nullptr : static_cast<char*>(ws);
  p->split_bytes = (ws && !sk) ? ws_bytes : 0;
}

// The most K steps one of G static slots runs when the t_sk tail tiles are
// split into S pieces (piece s of tile j is item s * t_sk + j, slot item % G).
int64_t tail_cost(int64_t t_sk, int64_t G, int KT, int S) {
  std::vector<int64_t> per(static_cast<size_t>(G), 0);
  for (int64_t q = 0; q < S * t_sk; ++q) {
    const int sp = static_cast<int>(q / t_sk);
    per[static_cast<size_t>(q % G)] += (((sp + 1) * KT / S) & ~1) - ((sp * KT / S) & ~1);
  }
  return *std::max_element(per.begin(), per.end());
}

// Stream-K tail (TLC_SCHED_STREAMK) for a launch of `grid` workgroups: the
// first floor(T / G) * G units whole, then each remaining tile in S pieces
// along K (2 <= S <= kSkMaxSplit, at least two K steps each), S chosen so
// that the slot with the most tail steps has the fewest, counting two steps
// of fix-up per extra piece; no tail unless that beats a round of whole
// tiles.  Only the kernel that runs whole 256 x 256 tiles has the tail;
// without it, or when the units fill the grid evenly, the schedule stays
// static.
tlc_status configure_tail(GemmParams* p, int32_t schedule, void* ws, int64_t ws_bytes, int grid,
                          int bm, int bn, int kind, const char* who) {
  p->sk_split = 0;
  if (schedule != TLC_SCHED_STREAMK || grid < 1 || p->n_tiles <= 0) return TLC_OK;
  const int KT = p->K / 64;
  const bool whole_tile_kernel = kind != KIND_MOE && bm == 256 && bn == 256 && p->M % 256 == 0 &&
                                 p->K % 64 == 0 && KT % 2 == 0 && p->split_bytes == 0;
  if (!whole_tile_kernel) return TLC_OK;
  const int64_t T = p->n_tiles, G = grid;
  const int64_t t_dp = T / G * G, t_sk = T - t_dp;
  if (t_sk == 0) return TLC_OK;
  int best = 0;
  int64_t best_cost = KT;
  for (int S = 2; S <= kSkMaxSplit && 2 * S <= KT; ++S) {
    const int64_t cost = tail_cost(t_sk, G, KT, S) + 2 * (S - 1);
    if (cost < best_cost) {
      best = S;
      best_cost = cost;
    }
  }
  if (best == 0) return TLC_OK;
  const int64_t need = t_sk * kSkBlockBytes;
  if (!ws || ws_bytes < need)
    return fail(TLC_ERR_INVALID_ARG, "%s: the stream-K tail of %lld tiles on %d workgroups needs a "
                "workspace of %lld bytes (tlc_streamk_workspace_bytes), got %lld", who,
                static_cast<long long>(t_sk), grid, static_cast<long long>(need),
                static_cast<long long>(ws ? ws_bytes : 0));
  p->sk_from = t_dp;
  p->sk_tiles = static_cast<int32_t>(t_sk);
  p->sk_split = best;
  p->sk_ws = static_cast<char*>(ws);
  return TLC_OK;
}

// Co-located landing: the chunks in landing order (rank+n_local, ... mod W)
// and the number of workgroups that copy them.  Default: the workgroups that
// the last round of units leaves idle anyway (rounds * grid - n_units, a
// multiple of 8); when that is under 32 the copy is on the critical path
// whoever does it, and every workgroup takes a share; a quarter of the grid
// when the unit count is only known on the device (n_units < 0).
// The peers' chunks in landing order (rank+n_local, ... mod world; the n_local
// chunks from `rank` on are already in place), chunk c raising flags[flag_base + c].
void fill_copy_chunks(CopyPlan* cp, void* const* dst, const void* const* src, int64_t bytes,
                      int world, int rank, int n_local, int flag_base) {
  cp->chunks = world - n_local;
  cp->vec = bytes / 16;
  for (int i = n_local; i < world; ++i) {
    const int c = (rank + i) % world;
    cp->src[i - n_local] = static_cast<const uint4*>(src[c]);
    cp->dst[i - n_local] = static_cast<uint4*>(dst[c]);
    cp->flag[i - n_local] = flag_base + c;
  }
}

// The copying workgroups have the lowest ids, so the dispatcher makes them
// resident first; they wait for nothing before they copy, and the workgroups
// that wait on their flags are dispatched after them.  That holds only while
// every copying workgroup can be resident at the same time: at most one
// 256 x 256 GEMM workgroup fits a compute unit (its LDS stages alone take 128
// KB), so copy_wgs is limited to the compute units (`resident`); more could
// leave copying workgroups waiting for compute units that workgroups spinning
// on their flags hold, until the wait times out.
tlc_status set_colocated(GemmParams* p, void* const* dst, const void* const* src, int64_t bytes,
                         int world, int rank, int n_local, int copy_wgs, int grid, int resident,
                         const char* who, int flag_base = 0, int64_t n_units = -1) {
  if (copy_wgs < 0 || copy_wgs > grid)
    return fail(TLC_ERR_INVALID_ARG, "%s: copy_wgs %d outside 0..grid %d", who, copy_wgs, grid);
  int cw = copy_wgs;
  if (cw == 0) {
    if (n_units >= 0) {
      const int64_t rounds = (n_units + grid - 1) / grid;
      cw = static_cast<int>((rounds * grid - n_units) / 8 * 8);
      if (cw < 32) cw = grid;
    } else {
      cw = grid / 4 / 8 * 8;
      if (cw < 8) cw = grid < 8 ? grid : 8;
    }
  }
  p->copy.wgs = world > n_local ? cw : 0;
  if (p->copy.wgs > resident)
    return fail(TLC_ERR_INVALID_ARG, "%s: %d co-located copying workgroups, more than the %d that "
                "can be resident at once (one per compute unit): pass copy_wgs <= %d, or a grid "
                "of at most %d", who, p->copy.wgs, resident, resident, resident);
  fill_copy_chunks(&p->copy, dst, src, bytes, world, rank, n_local, flag_base);
  // a workgroup's share is addressed with 32-bit byte offsets
  if (p->copy.wgs > 0 && (p->copy.vec + p->copy.wgs - 1) / p->copy.wgs >= (int64_t{1} << 27))
    return fail(TLC_ERR_UNSUPPORTED, "%s: co-located share of a %lld-byte chunk over %d workgroups "
                "exceeds 2 GiB", who, static_cast<long long>(bytes), p->copy.wgs);
  return TLC_OK;
}

// A caller grid must leave the reserved CUs free whenever kernels on other
// streams (a copy-stream landing, the scatter mode's sends) need them while
// the GEMM runs: checked against the largest part before any device call,
// and against the device's own count once it is known (cus > 0).
tlc_status check_grid(int grid, int reserve, int cus, const char* who) {
  if (grid < 0) return fail(TLC_ERR_INVALID_ARG, "%s: grid %d < 0", who, grid);
  if (reserve <= 0 || grid == 0) return TLC_OK;
  const int limit = (cus > 0 ? cus : kMaxCUs) - reserve;
  if (grid > limit)
    return fail(TLC_ERR_INVALID_ARG,
                "%s: grid %d leaves fewer than %d compute units free for the landing or send "
                "kernels (at most %d workgroups)", who, grid, reserve, limit);
  return TLC_OK;
}

// Persistent grid: every CU left free (dynamic: no more workgroups than
// units; stream-K: every CU, the tail spreads the last tiles over them), or
// the evenly spread static default.
int pick_grid(int requested, int32_t schedule, int64_t n_units, int avail) {
  if (requested > 0) return requested;
  if (avail < 1) avail = 1;
  if (schedule == TLC_SCHED_DYNAMIC)
    return static_cast<int>(n_units < avail ? (n_units > 0 ? n_units : 1) : avail);
  if (schedule == TLC_SCHED_STREAMK) return avail;
  return default_grid(n_units, avail);
}

}  // namespace

extern "C" {

tlc_status tlc_signals_alloc(tlc_signals** out) {
  if (!out) return fail(TLC_ERR_INVALID_ARG, "tlc_signals_alloc: NULL out");
  void* p = nullptr;
  tlc_status st = hip_check(hipExtMallocWithFlags(&p, sizeof(tlc_signals), hipDeviceMallocFinegrained),
                            "hipExtMallocWithFlags(fine-grained)");
  if (st) return st;
  st = hip_check(hipMemset(p, 0, sizeof(tlc_signals)), "hipMemset(signals)");
  if (!st) {
    static uint32_t table[TLC_EPOCH_MAX];
    for (uint32_t i = 0; i < TLC_EPOCH_MAX; ++i) table[i] = i + 1;
    st = hip_check(hipMemcpy(static_cast<tlc_signals*>(p)->epoch_table, table, sizeof(table),
                             hipMemcpyHostToDevice),
                   "hipMemcpy(epoch table)");
  }
  if (st) {
    (void)hipFree(p);
    return st;
  }
  st = hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");
  if (st) return st;
  *out = static_cast<tlc_signals*>(p);
  return ok();
}

tlc_status tlc_signals_free(tlc_signals* sig) {
  if (!sig) return ok();
  tlc_status st = hip_check(hipFree(sig), "hipFree(signals)");
  return st ? st : ok();
}

tlc_status tlc_signals_set(tlc_signals* sig, int32_t world, uint32_t value, void* stream) {
  if (!sig || world < 1 || world > TLC_MAX_WORLD)
    return fail(TLC_ERR_INVALID_ARG, "tlc_signals_set: bad arguments");
  tlc_status st = launch_signals_set(sig, world, value, stream);
  return st ? st : ok();
}

tlc_status tlc_signals_rewind(tlc_signals* sig, void* stream) {
  if (!sig) return fail(TLC_ERR_INVALID_ARG, "tlc_signals_rewind: NULL");
  tlc_status st = launch_signals_rewind(sig, stream);
  return st ? st : ok();
}

tlc_status tlc_signals_clear_status(tlc_signals* sig, void* stream) {
  if (!sig) return fail(TLC_ERR_INVALID_ARG, "tlc_signals_clear_status: NULL");
  tlc_status st = launch_status_clear(sig, stream);
  return st ? st : ok();
}

tlc_status tlc_read_status(const tlc_signals* sig, void* stream, int32_t* out) {
  if (!sig || !out) return fail(TLC_ERR_INVALID_ARG, "tlc_read_status: NULL");
  tlc_status st = hip_check(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize");
  if (st) return st;
  st = hip_check(hipMemcpy(out, sig->status, 4 * sizeof(int32_t), hipMemcpyDeviceToHost), "hipMemcpy(status)");
  return st ? st : ok();
}

tlc_status tlc_read_signals(const tlc_signals* sig, void* stream, tlc_signals* out) {
  if (!sig || !out) return fail(TLC_ERR_INVALID_ARG, "tlc_read_signals: NULL");
  tlc_status st = hip_check(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize");
  if (st) return st;
  st = hip_check(hipMemcpy(out, sig, sizeof(tlc_signals), hipMemcpyDeviceToHost), "hipMemcpy(signals)");
  return st ? st : ok();
}

tlc_status tlc_land(void* const* dst, const void* const* src, int64_t bytes_per_chunk, int32_t world,
                    int32_t rank, tlc_signals* sig, uint32_t epoch, int32_t land,
                    void* const* copy_streams, int32_t n_copy_streams) {
  if (world < 1 || world > TLC_MAX_WORLD || rank < 0 || rank >= world || !sig || bytes_per_chunk < 0)
    return fail(TLC_ERR_INVALID_ARG, "tlc_land: bad world/rank/signals/size");
  if (land == TLC_LAND_NONE) return fail(TLC_ERR_INVALID_ARG, "tlc_land: land must not be NONE");
  tlc_status st = check_land_args(land, src, dst, world, rank, bytes_per_chunk, "tlc_land",
                                  copy_streams, n_copy_streams, epoch);
  if (st) return st;
  DeviceInfo info;
  st = device_info(&info);
  if (st) return st;
  if (land == TLC_LAND_COLOCATED) {
    if (world < 2) return ok();
    // the GEMM kernel with no units: only its copying workgroups do work
    GemmParams p;
    memset(&p, 0, sizeof(p));
    p.do_wait = 1;
    p.sig = sig;
    p.epoch = epoch;
    st = set_colocated(&p, dst, src, bytes_per_chunk, world, rank, 1, 0, info.cus, info.cus,
                       "tlc_land");
    if (st) return st;
    st = launch_gemm(p, 256, 256, TLC_B_KN, KIND_DENSE, p.copy.wgs,
                     copy_streams && n_copy_streams > 0 ? copy_streams[0] : nullptr);
    return st ? st : ok();
  }
  st = enqueue_landing(land, dst, src, bytes_per_chunk, world, rank, 1, sig, epoch, copy_streams,
                       n_copy_streams, info);
  return st ? st : ok();
}

tlc_status tlc_ag_gemm(const tlc_ag_args* a, void* compute_stream, void* const* copy_streams,
                       int32_t n_copy_streams) {
  if (!a) return fail(TLC_ERR_INVALID_ARG, "tlc_ag_gemm: NULL args");
  tlc_status st = check_dense("tlc_ag_gemm", a->M, a->N, a->K, a->world, a->rank, a->rows_per_chunk,
                              a->bm, a->bn, a->b_layout, a->plan, a->n_tiles, a->a, a->b, a->c, a->sig);
  if (st) return st;
  st = check_schedule(a->schedule, a->workspace, a->workspace_bytes, "tlc_ag_gemm");
  if (st) return st;
  // Sub-chunks: each rank's chunk lands and is flagged as S pieces of R/S rows,
  // so W*S flags, the local rank's S pieces never waited for.
  const int S = a->sub_chunks > 1 ? a->sub_chunks : 1;
  if (a->sub_chunks < 0 || a->rows_per_chunk % S != 0 ||
      static_cast<int64_t>(a->world) * S > TLC_MAX_WORLD)
    return fail(TLC_ERR_INVALID_ARG, "tlc_ag_gemm: sub_chunks %d (rows_per_chunk %% S, world * S <= %d)",
                a->sub_chunks, TLC_MAX_WORLD);
  if (a->land != TLC_LAND_NONE && a->world > 1 && !a->a_src)
    return fail(TLC_ERR_INVALID_ARG, "tlc_ag_gemm: landing needs source and destination arrays");
  const int Wf = a->world * S, rf = a->rank * S;
  const int64_t chunk_bytes = static_cast<int64_t>(a->rows_per_chunk / S) * a->K * 2;
  void* dst[TLC_MAX_WORLD];
  const void* src[TLC_MAX_WORLD];
  for (int c = 0; c < Wf; ++c) {
    dst[c] = static_cast<char*>(a->a) + c * chunk_bytes;
    const int owner = c / S;
    const void* base = a->a_src ? a->a_src[owner] : nullptr;
    src[c] = (base && owner != a->rank) ? static_cast<const char*>(base) + (c % S) * chunk_bytes
                                        : nullptr;
  }
  st = check_land_args(a->land, src, dst, Wf, rf, chunk_bytes, "tlc_ag_gemm", copy_streams,
                       n_copy_streams, a->epoch, S);
  if (st) return st;
  st = check_grid(a->grid, Wf > S ? reserve_for(a->land) : 0, 0, "tlc_ag_gemm");
  if (st) return st;
  DeviceInfo info;
  st = device_info(&info);
  if (st) return st;
  st = check_grid(a->grid, Wf > S ? reserve_for(a->land) : 0, info.cus, "tlc_ag_gemm");
  if (st) return st;

  // The producer is always enqueued before the consumer: two streams may share
  // one hardware queue, and a GEMM queued ahead of its own landing there would
  // wait on flags that can never be raised.
  st = enqueue_landing(a->land, dst, src, chunk_bytes, Wf, rf, S, a->sig, a->epoch, copy_streams,
                       n_copy_streams, info);
  if (st) return st;
  const bool coloc = a->land == TLC_LAND_COLOCATED && Wf > S;
  if (a->n_tiles == 0 && !coloc) return ok();

  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.plan = a->plan;
  p.n_tiles = a->n_tiles;
  p.a = static_cast<const uint16_t*>(a->a);
  p.b = static_cast<const uint16_t*>(a->b);
  p.c = a->c;
  p.M = a->M;
  p.N = a->N;
  p.K = a->K;
  p.lda = a->K;
  p.ldb = a->b_layout == TLC_B_NK ? a->K : a->N;
  p.ldc = a->N;
  p.no_wait_mask = ((S == 32 ? 0u : (1u << S)) - 1u) << rf;
  // land == NONE with epoch 0: every chunk is resident, nothing to wait for
  p.do_wait = !(a->land == TLC_LAND_NONE && a->epoch == 0);
  p.sig = a->sig;
  p.epoch = a->epoch;
  p.timeout_ticks = ticks_for(a->timeout_ns, info);
  p.trace = a->trace;
  set_schedule(&p, a->schedule, a->workspace, a->workspace_bytes);
  const int avail = info.cus - (p.do_wait ? reserve_for(a->land) : 0);
  // no units (copy-only run of the co-located landing): one workgroup per
  // copying workgroup of a full grid
  int grid = a->n_tiles > 0 ? pick_grid(a->grid, a->schedule, a->n_tiles, avail)
                            : (a->grid > 0 ? a->grid : avail);
  if (coloc) {
    st = set_colocated(&p, dst, src, chunk_bytes, Wf, rf, S, a->copy_wgs, grid, info.cus,
                       "tlc_ag_gemm", 0,
                       a->n_tiles);
    if (st) return st;
    if (a->n_tiles == 0) grid = p.copy.wgs;
  }
  st = configure_tail(&p, a->schedule, a->workspace, a->workspace_bytes, grid, a->bm, a->bn,
                      KIND_DENSE, "tlc_ag_gemm");
  if (st) return st;
  p.xcd_remap = grid % 8 == 0;
  st = launch_gemm(p, a->bm, a->bn, a->b_layout, KIND_DENSE, grid, compute_stream);
  return st ? st : ok();
}

// The all-gather half of GEMM-AllReduce: the peers' reduced slices, landed
// into the output's other row chunks after the remote partials.
struct GatherPart {
  void* dst[TLC_MAX_WORLD];
  const void* src[TLC_MAX_WORLD];
  int32_t copy_wgs;
};

// The outgoing slices P[c], c != rank, in send order (rank+1, ..., rank-1 mod
// W), each once the GEMM has raised its ready flag.  With no tiles in the
// plan nothing would raise the flags: the slices are then sent as they are.
static tlc_status enqueue_sends(const tlc_rs_args* a, int64_t slice, const DeviceInfo& info) {
  const int64_t ticks = ticks_for(a->timeout_ns, info);
  hipStream_t s = static_cast<hipStream_t>(a->send_stream);
  if (a->send_land == TLC_LAND_CU) {
    SendParams sp;
    memset(&sp, 0, sizeof(sp));
    for (int i = 1; i < a->world; ++i) {
      const int c = (a->rank + i) % a->world;
      sp.order[i - 1] = c;
      sp.src[c] = reinterpret_cast<const uint4*>(a->partials + c * slice);
      sp.dst[c] = reinterpret_cast<uint4*>(a->send_dst[c]);
    }
    sp.n = a->world - 1;
    sp.vec_per_slice = slice / 4;
    sp.sig = a->sig;
    sp.epoch = a->epoch;
    sp.timeout_ticks = ticks;
    return launch_send_cu(sp, kSendCUWorkgroups, s);
  }
  const hipMemcpyKind kind =
      a->send_land == TLC_LAND_COPY_ENGINE ? hipMemcpyDeviceToDeviceNoCU : hipMemcpyDeviceToDevice;
  for (int i = 1; i < a->world; ++i) {
    const int c = (a->rank + i) % a->world;
    if (a->n_tiles > 0) {
      tlc_status st = launch_send_gate(a->sig, c, a->epoch, ticks, s);
      if (st) return st;
    }
    tlc_status st = hip_check(hipMemcpyAsync(a->send_dst[c], a->partials + c * slice,
                                             static_cast<size_t>(slice) * 4, kind, s),
                              "hipMemcpyAsync(send)");
    if (st) return st;
  }
  return TLC_OK;
}

static tlc_status rs_common(const tlc_rs_args* a, void* compute_stream, void* const* copy_streams,
                            int n_copy_streams, bool run_gemm, const GatherPart* g = nullptr) {
  if (!a) return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: NULL args");
  tlc_status st = check_dense("tlc_gemm_rs", a->M, a->N, a->K, a->world, a->rank, a->rows_per_chunk,
                              a->bm, a->bn, a->b_layout, a->plan, a->n_tiles, a->a, a->b,
                              a->partials, a->sig);
  if (st) return st;
  st = check_schedule(a->schedule, a->workspace, a->workspace_bytes, "tlc_gemm_rs");
  if (st) return st;
  if (a->N % 4 != 0) return fail(TLC_ERR_UNSUPPORTED, "tlc_gemm_rs: N %% 4 != 0");
  if (!a->out || !aligned16(a->out)) return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: out NULL or misaligned");
  const int64_t slice = static_cast<int64_t>(a->rows_per_chunk) * a->N;
  const int64_t slice_bytes = slice * 4;
  const int land = run_gemm ? a->land : TLC_LAND_NONE;
  // co-located: the reduce reads the peers' partials where they are
  const bool coloc = land == TLC_LAND_COLOCATED;
  const float* const* peer = coloc ? a->remote_src : a->landing;
  if (a->world > 1 && !peer)
    return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: NULL %s array", coloc ? "remote_src" : "landing");
  for (int s = 0; s < a->world; ++s) {
    if (s == a->rank) continue;
    if (!peer[s] || !aligned16(peer[s]))
      return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: %s[%d] NULL or misaligned",
                  coloc ? "remote_src" : "landing", s);
  }
  if (coloc && a->epoch < 1)
    return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: co-located landing needs epoch >= 1");
  if (!coloc) {
    st = check_land_args(land, reinterpret_cast<const void* const*>(a->remote_src),
                         reinterpret_cast<const void* const*>(a->landing), a->world, a->rank,
                         slice_bytes, "tlc_gemm_rs", copy_streams, n_copy_streams, a->epoch);
    if (st) return st;
  }
  if (g) {
    st = check_land_args(land, g->src, g->dst, a->world, a->rank, slice_bytes, "tlc_gemm_ar",
                         copy_streams, n_copy_streams, a->epoch);
    if (st) return st;
  }
  // sends of the partial slices to their owners (scatter mode's outgoing half)
  const bool sends = run_gemm && a->send_dst && a->world > 1;
  if (run_gemm && a->send_dst) {
    if (a->send_land != TLC_LAND_MEMCPY && a->send_land != TLC_LAND_COPY_ENGINE &&
        a->send_land != TLC_LAND_CU)
      return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: send_land %d (MEMCPY, COPY_ENGINE or CU)",
                  a->send_land);
    if (slice >= (int64_t{1} << 32))
      return fail(TLC_ERR_UNSUPPORTED, "tlc_gemm_rs: sends need rows_per_chunk * N < 2^32");
    if (a->send_land == TLC_LAND_CU && slice_bytes >= (int64_t{1} << 32))
      return fail(TLC_ERR_UNSUPPORTED, "tlc_gemm_rs: CU sends need slices of < 4 GiB");
    if (a->send_land == TLC_LAND_CU && a->n_tiles == 0)
      return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: CU sends need a plan with tiles");
    for (int c = 0; c < a->world; ++c) {
      if (c == a->rank) continue;
      if (!a->send_dst[c] || !aligned16(a->send_dst[c]))
        return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_rs: send_dst[%d] NULL or misaligned", c);
    }
  }
  // CUs the landing and the sends need beside the GEMM.  The scatter-mode GEMM
  // never waits, so the runtime's copies (memcpy and copy-engine landings and
  // sends) may share its CUs and it takes every one: a GEMM on all 256 CUs
  // instead of 224 runs the 4096 x 4096 x 2048 GEMM-RS in one round of tiles
  // instead of two.  Only the library's own copy kernels, sized for CUs of
  // their own (the CU landing, the CU sends), keep them free.
  int reserve = land == TLC_LAND_CU ? kReserveCUsLandCU : 0;
  if (sends && a->send_land == TLC_LAND_CU && reserve < kReserveCUsLandCU)
    reserve = kReserveCUsLandCU;
  if (run_gemm) {
    st = check_grid(a->grid, reserve, 0, "tlc_gemm_rs");
    if (st) return st;
  }
  DeviceInfo info;
  st = device_info(&info);
  if (st) return st;
  if (run_gemm) {
    st = check_grid(a->grid, reserve, info.cus, "tlc_gemm_rs");
    if (st) return st;
  }

  st = enqueue_landing(land, reinterpret_cast<void* const*>(a->landing),
                       reinterpret_cast<const void* const*>(a->remote_src), slice_bytes, a->world,
                       a->rank, 1, a->sig, a->epoch, copy_streams, n_copy_streams, info);
  if (st) return st;
  // the reduced slices of the peers raise flags[world + c]
  if (g) {
    st = enqueue_landing(land, g->dst, g->src, slice_bytes, a->world, a->rank, 1, a->sig, a->epoch,
                         copy_streams, n_copy_streams, info, a->world);
    if (st) return st;
  }
  // co-located all-gather: the GEMM's first workgroups copy the slices before
  // their first unit (the waiting kernel variant, with no chunk ever waited for)
  const bool coloc_gather = g && coloc && a->world > 1;

  if (run_gemm && (a->n_tiles > 0 || coloc_gather)) {
    GemmParams p;
    memset(&p, 0, sizeof(p));
    p.plan = a->plan;
    p.n_tiles = a->n_tiles;
    p.a = static_cast<const uint16_t*>(a->a);
    p.b = static_cast<const uint16_t*>(a->b);
    p.c = a->partials;
    p.M = a->M;
    p.N = a->N;
    p.K = a->K;
    p.lda = a->K;
    p.ldb = a->b_layout == TLC_B_NK ? a->K : a->N;
    p.ldc = a->N;
    p.do_wait = 0;
    p.sig = a->sig;
    p.epoch = a->epoch;
    p.timeout_ticks = ticks_for(a->timeout_ns, info);
    set_schedule(&p, a->schedule, a->workspace, a->workspace_bytes);
    if (sends) {
      p.rows_per_chunk = a->rows_per_chunk;
      p.notify_mask = ((a->world == 32) ? 0xFFFFFFFFu : ((1u << a->world) - 1u)) & ~(1u << a->rank);
      p.dest_total = static_cast<uint32_t>(slice);
    }
    const int avail = info.cus - reserve;
    int grid = a->n_tiles > 0 ? pick_grid(a->grid, a->schedule, a->n_tiles, avail)
                              : (a->grid > 0 ? a->grid : avail);
    if (coloc_gather) {
      p.do_wait = 1;
      p.no_wait_mask = 0xFFFFFFFFu;
      st = set_colocated(&p, const_cast<void* const*>(g->dst), g->src, slice_bytes, a->world,
                         a->rank, 1, g->copy_wgs, grid, info.cus, "tlc_gemm_ar", a->world,
                         a->n_tiles);
      if (st) return st;
      if (a->n_tiles == 0) grid = p.copy.wgs;
    }
    st = configure_tail(&p, a->schedule, a->workspace, a->workspace_bytes, grid, a->bm, a->bn,
                        sends ? KIND_RS_NOTIFY : KIND_DENSE, g ? "tlc_gemm_ar" : "tlc_gemm_rs");
    if (st) return st;
    p.xcd_remap = grid % 8 == 0;
    st = launch_gemm(p, a->bm, a->bn, a->b_layout, sends ? KIND_RS_NOTIFY : KIND_DENSE, grid,
                     compute_stream);
    if (st) return st;
  }
  // The sends are enqueued after the GEMM that raises their flags, so that a
  // hardware queue shared by the two streams never holds a gate ahead of it.
  if (sends) {
    st = enqueue_sends(a, slice, info);
    if (st) return st;
  }

  ReduceParams r;
  memset(&r, 0, sizeof(r));
  for (int s = 0; s < a->world; ++s)
    r.src[s] = s == a->rank ? a->partials + a->rank * slice : peer[s];
  r.out = a->out;
  r.n_vec4 = slice / 4;
  r.world = a->world;
  r.wait_mask = coloc ? 0u : ((a->world == 32) ? 0xFFFFFFFFu : ((1u << a->world) - 1u)) & ~(1u << a->rank);
  r.sig = a->sig;
  r.epoch = a->epoch;
  r.timeout_ticks = ticks_for(a->timeout_ns, info);
  int rgrid = info.cus * 2;  // 2 workgroups per CU: 7 % faster than 1 or 4 on the long slice
  const int64_t need = (r.n_vec4 + 1023) / 1024;  // 256 threads x 4 float4 per pass
  if (need < rgrid) rgrid = static_cast<int>(need > 0 ? need : 1);
  st = launch_reduce(r, rgrid, compute_stream);
  return st ? st : ok();
}

tlc_status tlc_gemm_rs(const tlc_rs_args* a, void* compute_stream, void* const* copy_streams,
                       int32_t n_copy_streams) {
  return rs_common(a, compute_stream, copy_streams, n_copy_streams, true);
}

tlc_status tlc_rs_reduce(const tlc_rs_args* a, void* compute_stream) {
  return rs_common(a, compute_stream, nullptr, 0, false);
}

tlc_status tlc_gemm_ar(const tlc_ar_args* a, void* compute_stream, void* const* copy_streams,
                       int32_t n_copy_streams) {
  if (!a) return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_ar: NULL args");
  const tlc_rs_args& r = a->rs;
  if (r.world < 1 || 2 * r.world > TLC_MAX_WORLD || r.rank < 0 || r.rank >= r.world)
    return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_ar: world %d (2 * world <= %d), rank %d", r.world,
                TLC_MAX_WORLD, r.rank);
  if (r.rows_per_chunk < 1 || r.N < 1)
    return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_ar: sizes must be >= 1");
  if (!a->c || !aligned16(a->c)) return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_ar: c NULL or misaligned");
  if (r.send_dst) return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_ar: send_dst must be NULL");
  if (r.land != TLC_LAND_NONE && r.world > 1 && !a->gathered_src)
    return fail(TLC_ERR_INVALID_ARG, "tlc_gemm_ar: landing needs gathered_src");
  const int64_t slice = static_cast<int64_t>(r.rows_per_chunk) * r.N;
  tlc_rs_args rr = r;
  rr.out = a->c + r.rank * slice;
  GatherPart g;
  memset(&g, 0, sizeof(g));
  for (int c = 0; c < r.world; ++c) {
    g.dst[c] = a->c + c * slice;
    g.src[c] = (a->gathered_src && c != r.rank) ? a->gathered_src[c] : nullptr;
  }
  g.copy_wgs = a->copy_wgs;
  return rs_common(&rr, compute_stream, copy_streams, n_copy_streams, true,
                   r.land == TLC_LAND_NONE ? nullptr : &g);
}

int64_t tlc_moe_plan_capacity(int32_t T, int32_t topk, int32_t experts, int32_t N, int32_t bm, int32_t bn) {
  if (T < 1 || topk < 1 || experts < 1 || N < 1 || bm < 1 || bn < 1) return 0;
  return moe_max_pairs(T, topk, experts, bm) * ((N + bn - 1) / bn);
}

int64_t tlc_moe_workspace_bytes(int32_t T, int32_t topk, int32_t experts, int32_t bm) {
  if (T < 1 || topk < 1 || experts < 1 || bm < 1) return 0;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  return up(static_cast<int64_t>(T) * 8) + up(moe_max_blocks(T) * experts * 4);
}

}  // extern "C"

// The routing with its workspace at `workspace` (caller's, or the static one).
static tlc_status moe_route_impl(const tlc_moe_route_args* a, void* workspace, void* stream) {
  if (a->world < 1 || a->world > TLC_MAX_WORLD || a->rank < 0 || a->rank >= a->world)
    return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route: world/rank");
  if (a->experts < 1 || a->experts > 64 || a->topk < 1 || a->topk > a->experts || a->topk > 16)
    return fail(TLC_ERR_UNSUPPORTED, "tlc_moe_route: experts %d (<= 64), topk %d (<= min(E, 16))",
                a->experts, a->topk);
  if (a->tokens_per_chunk < 1) return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route: tokens_per_chunk");
  const int64_t T = static_cast<int64_t>(a->world) * a->tokens_per_chunk;
  if (T > (1 << 20)) return fail(TLC_ERR_UNSUPPORTED, "tlc_moe_route: T > 2^20");
  if (a->N < 1 || !(a->bm == 128 || a->bm == 256) || a->bn < 1)
    return fail(TLC_ERR_UNSUPPORTED, "tlc_moe_route: N/bm/bn");
  if (a->order != TLC_ORDER_NATURAL && a->order != TLC_ORDER_RANK_OFFSET)
    return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route: order");
  if (!a->logits || !a->topk_idx || !a->gates || !a->counts || !a->offsets || !a->row_token ||
      !a->slot || !a->plan || !a->n_tiles_dev || !workspace)
    return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route: NULL array");
  const int64_t cap = tlc_moe_plan_capacity(static_cast<int32_t>(T), a->topk, a->experts, a->N, a->bm, a->bn);
  if (a->plan_cap < cap)
    return fail(TLC_ERR_CAPACITY, "tlc_moe_route: plan_cap %lld < %lld", static_cast<long long>(a->plan_cap),
                static_cast<long long>(cap));
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TLC_ERR_MISALIGNED, "tlc_moe_route: workspace not 256-byte aligned");
  // optional co-located landing of the token chunks by the top-k kernel
  void* dst[TLC_MAX_WORLD];
  int64_t chunk_bytes = 0;
  if (a->x_src) {
    if (!a->x || !a->sig)
      return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route: co-located landing needs x and sig");
    if (a->H < 8 || a->H % 8 != 0)
      return fail(TLC_ERR_UNSUPPORTED, "tlc_moe_route: co-located landing needs H %% 8 == 0 (H %d)", a->H);
    chunk_bytes = static_cast<int64_t>(a->tokens_per_chunk) * a->H * 2;
    for (int c = 0; c < a->world; ++c) dst[c] = static_cast<char*>(a->x) + c * chunk_bytes;
    const tlc_status st = check_land_args(TLC_LAND_COLOCATED, a->x_src, dst, a->world, a->rank,
                                          chunk_bytes, "tlc_moe_route", nullptr, 0, a->epoch);
    if (st) return st;
  }
  MoeDev d;
  memset(&d, 0, sizeof(d));
  if (a->x_src && a->world > 1) {
    fill_copy_chunks(&d.copy, dst, a->x_src, chunk_bytes, a->world, a->rank, 1, 0);
    // about 64 KB per copying workgroup; the routing's first kernel is
    // launched with that many workgroups after its own
    const int64_t per = (chunk_bytes + 65535) / 65536;
    if (per * d.copy.chunks > (1 << 30))
      return fail(TLC_ERR_UNSUPPORTED, "tlc_moe_route: co-located landing of %lld-byte chunks",
                  static_cast<long long>(chunk_bytes));
    d.copy.wgs = static_cast<int32_t>(per * d.copy.chunks);
    d.sig = a->sig;
    d.epoch = a->epoch;
  }
  d.logits = a->logits;
  d.T = static_cast<int32_t>(T);
  d.E = a->experts;
  d.k = a->topk;
  d.Tc = a->tokens_per_chunk;
  d.world = a->world;
  d.rank = a->rank;
  d.N = a->N;
  d.bm = a->bm;
  d.bn = a->bn;
  d.order = a->order;
  d.ntiles_n = (a->N + a->bn - 1) / a->bn;
  d.topk = a->topk_idx;
  d.gates = a->gates;
  d.counts = a->counts;
  d.offsets = a->offsets;
  d.row_token = a->row_token;
  d.slot = a->slot;
  d.plan = a->plan;
  d.n_tiles = a->n_tiles_dev;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  char* ws = static_cast<char*>(workspace);
  d.member = reinterpret_cast<unsigned long long*>(ws);
  ws += up(T * 8);
  d.blk = reinterpret_cast<int32_t*>(ws);
  DeviceInfo info;
  tlc_status st = device_info(&info);
  if (st) return st;
  st = launch_moe_route(d, stream);
  return st ? st : ok();
}

extern "C" {

tlc_status tlc_moe_route(const tlc_moe_route_args* a, void* stream) {
  if (!a) return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route: NULL args");
  return moe_route_impl(a, a->workspace, stream);
}

tlc_status tlc_moe_route_static(const tlc_moe_route_args* a, void* stream) {
  if (!a) return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route_static: NULL args");
  if (a->world < 1 || a->world > TLC_MAX_WORLD || a->tokens_per_chunk < 1 || a->topk < 1 ||
      a->experts < 1 || a->bm < 1)
    return fail(TLC_ERR_INVALID_ARG, "tlc_moe_route_static: sizes must be >= 1");
  const int64_t T = static_cast<int64_t>(a->world) * a->tokens_per_chunk;
  if (T > (1 << 20)) return fail(TLC_ERR_UNSUPPORTED, "tlc_moe_route_static: T > 2^20");
  const int64_t need = tlc_moe_workspace_bytes(static_cast<int32_t>(T), a->topk, a->experts, a->bm);
  if (need > kMoeStaticScratchBytes)
    return fail(TLC_ERR_CAPACITY, "tlc_moe_route_static: the routing needs %lld bytes of workspace, "
                "the static one holds %lld (use tlc_moe_route with a workspace)",
                static_cast<long long>(need), static_cast<long long>(kMoeStaticScratchBytes));
  void* ws = nullptr;
  tlc_status st = moe_static_scratch(&ws);
  if (st) return st;
  return moe_route_impl(a, ws, stream);
}

int64_t tlc_moe_static_workspace_bytes(void) { return kMoeStaticScratchBytes; }

tlc_status tlc_ag_moe(const tlc_moe_args* a, void* compute_stream, void* const* copy_streams,
                      int32_t n_copy_streams) {
  if (!a) return fail(TLC_ERR_INVALID_ARG, "tlc_ag_moe: NULL args");
  if (a->world < 1 || a->world > TLC_MAX_WORLD || a->rank < 0 || a->rank >= a->world)
    return fail(TLC_ERR_INVALID_ARG, "tlc_ag_moe: world/rank");
  if (a->experts < 1 || a->topk < 1 || a->tokens_per_chunk < 1 || a->H < 1 || a->N < 1)
    return fail(TLC_ERR_INVALID_ARG, "tlc_ag_moe: sizes must be >= 1");
  if (a->H % 64 != 0 || a->N % 8 != 0)
    return fail(TLC_ERR_UNSUPPORTED, "tlc_ag_moe: H %% 64 and N %% 8 must be 0");
  if (!((a->bm == 256 && a->bn == 256) || (a->bm == 128 && a->bn == 128)))
    return fail(TLC_ERR_UNSUPPORTED, "tlc_ag_moe: tile %dx%d not built", a->bm, a->bn);
  if (a->w_layout != TLC_B_KN && a->w_layout != TLC_B_NK)
    return fail(TLC_ERR_INVALID_ARG, "tlc_ag_moe: w_layout");
  const int64_t T = static_cast<int64_t>(a->world) * a->tokens_per_chunk;
  if (T * a->H >= (1LL << 31)) return fail(TLC_ERR_UNSUPPORTED, "tlc_ag_moe: T*H >= 2^31");
  if (a->topk > a->experts || T * a->topk >= (1LL << 31))
    return fail(TLC_ERR_UNSUPPORTED, "tlc_ag_moe: topk %d (<= experts), T*topk < 2^31", a->topk);
  if (a->plan_cap < 0) return fail(TLC_ERR_INVALID_ARG, "tlc_ag_moe: plan_cap < 0");
  if (!a->plan || !a->n_tiles_dev || !a->row_token || !a->x || !a->w || !a->y || !a->sig)
    return fail(TLC_ERR_INVALID_ARG, "tlc_ag_moe: NULL array");
  if (!aligned16(a->x) || !aligned16(a->w) || !aligned16(a->y))
    return fail(TLC_ERR_MISALIGNED, "tlc_ag_moe: operands must be 16-byte aligned");
  if (check_schedule(a->schedule, nullptr, 0, "tlc_ag_moe")) return TLC_ERR_INVALID_ARG;
  const int64_t chunk_bytes = static_cast<int64_t>(a->tokens_per_chunk) * a->H * 2;
  void* dst[TLC_MAX_WORLD];
  for (int c = 0; c < a->world; ++c) dst[c] = static_cast<char*>(a->x) + c * chunk_bytes;
  tlc_status st = check_land_args(a->land, a->x_src, dst, a->world, a->rank, chunk_bytes, "tlc_ag_moe",
                                  copy_streams, n_copy_streams, a->epoch);
  if (st) return st;
  // The grouped GEMM's whole-tile kernel (H / 64 even) leaves room on every CU
  // for the runtime's copy and flag-transfer workgroups (a fifth of the
  // registers or more, 32 KB of LDS, most wavefront slots), so beside the memcpy and
  // copy-engine landings it waits on flags without a reserve and takes every
  // CU; the 8-wavefront fallback (H / 64 odd) fills its CUs, and the CU landing
  // kernel is sized for CUs of its own: those keep the reserve.
  const bool shares_cus = (a->H / 64) % 2 == 0 && a->land != TLC_LAND_CU;
  const int moe_reserve = (a->world > 1 && !shares_cus) ? reserve_for(a->land) : 0;
  st = check_grid(a->grid, moe_reserve, 0, "tlc_ag_moe");
  if (st) return st;
  DeviceInfo info;
  st = device_info(&info);
  if (st) return st;
  st = check_grid(a->grid, moe_reserve, info.cus, "tlc_ag_moe");
  if (st) return st;
  st = enqueue_landing(a->land, dst, a->x_src, chunk_bytes, a->world, a->rank, 1, a->sig, a->epoch,
                       copy_streams, n_copy_streams, info);
  if (st) return st;

  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.plan = a->plan;
  p.n_tiles_dev = a->n_tiles_dev;
  p.n_tiles = a->plan_cap;
  p.a = static_cast<const uint16_t*>(a->x);
  p.b = static_cast<const uint16_t*>(a->w);
  p.c = a->y;
  p.row_token = a->row_token;
  p.a_rows = T;
  p.M = static_cast<int32_t>(T * a->topk);
  p.N = a->N;
  p.K = a->H;
  p.lda = a->H;
  p.ldb = a->w_layout == TLC_B_NK ? a->H : a->N;
  p.ldc = a->N;
  p.b_expert_stride = static_cast<int64_t>(a->H) * a->N;
  p.no_wait_mask = 1u << a->rank;
  p.do_wait = !(a->land == TLC_LAND_NONE && a->epoch == 0);
  p.sig = a->sig;
  p.epoch = a->epoch;
  p.timeout_ticks = ticks_for(a->timeout_ns, info);
  set_schedule(&p, a->schedule, nullptr, 0);
  const int avail = info.cus - (p.do_wait ? moe_reserve : 0);
  // The tile count is only known on the device: use every available CU.
  int grid = a->grid > 0 ? a->grid : (avail >= 8 ? avail / 8 * 8 : avail);
  if (a->land == TLC_LAND_COLOCATED) {
    st = set_colocated(&p, dst, a->x_src, chunk_bytes, a->world, a->rank, 1, a->copy_wgs, grid,
                       info.cus, "tlc_ag_moe");
    if (st) return st;
  }
  p.xcd_remap = grid % 8 == 0;
  st = launch_gemm(p, a->bm, a->bn, a->w_layout, KIND_MOE, grid, compute_stream);
  return st ? st : ok();
}

int64_t tlc_wall_clock_khz(void) {
  DeviceInfo info;
  if (device_info(&info)) return 0;
  return info.wall_khz;
}

const char* tlc_status_string(tlc_status s) {
  switch (s) {
    case TLC_OK: return "ok";
    case TLC_ERR_INVALID_ARG: return "invalid argument";
    case TLC_ERR_UNSUPPORTED: return "unsupported";
    case TLC_ERR_MISALIGNED: return "misaligned";
    case TLC_ERR_CAPACITY: return "capacity too small";
    case TLC_ERR_HIP: return "HIP runtime error";
    case TLC_ERR_TIMEOUT: return "timeout waiting for a chunk";
    case TLC_ERR_BAD_PLAN: return "plan entry outside the output";
    default: return "unknown status";
  }
}

const char* tlc_last_error(void) { return g_err; }

int32_t tlc_version(void) { return 132; }

}  // extern "C"
