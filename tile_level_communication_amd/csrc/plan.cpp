// Host tile planner: the order in which the persistent GEMM visits its tiles.
//
// Gather mode follows the rank-offset start of DITRON's distributed swizzle
// (paper notes, §3.2: execution starts at rank_id mod local_world_size, and the
// compiler issues remote fetches early so local HBM acts as a cache of remote
// memory).  Scatter mode produces remote-bound tiles first and the local slice
// last (§3.2 scatter mode; Triton-Distributed talk, swizzling section).  Tiles
// that straddle chunk boundaries are keyed by the last chunk they wait for
// (gather) or the first destination they feed (scatter), per the talk's
// section on non-perfect tile scheduling.  Inside one key the tiles go band by
// band (group_m m-tiles wide), column by column, keeping operand reuse close in
// time (AutoOverlap §5.4 / Fig. 6, intra-chunk swizzle for locality).
//
// Tiles whose key is at or past split_from are cut into split_k K ranges that
// follow each other in the plan.  This is not from the pages: a 256 x 256 tile
// over K = 5120 is a long unit of work, and the tiles that depend on the last
// chunk would otherwise run on only as many compute units as that chunk has
// tiles, after everything else has finished.
#include <algorithm>
#include <vector>

#include "tlc_internal.h"

namespace {

struct Keyed {
  int32_t key, band, nt, mt;
  tlc_tile tile;
};

bool key_less(const Keyed& x, const Keyed& y) {
  if (x.key != y.key) return x.key < y.key;
  if (x.band != y.band) return x.band < y.band;
  if (x.nt != y.nt) return x.nt < y.nt;
  return x.mt < y.mt;
}

int32_t mod(int64_t a, int32_t w) {
  int64_t r = a % w;
  return static_cast<int32_t>(r < 0 ? r + w : r);
}

}  // namespace

extern "C" tlc_status tlc_chunk_plan(const tlc_plan_desc* d, tlc_tile* tiles, int64_t cap,
                                     int64_t* n_tiles, int32_t* landing_order) {
  using tlc::fail;
  if (!d || !n_tiles) return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: NULL desc or n_tiles");
  if (d->mode != TLC_MODE_AG && d->mode != TLC_MODE_RS)
    return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: mode %d is not AG or RS", d->mode);
  if (d->world < 1 || d->world > TLC_MAX_WORLD)
    return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: world %d outside 1..%d", d->world,
                TLC_MAX_WORLD);
  if (d->rank < 0 || d->rank >= d->world)
    return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: rank %d outside 0..%d", d->rank,
                d->world - 1);
  if (d->M < 1 || d->N < 1 || d->rows_per_chunk < 1 || d->bm < 1 || d->bn < 1 || d->group_m < 1)
    return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: sizes must be >= 1");
  if (static_cast<int64_t>(d->world) * d->rows_per_chunk != d->M)
    return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: M=%d != world %d * rows_per_chunk %d", d->M,
                d->world, d->rows_per_chunk);
  if (d->order != TLC_ORDER_NATURAL && d->order != TLC_ORDER_RANK_OFFSET)
    return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: order %d unknown", d->order);
  if (d->split_k < 0 || d->split_k > 255 || d->split_from < 0)
    return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: split_k %d outside 0..255 or split_from %d < 0",
                d->split_k, d->split_from);
  const int32_t SC = d->sub_chunks > 1 ? d->sub_chunks : 1;
  if (d->sub_chunks < 0 || (SC > 1 && (d->mode != TLC_MODE_AG || d->rows_per_chunk % SC != 0 ||
                                       static_cast<int64_t>(d->world) * SC > TLC_MAX_WORLD)))
    return fail(TLC_ERR_INVALID_ARG,
                "tlc_chunk_plan: sub_chunks %d needs gather mode, rows_per_chunk %% S == 0, "
                "world * S <= %d", d->sub_chunks, TLC_MAX_WORLD);

  // with sub-chunks, the plan of world * S chunks of R / S rows, local chunk rank * S
  const int32_t W = d->world * SC, r = d->rank * SC, R = d->rows_per_chunk / SC;
  const int64_t mtiles = (d->M + d->bm - 1) / d->bm;
  const int64_t ntiles = (d->N + d->bn - 1) / d->bn;
  const int32_t S = d->split_k >= 2 ? d->split_k : 1;
  std::vector<Keyed> v;
  v.reserve(static_cast<size_t>(mtiles * ntiles));
  for (int64_t mt = 0; mt < mtiles; ++mt) {
    const int32_t m0 = static_cast<int32_t>(mt * d->bm);
    const int32_t rows = std::min<int32_t>(d->bm, d->M - m0);
    const int32_t c_first = m0 / R, c_last = (m0 + rows - 1) / R;
    uint32_t mask = 0;
    int32_t key_ag = 0, key_rs = W;
    for (int32_t c = c_first; c <= c_last; ++c) {
      mask |= 1u << c;
      key_ag = std::max(key_ag, mod(c - r, W));       // consume position, latest
      key_rs = std::min(key_rs, mod(c - r - 1, W));   // send position, earliest
    }
    int32_t key = d->order == TLC_ORDER_NATURAL ? 0 : (d->mode == TLC_MODE_AG ? key_ag : key_rs);
    for (int64_t nt = 0; nt < ntiles; ++nt) {
      Keyed k;
      k.key = key;
      k.band = static_cast<int32_t>(mt / d->group_m);
      k.nt = static_cast<int32_t>(nt);
      k.mt = static_cast<int32_t>(mt);
      k.tile.m0 = m0;
      k.tile.n0 = static_cast<int32_t>(nt * d->bn);
      k.tile.m_rows = rows;
      k.tile.n_cols = std::min<int32_t>(d->bn, d->N - k.tile.n0);
      k.tile.expert = -1;
      k.tile.chunk_mask = mask;
      k.tile.key = key;
      k.tile.split = 0;
      v.push_back(k);
    }
  }
  std::sort(v.begin(), v.end(), key_less);

  int64_t count = 0;
  for (const Keyed& k : v) count += (S > 1 && k.key >= d->split_from) ? S : 1;
  *n_tiles = count;
  if (landing_order)
    for (int32_t i = SC; i < W; ++i) landing_order[i - SC] = (r + i) % W;
  if (!tiles) return tlc::ok();
  if (cap < count)
    return fail(TLC_ERR_CAPACITY, "tlc_chunk_plan: capacity %lld < %lld units",
                static_cast<long long>(cap), static_cast<long long>(count));
  int64_t out = 0;
  uint32_t fix = 0;
  for (const Keyed& k : v) {
    if (S > 1 && k.key >= d->split_from) {
      if (fix > 0xFFFFu)
        return fail(TLC_ERR_INVALID_ARG, "tlc_chunk_plan: more than 65536 split tiles");
      for (int32_t u = 0; u < S; ++u) {
        tiles[out] = k.tile;
        tiles[out].split = static_cast<uint32_t>(S) | (static_cast<uint32_t>(u) << 8) | (fix << 16);
        ++out;
      }
      ++fix;
    } else {
      tiles[out++] = k.tile;
    }
  }
  return tlc::ok();
}

extern "C" int64_t tlc_split_workspace_bytes(int64_t n_split_tiles, int32_t split_k, int32_t bm,
                                             int32_t bn) {
  if (n_split_tiles <= 0 || split_k < 2 || bm < 1 || bn < 1) return 0;
  return n_split_tiles * tlc::split_block_bytes(split_k, bm, bn);
}

extern "C" int64_t tlc_streamk_workspace_bytes(int32_t grid) {
  if (grid < 0) return -1;
  return static_cast<int64_t>(grid == 0 ? 256 : grid) * tlc::kSkBlockBytes;
}

namespace tlc {
int64_t split_block_bytes(int32_t split_k, int32_t bm, int32_t bn) {
  return 256 + static_cast<int64_t>(split_k) * bm * bn * 4;
}
}  // namespace tlc
