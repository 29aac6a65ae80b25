// Host harness for the tile planner under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++ by tests/test_plan_sanitizers.py;
// no device code).  It walks a grid of plan descriptors, valid and invalid,
// and checks what every plan must satisfy whatever its order: each output tile
// appears once (or once per K range of a split tile, ranges 0..S-1 adjacent),
// tiles lie inside the output, keys never decrease along the plan, the chunk
// mask covers exactly the chunks of the tile's rows, and the landing order
// lists every chunk but the local ones once.  Exit status 0 when all hold.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <set>
#include <tuple>
#include <vector>

#include "tlc.h"

namespace tlc {
// the library's error reporting lives with the device code; the planner only
// needs the status to come back
tlc_status fail(tlc_status s, const char*, ...) { return s; }
tlc_status ok() { return TLC_OK; }
}  // namespace tlc

static int g_fail = 0;
static long g_plans = 0;

static void check(bool c, const char* what, const tlc_plan_desc& d) {
  if (c) return;
  if (++g_fail <= 20)
    std::fprintf(stderr, "FAIL %s: mode %d world %d rank %d M %d N %d R %d bm %d bn %d order %d gm %d "
                 "split %d/%d sub %d\n", what, d.mode, d.world, d.rank, d.M, d.N, d.rows_per_chunk, d.bm,
                 d.bn, d.order, d.group_m, d.split_k, d.split_from, d.sub_chunks);
}

static void run_valid(const tlc_plan_desc& d) {
  int64_t n = -1;
  std::vector<int32_t> land(TLC_MAX_WORLD, -1);
  tlc_status s = tlc_chunk_plan(&d, nullptr, 0, &n, land.data());
  check(s == TLC_OK && n > 0, "count pass", d);
  if (s != TLC_OK || n <= 0) return;
  // one unit short: refused, nothing written past the array
  if (n > 1) {
    std::vector<tlc_tile> small(static_cast<size_t>(n - 1));
    int64_t n2 = -1;
    check(tlc_chunk_plan(&d, small.data(), n - 1, &n2, nullptr) == TLC_ERR_CAPACITY, "capacity", d);
  }
  std::vector<tlc_tile> t(static_cast<size_t>(n));
  int64_t n3 = -1;
  s = tlc_chunk_plan(&d, t.data(), n, &n3, land.data());
  check(s == TLC_OK && n3 == n, "fill pass", d);
  if (s != TLC_OK) return;
  ++g_plans;
  const int S = d.split_k >= 2 ? d.split_k : 1;
  const int SC = d.sub_chunks > 1 ? d.sub_chunks : 1;
  const int W = d.world * SC, R = d.rows_per_chunk / SC;
  std::set<std::tuple<int, int, int>> seen;
  int32_t prev_key = -1;
  for (int64_t i = 0; i < n; ++i) {
    const tlc_tile& x = t[static_cast<size_t>(i)];
    check(x.m0 >= 0 && x.n0 >= 0 && x.m_rows >= 1 && x.n_cols >= 1 && x.m0 + x.m_rows <= d.M &&
              x.n0 + x.n_cols <= d.N && x.m_rows <= d.bm && x.n_cols <= d.bn,
          "tile inside the output", d);
    check(x.key >= prev_key, "keys in order", d);
    prev_key = x.key;
    uint32_t want = 0;
    for (int c = x.m0 / R; c <= (x.m0 + x.m_rows - 1) / R; ++c) want |= 1u << c;
    check(x.chunk_mask == want, "chunk mask", d);
    const int sk = x.split ? static_cast<int>(x.split & 0xFF) : 1;
    const int si = x.split ? static_cast<int>((x.split >> 8) & 0xFF) : 0;
    check(sk == 1 || sk == S, "split factor", d);
    check(seen.insert(std::make_tuple(x.m0, x.n0, si)).second, "tile once per K range", d);
    if (x.split && si > 0) {
      const tlc_tile& p = t[static_cast<size_t>(i - 1)];
      check(p.m0 == x.m0 && p.n0 == x.n0 && ((p.split >> 8) & 0xFF) == static_cast<uint32_t>(si - 1),
            "K ranges adjacent", d);
    }
  }
  const int64_t mt = (d.M + d.bm - 1) / d.bm, nt = (d.N + d.bn - 1) / d.bn;
  check(static_cast<int64_t>(seen.size()) == n && n >= mt * nt && n <= mt * nt * S, "tile count", d);
  std::set<int> l;
  for (int i = 0; i < W - SC; ++i) l.insert(land[static_cast<size_t>(i)]);
  bool ok = static_cast<int>(l.size()) == W - SC;
  for (int c : l) ok = ok && c >= 0 && c < W && c / SC != d.rank;
  check(ok, "landing order", d);
}

int main() {
  const int worlds[] = {1, 2, 3, 8, 32};
  const int rows[] = {1, 7, 64, 256, 300};
  const int cols[] = {1, 8, 200, 520};
  const int tiles[] = {128, 256};
  for (int mode : {TLC_MODE_AG, TLC_MODE_RS})
    for (int w : worlds)
      for (int rank : {0, w / 2, w - 1})
        for (int R : rows)
          for (int N : cols)
            for (int tile : tiles)
              for (int order : {TLC_ORDER_NATURAL, TLC_ORDER_RANK_OFFSET})
                for (int gm : {1, 3, 8})
                  for (int split : {0, 2, 5})
                    for (int sub : {0, 2}) {
                      if (sub > 1 && (mode != TLC_MODE_AG || R % sub != 0 || w * sub > TLC_MAX_WORLD))
                        continue;
                      tlc_plan_desc d;
                      std::memset(&d, 0, sizeof(d));
                      d.mode = mode; d.world = w; d.rank = rank; d.M = w * R; d.N = N;
                      d.rows_per_chunk = R; d.bm = tile; d.bn = tile; d.order = order; d.group_m = gm;
                      d.split_k = split; d.split_from = split ? (w - 1) : 0; d.sub_chunks = sub;
                      run_valid(d);
                    }
  // invalid descriptors: refused with INVALID_ARG, nothing written
  tlc_plan_desc base;
  std::memset(&base, 0, sizeof(base));
  base.mode = TLC_MODE_AG; base.world = 4; base.rank = 1; base.M = 1024; base.N = 512;
  base.rows_per_chunk = 256; base.bm = 256; base.bn = 256; base.order = TLC_ORDER_RANK_OFFSET;
  base.group_m = 4;
  const int n_bad = 11;
  for (int b = 0; b < n_bad; ++b) {
    tlc_plan_desc d = base;
    switch (b) {
      case 0: d.mode = 7; break;
      case 1: d.world = 0; break;
      case 2: d.world = TLC_MAX_WORLD + 1; break;
      case 3: d.rank = 4; break;
      case 4: d.rank = -1; break;
      case 5: d.M = 1000; break;
      case 6: d.bm = 0; break;
      case 7: d.order = 9; break;
      case 8: d.split_k = 300; break;
      case 9: d.sub_chunks = 3; break;
      case 10: d.group_m = 0; break;
    }
    tlc_tile sentinel[4];
    std::memset(sentinel, 0x5A, sizeof(sentinel));
    int64_t n = 12345;
    const tlc_status s = tlc_chunk_plan(&d, sentinel, 4, &n, nullptr);
    bool untouched = true;
    for (size_t i = 0; i < sizeof(sentinel); ++i)
      untouched = untouched && reinterpret_cast<unsigned char*>(sentinel)[i] == 0x5A;
    check(s == TLC_ERR_INVALID_ARG && untouched, "invalid descriptor refused", d);
  }
  int64_t n = 0;
  check(tlc_chunk_plan(nullptr, nullptr, 0, &n, nullptr) == TLC_ERR_INVALID_ARG, "NULL desc", base);
  std::printf("plans %ld failures %d\n", g_plans, g_fail);
  return g_fail == 0 ? 0 : 1;
}
