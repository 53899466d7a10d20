// mask_check.cpp -- host-side check of the range-tiled kernels' element masks.
//
// The tile steps evaluate a range mask as one run of positions per lane
// (PosRun: lo .. lo+span-1), shifted once per tile to a base so that each
// element is base + c with c a compile-time offset.  This program checks,
// exhaustively over small sizes, windows, offsets and both causal settings,
// that the run and its shifted form say exactly what the kernels' visibility
// predicate range_ok says (key j < Lk; j <= i when causal; i - w < j, plus
// j < i + w without causal, for a window w > 0), for the query-major mask
// (lane = query) and the key-major one (lane = key, rows q < L at position
// q + shift).  Exit status 0 = all checks passed.
#include <cstdio>

#include "../../exact_tiled_attention_flash_amd/csrc/fa_bwd_tile.hpp"

using namespace fa;
using fa::bwdtile::RangeMaskK;

static long failures = 0, checks = 0;

static void expect(bool got, bool want, const char* what, int a, int b, int c, int d, int e) {
  ++checks;
  if (got != want) {
    if (failures < 20) std::printf("FAIL %s: %d %d %d %d %d: got %d want %d\n", what, a, b, c, d, e, got, want);
    ++failures;
  }
}

template <bool CAUSAL>
static void check_query_major() {
  for (int Lk = 0; Lk <= 24; ++Lk)
    for (int w = 0; w <= 30; ++w)
      for (int i = -40; i <= 70; ++i) {
        const RangeMaskQ<CAUSAL> m{Lk, w, i};
        const PosRun r = m.run();
        for (int j = 0; j <= 90; ++j) expect(r(j), range_ok<CAUSAL>(j, i, Lk, w), "query-major", Lk, w, i, j, 0);
        // shifted to a tile base, evaluated at base + c
        for (int base = 0; base <= 40; base += 4) {
          PosRun s = r;
          s.lo -= base;
          for (int c = 0; c <= 63; ++c)
            expect(s(c), range_ok<CAUSAL>(base + c, i, Lk, w), "query-major at base", Lk, w, i, base, c);
        }
      }
}

template <bool CAUSAL>
static void check_key_major() {
  for (int L = 0; L <= 24; ++L)
    for (int w = 0; w <= 30; ++w)
      for (int shift = -40; shift <= 40; ++shift)
        for (int j = 0; j <= 50; ++j) {
          const RangeMaskK<CAUSAL> m{L, shift, w, j};
          const PosRun r = m.run();
          for (int q = 0; q <= 60; ++q) {
            const bool want = q < L && range_ok<CAUSAL>(j, q + shift, j + 1, w);
            expect(r(q), want, "key-major", L, w, shift, j, q);
          }
        }
}

int main() {
  check_query_major<false>();
  check_query_major<true>();
  check_key_major<false>();
  check_key_major<true>();
  std::printf("%ld checks, %ld failures\n", checks, failures);
  return failures ? 1 : 0;
}
