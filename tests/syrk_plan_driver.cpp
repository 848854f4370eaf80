// Host checks of the Hessian kernels' work decomposition (syrk_plan.h), run by
// tests/test_syrk_plan.py.  Prints one line per failure and a summary line;
// exits nonzero on any failure.
#include <stdio.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <set>
#include <utility>
#include <vector>

#include "syrk_plan.h"

using namespace gptq;

static long failures = 0;
#define CHECK(cond, ...)           \
  do {                             \
    if (!(cond)) {                 \
      if (failures < 20) {         \
        printf("FAIL: " __VA_ARGS__); \
        printf("\n");              \
      }                            \
      ++failures;                  \
    }                              \
  } while (0)

// Every order must hit each tile of its grid exactly once.
static void check_orders(int max_nbt) {
  for (int nbt = 1; nbt <= max_nbt; ++nbt) {
    const int T = nbt * (nbt + 1) / 2;
    std::vector<int> seen_st(nbt * nbt, 0), seen_od(nbt * nbt, 0), seen_up(nbt * nbt, 0);
    for (int i = 0; i < T; ++i) {
      int I = -1, J = -1;
      decode_supertiles(i, nbt, T, I, J);
      CHECK(0 <= I && I <= J && J < nbt, "supertiles nbt=%d i=%d -> (%d, %d)", nbt, i, I, J);
      if (0 <= I && I <= J && J < nbt) ++seen_st[I * nbt + J];
      decode_offdiag_first(i, nbt, I, J);
      CHECK(0 <= I && I <= J && J < nbt, "offdiag_first nbt=%d i=%d -> (%d, %d)", nbt, i, I, J);
      if (0 <= I && I <= J && J < nbt) ++seen_od[I * nbt + J];
      CHECK(i < nbt * (nbt - 1) / 2 ? I < J : I == J, "offdiag_first order nbt=%d i=%d", nbt, i);
      decode_upper(i, nbt, I, J);
      CHECK(0 <= I && I <= J && J < nbt, "upper nbt=%d i=%d -> (%d, %d)", nbt, i, I, J);
      if (0 <= I && I <= J && J < nbt) ++seen_up[I * nbt + J];
    }
    for (int I = 0; I < nbt; ++I)
      for (int J = I; J < nbt; ++J) {
        CHECK(seen_st[I * nbt + J] == 1, "supertiles nbt=%d tile (%d, %d) hit %d times", nbt, I, J, seen_st[I * nbt + J]);
        CHECK(seen_od[I * nbt + J] == 1, "offdiag_first nbt=%d tile (%d, %d) hit %d times", nbt, I, J,
              seen_od[I * nbt + J]);
        CHECK(seen_up[I * nbt + J] == 1, "upper nbt=%d tile (%d, %d) hit %d times", nbt, I, J, seen_up[I * nbt + J]);
      }
    const int T2 = nbt * nbt;
    std::vector<int> seen_sq(T2, 0);
    for (int i = 0; i < T2; ++i) {
      int I = -1, J = -1;
      decode_square_supertiles(i, nbt, T2, I, J);
      CHECK(0 <= I && I < nbt && 0 <= J && J < nbt, "square nbt=%d i=%d -> (%d, %d)", nbt, i, I, J);
      if (0 <= I && I < nbt && 0 <= J && J < nbt) ++seen_sq[I * nbt + J];
    }
    for (int t = 0; t < T2; ++t) CHECK(seen_sq[t] == 1, "square nbt=%d tile %d hit %d times", nbt, t, seen_sq[t]);
  }
}

struct PlanArgs : SyrkPlan {
  int tokens;
};

// The items of a plan: each partial slot written by exactly one item, each
// tile's token pieces a partition of [0, tokens), and tile_slots naming
// exactly the slots of the tile's items.
static void check_plan(int64_t n, int64_t tokens, bool bf16, bool cross, int cus) {
  PlanArgs a;
  static_cast<SyrkPlan&>(a) = syrk_plan(n, tokens, bf16, cross, cus);
  a.tokens = (int)tokens;
  const int64_t items = ((int64_t)a.full + (int64_t)(a.T - a.full) * a.P) * a.S;
  CHECK(a.S >= 1 && a.P >= 1 && a.full >= 0 && a.full <= a.T, "plan n=%lld tokens=%lld: S %d P %d full %d T %d",
        (long long)n, (long long)tokens, a.S, a.P, a.full, a.T);
  CHECK((int64_t)a.S * a.tps >= tokens && (int64_t)(a.S - 1) * a.tps < tokens,
        "plan n=%lld tokens=%lld: %d splits of %d tokens", (long long)n, (long long)tokens, a.S, a.tps);
  CHECK(a.P == 1 || (int64_t)a.P * a.tpp >= a.tps, "plan n=%lld tokens=%lld: %d pieces of %d for %d", (long long)n,
        (long long)tokens, a.P, a.tpp, a.tps);
  std::vector<int> slot_hits(a.slots, 0);
  std::map<int, std::vector<std::pair<int, int>>> ranges;
  std::map<int, std::set<int>> tile_slot_set;
  for (int64_t b = 0; b < items; ++b) {
    const SyrkItem it = decode_item(a, (int)b);
    const bool ok = it.tile >= 0 && it.tile < a.T && it.slot >= 0 && it.slot < a.slots && 0 <= it.t0 &&
                    it.t0 <= it.t1 && it.t1 <= tokens;
    CHECK(ok, "item n=%lld tokens=%lld b=%lld -> tile %d slot %d [%d, %d)", (long long)n, (long long)tokens,
          (long long)b, it.tile, it.slot, it.t0, it.t1);
    if (!ok) continue;
    ++slot_hits[it.slot];
    ranges[it.tile].push_back({it.t0, it.t1});
    tile_slot_set[it.tile].insert(it.slot);
  }
  for (int64_t s = 0; s < a.slots; ++s)
    CHECK(slot_hits[s] == 1, "plan n=%lld tokens=%lld: slot %lld written %d times", (long long)n, (long long)tokens,
          (long long)s, slot_hits[s]);
  CHECK((int)ranges.size() == a.T, "plan n=%lld tokens=%lld: %d of %d tiles have items", (long long)n,
        (long long)tokens, (int)ranges.size(), a.T);
  for (auto& kv : ranges) {
    // the tile's non-empty token ranges, in order, must tile [0, tokens)
    std::vector<std::pair<int, int>> rs;
    for (auto& r : kv.second)
      if (r.first < r.second) rs.push_back(r);
    std::sort(rs.begin(), rs.end());
    int64_t at = 0;
    for (auto& r : rs) {
      CHECK(r.first == at, "plan n=%lld tokens=%lld: tile %d has a gap or overlap at token %lld", (long long)n,
            (long long)tokens, kv.first, (long long)at);
      at = r.second;
    }
    CHECK(at == tokens, "plan n=%lld tokens=%lld: tile %d covers tokens up to %lld", (long long)n, (long long)tokens,
          kv.first, (long long)at);
    int first = -1, count = -1;
    tile_slots(a, kv.first, first, count);
    std::set<int> want;
    for (int s = first; s < first + count; ++s) want.insert(s);
    CHECK(want == tile_slot_set[kv.first], "plan n=%lld tokens=%lld: tile %d slots [%d, +%d) differ from its items'",
          (long long)n, (long long)tokens, kv.first, first, count);
  }
}

int main() {
  check_orders(139);
  long plans = 0;
  const int64_t widths[] = {1, 7, 100, 255, 256, 257, 512, 700, 1024, 1100, 2048, 4096, 5120, 11008};
  const int64_t tokens[] = {1, 5, 33, 1023, 1024, 1025, 4096, 8192, 8193, 20000, 65536, 131072, 262144};
  for (int64_t n : widths)
    for (int64_t t : tokens)
      for (int bf16 = 0; bf16 < 2; ++bf16)
        for (int cross = 0; cross < 2; ++cross)
          for (int cus : {256, 304, 80}) {
            check_plan(n, t, bf16 != 0, cross != 0, cus);
            ++plans;
          }
  printf("orders 1..139, plans %ld, failures %ld\n", plans, failures);
  return failures != 0;
}
