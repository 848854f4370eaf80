// Work decomposition of the Hessian kernels and of their cross mode
// (k_hessian.hip): the plan of token splits and pieces, the work item ->
// (tile, token range, partial slot) map, the partial slots each tile sums, and
// the orders in which items take tiles.  Plain C++ with no device types: the
// constexpr maps are compiled for the device inside the kernels and for the
// host by the CPU tests, which check that every order is a bijection onto the
// tiles and that the items of a tile cover its tokens and slots exactly once.
#pragma once

#include <stdint.h>

namespace gptq {

constexpr int TB = 256;     // bf16 tile
constexpr int KB = 32;      // bf16 tokens per LDS stage
constexpr int TF = 128;     // fp32 tile
constexpr int KT_F32 = 16;  // fp32 tokens per LDS stage

constexpr int smin(int a, int b) { return a < b ? a : b; }
constexpr int smax(int a, int b) { return a > b ? a : b; }

struct SyrkPlan {
  int tile, nbt, T, S, tps, full, P, tpp;
  int64_t slots;
};

// Work decomposition.  bf16: with fewer than three upper tiles per CU the
// tokens are split 8 ways (one split per XCD), else not at all.  A split runs
// on the CUs of one XCD: whole tiles go out in full rounds of cus/8, and the
// tiles left over for a last partial round are cut into token pieces so that
// they fill that round.  fp32 (small problems): enough items for the chip
// with at least 512 tokens per split.  cus: the device's compute units.
inline SyrkPlan syrk_plan(int64_t n, int64_t tokens, bool bf16, bool cross, int cus) {
  SyrkPlan p{};
  p.tile = bf16 ? TB : TF;
  p.nbt = (int)((n + p.tile - 1) / p.tile);
  p.T = cross ? p.nbt * p.nbt : p.nbt * (p.nbt + 1) / 2;
  const int kt = bf16 ? KB : KT_F32;
  int64_t s;
  if (bf16) {
    s = (p.T >= 768 || tokens < 8 * 4 * KB) ? 1 : 8;
  } else {
    const int64_t target = 1024;
    s = (target + p.T - 1) / p.T;
    const int64_t max_s = (tokens + 511) / 512;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
  }
  int64_t per = (tokens + s - 1) / s;
  per = (per + kt - 1) / kt * kt;
  s = (tokens + per - 1) / per;
  if (s < 1) s = 1;
  p.S = (int)s;
  p.tps = (int)per;
  p.full = p.T;
  p.P = 1;
  p.tpp = p.tps;
  if (bf16 && p.S == 8) {
    const int per_xcd = smax(1, cus / 8);
    const int left = p.T % per_xcd;
    const int pieces = left > 0 ? per_xcd / left : 1;
    if (left > 0 && pieces > 1 && p.tps / pieces >= 4 * KB) {
      p.full = p.T - left;
      p.P = pieces;
      p.tpp = (p.tps / pieces + KB - 1) / KB * KB;
    }
  }
  p.slots = (int64_t)p.full * p.S + (int64_t)(p.T - p.full) * p.S * p.P;
  return p;
}

// Work item b -> (tile, token range, partial slot).  Split s = b % S: with
// S = 8 the dispatcher's round robin over the 8 XCDs sends every item of
// split s to the same XCD, which then streams only that eighth of X through
// its L2.  Units u = b / S below `full` are whole tiles (u = tile).  The last
// T - full tiles would leave most CUs of an XCD idle in a final partial
// round, so each of their splits is cut into P token pieces, giving
// (T - full) * P short items per XCD instead.  Slots: whole tiles tile * S + s;
// pieced tiles after them, (tile, s, piece) in token order.  A is any struct
// with the plan's fields (the kernels' arguments, or a SyrkPlan with tokens).
struct SyrkItem {
  int tile, slot, t0, t1;
};

template <class A>
[[gnu::always_inline]] constexpr SyrkItem decode_item(const A& a, int b) {
  SyrkItem it;
  const int s = b % a.S, u = b / a.S;
  const int t0 = s * a.tps, t1 = smin(a.tokens, t0 + a.tps);
  if (u < a.full) {
    it.tile = u;
    it.slot = u * a.S + s;
    it.t0 = t0;
    it.t1 = t1;
  } else {
    const int L = a.T - a.full, v = u - a.full;
    const int k = v % L, piece = v / L;
    it.tile = a.full + k;
    it.slot = a.full * a.S + (k * a.S + s) * a.P + piece;
    it.t0 = smin(t1, t0 + piece * a.tpp);
    it.t1 = smin(t1, it.t0 + a.tpp);
  }
  return it;
}

// Partial slots of a tile, in summation order.
template <class A>
[[gnu::always_inline]] constexpr void tile_slots(const A& a, int tile, int& first, int& count) {
  if (tile < a.full) {
    first = tile * a.S;
    count = a.S;
  } else {
    first = a.full * a.S + (tile - a.full) * a.S * a.P;
    count = a.S * a.P;
  }
}

// Off-diagonal tiles first (row-major), the cheaper diagonal tiles last: the
// dispatcher hands items out in order, so the last partial round of work
// items consists of short ones.
[[gnu::always_inline]] constexpr void decode_offdiag_first(int t, int nbt, int& I, int& J) {
  const int noff = nbt * (nbt - 1) / 2;
  if (t >= noff) {
    I = J = t - noff;
    return;
  }
  int i = 0, base = 0;
  while (base + (nbt - 1 - i) <= t) {
    base += nbt - 1 - i;
    ++i;
  }
  I = i;
  J = i + 1 + (t - base);
}

// One token split (many tiles): the items of a round go to the 8 XCDs in turn,
// so an XCD's 32 concurrent tiles are every eighth item.  Tiles are therefore
// numbered by supertiles of 4 block rows x 8 block columns, the supertiles that
// lie wholly above the diagonal first (32 tiles each, row-major), the rest
// after them, and item i of a full round of 256 takes tile 32 (8 (m / 32) + x) +
// m % 32 with x = i % 8 and m = i / 8: each XCD runs one whole supertile at a
// time, whose 32 tiles read 12 column blocks of X between them instead of about
// 33 in row-major order, so its L2 streams X far fewer times.  Items of the
// last, partial round keep their own numbers.  A bijection onto the tiles.
[[gnu::always_inline]] constexpr bool full_supertile(int a, int b, int nbt) {
  return 4 * a + 4 <= nbt && 8 * b + 8 <= nbt && 8 * b >= 4 * a + 3;
}

[[gnu::always_inline]] constexpr void decode_supertiles(int i, int nbt, int T, int& I, int& J) {
  const int R = T / 256;
  int t = i;
  if (i < R * 256) {
    const int x = i & 7, m = i >> 3;
    t = 32 * (8 * (m >> 5) + x) + (m & 31);
  }
  int base = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int a = 0; 4 * a < nbt; ++a) {
      const int i0 = 4 * a, i1 = smin(i0 + 4, nbt);
      for (int b = i0 / 8; 8 * b < nbt; ++b) {
        if ((pass == 0) != full_supertile(a, b, nbt)) continue;
        const int j0 = 8 * b, j1 = smin(j0 + 8, nbt);
        int cnt = 0;
        for (int r = i0; r < i1; ++r) cnt += smax(0, j1 - smax(j0, r));
        if (t < base + cnt) {
          int k = t - base;
          for (int r = i0; r < i1; ++r) {
            const int w = smax(0, j1 - smax(j0, r));
            if (k < w) {
              I = r;
              J = smax(j0, r) + k;
              return;
            }
            k -= w;
          }
        }
        base += cnt;
      }
    }
  }
  I = J = 0;  // not reached for i < T
}

[[gnu::always_inline]] constexpr void decode_upper(int t, int nbt, int& I, int& J) {
  // row-major enumeration of upper tiles: row I holds nbt - I tiles
  int i = 0, base = 0;
  while (base + (nbt - i) <= t) {
    base += nbt - i;
    ++i;
  }
  I = i;
  J = i + (t - base);
}

// Cross term with one token split: the square tile grid in supertiles of 4
// block rows x 8 block columns (the whole ones first, row-major), then the
// tiles outside them row-major; rounds of 256 items are spread over the XCDs
// as in decode_supertiles, so each XCD runs one supertile at a time.  A
// bijection onto the nbt^2 tiles.
[[gnu::always_inline]] constexpr void decode_square_supertiles(int i, int nbt, int T, int& I, int& J) {
  const int R = T / 256;
  int t = i;
  if (i < R * 256) {
    const int x = i & 7, m = i >> 3;
    t = 32 * (8 * (m >> 5) + x) + (m & 31);
  }
  const int SR = nbt / 4, SC = nbt / 8;
  const int F = SR * SC * 32;
  if (t < F) {
    const int sup = t >> 5, w = t & 31;
    I = 4 * (sup / SC) + (w >> 3);
    J = 8 * (sup % SC) + (w & 7);
    return;
  }
  int k = t - F;
  const int wA = nbt - 8 * SC;  // columns right of the whole supertiles, rows inside them
  if (k < 4 * SR * wA) {
    I = k / wA;
    J = 8 * SC + k % wA;
    return;
  }
  k -= 4 * SR * wA;
  I = 4 * SR + k / nbt;
  J = k % nbt;
}

}  // namespace gptq
