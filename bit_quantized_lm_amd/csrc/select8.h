// The eight best of one block row of 64 coarse scores, as the many-row coarse
// kernel selects them one list per thread: plain constexpr C++ (usable on the
// device and on the host), so the host tests run this same code against a
// sort.  Internal to the library (not part of the public ABI).
#pragma once

#include <stdint.h>

namespace dh {

constexpr uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }
constexpr uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Compare-exchange of two keys, the larger first.
constexpr void cx_desc(uint32_t& a, uint32_t& b) {
  const uint32_t hi = umax32(a, b);
  b = umin32(a, b);
  a = hi;
}

// Eight keys sorted descending: Batcher's odd-even merge sort (19 comparators).
constexpr void sort8_desc(uint32_t (&v)[8]) {
  constexpr int P[19][2] = {{0, 1}, {2, 3}, {4, 5}, {6, 7}, {0, 2}, {1, 3}, {4, 6}, {5, 7}, {1, 2}, {5, 6},
                            {0, 4}, {1, 5}, {2, 6}, {3, 7}, {2, 4}, {3, 5}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
  for (int i = 0; i < 19; ++i) cx_desc(v[P[i][0]], v[P[i][1]]);
}

// A bitonic sequence of eight keys sorted descending (12 comparators).
constexpr void bitonic8_desc(uint32_t (&v)[8]) {
#pragma unroll
  for (int d = 4; d > 0; d >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & d) == 0) cx_desc(v[i], v[i + d]);
}

// The eight best of a row of 64 keys taken as eight runs of eight.
// load_at(r, raw) fills raw[0..7] with the keys of run r (each column once
// over the eight runs) and tag_at(r, e) is 63 - the column of element e of
// run r; key_at(c) is column c's key, for the rebuild's loop over a run-time
// column.  slot[i] receives 63 - column of the i-th best (score desc, column
// asc), or 64 where fewer than i + 1 columns exist.
//
// Replacing each key's low 6 bits by 63 - column makes the keys of a row
// distinct and, between scores whose keys differ above bit 5, orders them as
// (score desc, column asc).  The runs are sorted by Batcher's network and
// merged into the eight largest (bitonic merge of the current eight with the
// next run reversed), tracking the largest key left out.  That is the exact
// list unless two of the eight, or the eighth and the best key left out,
// agree above bit 5 (scores within 63 units in the last place of each
// other); such a list is rebuilt with 64-bit keys (full key, then 63 -
// column) over the columns whose keys reach the eighth's upper bits.
// kRolled: the run loop is not unrolled (small code, for an epilogue that
// runs once per kernel and would otherwise wait on instruction fetch), and
// run r + 1 is loaded before run r is merged, so that its loads (from LDS in
// the kernel) are in flight during the merge.
template <bool kRolled, class LoadAt, class TagAt, class KeyAt>
constexpr void select8_runs(LoadAt load_at, TagAt tag_at, KeyAt key_at, uint32_t (&slot)[8]) {
  uint32_t run[8] = {}, ninth = 0u;   // merging into zeros keeps the first run as it is
  auto merge = [&](uint32_t(&ch)[8]) {
    sort8_desc(ch);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t hi = umax32(run[i], ch[7 - i]);
      ninth = umax32(ninth, umin32(run[i], ch[7 - i]));
      run[i] = hi;
    }
    bitonic8_desc(run);
  };
  auto tagged = [&](int r, const uint32_t(&raw)[8], uint32_t(&ch)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ch[e] = (raw[e] & ~63u) | (uint32_t)tag_at(r, e);
  };
  if constexpr (kRolled) {
    uint32_t raw[8] = {};
    load_at(0, raw);
#pragma unroll 1
    for (int r = 0; r < 8; ++r) {
      uint32_t ch[8] = {};
      tagged(r, raw, ch);
      load_at(r < 7 ? r + 1 : 7, raw);   // the last iteration reads run 7 again, unused
      merge(ch);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      uint32_t raw[8] = {}, ch[8] = {};
      load_at(r, raw);
      tagged(r, raw, ch);
      merge(ch);
    }
  }
  // exact unless upper parts agree where the order or the cut depends on them
  const uint32_t p8 = run[7] >> 6;
  bool exact = (ninth >> 6) < p8 || p8 == 0u;
#pragma unroll
  for (int i = 0; i < 7; ++i) exact &= (run[i] >> 6) != (run[i + 1] >> 6) || (run[i + 1] >> 6) == 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) slot[i] = run[i] >> 6 ? run[i] & 63u : 64u;
  if (!exact) {
    unsigned long long top[8] = {};
    for (int c = 0; c < 64; ++c) {
      const uint32_t k = key_at(c);
      if (k != 0u && (k >> 6) >= p8) {
        unsigned long long t = ((unsigned long long)k << 32) | (uint32_t)(63 - c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const unsigned long long u = top[i];
          const bool gt = t > u;
          top[i] = gt ? t : u;
          t = gt ? u : t;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) slot[i] = top[i] ? (uint32_t)(top[i] & 63ull) : 64u;
  }
}

// key[c]: the order-preserving unsigned image of column c's score (0 for a
// column that does not exist), held in registers (indexed by constants only);
// key_at(c) the same value, for the rebuild's loop.  Runs are eight
// consecutive columns.
template <class KeyAt>
constexpr void select8_row(const uint32_t (&key)[64], KeyAt key_at, uint32_t (&slot)[8]) {
  select8_runs<false>(
      [&](int r, uint32_t(&raw)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) raw[e] = key[8 * r + e];
      },
      [](int r, int e) { return 63 - 8 * r - e; }, key_at, slot);
}

}  // namespace dh
