// Host check of the per-thread top-8 selection (select8.h), the code the
// many-row coarse kernels run (unrolled over consecutive columns, and rolled
// over the fp16 kernel's runs): against a sort by (key desc, column asc) on
// random rows, rows with exact ties, rows with near-ties (keys a few units
// apart, so their upper 26 bits agree), rows with missing columns (key 0) and
// rows with a planted cut (the 8th and 9th keys within 63 units, the other
// seven far above, so only the check of the best key left out catches it),
// plus the sorting networks on all 256 zero-one inputs.  Exit status 0 = all
// agree.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../bit_quantized_lm_amd/csrc/select8.h"

static uint32_t key_of(float f) {   // order-preserving unsigned image of a float
  f += 0.0f;                        // -0 as +0
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

int main() {
  int failures = 0;
  for (int bits = 0; bits < 256; ++bits) {   // zero-one principle for the network
    uint32_t v[8];
    for (int i = 0; i < 8; ++i) v[i] = (bits >> i) & 1u;
    dh::sort8_desc(v);
    for (int i = 0; i < 7; ++i) failures += v[i] < v[i + 1];
  }
  std::mt19937_64 rng(17);
  std::normal_distribution<float> nrm(0.f, 1.f);
  long slow = 0;
  for (int trial = 0; trial < 300000; ++trial) {
    const int mode = trial % 6;
    uint32_t key[64];
    const float base = nrm(rng);
    for (int c = 0; c < 64; ++c) {
      float s = nrm(rng);
      if (mode == 1) s = std::round(s * 2.f);                       // many exact ties
      if (mode == 2) s = base;                                      // one value, then nudged
      if (mode == 4) s = (c % 5 == 0) ? base : s * 1e-3f;           // a repeated maximum
      key[c] = key_of(s);
      if (mode == 2 || mode == 3) key[c] += (uint32_t)(rng() % 64);  // near-ties within 63 units
    }
    const int nvalid = mode == 5 ? 1 + (int)(rng() % 64) : 64;
    for (int c = nvalid; c < 64; ++c) key[c] = 0u;
    if (trial % 7 == 6) {   // a planted cut: the 8th and 9th within 63 units, their columns in the wrong order
      int perm[64];
      for (int c = 0; c < 64; ++c) perm[c] = c;
      for (int c = 63; c > 0; --c) std::swap(perm[c], perm[rng() % (c + 1)]);
      for (int c = 0; c < 64; ++c) key[c] = key_of(nrm(rng) * 0.1f);
      const uint32_t K = key_of(4.0f) & ~63u;
      for (int i = 0; i < 7; ++i) key[perm[i]] = K + 64u * 1000u * (uint32_t)(i + 1);
      const int c8 = std::max(perm[7], perm[8]), c9 = std::min(perm[7], perm[8]);
      key[c8] = K + 40u;   // the 8th, at the higher column
      key[c9] = K + 10u;   // the 9th: its column tag puts it above the 8th
    }
    uint32_t slot[8], slot2[8];
    dh::select8_row(key, [&](int c) { return key[c]; }, slot);
    // the rolled form over runs of non-consecutive columns (the fp16 kernel's
    // LDS pieces: run r = columns g, g + 16, g + 32, g + 48 for g = 2r, 2r + 1)
    auto col_of = [](int r, int e) { return 16 * (e & 3) + 2 * r + (e >> 2); };
    dh::select8_runs<true>(
        [&](int r, uint32_t(&raw)[8]) {
          for (int e = 0; e < 8; ++e) raw[e] = key[col_of(r, e)];
        },
        [&](int r, int e) { return 63 - col_of(r, e); }, [&](int c) { return key[c]; }, slot2);
    std::vector<int> cols;
    for (int c = 0; c < 64; ++c)
      if (key[c]) cols.push_back(c);
    std::stable_sort(cols.begin(), cols.end(), [&](int a, int b) { return key[a] > key[b]; });
    bool fast = true;
    for (int i = 0; i < 8; ++i) {
      const uint32_t want = i < (int)cols.size() ? (uint32_t)(63 - cols[i]) : 64u;
      if (slot[i] != want || slot2[i] != want) {
        if (failures < 10)
          std::printf("trial %d mode %d slot %d: got %u / %u (rolled) want %u\n", trial, mode, i, slot[i], slot2[i],
                      want);
        ++failures;
      }
    }
    for (int i = 0; i + 1 < (int)cols.size() && i < 8; ++i) fast &= (key[cols[i]] >> 6) != (key[cols[i + 1]] >> 6);
    slow += !fast;
  }
  std::printf("%s (%d failures; rows with agreeing upper bits: %ld)\n", failures ? "FAIL" : "ok", failures, slow);
  return failures ? 1 : 0;
}
