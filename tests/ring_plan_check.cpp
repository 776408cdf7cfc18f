// Host check of the many-row coarse kernel's DMA ring schedule (ring_plan.h):
// for every row-tile count, every row length K the kernel takes up to 40960,
// every wave part and block and every stage, each DMA op must read inside its
// source buffer and write inside its LDS ring, the LDS must fit, and every
// wait count must complete the ops the next stage reads (counted here op by
// op, independently of big_wait's closed form).  Exit status 0 = all hold.
#include <cstdio>

#include "../bit_quantized_lm_amd/csrc/ring_plan.h"

using namespace dh;

static int failures = 0;
#define CHECK(c, ...)                                 \
  do {                                                \
    if (!(c)) {                                       \
      if (failures < 20) std::printf(__VA_ARGS__);    \
      ++failures;                                     \
    }                                                 \
  } while (0)

template <int MT>
void check_shape() {
  using S = BigShape<MT>;
  constexpr int NBUF = S::XD + 1, SPB = S::SPB;
  const size_t lds = big_lds_bytes(MT, S::XD, S::CD, S::BPW, S::GPS);
  CHECK(lds <= 160 * 1024, "MT %d: LDS %zu\n", MT, lds);
  CHECK((size_t)S::BPW * 16 * MT * 68 * 4 <= lds, "MT %d: score area\n", MT);
  CHECK(S::W * 64 <= 1024 && S::GPS * SPB == 4, "MT %d: shape\n", MT);
  // ops a wave of part P issues in stage j (x first, then zero-point, then codes)
  auto ops = [&](int P, int j) {
    return S::nx(P) + (stage_has_byte_ops<MT>(j) ? S::nb(P) + S::nc(P) : 0);
  };
  auto ops_after = [&](int P, int s0, int after_in_s0, int s1) {   // after an op of stage s0, to the end of s1
    int n = after_in_s0;
    for (int s = s0 + 1; s <= s1; ++s) n += ops(P, s);
    return n;
  };
  for (int P = 0; P < S::WPB; ++P) {
    for (int Q = 0; Q < SPB; ++Q) {
      const int w = P == 0 ? big_wait<MT, 0>(Q) : big_wait<MT, 1>(Q);
      CHECK(w >= 0 && w <= 63, "MT %d P %d: wait %d\n", MT, P, w);
    }
  }
  for (int K = 512; K <= 40960; K += 512) {
    const int NG4 = K / 512, NGRP = K / 128, NST = SPB * NG4;
    for (int P = 0; P < S::WPB; ++P) {
      auto wait_at = [&](int j) {   // the count waited for at the end of stage j
        const int Q = ((j % SPB) + SPB) % SPB;
        return P == 0 ? big_wait<MT, 0>(Q) : big_wait<MT, 1>(Q);
      };
      for (int lb = 0; lb < S::BPW; ++lb) {
        for (int j = -S::PRO; j < NST; ++j) {
          for (int k = 0; k < S::nx(P); ++k) {
            const XOp o = x_op<MT>(j, lb, k, NGRP);
            CHECK(o.slab >= 0 && o.slab < NGRP && o.chunk >= 0 && o.chunk < 4 * MT && o.dst >= 0 &&
                      o.dst < NBUF * S::GPS * 4 * MT,
                  "MT %d K %d P %d lb %d j %d k %d: x op slab %d chunk %d dst %d\n", MT, K, P, lb, j, k, o.slab,
                  o.chunk, o.dst);
          }
          if (stage_has_byte_ops<MT>(j)) {
            const int GB = zp_group<MT>(j, NG4), GC = code_group<MT>(j, NG4), cs = code_slot<MT>(j);
            CHECK(GB >= 0 && GB < NG4 && GC >= 0 && GC < NG4 && cs >= 0 && cs < S::CD,
                  "MT %d K %d j %d: byte ops GB %d GC %d slot %d\n", MT, K, j, GB, GC, cs);
            for (int k = 0; k < S::nb(P); ++k) CHECK(lb * S::nb(P) + k < 4, "MT %d: zero-point chunk\n", MT);
          }
        }
      }
      // stage j reads its slabs from slot j mod NBUF: they were fetched by
      // stage j - XD and completed by the wait at the end of stage j - XW
      if (S::nx(P)) {
        for (int j = 0; j < NST; ++j) {
          const int s = j - S::XD;
          if (s < -S::PRO) continue;
          const int after = stage_has_byte_ops<MT>(s) ? S::nb(P) + S::nc(P) : 0;
          const int need = ops_after(P, s, after, j - S::XW);
          CHECK(wait_at(j - S::XW) <= need, "MT %d K %d P %d: slabs of stage %d not waited for\n", MT, K, P, j);
          for (int t = 0; t < S::GPS; ++t) {   // the slot holds stage j when it is read
            const XOp o = x_op<MT>(s, 0, t * 4 * MT / S::BPW, NGRP);
            CHECK(o.dst / (4 * MT) == (j % NBUF) * S::GPS + t, "MT %d: slot of stage %d\n", MT, j);
          }
          for (int s2 = s + 1; s2 <= j; ++s2) {   // nothing else lands in that slot before it is read
            const XOp o = x_op<MT>(s2, 0, 0, NGRP);
            CHECK(o.dst / (4 * MT) / S::GPS != j % NBUF, "MT %d: slot of stage %d overwritten at %d\n", MT, j, s2);
          }
        }
      }
      // byte group G + 1's codes and zero-point slab complete at the end of
      // byte group G (its last stage)
      for (int G = 0; G + 1 < NG4; ++G) {
        const int end = SPB * G + SPB - 1;
        if (S::nc(P)) {
          const int sc = SPB * (G + 1 - S::CD) + 1;
          CHECK(code_group<MT>(sc, NG4) == G + 1 && stage_has_byte_ops<MT>(sc), "MT %d: code stage\n", MT);
          if (sc >= -S::PRO) CHECK(wait_at(end) <= ops_after(P, sc, 0, end), "MT %d K %d: codes of %d\n", MT, K, G + 1);
        }
        if (S::nb(P)) {
          const int sb = SPB * G + 1;
          CHECK(zp_group<MT>(sb, NG4) == G + 1, "MT %d: zero-point stage\n", MT);
          CHECK(wait_at(end) <= ops_after(P, sb, S::nc(P), end), "MT %d K %d: zero point of %d\n", MT, K, G + 1);
        }
      }
    }
  }
}

int main() {
  check_shape<1>();
  check_shape<2>();
  check_shape<3>();
  check_shape<4>();
  check_shape<5>();
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
