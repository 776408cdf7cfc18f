// Host check of the many-row coarse kernel's DMA ring schedule (ring_plan.h):
// for every row-tile count, every row length K the kernel takes up to 40960,
// every wave part and block and every stage, each DMA op must read inside its
// source buffer and write inside its LDS ring, the LDS must fit, and every
// wait count must complete the ops the next stage reads (counted here op by
// op, independently of big_wait's closed form).  Exit status 0 = all hold.
#include <cstdio>
#include <vector>

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


// The fp16 many-row kernel's schedule (dh::h16_*), simulated op by op: every
// wave's ops in issue order, each wait completing all but the last
// h16_wait(MT, q) of them.  Checked: every op in bounds; at the end of stage
// j each wave's ops of slab j + 1 complete (every chunk of it fetched by some
// wave), at the end of a byte group's last stage its ops of the next byte
// group's codes and zero-point chunk complete; no x op writes a slot that the
// current or the next stage reads; byte ops (which rewrite the code slot and a
// zero-point slot) are issued only after the barrier that ends the byte
// group's first stage, by which every wave has read the byte group's codes,
// pairs and zero-point slab into registers.
template <int MT>
void check_h16(int K) {
  constexpr int W = kH16Blocks, SLOTS = kH16Slots;
  const int NG4 = K / 512, NST = 4 * NG4;
  CHECK(h16_ring_bytes(MT) <= 160 * 1024 && (size_t)W * 16 * MT * 64 * 4 <= 160 * 1024, "h16 MT %d: LDS\n", MT);
  CHECK(h16_wait(MT, 0) <= 63 && h16_wait(MT, 1) <= 63, "h16 MT %d: wait range\n", MT);
  struct Op {
    int kind;   // 0: x chunk, 1: zero-point chunk, 2: code or pair chunk
    int data;   // x: slab * 64 + chunk; zero point: byte group * 4 + chunk; codes: byte group * 16 + chunk
    int slot;   // x: ring slot; zero point: slot 0 or 1; codes: 0
  };
  for (int w = 0; w < W; ++w) {
    std::vector<Op> ops;
    std::vector<char> done;
    auto issue_x = [&](int j) {
      const int slab = h16_slab(j, NST);
      CHECK(slab >= 0 && slab < NST, "h16 MT %d K %d: slab %d of stage %d\n", MT, K, slab, j);
      for (int k = 0; k < h16_xops(MT); ++k) {
        const int c = h16_xchunk(MT, w, k);
        CHECK(c >= 0 && c < 4 * MT, "h16 MT %d: chunk %d\n", MT, c);
        ops.push_back({0, slab * 64 + c, j % SLOTS});
        done.push_back(0);
      }
    };
    auto issue_bytes = [&](int G) {
      const int Gc = h16_byte_group(G, NG4);
      CHECK(Gc >= 0 && Gc < NG4, "h16 MT %d K %d: byte group %d\n", MT, K, Gc);
      ops.push_back({1, Gc * 4 + (w & 3), Gc & 1});
      done.push_back(0);
      for (int k = 0; k < kCodeChunks; ++k) {
        ops.push_back({2, Gc * 16 + k, 0});
        done.push_back(0);
      }
    };
    auto wait = [&](int n) {   // all but the last n complete
      for (int i = 0; i + n < (int)ops.size(); ++i) done[i] = 1;
    };
    auto complete = [&](int kind, int data, int slot) {   // the latest issue of that data into that slot
      int last = -1;
      for (int i = 0; i < (int)ops.size(); ++i)
        if (ops[i].kind == kind && ops[i].data == data && ops[i].slot == slot) last = i;
      return last >= 0 && done[last];
    };
    // ops issued at stage j must not target the slot read in stage j or j + 1
    auto check_targets = [&](size_t from, int j) {
      for (size_t i = from; i < ops.size(); ++i)
        if (ops[i].kind == 0) {
          CHECK(ops[i].slot != j % SLOTS && (j + 1 >= NST || ops[i].slot != (j + 1) % SLOTS),
                "h16 MT %d K %d: stage %d writes a slot in use\n", MT, K, j);
        } else {
          CHECK((j & 3) >= 1, "h16 MT %d K %d: byte ops in the first stage of a byte group\n", MT, K);
        }
    };
    for (int j = 0; j < kH16XD; ++j) issue_x(j);
    issue_bytes(0);
    wait(0);
    for (int j = 0; j < NST; ++j) {
      const int q = j & 3, G = j >> 2;
      if (q == 0) {   // byte group G's codes and zero-point chunk, and slab j, complete
        for (int k = 0; k < kCodeChunks; ++k)
          CHECK(complete(2, G * 16 + k, 0), "h16 MT %d K %d w %d: codes of %d\n", MT, K, w, G);
        CHECK(complete(1, G * 4 + (w & 3), G & 1), "h16 MT %d K %d w %d: zero point of %d\n", MT, K, w, G);
      }
      const size_t from = ops.size();
      issue_x(j + kH16XD);
      if (q == 1) issue_bytes(G + 1);
      check_targets(from, j);
      wait(h16_wait(MT, q));
      if (j + 1 < NST)
        for (int k = 0; k < h16_xops(MT); ++k)
          CHECK(complete(0, (j + 1) * 64 + h16_xchunk(MT, w, k), (j + 1) % SLOTS), "h16 MT %d K %d w %d: slab %d\n",
                MT, K, w, j + 1);
    }
  }
  for (int c = 0; c < 4 * MT; ++c) {   // every chunk of a slab is some wave's
    bool any = false;
    for (int w = 0; w < W; ++w)
      for (int k = 0; k < h16_xops(MT); ++k) any |= h16_xchunk(MT, w, k) == c;
    CHECK(any, "h16 MT %d: chunk %d unfetched\n", MT, c);
  }
}

int main() {
  check_shape<1>();
  check_shape<2>();
  check_shape<3>();
  check_shape<4>();
  check_shape<5>();
  for (int K = 512; K <= 16384; K += 512) {   // the fp16 kernel's row lengths
    check_h16<3>(K);
    check_h16<4>(K);
    check_h16<5>(K);
  }
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
