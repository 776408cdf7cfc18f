// Host check of the many-row coarse kernels' DMA ring schedules (ring_plan.h):
// for every row-tile count, every row length the kernel takes up to 40960,
// every wave and every stage, each DMA op must read inside its source buffer
// and write inside its LDS ring, the LDS must fit, and every LDS read must
// find its data in place and not rewritten while it is read (simulated op by
// op, independently of big_wait's closed form).  Exit status 0 = all hold.
#include <cstdio>
#include <utility>
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

// The many-row kernel's schedule for one shape S and one row length (NG4
// byte groups), simulated op by op.  Every wave (part P, block lb) issues its
// ops of each stage in order; the prologue's stages -PRO .. -1 end with one
// wait and a barrier, every main stage with the wait big_wait(j mod SPB) and
// a barrier.  A wait completes all but the last n of the wave's ops; an op
// may land at any time between its issue and the wait that completes it.
// Every LDS chunk is written by one wave only.  Time runs in half stages:
// 2j is the start of stage j (the byte group's reads of its codes and
// zero-point slab, before the stage issues anything), 2j + 1 the rest of it
// (its ops, then its compute); the barrier ending stage j is at 2j + 2.  A
// read of chunk T expecting data d during times t0 .. t1 holds when the last
// op into T issued before t0 carries d and is complete at a barrier no later
// than t0, and no op into T with other data is issued in t0 .. t1.  The
// reads: stage r reads the GPS x slabs of its groups during 2r + 1 (the
// first of them from 2r - 1 on when XW = 2: the next stage's first fragments
// are read before the barrier); byte group G's first stage reads the codes
// and pairs of every block and the zero-point slab of G at 2 SPB G.  Where
// one wave reads a block's codes (WPB = 1) it refills their slot in that same
// stage, after those reads.
struct SimOp {
  int time, data, done;   // time: 2 stage + 1; done: the time of the barrier completing it, or a large value
  int wave;
};
template <class S>
void check_big_k(int NG4) {
  constexpr int NBUF = S::XD + 1, SPB = S::SPB, MT = S::MT;
  const int NGRP = S::QPB * NG4, NST = SPB * NG4;
  // LDS chunk ids: x ring, then codes [slot][block][chunk], then zero point [slot][chunk]
  const int nx_chunks = NBUF * S::GPS * 4 * MT, ncode = S::CD * S::BPW * kCodeChunks;
  const int T_CODE = nx_chunks, T_ZP = nx_chunks + ncode, NT = T_ZP + S::ZPS * 4;
  std::vector<std::vector<SimOp>> tgt(NT);
  std::vector<int> writer(NT, -1);
  struct WaveState {
    std::vector<std::pair<int, int>> ops;   // (target, index in tgt[target])
    size_t done = 0;
  };
  std::vector<WaveState> waves(S::WPB * S::BPW);
  auto issue = [&](int wid, int j, int T, int data) {
    CHECK(T >= 0 && T < NT, "%d/%d NG4 %d: target %d\n", MT, S::QPB, NG4, T);
    if (T < 0 || T >= NT) return;
    CHECK(writer[T] < 0 || writer[T] == wid, "%d/%d: chunk %d written by two waves\n", MT, S::QPB, T);
    writer[T] = wid;
    tgt[T].push_back({2 * j + 1, data, 1 << 30, wid});
    waves[wid].ops.push_back({T, (int)tgt[T].size() - 1});
  };
  auto wait = [&](int wid, int n, int j) {
    WaveState& w = waves[wid];
    for (; w.done + n < w.ops.size(); ++w.done) tgt[w.ops[w.done].first][w.ops[w.done].second].done = 2 * j + 2;
  };
  // only: the one wave that reads the chunk (-1: every wave reads it).  An
  // op of another wave is ordered after the read only by a barrier, so for
  // it the read lasts to the end of its stage (t1 | 1); the reading wave's
  // own ops follow its reads in program order.
  auto read = [&](int T, int data, int t0, int t1, int only, const char* what) {
    const std::vector<SimOp>& v = tgt[T];
    int last = -1;
    for (int i = 0; i < (int)v.size(); ++i) {
      if (v[i].time < t0) last = i;
      else if (v[i].time <= (v[i].wave == only ? t1 : t1 | 1))
        CHECK(v[i].data == data, "%d/%d NG4 %d: %s chunk %d rewritten at time %d while read in %d..%d\n", MT,
              S::QPB, NG4, what, T, v[i].time, t0, t1);
    }
    CHECK(last >= 0 && v[last].data == data && v[last].done <= t0,
          "%d/%d NG4 %d: %s chunk %d (data %d) not in place for times %d..%d\n", MT, S::QPB, NG4, what, T, data, t0,
          t1);
  };
  auto issue_stage = [&](int j) {
    for (int P = 0; P < S::WPB; ++P)
      for (int lb = 0; lb < S::BPW; ++lb) {
        const int wid = P * S::BPW + lb;
        for (int k = 0; k < S::nx(P); ++k) {
          const XOp o = x_op<S>(j, lb, k, NGRP);
          CHECK(o.slab >= 0 && o.slab < NGRP && o.chunk >= 0 && o.chunk < 4 * MT,
                "%d/%d NG4 %d j %d: x op slab %d chunk %d\n", MT, S::QPB, NG4, j, o.slab, o.chunk);
          issue(wid, j, o.dst, o.slab * 64 + o.chunk);
        }
        if (stage_has_zp_ops<S>(j)) {
          const int GB = zp_group<S>(j, NG4), zs = zp_slot<S>(j);
          CHECK(GB >= 0 && GB < NG4 && zs >= 0 && zs < S::ZPS, "%d/%d NG4 %d j %d: zero-point ops GB %d slot %d\n", MT,
                S::QPB, NG4, j, GB, zs);
          for (int k = 0; k < S::nb(P); ++k) {
            const int c = lb * S::nb(P) + k;
            CHECK(c < 4, "%d/%d: zero-point chunk %d\n", MT, S::QPB, c);
            issue(wid, j, T_ZP + zs * 4 + c, GB * 4 + c);
          }
        }
        if (stage_has_code_ops<S>(j)) {
          const int GC = code_group<S>(j, NG4), cs = code_slot<S>(j);
          CHECK(GC >= 0 && GC < NG4 && cs >= 0 && cs < S::CD, "%d/%d NG4 %d j %d: code ops GC %d slot %d\n", MT,
                S::QPB, NG4, j, GC, cs);
          CHECK(S::CODE == S::BYTE || S::WPB == 1, "%d/%d: codes refilled before a barrier with two waves a block\n",
                MT, S::QPB);
          for (int k = 0; k < S::nc(P); ++k) issue(wid, j, T_CODE + (cs * S::BPW + lb) * kCodeChunks + k, GC * 16 + k);
        }
      }
  };
  auto wait_stage = [&](int j, int Q) {
    for (int P = 0; P < S::WPB; ++P)
      for (int lb = 0; lb < S::BPW; ++lb) wait(P * S::BPW + lb, P == 0 ? big_wait<S, 0>(Q) : big_wait<S, 1>(Q), j);
  };
  for (int j = -S::PRO; j < 0; ++j) issue_stage(j);
  wait_stage(-1, SPB - 1);
  for (int j = 0; j < NST; ++j) {
    issue_stage(j);
    wait_stage(j, j % SPB);
  }
  // the reads, checked against the whole history (a read looks only at the
  // ops issued up to the end of its window, and at the barrier before it)
  for (int G = 0; G < NG4; ++G) {   // byte group G's codes, pairs and zero-point slab, read at its start
    const int j = SPB * G;
    for (int lb = 0; lb < S::BPW; ++lb)
      for (int k = 0; k < kCodeChunks; ++k)
        read(T_CODE + ((G % S::CD) * S::BPW + lb) * kCodeChunks + k, G * 16 + k, 2 * j, 2 * j,
             S::WPB == 1 ? lb : -1, "code");   // read by the block's waves
    for (int c = 0; c < 4; ++c) read(T_ZP + (G % S::ZPS) * 4 + c, G * 4 + c, 2 * j, 2 * j, -1, "zero-point");
  }
  for (int j = 0; j < NST; ++j)
    for (int t = 0; t < S::GPS; ++t) {
      const int r0 = t == 0 && S::XW == 2 && j > 0 ? j - 1 : j;   // read during stages r0 .. j
      for (int cc = 0; cc < 4 * MT; ++cc)
        read(((j % NBUF) * S::GPS + t) * 4 * MT + cc, (S::GPS * j + t) * 64 + cc, 2 * r0, 2 * j + 1, -1, "x");
    }
}

template <class S>
void check_big() {
  const size_t lds = big_lds_bytes<S>();
  CHECK(lds <= 160 * 1024, "%d/%d: LDS %zu\n", S::MT, S::QPB, lds);
  CHECK((size_t)S::BPW * 16 * S::MT * 68 * 4 <= lds, "%d/%d: score area\n", S::MT, S::QPB);
  CHECK(S::W * 64 <= 1024 && S::GPS * S::SPB == S::QPB, "%d/%d: shape\n", S::MT, S::QPB);
  for (int Q = 0; Q < S::SPB; ++Q)
    for (int w : {big_wait<S, 0>(Q), big_wait<S, 1>(Q)}) CHECK(w >= 0 && w <= 63, "%d/%d: wait %d\n", S::MT, S::QPB, w);
  for (int NG4 = 1; NG4 <= 80; ++NG4) check_big_k<S>(NG4);   // row lengths up to 40960
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
  constexpr int W = h16_waves(MT), SLOTS = kH16Slots, WPB = 4 / h16_ntw(MT);
  const int NG4 = K / 512, NST = 4 * NG4;
  CHECK(h16_ring_bytes(MT) <= 160 * 1024 && (size_t)kH16Blocks * 16 * MT * 64 * 4 <= 160 * 1024, "h16 MT %d: LDS\n",
        MT);
  CHECK(h16_wait(MT, 0) <= 63 && h16_wait(MT, 1) <= 63, "h16 MT %d: wait range\n", MT);
  struct Op {
    int kind;   // 0: x chunk, 1: zero-point chunk, 2: code or pair chunk
    int data;   // x: slab * 64 + chunk; zero point: byte group * 4 + chunk; codes: byte group * 16 + chunk
    int slot;   // x: ring slot; zero point: slot 0 or 1; codes: the block (its code slot)
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
      for (int k = 0; k < h16_code_ops(MT); ++k) {
        const int ch = h16_code_chunk(MT, w % WPB, k);
        CHECK(ch >= 0 && ch < kCodeChunks, "h16: code chunk %d\n", ch);
        ops.push_back({2, Gc * 16 + ch, w / WPB});
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
      if (q == 0) {   // byte group G's codes (the chunks this wave reads) and zero-point chunk complete
        for (int k = 0; k < h16_code_ops(MT); ++k)
          CHECK(complete(2, G * 16 + h16_code_chunk(MT, w % WPB, k), w / WPB), "h16 MT %d K %d w %d: codes of %d\n",
                MT, K, w, G);
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
  for (int p = 0; p < WPB; ++p) {   // a wave fetches the chunks it reads: both halves of its tiles, and the pairs
    bool got[kCodeChunks] = {};
    for (int k = 0; k < h16_code_ops(MT); ++k) got[h16_code_chunk(MT, p, k)] = true;
    const int ntw = h16_ntw(MT);
    for (int h = 0; h < 2; ++h)
      for (int t = ntw * p; t < ntw * p + ntw; ++t)
        CHECK(got[h * 4 + t], "h16 MT %d: part %d misses chunk %d\n", MT, p, h * 4 + t);
    CHECK(got[8], "h16 MT %d: part %d misses the pairs\n", MT, p);
  }
  for (int c = 0; c < 4 * MT; ++c) {   // every chunk of a slab is some wave's
    bool any = false;
    for (int w = 0; w < W; ++w)
      for (int k = 0; k < h16_xops(MT); ++k) any |= h16_xchunk(MT, w, k) == c;
    CHECK(any, "h16 MT %d: chunk %d unfetched\n", MT, c);
  }
}

int main() {
  check_big<BigShape<1>>();
  check_big<BigShape<2>>();
  check_big<BigShape<3>>();
  check_big<BigShape<4>>();
  check_big<BigShape<5>>();
  check_big<BigShape<3, 2>>();   // a 4-bit head's two halves per byte group
  check_big<BigShape<4, 2>>();
  check_big<BigShape<5, 2>>();
  for (int K = 512; K <= 16384; K += 512) {   // the fp16 kernel's row lengths
    check_h16<3>(K);
    check_h16<4>(K);
    check_h16<5>(K);
  }
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
