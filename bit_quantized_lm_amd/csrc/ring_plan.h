// DMA ring schedule of the many-row coarse kernel: its shape per row-tile
// count, the wait counts, and the source and destination of every DMA op a
// wave issues.  Plain constexpr C++ with no HIP types, so the host tests
// compile it and check every op of every stage against the buffers it
// addresses.  Internal to the library (not part of the public ABI).
#pragma once

#include <stddef.h>

namespace dh {

constexpr int kMaxMT = 5;            // 16-row tiles per launch (80 rows)
constexpr int kCodeChunks = 9;       // 1 KB chunks of one block's byte group: 8 code + 1 pair
constexpr int kZpEntries = 256;      // zero-point slab entries (16 bytes)

// Groups of 128 k a byte group of the many-row kernel holds: a 2-bit head's
// four quarters; a 4-bit head's two halves (the code of k in one nibble, of
// K/2 + k in the other) from three row tiles on.  With one or two row tiles
// a 4-bit head keeps the 2-bit head's four stages per byte group, the last
// two without codes, so that its codes, in the single code slot there, have
// three stages to arrive instead of one.
constexpr int big_qpb(bool half, int MT) { return half && MT >= 3 ? 2 : 4; }

template <int MT_, int QPB_ = 4>
struct BigShape {
  static constexpr int MT = MT_;                    // 16-row tiles
  static constexpr int QPB = QPB_;                  // groups per byte group
  static constexpr int WPB = MT >= 3 ? 2 : 1;       // waves per block
  static constexpr int BPW = 4;                     // blocks per workgroup
  static constexpr int NTW = 4 / WPB;               // column tiles per wave
  static constexpr int W = BPW * WPB;               // waves per workgroup
  // x slabs and byte groups of codes requested ahead.  One or two row tiles
  // run four waves per workgroup: with one byte group of codes ahead (its
  // slot refilled after the first group of the byte group has read it) and,
  // at two tiles, three slabs, two workgroups fit a CU's LDS, so each SIMD
  // runs two waves instead of one (M = 16: 59.9 -> 43.7 us, M = 32: 76.6 ->
  // 58.2 us).  From three tiles on, two waves per block already fill that
  // (two workgroups of two blocks per CU, with one x slab ahead, measured
  // 2-3 % slower at M = 48 and 72 on the same box).
  // From four row tiles on a stage (the unit of the x ring, of the DMA
  // schedule and of the barriers) is two groups, so the eight waves meet at
  // half as many barriers; below, a stage is one group.  XD and XW count stages.
  static constexpr int GPS = MT >= 4 ? 2 : 1;       // groups per stage
  static constexpr int SPB = QPB / GPS;             // stages per byte group: 4, 2 or 1
  static constexpr int XD = MT >= 4 ? 1 : MT == 3 ? 5 : MT == 2 ? 3 : 6;
  static constexpr int CD = MT <= 2 ? 1 : 2;
  static constexpr int XW = XD >= 4 ? 2 : 1;        // stage's slabs completed XW stages ahead
  // Byte ops (zero-point slab, codes and pairs) are issued at the stages with
  // j mod SPB == BYTE, right after a barrier that every wave passes holding
  // the codes it read from the slot they refill.  With several stages per
  // byte group that is the barrier after the byte group's first stage, and
  // the codes of byte group G + CD go into the slot of G.  With one stage per
  // byte group it is the barrier that ended the previous byte group: the
  // codes of G + CD - 1 go into the slot of G - 1 (LAG = 1), and the
  // zero-point slab, read at the start of each byte group, has two slots.
  static constexpr int BYTE = 1 % SPB;
  static constexpr int LAG = SPB == 1 ? 1 : 0;
  static constexpr int ZPS = SPB == 1 ? 2 : 1;      // zero-point slots
  // With one wave per block a block's code slot is read by that wave alone,
  // at the start of the byte group: the wave refills it right after its own
  // reads (j mod SPB == 0, its LDS reads waited for), a stage earlier than
  // a barrier would allow; the zero-point slab, read by every wave, keeps
  // stage BYTE.
  static constexpr int CODE = WPB == 1 ? 0 : BYTE;
  // prologue stages: the x slabs of stages 0 .. XD - 1 and the codes of byte
  // groups 0 .. CD - LAG - 1 (issued at stage SPB (G - CD + LAG) + CODE)
  static constexpr int PRO_C = SPB * (CD - LAG) - CODE;
  static constexpr int PRO = XD > PRO_C ? XD : PRO_C;
  // DMA ops per iteration of a wave of part p.  With two waves per block the
  // parts issue different streams: part 1 the x slabs (chunks lb + BPW k),
  // part 0 its block's codes and scale pairs and its share of the zero-point
  // slab.  A wave's vmcnt completes in issue order, so a wait for an x slab
  // (an L2 read) never waits behind code bytes on their way from HBM, and the
  // codes get their full distance (CD byte groups) before anyone waits for
  // them.  With one wave per block every wave issues both.
  static constexpr int nx(int p) { return WPB == 1 || p == 1 ? GPS * 4 * MT / BPW : 0; }
  static constexpr int nc(int p) { return p == 0 ? kCodeChunks : 0; }
  static constexpr int nb(int p) { return p == 0 ? 4 / BPW : 0; }
};

template <class S>
constexpr size_t big_lds_bytes() {
  return (size_t)(S::XD + 1) * S::GPS * 4096 * S::MT + (size_t)S::CD * S::BPW * kCodeChunks * 1024 +
         (size_t)S::ZPS * kZpEntries * 16;
}

// floor(j / SPB) for any stage j (the prologue's are negative)
template <class S>
constexpr int stage_byte_group(int j) {
  return j >= 0 ? j / S::SPB : -((-j + S::SPB - 1) / S::SPB);
}
template <class S>
constexpr int stage_mod(int j) { return j - S::SPB * stage_byte_group<S>(j); }

// One stage's x-slab ops: stage j fetches the slabs of stage gx = j + XD into
// slot gx mod NBUF; before the start (gx < 0, prologue) a slot's first stage,
// which that slot receives again later.  Op k of a wave of block lb is chunk
// c = lb + BPW k of the stage's GPS slabs: slab t = c / (4 MT), chunk cc.
// NGRP: the slabs (groups) of the row, QPB per byte group.
struct XOp {
  int slab;    // source slab (group) index, clamped to the last group
  int chunk;   // 1 KB chunk of the slab (64 entries of 16 bytes)
  int dst;     // destination: 1 KB chunk index in the x ring
};
template <class S>
constexpr XOp x_op(int j, int lb, int k, int NGRP) {
  constexpr int NBUF = S::XD + 1, MT = S::MT;
  int gx = j + S::XD;
  if (gx < 0) gx = (gx % NBUF + NBUF) % NBUF;
  const int xslot = gx % NBUF;
  const int c = lb + S::BPW * k, t = c / (4 * MT), cc = c - t * 4 * MT;
  const int g = S::GPS * gx + t < NGRP - 1 ? S::GPS * gx + t : NGRP - 1;
  return XOp{g, cc, (xslot * S::GPS + t) * 4 * MT + cc};
}

// Whether stage j issues the zero-point slab's ops, and the codes' (after
// the zero-point slab's where a stage issues both).
template <class S>
constexpr bool stage_has_zp_ops(int j) {
  return stage_mod<S>(j) == S::BYTE;
}
template <class S>
constexpr bool stage_has_code_ops(int j) {
  return stage_mod<S>(j) == S::CODE;
}
// Byte group whose zero-point slab stage j fetches (the next one, clamped),
// and its slot.
template <class S>
constexpr int zp_group(int j, int NG4) {
  const int GB = stage_byte_group<S>(j) + 1;
  return GB < 0 ? 0 : GB < NG4 ? GB : NG4 - 1;
}
template <class S>
constexpr int zp_slot(int j) {
  return ((stage_byte_group<S>(j) + 1) % S::ZPS + S::ZPS) % S::ZPS;
}
// Byte group whose codes stage j fetches (CD - LAG ahead, clamped: a
// prologue stage before the first byte group's fetches byte group 0 into a
// slot that receives its own byte group later) and its slot.
template <class S>
constexpr int code_slot(int j) {
  return ((stage_byte_group<S>(j) + S::CD - S::LAG) % S::CD + S::CD) % S::CD;
}
template <class S>
constexpr int code_group(int j, int NG4) {
  const int GC = stage_byte_group<S>(j) + S::CD - S::LAG;
  return GC < 0 ? 0 : GC < NG4 ? GC : NG4 - 1;
}

// Ops a wave of part P may leave outstanding at the end of a stage with
// j mod SPB == Q: those issued after X(j + XW) and, for the byte group's last
// stage (Q == SPB - 1), after the zero-point slab and the codes of the next
// byte group, issued at stages BYTE and CODE + SPB (1 - CD + LAG) (relative
// to j - Q).  The prologue's final wait (X(XW - 1), codes and zero-point
// slab of byte group 0) is the Q == SPB - 1 case.
template <class S, int P>
constexpr int big_wait(int Q) {
  auto zc = [&](int j) { return stage_mod<S>(j) == S::BYTE ? S::nb(P) : 0; };
  auto cc = [&](int j) { return stage_mod<S>(j) == S::CODE ? S::nc(P) : 0; };
  auto cb = [&](int j) { return zc(j) + cc(j); };
  auto ops = [&](int j) { return S::nx(P) + cb(j); };
  auto after = [&](int j0, int in_iter) {   // ops after one issued in iteration j0
    int n = in_iter;
    for (int j = j0 + 1; j <= Q; ++j) n += ops(j);
    return n;
  };
  int best = 1 << 20;
  auto take = [&](int n) { best = n < best ? n : best; };
  if (S::nx(P)) take(after(Q + S::XW - S::XD, cb(Q + S::XW - S::XD)));
  if (Q == S::SPB - 1) {
    const int j0 = Q + 1 - S::SPB;   // the byte group's first stage
    const int jb = j0 + S::BYTE;     // the zero-point slab's stage
    if (S::nc(P)) take(after(j0 + S::CODE + S::SPB * (1 - S::CD + S::LAG), 0));   // codes: last in their stage
    if (S::nb(P)) take(after(jb, cc(jb)));   // followed by that stage's codes, if any
  }
  return best < 63 ? best : 63;   // 63: nothing this iteration must complete
}

// DMA schedule of the fp16 many-row kernel: kH16Blocks 64-column blocks a
// workgroup, each held by 4 / h16_ntw(MT) waves of h16_ntw(MT) column tiles
// (two waves a block up to four row tiles, where their registers allow four
// waves per SIMD; one at five); every wave issues the same number of ops in
// the same order.  Stage j = 4G + q (quarter q of byte group G) reads x slab
// j (group 4G + q) from slot j mod kH16Slots.  At its start a wave issues
// h16_xops(MT) ops of slab j + kH16XD (clamped to the last slab) into that
// slab's slot, and at q == 1 its byte ops for byte group G + 1 (clamped): one
// zero-point op (chunk wave mod 4 into zero-point slot (G + 1) mod 2), then
// the code chunks of its tiles and the block's pair chunk (h16_code_chunk)
// into its block's code slot.  At the end of the stage it waits until at
// most h16_wait(MT, q) of its ops are outstanding and meets the others at a
// barrier.  Chunks that several waves fetch (x chunks past the slab's, the
// zero-point chunks, a block's pair chunk) are the same bytes into the same
// place.
constexpr int kH16Blocks = 8;
constexpr int kH16XD = 2;
constexpr int kH16Slots = kH16XD + 1;
constexpr int h16_ntw(int MT) { return MT >= 5 ? 4 : 2; }                 // column tiles a wave
constexpr int h16_waves(int MT) { return kH16Blocks * 4 / h16_ntw(MT); }   // waves a workgroup
// a wave's code ops: every chunk of its block (one wave a block), or its two
// tiles' chunks of the two halves and the pair chunk
constexpr int h16_code_ops(int MT) { return h16_ntw(MT) == 4 ? kCodeChunks : 5; }
constexpr int h16_byte_ops(int MT) { return 1 + h16_code_ops(MT); }
constexpr int h16_xops(int MT) { return (4 * MT + h16_waves(MT) - 1) / h16_waves(MT); }
// chunk of a slab (of 4 MT) that op k of a wave fetches: past the slab, a
// repeat of chunk c - 4 MT (the same bytes into the same place)
constexpr int h16_xchunk(int MT, int wave, int k) {
  const int c = wave + h16_waves(MT) * k;
  return c >= 4 * MT ? c - 4 * MT : c;
}
// code chunk (h * 4 + t: half h of column tile t; 8: the block's pairs) of
// code op k of the wave of part p of its block (tiles p NTW .. p NTW + NTW - 1)
constexpr int h16_code_chunk(int MT, int p, int k) {
  return h16_ntw(MT) == 4 ? k : k < 4 ? (k >> 1) * 4 + 2 * p + (k & 1) : 8;
}
constexpr int h16_slab(int j, int nstage) { return j < nstage ? j : nstage - 1; }
constexpr int h16_byte_group(int G, int NG4) { return G < NG4 ? G : NG4 - 1; }
// Ops issued after slab j + 1's (and, at q == 3, after byte group G + 1's)
// by the end of stage j: the byte ops of stage j - 1 when it had q == 1, and
// this stage's x ops and, at q == 1, its byte ops.
constexpr int h16_wait(int MT, int q) { return q == 1 || q == 2 ? h16_xops(MT) + h16_byte_ops(MT) : h16_xops(MT); }
constexpr size_t h16_ring_bytes(int MT) {
  return (size_t)kH16Slots * MT * 4096 + (size_t)kH16Blocks * kCodeChunks * 1024 + (size_t)2 * kZpEntries * 16;
}

}  // namespace dh
