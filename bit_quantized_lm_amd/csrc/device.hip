// Device side of the draft-head library: HIP kernels for gfx950 (MI355X) and
// the validating C entry points that launch them.
//
// Per call (radiance_drafthead.py page, `_apply_head_int2`):
//   coarse_*_kernel scores x against the 2-bit weight and keeps the top KCAND
//                   columns of every 64-column block (`_draft_head_int2` + `_emit`)
//   rerank_kernel   row top-R of the candidates (`bm.topk` + `bi.gather`), then the
//                   exact fp32 dot of x with each one's bf16 row (`_rerank_exact`)
//   argmax_kernel   best reranked candidate per row
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "../../include/drafthead.h"
#include "common.h"
#include "ring_plan.h"
#include "select8.h"

namespace {

using dh::BigShape;
using dh::big_lds_bytes;
using dh::big_wait;
using dh::kCodeChunks;
using dh::kMaxMT;
using dh::kZpEntries;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Decode quarter q of two code dwords into four bf16 pairs holding v * 2^(2q-133).
//
// Code v of quarter q sits in bits 2q..2q+1 of each byte.  Masking a byte pair
// (bytes 0 and 2, or bytes 1 and 3 after a shift right by 8) with
// 0x00030003 << 2q leaves each code in place in a bf16 halfword whose exponent
// field is zero: for q < 3 that is the denormal v * 2^(2q-133); for q = 3 the
// code's high bit is the exponent's low bit, and 0x40 / 0x80 / 0xC0 read as
// 2^-127 / 2^-126 / 1.5 * 2^-126, i.e. again exactly v * 2^(6-133).  So one AND
// decodes two weights with no 1.0 bias to cancel (the page's bit-pattern
// decode produced 1 + v/4; this one produces v scaled by a power of two).
// The matrix cores keep bf16 denormal inputs, and x is staged scaled by 2^64
// so that the products stay normal fp32 values.  Element order of the result:
// byte {0, 2, 1, 3} of d0 then {0, 2, 1, 3} of d1 (the x fragments are staged
// in the same order); o0, o1 are d0 >> 8 and d1 >> 8.
__device__ __forceinline__ bf16x8 decode_quarter(uint32_t d0, uint32_t o0, uint32_t d1, uint32_t o1,
                                                 uint32_t mask) {
  u32x4 v = {d0 & mask, o0 & mask, d1 & mask, o1 & mask};
  return __builtin_bit_cast(bf16x8, v);
}

// A 4-bit head as draft_head_tile_int4 lays it out: the page's own code
// bytes (the code of k in bits 0..3, that of K/2 + k in bits 4..7), tiled as
// a 2-bit head of length 2K, whose quarters 0 and 1 cover the same k as the
// two nibbles (byte j, quarter q of that form: k' = j + q K/2).  Half H of a
// byte pair masked in place with 0x000F000F << 4H is a bf16 halfword holding
// v * 2^(4H-133): for H = 1 the code's high bit is the exponent's low bit,
// which reads the same way (a pattern b < 256 is the value b * 2^-133, as in
// quarter 3 above).  One AND per two weights, as for a quarter.
template <int H>
__device__ __forceinline__ bf16x8 decode_half4(uint32_t d0, uint32_t o0, uint32_t d1, uint32_t o1) {
  return decode_quarter(d0, o0, d1, o1, 0x000F000Fu << (4 * H));
}

constexpr int kXScaleLog2 = 64;   // x is staged as x * 2^64

// Multiplier turning the MFMA sum D = sum x 2^64 v 2^(2q-133) of quarter q into
// (S/4) sum x v: S * 2^(133 - 64 - 2q - 2).
__device__ __forceinline__ float quarter_scale(float S, int q) {
  return __builtin_ldexpf(S, 133 - kXScaleLog2 - 2 - 2 * q);
}
// The same for half H of a 4-bit head (decode_half4, v 2^(4H-133)): (S/16)
// sum x v, the page's 4-bit weight (S/16) v before its zero point.
__device__ __forceinline__ float half4_scale(float S, int H) {
  return __builtin_ldexpf(S, 133 - kXScaleLog2 - 4 - 4 * H);
}

// bf16 x (bits) scaled by 2^64, exactly (|x| < 2^63 stays finite).
__device__ __forceinline__ uint32_t scale_x_pair(uint32_t w) {
  const float lo = __builtin_ldexpf(lo_bf16(w), kXScaleLog2);
  const float hi = __builtin_ldexpf(hi_bf16(w), kXScaleLog2);
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// ---------------------------------------------------------------------------
// Coarse pass building blocks.
//
// A wave computes coarse scores of 64-column blocks for up to 16*MT rows with
// bf16 MFMA 16x16x32: the A operand is x * 2^64 (rows), the B operand the
// decoded codes v 2^(2q-133) (decode_quarter), one 16-column tile per MFMA,
// four tiles per block.  Lane (hh, nn) = (lane / 16, lane % 16) supplies row
// nn of A and column nn of B for k-slots 8hh..8hh+7; the accumulator holds
// rows 4hh + r, column nn.  K is walked as groups (byte group G, quarter q):
// code byte j of byte group G (j / 128 = G) carries one code of each of the
// groups q*NG4 + G.  After a group's MFMAs the accumulator takes the page's
// premultiplied pair, S * p - ZS * X with p = sum_k x (1 + v/4) and X =
// sum_k x, written for codes without the 1.0 bias: (S/4) sum_k x v - (ZS - S) X.
//
// x fragments live in LDS in the decode order: fragment f = (h*2 + e)*4 + s of
// a group holds x at k = q*K/4 + 128*G + 64h + 16s + 8e + {0,2,1,3,4,6,5,7}.

// Arguments of the rerank (row top-R of the candidates, exact logits, and
// with the argmax the per-row arrival counters).
// The rows the exact rerank reads: bf16 rows; e4m3 rows with a per-row fp32
// scale; or NVFP4 rows (e2m1 nibbles, an e4m3 scale per 16 elements, one
// global fp32 scale).
enum RowKind { kRowsBf16 = 0, kRowsE4m3 = 1, kRowsNvfp4 = 2 };
struct RowSrc {
  const void* w;          // bf16 rows (ldw elements), e4m3 rows (ldw bytes) or NVFP4 rows (ldw bytes)
  int64_t ldw;
  const float* wscale;    // e4m3: per-row scale
  const uint8_t* bscale;  // NVFP4: e4m3 scale per 16 elements, rows of lds bytes
  int64_t lds;
  const float* gscale;    // NVFP4: the global scale (one float)
  int kind;
};

struct RerankArgs {
  const uint16_t* x;
  RowSrc src;
  int K, N;
  const float* cand_val;
  const int32_t* cand_id;
  int nblk, kcand, R;
  int32_t* rr_id;
  float* rr_val;
  int32_t* out_id;
  float* out_val;
  unsigned long long* hand;   // per-row hand-off words (rows split over several workgroups)
  uint16_t* row_out;          // optional bf16 row [M][N]: each reranked id's exact value is written over it
  const float* bmax;          // optional [M][nblk]: the block maxima, contiguous (else read at slot b*kcand)
};

struct CoarseArgs {
  const uint16_t* x;
  int M, K, N, nblk;
  const u32x4* tiled;
  const u32x4* pairs;
  int kcand;
  float* cand_val;
  int32_t* cand_id;
  float* coarse_out;
  uint16_t* row_out;   // optional bf16 row [M][N] for the caller (the rerank scatters the exact values)
  int topk_only;       // row_out holds -inf instead of the coarse scores
  unsigned long long* hand;   // per-row hand-off words of the rerank; workgroup 0 zeroes hand[0..ncnt)
  int ncnt;
  int kx;          // row length of x: K, or K / 2 for a 4-bit head run at length K (x' = (x, x))
  int half_pairs;  // a 4-bit head (draft_head_tile_int4): code nibbles, pairs of quarters 0 and 1 only
  float* bmax;     // optional [M][nblk]: each block's maximum (its slot 0's value) once more, contiguous
};

// The rerank's per-row hand-off words are only ever written with agent-scope
// atomics (a plain store would leave a dirty L2 line whose later write-back
// could undo atomic updates made meanwhile on other XCDs).  The coarse kernel
// of each call zeroes them; the next kernel on the stream sees the zeros
// (kernel boundary).
__device__ __forceinline__ void zero_counters(const CoarseArgs& A) {
  if (blockIdx.x == 0 && (int)threadIdx.x < A.ncnt)
    __hip_atomic_store(A.hand + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A 4-bit head's pairs (draft_head_tile_int4): per (column, byte group) the
// head's own (S, ZS) of its two halves, in the slots of quarters 0 and 1;
// quarters 2 and 3 hold nothing (zero pairs: no code part, no zero point).
__device__ __forceinline__ u32x4 half_pairs4(u32x2 p) { return u32x4{p[0], p[1], 0u, 0u}; }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The optional outputs of a coarse score: the fp32 row, and the bf16 row the
// page hands to its caller (`_draft_head_int2`'s store of Y: the coarse score
// rounded to bf16, or -inf everywhere for a top-k caller), into which the
// rerank then writes the exact values.
// Whether the call wants the optional full outputs (uniform).  The epilogues
// test it once and store in a loop of their own, so that the common case runs
// no per-score branch.
__device__ __forceinline__ bool wants_scores(const CoarseArgs& A) { return A.coarse_out || A.row_out; }
__device__ __forceinline__ void store_scores(const CoarseArgs& A, int m, int n, float sv) {
  if (A.coarse_out) A.coarse_out[(size_t)m * A.N + n] = sv;
  if (A.row_out) A.row_out[(size_t)m * A.N + n] = (uint16_t)(A.topk_only ? 0xFF80u : f32_to_bf16_rne(sv));
}

// One group: MFMAs of the (h, e) fragments for all tiles, then the scale update.
// `xb` points at this lane's fragment 0 of the group (A row nn, k-slot hh),
// fragment f of M-tile i at xb[f * fstride + 16 * i]; `Xg` at the group's X[row].
// MFMA phase of one group (quarter Q of a byte group; Q < 0: quarter `q`
// known at run time): cg = sum over the group's k of x 2^64 * v 2^(2q-133);
// with kHalf, half q of a 4-bit head's bytes (v 2^(4q-133), decode_half4).
// The wave covers NT 16-column tiles; raw8 holds raw >> 8 (the odd byte pairs
// moved down), computed once per byte group.
template <int MT, int Q, int NT, bool kHalf = false>
__device__ __forceinline__ void group_mma(f32x4 (&cg)[MT][NT], const u32x4 (&raw)[2][NT],
                                          const u32x4 (&raw8)[2][NT], const u32x4* xb, int fstride,
                                          int q = Q) {
  const uint32_t mask = kHalf ? 0x000F000Fu << (4 * q) : 0x00030003u << (2 * q);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) cg[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      bf16x8 a[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        a[i] = __builtin_bit_cast(bf16x8, xb[(h * 2 + e) * 4 * fstride + 16 * i]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 bv = decode_quarter(raw[h][t][2 * e], raw8[h][t][2 * e], raw[h][t][2 * e + 1],
                                         raw8[h][t][2 * e + 1], mask);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          cg[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bv, cg[i][t], 0, 0, 0);
      }
    }
  }
}

// Scale phase of one group: acc += (S/4) sum x v - (ZS - S) sum x, with S, ZS
// the group's premultiplied pair (the page's S * p - ZS * X written for codes
// decoded without the 1.0 bias; with kHalf a 4-bit head's half, (S/16) sum x v).
// Rows 16i + 4hh + r, r < MR.
template <int MT, int MR, int Q, int NT, bool kHalf = false>
__device__ __forceinline__ void group_scale(f32x4 (&acc)[MT][NT], const f32x4 (&cg)[MT][NT],
                                            const u32x4 (&sz)[NT], const float* Xg, int hh, int q = Q) {
  float X[MT][MR];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < MR; ++r) X[i][r] = Xg[16 * i + 4 * hh + r];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint32_t pr;
    if constexpr (Q >= 0) pr = sz[t][Q];
    else pr = q == 0 ? sz[t][0] : q == 1 ? sz[t][1] : q == 2 ? sz[t][2] : sz[t][3];
    const float S = lo_bf16(pr);
    const float Sq = kHalf ? half4_scale(S, q) : quarter_scale(S, q), nzp = S - hi_bf16(pr);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < MR; ++r)
        acc[i][t][r] = __builtin_fmaf(nzp, X[i][r], __builtin_fmaf(Sq, cg[i][t][r], acc[i][t][r]));
  }
}

template <int MT, int MR, int Q, int NT>
__device__ __forceinline__ void coarse_group(f32x4 (&acc)[MT][NT], const u32x4 (&raw)[2][NT],
                                             const u32x4 (&raw8)[2][NT], const u32x4 (&sz)[NT],
                                             const u32x4* xb, int fstride, const float* Xg, int hh,
                                             int q = Q) {
  f32x4 cg[MT][NT];
  group_mma<MT, Q, NT>(cg, raw, raw8, xb, fstride, q);
  group_scale<MT, MR, Q, NT>(acc, cg, sz, Xg, hh, q);
}

template <int NT>
__device__ __forceinline__ void shift_codes(const u32x4 (&raw)[2][NT], u32x4 (&raw8)[2][NT]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) raw8[h][t][c] = raw[h][t][c] >> 8;
}

// All-reduce max / min over each 16-lane row of the wave with DPP lane moves
// (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror), which
// fold into the max / min instructions: every lane of the row ends with the
// row's result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, dpp_row<0xB1>(v));
  v = max(v, dpp_row<0x4E>(v));
  v = max(v, dpp_row<0x141>(v));
  v = max(v, dpp_row<0x140>(v));
  return v;
}
__device__ __forceinline__ uint32_t row16_min(uint32_t v) {
  v = min(v, dpp_row<0xB1>(v));
  v = min(v, dpp_row<0x4E>(v));
  v = min(v, dpp_row<0x141>(v));
  v = min(v, dpp_row<0x140>(v));
  return v;
}

// fp32 <-> unsigned key with the same order (finite values and -inf; key 0
// is below every value and marks a column past N).
__device__ __forceinline__ uint32_t f32_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// f32_key(f) where ok, else 0, computed without a branch (a guarded key
// makes the compiler wrap each one in a masked region of its own).
__device__ __forceinline__ uint32_t f32_key_if(bool ok, float f) { return f32_key(f + 0.0f) & (0u - (uint32_t)ok); }
__device__ __forceinline__ float key_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// (a & mask) | (b & ~mask): one bitfield-insert, and no branch.
__device__ __forceinline__ uint32_t bsel(uint32_t mask, uint32_t a, uint32_t b) {
  return (a & mask) | (b & ~mask);
}

// Epilogue of one block: optional full rows, then the top-kcand of the block
// (`_emit`), ordered by value desc, column asc.  The four rows
// m0 + 16i + 4hh + r of one pass (i, r) are handled at once, one per 16-lane
// row.  Each lane first sorts its four scores (stable, so equal scores keep
// column order); every round then takes the row's largest head and the
// lowest column among the lanes holding it, lane cc of the row keeps round
// cc's result, and the winning lane advances.  Rounds are branch-free and up
// to four passes run interleaved, so their cross-lane chains overlap.
// value(i, r, t): the coarse score of row m0 + 16i + 4hh + r, column
// 64b + 16t + nn.  Passes with r % rstep != rfirst are left to another wave.
// Slots past the block's valid columns get (-inf, -1).
// The selection rounds, for NB lists at a time per 16-lane row: lane nn of a
// row holds keys k[t] of columns c[t] (t = 0..3).  Each lane first sorts its
// four (stable on equal keys); each round then takes the row's largest head
// (row16_max) and the lowest column holding it (row16_min), lane cc keeps
// round cc's result and the winning lane advances.  On return lane nn holds
// the list's entry 16 sl + nn in kk[sl], kc[sl] (key 0: none).
template <int NB>
__device__ __forceinline__ void row16_select(uint32_t (&k)[NB][4], uint32_t (&c)[NB][4], int kcand, int nn,
                                             uint32_t (&kk)[NB][4], uint32_t (&kc)[NB][4]) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int t = 0; t < 4; ++t) kk[j][t] = kc[j][t] = 0u;
    auto ce = [&](int p) {   // neighbours p, p + 1: stable on equal keys
      const uint32_t sw = k[j][p + 1] > k[j][p] ? ~0u : 0u;
      const uint32_t tk = k[j][p], tc = c[j][p];
      k[j][p] = bsel(sw, k[j][p + 1], tk);
      c[j][p] = bsel(sw, c[j][p + 1], tc);
      k[j][p + 1] = bsel(sw, tk, k[j][p + 1]);
      c[j][p + 1] = bsel(sw, tc, c[j][p + 1]);
    };
    ce(0);
    ce(1);
    ce(2);
    ce(0);
    ce(1);
    ce(0);
  }
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    if (16 * sl >= kcand) break;
    const int nround = min(16, kcand - 16 * sl);
    for (int cc = 0; cc < nround; ++cc) {
      const uint32_t own = cc == nn ? ~0u : 0u;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint32_t mx = row16_max(k[j][0]);
        const uint32_t mc = row16_min(k[j][0] == mx ? c[j][0] : 64u);
        const uint32_t win = c[j][0] == mc ? ~0u : 0u;   // the winner's next score becomes its head
        k[j][0] = bsel(win, k[j][1], k[j][0]);
        k[j][1] = bsel(win, k[j][2], k[j][1]);
        k[j][2] = bsel(win, k[j][3], k[j][2]);
        k[j][3] = k[j][3] & ~win;
        c[j][0] = bsel(win, c[j][1], c[j][0]);
        c[j][1] = bsel(win, c[j][2], c[j][1]);
        c[j][2] = bsel(win, c[j][3], c[j][2]);
        c[j][3] = bsel(win, 64u, c[j][3]);
        kk[j][sl] = bsel(own, mx, kk[j][sl]);
        kc[j][sl] = bsel(own, mc, kc[j][sl]);
      }
    }
  }
}

// Lane nn's entries of the list of (row m, block b): slots 16 sl + nn.
__device__ __forceinline__ void write_list(const CoarseArgs& A, int m, int b, const uint32_t (&kk)[4],
                                           const uint32_t (&kc)[4], int nn) {
  const float NEG_INF = -__builtin_inff();
  const size_t base = (size_t)m * A.nblk * A.kcand + (size_t)b * A.kcand;
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    const int cs = 16 * sl + nn;
    if (cs < A.kcand) {
      A.cand_val[base + cs] = kk[sl] ? key_f32(kk[sl]) : NEG_INF;
      A.cand_id[base + cs] = kk[sl] ? b * 64 + (int)kc[sl] : -1;
    }
  }
  if (A.bmax && nn == 0) A.bmax[(size_t)m * A.nblk + b] = kk[0] ? key_f32(kk[0]) : NEG_INF;
}

// Top-kcand of block b for the rows a wave's accumulators hold: rows m0 + 16 i
// + 4 hh + r, one list per 16-lane row and pass, up to four passes at once
// so that the cross-lane chains overlap.  Keys are order-preserving unsigned
// images of the fp32 scores; ties go to the lower column.
template <int MT, int MR, class Value>
__device__ __forceinline__ void block_select(Value value, const CoarseArgs& A, int b, int hh, int nn,
                                             int rfirst = 0, int rstep = 1, int m0 = 0) {
  constexpr int NP = MT * MR, NB = NP < 4 ? NP : 4;   // passes, passes per batch
#pragma unroll
  for (int p0 = 0; p0 < NP; p0 += NB) {
    uint32_t k[NB][4], c[NB][4], kk[NB][4], kc[NB][4];
    bool live[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int pi = p0 + j, i = pi / MR, r = pi % MR;
      live[j] = pi < NP && m0 + 16 * i + r < A.M && r % rstep == rfirst;   // wave-uniform
      const int m = m0 + 16 * i + 4 * hh + r;
      const bool row_ok = live[j] && m < A.M;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = b * 64 + 16 * t + nn;
        const bool ok = row_ok && n < A.N;
        k[j][t] = f32_key_if(ok, pi < NP ? value(i, r, t) : 0.f);   // -0 counts as +0, as in a float compare
        c[j][t] = 16 * t + nn;
      }
    }
    if (wants_scores(A)) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int pi = p0 + j, i = pi / MR, r = pi % MR;
        const int m = m0 + 16 * i + 4 * hh + r;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int n = b * 64 + 16 * t + nn;
          if (live[j] && m < A.M && n < A.N) store_scores(A, m, n, value(i, r, t));
        }
      }
    }
    bool any = false;
#pragma unroll
    for (int j = 0; j < NB; ++j) any |= live[j];
    if (!any) continue;
    row16_select<NB>(k, c, A.kcand, nn, kk, kc);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int pi = p0 + j, i = pi / MR, r = pi % MR;
      const int m = m0 + 16 * i + 4 * hh + r;
      if (live[j] && m < A.M) write_list(A, m, b, kk[j], kc[j], nn);
    }
  }
}

// The resident kernel's selection: the lists of all (block, row) pairs of the
// workgroup, read from LDS (sc: [kBlocks][MP][64] scores), packed densely
// onto the 16-lane rows of the waves (list q = 4 (wave + W pass) + hh is row
// q % M of block q / M), so that each selection round serves four lists.
template <int MP, int kBlocks, int W>
__device__ __forceinline__ void res_select(const float* sc, const CoarseArgs& A, int b0, int wave, int hh,
                                           int nn) {
  constexpr int NB = (kBlocks * MP + 4 * W - 1) / (4 * W);   // passes per wave
  const int nl = kBlocks * A.M;
  if (4 * wave >= nl) return;   // wave-uniform: no list in any pass
  uint32_t k[NB][4], c[NB][4], kk[NB][4], kc[NB][4];
  int lbq[NB], mq[NB];
  bool live[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int q = 4 * (wave + W * j) + hh;
    lbq[j] = q / A.M;
    mq[j] = q - lbq[j] * A.M;
    live[j] = q < nl && b0 + lbq[j] < A.nblk;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = (b0 + lbq[j]) * 64 + 16 * t + nn;
      const bool ok = live[j] && n < A.N;
      const int li = live[j] ? lbq[j] * MP + mq[j] : 0;   // a row in the score area either way
      k[j][t] = f32_key_if(ok, sc[li * 64 + 16 * t + nn]);   // -0 counts as +0, as in a float compare
      c[j][t] = 16 * t + nn;
    }
  }
  if (wants_scores(A)) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = (b0 + lbq[j]) * 64 + 16 * t + nn;
        if (live[j] && n < A.N) store_scores(A, mq[j], n, sc[(lbq[j] * MP + mq[j]) * 64 + 16 * t + nn]);
      }
  }
  row16_select<NB>(k, c, A.kcand, nn, kk, kc);
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (live[j]) write_list(A, mq[j], b0 + lbq[j], kk[j], kc[j], nn);
}

// Convert 8 natural-order bf16 x values into the decode order {0,2,1,3,4,6,5,7},
// scaled by 2^64, and return the fp32 sum of the unscaled values.
__device__ __forceinline__ u32x4 permute_x(const u32x4 v, float& sum) {
  u32x4 o;
  o[0] = scale_x_pair((v[0] & 0xFFFFu) | (v[1] << 16));
  o[1] = scale_x_pair((v[0] >> 16) | (v[1] & 0xFFFF0000u));
  o[2] = scale_x_pair((v[2] & 0xFFFFu) | (v[3] << 16));
  o[3] = scale_x_pair((v[2] >> 16) | (v[3] & 0xFFFF0000u));
  sum = lo_bf16(v[0]) + hi_bf16(v[0]) + lo_bf16(v[1]) + hi_bf16(v[1]) + lo_bf16(v[2]) +
        hi_bf16(v[2]) + lo_bf16(v[3]) + hi_bf16(v[3]);
  return o;
}

// Sum over the 16 lanes of a DPP row (the 16 pieces of one group of one row),
// by DPP moves (lane pairs 1 apart, 2 apart, then the half rows and the row
// mirrored): the tree of an xor butterfly, so every lane gets the same sum,
// without the LDS round trips of a shuffle.
__device__ __forceinline__ float row16_sum(float s) {
  s += __uint_as_float(dpp_row<0xB1>(__float_as_uint(s)));
  s += __uint_as_float(dpp_row<0x4E>(__float_as_uint(s)));
  s += __uint_as_float(dpp_row<0x141>(__float_as_uint(s)));
  s += __uint_as_float(dpp_row<0x140>(__float_as_uint(s)));
  return s;
}

// Lane l's value, in every lane (a lane read, not a shuffle through LDS).
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Maximum over the wave (every lane active): over each DPP row, then the
// four rows' by lane reads.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_row<0xB1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_row<0x4E>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_row<0x141>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_row<0x140>(__float_as_uint(v))));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// ---------------------------------------------------------------------------
// Coarse kernel, x resident in LDS (M <= 8 and the whole x fits).
//
// 4/NT waves share a 64-column block, each computing NT of its four 16-column
// tiles, so a wave needs few registers and many waves fit per SIMD.  The
// workgroup stages all of x once (MP rows, MP = the next power of two >= M;
// lanes whose A row nn >= MP read row nn & (MP-1), whose results are never
// used) with the group sums X.  Then every wave streams its tiles with no
// further barrier, keeping the codes and scale pairs of the next byte groups
// in flight in a ring of D register sets (D-1 groups ahead at one row, D from
// two rows on).  At the end the scores of every tile meet in LDS and the
// workgroup's (block, row) lists are selected, four per wave at a time.
// LDS: x fragments [group it = 4G + q][f][MP] (16 bytes each), X[it][MP], then
// the block scores [block][MP rows][64 columns].
constexpr int kResDepth = 2;   // ring sets of byte groups held in registers

// Two tiles per wave, so that four waves fit each SIMD and hide each other's
// latency (four tiles per wave, two waves per SIMD, measured 1.1-4.0 us
// slower at three to eight rows).  Eight waves (four blocks) per workgroup up
// to four rows, two workgroups per CU; sixteen (eight blocks) at eight rows,
// where x of eight rows leaves LDS for one workgroup per CU.
constexpr int res_nt(int MP) { return 2; }
constexpr int res_waves_of(int MP) { return MP == 8 ? 16 : 8; }

template <int MP>
constexpr int res_waves() { return res_waves_of(MP); }
// Waves per SIMD the grid needs to be resident at once (1940 blocks at the
// page's N): four.
template <int MP>
constexpr int res_min_waves() { return 4; }

template <int MP, bool kHalf>
__global__ __launch_bounds__(64 * res_waves<MP>()) __attribute__((amdgpu_waves_per_eu(res_min_waves<MP>())))
void coarse_resident_kernel(CoarseArgs A) {
  constexpr int kResWaves = res_waves<MP>();
  constexpr int kResThreads = 64 * kResWaves;
  constexpr int NT = res_nt(MP), D = kResDepth;
  constexpr int kWavesPerBlock = 4 / NT;
  constexpr int kBlocks = kResWaves / kWavesPerBlock;
  constexpr int MR = MP < 4 ? MP : 4;  // accumulator rows r that can hold a live row
  extern __shared__ __align__(16) unsigned char smem[];
  const int NG4 = A.K >> 9, Q4 = A.K >> 2;
  // x rows of length kx < K (a 4-bit head in the tiles of a 2-bit head of
  // length 2K): only quarters 0 and 1, its two halves, carry codes, so only
  // their x is staged (QN = 2 quarters per byte group; else 4).
  const int QN = A.kx < A.K ? 2 : 4, NGS = A.kx >> 7;   // staged quarters, staged groups
  u32x4* xs = reinterpret_cast<u32x4*>(smem);                               // [NGS][16][MP]
  float* Xs = reinterpret_cast<float*>(smem + (size_t)NGS * 16 * MP * 16);      // [NGS][MP]
  float* sel = Xs + (size_t)NGS * MP;                                          // [kBlocks][MP][64]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 4, nn = lane & 15;
  const int lblk = wave / kWavesPerBlock, part = wave % kWavesPerBlock;
  const int b = blockIdx.x * kBlocks + lblk;
  const bool blk_ok = b < A.nblk;
  zero_counters(A);

  // A wave past the last block reads block 0 (valid memory) and writes nothing.
  const u32x4* tp = A.tiled + (size_t)(blk_ok ? b : 0) * NG4 * 512 + NT * part * 64;
  const u32x4* pp = A.pairs + (size_t)(blk_ok ? b : 0) * NG4 * 64 + NT * part * 16;
  const u32x2* pp2 = reinterpret_cast<const u32x2*>(A.pairs) + (size_t)(blk_ok ? b : 0) * NG4 * 64 + NT * part * 16;
  // codes and scale pairs are read once per call: nontemporal loads keep them
  // from displacing x and the candidates in the caches
  auto load_codes = [&](int G, u32x4 (&raw)[2][NT], u32x4 (&sz)[NT]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < NT; ++t) raw[h][t] = __builtin_nontemporal_load(tp + ((G * 2 + h) * 4 + t) * 64 + lane);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (kHalf) sz[t] = half_pairs4(__builtin_nontemporal_load(pp2 + (G * 4 + t) * 16 + nn));
      else sz[t] = __builtin_nontemporal_load(pp + (G * 4 + t) * 16 + nn);
    }
  };

  u32x4 rw[D][2][NT], sw[D][NT];   // ring: set (G mod D) holds byte group G

  // stage x: piece i = (m, k0 = 8p) for all MP rows (zero rows past M).  Loads
  // are issued kBatch at a time from clamped (always valid) addresses: at
  // K = 5120 all of x in one round (1.0 us less at four rows than rounds of
  // four loads).  The
  // first byte groups' codes are requested right after the first batch of x,
  // so that x (from L2) is not waited for behind them.
  {
    constexpr int kBatch = MP <= 2 ? 4 : 5;
    const int per_row = A.kx >> 3;
    const int total = MP * per_row;
    auto issue_x = [&](int base, u32x4 (&v)[kBatch]) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = min(base + tid + j * kResThreads, total - 1);
        const int m = i / per_row, k0 = (i - m * per_row) * 8;
        v[j] = *reinterpret_cast<const u32x4*>(A.x + (size_t)(m < A.M ? m : 0) * A.kx + k0);
      }
    };
    // Only the LDS writes are predicated: a load whose value were used only
    // under the predicate could be sunk by the compiler behind the code loads.
    auto use_x = [&](int base, const u32x4 (&v)[kBatch]) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = base + tid + j * kResThreads;
        const int ic = min(i, total - 1);
        const int m = ic / per_row, k0 = (ic - m * per_row) * 8;
        const u32x4 vm = m < A.M ? v[j] : u32x4{0u, 0u, 0u, 0u};
        const int q = k0 / Q4, G = (k0 - q * Q4) >> 7, p = (k0 >> 3) & 15;
        const int it = G * QN + q;
        float sum;
        const u32x4 o = permute_x(vm, sum);
        sum = row16_sum(sum);
        if (i < total) {   // uniform per 16-lane row: total is a multiple of 16
          const int h = p >> 3, s = (p >> 1) & 3, e = p & 1;
          xs[(it * 16 + (h * 2 + e) * 4 + s) * MP + m] = o;
          if (p == 0) Xs[it * MP + m] = sum;
        }
      }
    };
    u32x4 v[kBatch];
    issue_x(0, v);
    // The first D-1 byte groups at one row; from two rows on the first D,
    // unconditionally (a guarded load makes the compiler wait for it before
    // x can be used; with a single byte group, K = 512, the second set
    // re-reads the first).
    if constexpr (MP == 1) {
#pragma unroll
      for (int d = 0; d < D - 1; ++d)
        if (d < NG4) load_codes(d, rw[d], sw[d]);
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) load_codes(min(d, NG4 - 1), rw[d], sw[d]);
    }
    use_x(0, v);
    for (int base = kResThreads * kBatch; base < total; base += kResThreads * kBatch) {
      issue_x(base, v);
      use_x(base, v);
    }
  }
  __syncthreads();

  f32x4 acc[1][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int arow = nn & (MP - 1);
  auto byte_group = [&](int G, const u32x4 (&raw)[2][NT], const u32x4 (&sz)[NT]) {
    const u32x4* xb = xs + (size_t)(G * QN * 16 + hh) * MP + arow;
    const float* Xg = Xs + G * QN * MP + ((4 * hh) & (MP - 1));
    u32x4 raw8[2][NT];
    shift_codes(raw, raw8);
    // each group's scale update is issued after the next group's MFMAs, so it
    // does not wait on results that were just issued
    f32x4 c0[1][NT], c1[1][NT];
    if constexpr (kHalf) {   // a 4-bit head: its two halves, whole codes
      group_mma<1, 0, NT, true>(c0, raw, raw8, xb, MP);
      group_mma<1, 1, NT, true>(c1, raw, raw8, xb + 16 * MP, MP);
      group_scale<1, MR, 0, NT, true>(acc, c0, sz, Xg, 0);
      group_scale<1, MR, 1, NT, true>(acc, c1, sz, Xg + MP, 0);
    } else {
      group_mma<1, 0, NT>(c0, raw, raw8, xb, MP);
      group_mma<1, 1, NT>(c1, raw, raw8, xb + 16 * MP, MP);
      group_scale<1, MR, 0, NT>(acc, c0, sz, Xg, 0);
      group_mma<1, 2, NT>(c0, raw, raw8, xb + 32 * MP, MP);
      group_scale<1, MR, 1, NT>(acc, c1, sz, Xg + MP, 0);
      group_mma<1, 3, NT>(c1, raw, raw8, xb + 48 * MP, MP);
      group_scale<1, MR, 2, NT>(acc, c0, sz, Xg + 2 * MP, 0);
      group_scale<1, MR, 3, NT>(acc, c1, sz, Xg + 3 * MP, 0);
    }
  };
  // Two forms of the same stream.  From two rows on, each ring set is
  // refilled right after its byte group is done, so D byte groups are in
  // flight while one is waited for.  Its steady state loads unconditionally,
  // so that every wait is exact (a guarded load makes the compiler wait as if
  // it had not been issued), and scheduling barriers keep the loads where
  // they are (sunk towards their first use they would no longer be ahead;
  // mixed into the byte group's work they would need other registers than
  // the ring's, copied back after a wait).  At one row that form needs more
  // than the 128 registers that four waves per SIMD allow (the compiler then
  // spills), so one row keeps the guarded form, D-1 byte groups ahead (its
  // extra waits measured no slower there than exact ones).
  if constexpr (MP == 1) {
    for (int G0 = 0; G0 < NG4; G0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int G = G0 + d;
        if (G + D - 1 < NG4) load_codes(G + D - 1, rw[(d + D - 1) % D], sw[(d + D - 1) % D]);
        if (G < NG4) byte_group(G, rw[d], sw[d]);
      }
    }
  } else {
    int G0 = 0;
    for (; G0 + 2 * D - 1 < NG4; G0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        byte_group(G0 + d, rw[d], sw[d]);
        __builtin_amdgcn_sched_barrier(0);
        load_codes(G0 + d + D, rw[d], sw[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < 2 * D - 1; ++d) {
      const int G = G0 + d;
      if (G < NG4) byte_group(G, rw[d % D], sw[d % D]);
      if (G + D < NG4) load_codes(G + D, rw[d % D], sw[d % D]);
    }
  }

  // Every wave puts the scores of its tiles' live rows in LDS; after one
  // barrier the (block, row) lists are selected four at a time per wave.
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const int row = 4 * hh + r;
      if (row < MP) sel[(lblk * MP + row) * 64 + 16 * (NT * part + t) + nn] = acc[0][t][r];
    }
  __syncthreads();
  res_select<MP, kBlocks, kResWaves>(sel, A, blockIdx.x * kBlocks, wave, hh, nn);
}

// ---------------------------------------------------------------------------
// Coarse kernel for more rows (up to 80 per launch, MT 16-row tiles).
//
// The page's accumulator form, S * p - ZS * X per group, is computed in two
// parts.  The code part, (S/4) sum_k x v, is one MFMA chain per group, scaled
// on the accumulator with one FMA per score.  The zero-point part, the sum
// over groups of (S - ZS) X, is itself a small matrix product: per byte group
// one more MFMA per tile, whose live k-slots pair each quarter's S - ZS with
// that group's sum X.  S - ZS is exact in bf16 (ZS lies in [S, 2S), so the
// difference is a multiple of S's last place and smaller than S), and X is
// split into three bf16 parts whose sum is X to 2^-27 relative, so every
// product is exact and only fp32 sums round.
//
// prep_x_kernel writes x for one launch into the caller's workspace in the
// order the kernel consumes it, rows >= M zero (MP = 16 MT rows; QPB groups
// per byte group, dh::big_qpb: four quarters, or a 4-bit head's two halves):
//   x slab of group g = QPB G + q (byte group G, quarter q): 16 fragments x
//     MP rows, 16 bytes each, x * 2^64 in decode order (256 MT entries);
//   zero-point slab of byte group G: 256 entries; entry hh*MP + m (hh < 2)
//     holds row m's k-slots 8hh..8hh+7 of that product:
//     X_hi(q0..q3) X_mid(q0..q3) | X_lo(q0..q3) 0 0 0 0 (X of q >= QPB: 0).
//
// Workgroup = 4 blocks of 64 columns.  From MT = 3 on, two waves share a
// block, wave (block lb, part p) holding column tiles 2p and 2p + 1 for all
// MT row tiles, so each weight fragment is decoded once (a split by rows
// would have both waves decode every fragment) and the two waves a SIMD runs
// (lb and lb + 4) hide each other's latency; their scores meet in LDS for the
// selection.  Below that, one wave per block holds all four column tiles and
// two workgroups share a CU.
// Each group's scale update (one FMA per score) is issued during the next
// group's MFMAs, component ks of every tile in k-slice ks, so the VALU work
// runs beside the matrix cores instead of between two MFMA phases.
//
// Every global read of the main loop is a direct-to-LDS DMA.  Stage j (GPS
// groups, GPS = 1 or 2, SPB = QPB / GPS stages per byte group; j < 0: the
// prologue) issues, in this order and every time, even where the data does
// not exist (then a harmless copy into a slot that is free, or that later
// receives the same bytes):
//   X(j + XD)  the wave's chunks of that stage's x slabs               NX ops
//   at j = SPB G + 1 (after every wave read byte group G's codes; with one
//   stage per byte group, at j = G, after the barrier that ended G - 1):
//   B(G + 1)   its chunks of byte group G + 1's zero-point slab       NB ops
//   C(G + CD)  the wave's chunks of that byte group's codes/pairs      NC ops
//              (G + CD - 1 with one stage per byte group)
// and ends with one vmcnt wait that completes X(j + XW) and, at the end of a
// byte group, C and B of the next one, then a barrier.  With XW = 2 the
// next stage's first x fragments are read before that barrier.  The number
// of ops issued after any op depends only on j mod SPB, so every wait count
// is a constant (big_wait).  Completions are counted in issue order, so with two
// waves per block the x slabs and the codes are issued by different waves
// (BigShape::nx, nc): a wait for an x slab (an L2 hit) never waits for code
// bytes still on their way from HBM, and the codes have CD byte groups to
// arrive.  With one wave per block (one or two row tiles) both streams share
// the wave's counter, and x runs XD = 3..6 stages (groups) ahead.
// Workspace of one launch with MT row tiles: x slabs, zero-point slabs, then
// the rows' scale exponents (fp16 kernel).
constexpr size_t kFexpBytes = 512;
size_t big_workspace_bytes(int MT, int K) {
  return (size_t)(K / DH_GROUP) * 4096 * MT + (size_t)(K / 512) * kZpEntries * 16 + kFexpBytes;
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One direct-to-LDS DMA op: lane l's 16 bytes at base + voff land at
// lds + 16 l (base and lds wave-uniform; voff = 16 l).  The nontemporal form
// is for data read once per call (codes, scale pairs).
__device__ __forceinline__ void dma16(uint32_t voff, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_nt(uint32_t voff, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// One wave per (m, G): lane q * 16 + p takes piece p (8 consecutive k) of
// group 4G + q of row m, so every lane issues one load and one store and the
// 16 lanes of a group sum its x in one DPP reduction; lanes 0 and 1 gather the
// four group sums for the zero-point slab.  x has rows of kx elements;
// element k of x' is x[k mod kx] (kx = K, or K/2).
__global__ __launch_bounds__(256) void prep_x_kernel(const uint16_t* __restrict__ x, int M, int MP, int K, int kx,
                                                     int qpb, u32x4* __restrict__ xslab, u32x4* __restrict__ zslab) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int NG4 = K >> 9, Q4 = K >> 2;
  if (w >= MP * NG4) return;   // whole waves leave together
  const int G = w % NG4, m = w / NG4, q = lane >> 4, p = lane & 15;
  const int h = p >> 3, s = (p >> 1) & 3, e = p & 1, f = (h * 2 + e) * 4 + s;
  const int k = q * Q4 + 128 * G + 8 * p;
  const u32x4 v = m < M ? *reinterpret_cast<const u32x4*>(x + (size_t)m * kx + (k < kx ? k : k - kx))
                        : u32x4{0u, 0u, 0u, 0u};
  float sum;
  const u32x4 xv = permute_x(v, sum);
  if (q < qpb) xslab[((size_t)(qpb * G + q) * 16 + f) * MP + m] = xv;
  sum = row16_sum(sum);
  float X[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) X[u] = u < qpb ? lane_value(sum, 16 * u) : 0.f;
  if (lane < 2) {
    uint32_t part[3][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float r = X[u];
#pragma unroll
      for (int c = 0; c < 3; ++c) {   // r - bf16(r) is exact in fp32
        part[c][u] = f32_to_bf16_rne(r);
        r -= __uint_as_float(part[c][u] << 16);
      }
    }
    const u32x4 o = lane == 0 ? u32x4{part[0][0] | part[0][1] << 16, part[0][2] | part[0][3] << 16,
                                      part[1][0] | part[1][1] << 16, part[1][2] | part[1][3] << 16}
                              : u32x4{part[2][0] | part[2][1] << 16, part[2][2] | part[2][3] << 16, 0u, 0u};
    zslab[(size_t)G * kZpEntries + lane * MP + m] = o;
  }
}

struct BigArgs {
  CoarseArgs c;
  const u32x4* xslab;
  const u32x4* zslab;
};

// The many-row kernel's score area in LDS holds, per (block, row), the 64
// order-preserving keys of the row's coarse scores (f32_key of the score, -0
// as +0; 0 for a column past N), rows kScStride words apart: a multiple of
// four, so a row is read in 16-byte pieces, and 68 mod 64 = 4, so the rows of
// sixteen neighbouring lists cover the 64 banks once.
constexpr int kScStride = 68;

// The top-kcand list (kcand <= 8) of row m, block b, selected by this thread
// alone from the row's 64 keys in LDS: load_at(r, raw) the keys of run r,
// tag_at(r, e) 63 - the column of its element e, key_at(c) column c's key (select8_runs;
// the run loop is rolled: the epilogue runs once per kernel, and its
// unrolled code would mostly wait for instruction fetch).  The values written
// are the keys' scores times `scale` (a power of two: exact, order kept).
template <class LoadAt, class TagAt, class KeyAt>
__device__ __forceinline__ void emit_list8(LoadAt load_at, TagAt tag_at, KeyAt key_at, const CoarseArgs& A, int m,
                                           int b, float scale = 1.0f) {
  uint32_t slot[8];   // 63 - column, or 64 for an empty slot
  dh::select8_runs<true>(load_at, tag_at, key_at, slot);
  float val[8];
  int32_t id[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ok = slot[i] < 64u;
    const int col = 63 - (int)(ok ? slot[i] : 63u);
    // read for every slot (column 0 for an empty one) and selected by bits,
    // so that the eight reads are in flight together (a conditional read
    // becomes a branch and a wait of its own)
    const uint32_t kv = key_at(col), okm = 0u - (uint32_t)ok;
    val[i] = __uint_as_float((__float_as_uint(key_f32(kv) * scale) & okm) | (0xFF800000u & ~okm));   // else -inf
    id[i] = (int)(((uint32_t)(b * 64 + col) & okm) | ~okm);                                 // else -1
  }
  const size_t base = ((size_t)m * A.nblk + b) * A.kcand;
  if (A.bmax) A.bmax[(size_t)m * A.nblk + b] = val[0];
  if (A.kcand == 8) {   // 32-byte aligned: the list is two 16-byte pieces
    reinterpret_cast<f32x4*>(A.cand_val + base)[0] = f32x4{val[0], val[1], val[2], val[3]};
    reinterpret_cast<f32x4*>(A.cand_val + base)[1] = f32x4{val[4], val[5], val[6], val[7]};
    reinterpret_cast<u32x4*>(A.cand_id + base)[0] =
        u32x4{(uint32_t)id[0], (uint32_t)id[1], (uint32_t)id[2], (uint32_t)id[3]};
    reinterpret_cast<u32x4*>(A.cand_id + base)[1] =
        u32x4{(uint32_t)id[4], (uint32_t)id[5], (uint32_t)id[6], (uint32_t)id[7]};
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < A.kcand) {
        A.cand_val[base + i] = val[i];
        A.cand_id[base + i] = id[i];
      }
  }
}

// Top-kcand lists (kcand <= 8) of every (block, row) pair of a many-row
// workgroup, one list per thread, from the keys in LDS (row lb * MP + m).
// Each key's low 6 bits are replaced by 63 - column, so the keys of a row are
// distinct and, between scores whose keys differ above bit 5, order as (score
// desc, column asc).  Eight sorted runs of eight (Batcher's network) are merged
// into the eight largest (bitonic merge of the current eight with the next
// run reversed), tracking the largest key left out.  That is the exact list
// unless two of the eight, or the eighth and the best key left out, agree
// above bit 5 (scores within 63 units in the last place of each other); such
// a list is rebuilt with 64-bit keys (full key, then 63 - column) over the
// columns whose keys reach the eighth's upper bits.
// Lists go to the first min(W, 4) waves (one per SIMD) while they fit, else
// to all W; wave w takes the consecutive lists w * cnt .. w * cnt + cnt - 1.
template <int MP, int BPW>
__device__ __forceinline__ void lane_select8(const uint32_t* sk, const CoarseArgs& A, int b0, int wave, int W,
                                             int lane) {
  const int nl = BPW * A.M;
  const int nw = nl <= 64 * min(W, 4) ? min(W, 4) : W;
  const int cnt = (nl + nw - 1) / nw;
  if (wave >= nw) return;
  for (int j = lane; j < cnt; j += 64) {
    const int q = wave * cnt + j;
    if (q >= nl) break;
    const int lb = q / A.M, m = q - lb * A.M;
    const int b = b0 + lb;
    if (b >= A.nblk) continue;
    const uint32_t* row = sk + (lb * MP + m) * kScStride;
    emit_list8(
        [&](int r, uint32_t(&raw)[8]) {   // run r: columns 8r .. 8r + 7
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * r + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) raw[4 * h + e] = v[e];
          }
        },
        [](int r, int e) { return 63 - 8 * r - e; }, [&](int c) { return row[c]; }, A, m, b);
  }
}

// Top-kcand lists (any kcand) of every (block, row) pair of a many-row
// workgroup from the keys in LDS, by the 16-lane selection rounds: four lists
// per wave and pass (list q = 4 (wave + W pass) + hh is row q % M of block
// q / M), four passes at a time.
template <int MP, int W, int BPW>
__device__ __forceinline__ void big_select(const uint32_t* sk, const CoarseArgs& A, int b0, int wave, int hh,
                                           int nn) {
  constexpr int NB = 4;
  const int nl = BPW * A.M;
  for (int p0 = 0; 4 * (wave + W * p0) < nl; p0 += NB) {   // wave-uniform
    uint32_t k[NB][4], c[NB][4], kk[NB][4], kc[NB][4];
    int lbq[NB], mq[NB];
    bool live[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int q = 4 * (wave + W * (p0 + j)) + hh;
      lbq[j] = q / A.M;
      mq[j] = q - lbq[j] * A.M;
      live[j] = q < nl && b0 + lbq[j] < A.nblk;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        k[j][t] = live[j] ? sk[(lbq[j] * MP + mq[j]) * kScStride + 16 * t + nn] : 0u;
        c[j][t] = 16 * t + nn;
      }
    }
    row16_select<NB>(k, c, A.kcand, nn, kk, kc);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (live[j]) write_list(A, mq[j], b0 + lbq[j], kk[j], kc[j], nn);
  }
}

// MFMA phase of one group (quarter Q) for the MT row tiles and the wave's NTW
// column tiles: cg = sum over the group's k of x 2^64 * v 2^(2Q-133).  On
// entry a[0] holds k-slice 0's x fragments; each slice's MFMAs issue while the
// next slice's fragments are read (with kNext the last slice reads slice 0 of
// the next group, from xn).  Beside them runs the previous group's scale
// update, acc += sp * cp, component ks of every tile in slice ks.  A
// scheduling barrier per slice keeps one slice's decoded operands live at a
// time.  xb, xn: this lane's fragment 0 (A row nn, k-slot hh) in this group's
// slab and the next one's.
// kMode 0: quarter Q of a 2-bit head; 1: half Q (0 or 1) of a 4-bit head,
// whole codes (decode_half4); 2: a 4-bit head's quarter 2 or 3 where its byte
// groups keep four stages: no codes, no fragments, no MFMA, cg left as it is.
// kUpd: the previous group had sums to scale (not so after a kMode 2 group).
template <int MT, int NTW, int Q, int MP, bool kNext, int kMode, bool kUpd>
__device__ __forceinline__ void big_group_mma(f32x4 (&cg)[MT][NTW], f32x4 (&acc)[MT][NTW],
                                              const f32x4 (&cp)[MT][NTW], const float (&sp)[NTW],
                                              u32x4 (&a)[2][MT], const u32x4 (&raw)[2][NTW],
                                              const u32x4 (&raw8)[2][NTW], const u32x4* xb, const u32x4* xn) {
  constexpr uint32_t mask = 0x00030003u << (2 * Q);
  constexpr bool kMma = kMode != 2;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int h = ks >> 1, e = ks & 1;
    if (ks < 3) {
      const int f = (((ks + 1) >> 1) * 2 + ((ks + 1) & 1)) * 4;
      if constexpr (kMma) {
#pragma unroll
        for (int i = 0; i < MT; ++i) a[(ks + 1) & 1][i] = xb[f * MP + 16 * i];
      }
    } else if (kNext && (kMma || Q == 3)) {
#pragma unroll
      for (int i = 0; i < MT; ++i) a[0][i] = xn[16 * i];
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      bf16x8 bv;
      if constexpr (kMode == 0)
        bv = decode_quarter(raw[h][t][2 * e], raw8[h][t][2 * e], raw[h][t][2 * e + 1], raw8[h][t][2 * e + 1],
                            mask);
      else if constexpr (kMode == 1)
        bv = decode_half4<Q & 1>(raw[h][t][2 * e], raw8[h][t][2 * e], raw[h][t][2 * e + 1],
                                 raw8[h][t][2 * e + 1]);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if constexpr (kMma)
          cg[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[ks & 1][i]), bv,
                                                             ks ? cg[i][t] : f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if constexpr (kUpd) acc[i][t][ks] = __builtin_fmaf(sp[t], cp[i][t][ks], acc[i][t][ks]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One wave's share of a block: part P holds column tiles P NTW .. P NTW +
// NTW - 1 of the block, all MT row tiles and the whole of K; then the
// block's selection (from LDS when two waves share the block).
template <int MT, int P, bool kHalf>
__device__ __forceinline__ void big_wave(const BigArgs& BA, unsigned char* smem) {
  constexpr int QPB = dh::big_qpb(kHalf, MT);   // groups (stages' worth of x slabs) per byte group
  using S = BigShape<MT, QPB>;
  constexpr int MP = 16 * MT, XD = S::XD, NBUF = XD + 1, W = S::W, WPB = S::WPB, CD = S::CD, BPW = S::BPW;
  constexpr int NTW = S::NTW, T0 = P * NTW;
  const CoarseArgs& A = BA.c;
  constexpr int GPS = S::GPS, SPB = S::SPB;
  u32x4* xs = reinterpret_cast<u32x4*>(smem);     // [NBUF][GPS][16][MP]
  u32x4* cs = xs + NBUF * GPS * 16 * MP;          // [CD slots][BPW blocks][9 chunks][64]
  u32x4* zs = cs + CD * BPW * kCodeChunks * 64;   // [ZPS][256]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 4, nn = lane & 15;
  const int lb = wave & (BPW - 1);
  const int b = blockIdx.x * BPW + lb;
  const bool blk_ok = b < A.nblk;
  const int NG4 = A.K >> 9, NGRP = QPB * NG4;
  if constexpr (P == 0) zero_counters(A);

  // A block past the last one streams block 0 (valid memory) and writes nothing.
  const u32x4* tp = A.tiled + (size_t)(blk_ok ? b : 0) * NG4 * 512;
  // pairs: 1 KB per byte group, or 512 B with half pairs (fetched by lanes
  // 0-31 and again by lanes 32-63 into the chunk's second half, unread)
  constexpr int PB = kHalf ? 32 : 64;
  const u32x4* pp = A.pairs + (size_t)(blk_ok ? b : 0) * NG4 * PB;
  const uint32_t voff = lane * 16, voff_p = (lane % PB) * 16;
  const uint32_t xs_l = lds_addr(xs), zs_l = lds_addr(zs);
  const uint32_t cs_l = lds_addr(cs + lb * kCodeChunks * 64);

  // Issue stage j's ops.  Data past the end is replaced by a copy of the
  // last slab or byte group into a slot nothing reads before the main loop
  // ends; data before the start (prologue stages ahead of X(0) or B(0)) by
  // the bytes its slot is about to receive.
  auto issue = [&](int j) {
#pragma unroll
    for (int k = 0; k < S::nx(P); ++k) {   // chunks lb + BPW k of the stage's GPS slabs
      const dh::XOp o = dh::x_op<S>(j, lb, k, NGRP);
      dma16(voff, BA.xslab + (size_t)o.slab * 256 * MT + o.chunk * 64, xs_l + o.dst * 1024);
    }
    if (dh::stage_has_zp_ops<S>(j)) {
      // the zero-point slab before the codes: it is waited for at the byte
      // group's end, the codes (issued after it, so not waited for with it)
      // CD byte groups later
      const int GB = dh::zp_group<S>(j, NG4);
      const uint32_t zslot = (uint32_t)dh::zp_slot<S>(j);
#pragma unroll
      for (int k = 0; k < S::nb(P); ++k) {   // zero-point chunks lb nb + k of four
        const int c = lb * S::nb(P) + k;
        dma16(voff, BA.zslab + (size_t)GB * kZpEntries + c * 64, zs_l + zslot * 4096 + c * 1024);
      }
    }
    if (dh::stage_has_code_ops<S>(j)) {
      // with one wave per block (S::CODE == 0) the slot refilled here is the
      // one this wave has just read: its LDS reads must have returned
      if constexpr (S::CODE == 0) __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
      const int GC = dh::code_group<S>(j, NG4);
      const uint32_t cslot = (uint32_t)dh::code_slot<S>(j);
#pragma unroll
      for (int k = 0; k < S::nc(P); ++k) {
        const int c = k;
        const uint32_t dst = cs_l + cslot * BPW * kCodeChunks * 1024 + c * 1024;
        if (c < 8) dma16_nt(voff, tp + (GC * 8 + c) * 64, dst);
        else dma16_nt(voff_p, pp + GC * PB, dst);
      }
    }
  };

#pragma unroll
  for (int j = -S::PRO; j < 0; ++j) issue(j);
  wait_vm<big_wait<S, P>(SPB - 1)>();
  __syncthreads();

  // cgs[Q & 1] receives group Q's MFMA sums; the other set still holds the
  // previous group's, scaled into acc (by sp) during group Q.
  f32x4 acc[MT][NTW], cgs[2][MT][NTW];
  float sp[NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = cgs[1][i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NTW; ++t) sp[t] = 0.f;
  const u32x4* xl = xs + hh * MP + nn;   // this lane's fragment 0 in slab 0
  u32x4 a[2][MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) a[0][i] = xl[16 * i];

  for (int G = 0; G < NG4; ++G) {
    // byte group G's codes and scale pairs of the wave's column tiles, into
    // registers (the slot is refilled with byte group G + CD after this
    // iteration's barrier)
    const u32x4* cw = cs + ((G % CD) * BPW + lb) * kCodeChunks * 64;
    u32x4 raw[2][NTW], sz[NTW];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < NTW; ++t) raw[h][t] = cw[(h * 4 + T0 + t) * 64 + lane];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      if constexpr (kHalf) sz[t] = half_pairs4(reinterpret_cast<const u32x2*>(cw + 512)[(T0 + t) * 16 + nn]);
      else sz[t] = cw[512 + (T0 + t) * 16 + nn];
    }

    // zero-point part of byte group G
    {
      u32x4 za[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) za[i] = zs[(G % S::ZPS) * kZpEntries + (hh & 1) * MP + 16 * i + nn];
      if (hh >= 2) {
#pragma unroll
        for (int i = 0; i < MT; ++i) za[i] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        uint32_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = __float_as_uint(lo_bf16(sz[t][q]) - hi_bf16(sz[t][q]));
        const uint32_t p01 = (d[0] >> 16) | (d[1] & 0xFFFF0000u);
        const uint32_t p23 = (d[2] >> 16) | (d[3] & 0xFFFF0000u);
        const u32x4 zb = u32x4{p01, p23, p01, p23};   // slots 8..15 meet zero x parts
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, za[i]),
                                                             __builtin_bit_cast(bf16x8, zb), acc[i][t], 0, 0, 0);
      }
    }

    u32x4 raw8[2][NTW];
    shift_codes(raw, raw8);
    // one group's MFMAs (quarter Q, the stage's slab t), its scale kept for
    // the next group
    auto group = [&](auto qc, int j) {
      constexpr int Q = decltype(qc)::value, t = Q % GPS;
      float sq[NTW];
      // a 4-bit head decodes whole codes in quarters 0 and 1 (the halves of
      // its K) and, where its byte groups keep four stages, has nothing in
      // quarters 2 and 3 (after which no sums are left to scale)
      constexpr int kMode = kHalf ? (Q < 2 ? 1 : 2) : 0;
      constexpr bool kUpd = !(kHalf && QPB == 4 && (Q == 0 || Q == 3));
#pragma unroll
      for (int u = 0; u < NTW; ++u)
        sq[u] = kMode == 0 ? quarter_scale(lo_bf16(sz[u][Q]), Q) : kMode == 1 ? half4_scale(lo_bf16(sz[u][Q]), Q) : 0.f;
      const u32x4* xb = xl + ((j % NBUF) * GPS + t) * 16 * MP;
      const u32x4* xn = t + 1 < GPS ? xb + 16 * MP : xl + ((j + 1) % NBUF) * GPS * 16 * MP;
      big_group_mma<MT, NTW, Q, MP, (t + 1 < GPS) || S::XW == 2, kMode, kUpd>(cgs[Q & 1], acc, cgs[(Q + 1) & 1],
                                                                              sp, a, raw, raw8, xb, xn);
#pragma unroll
      for (int u = 0; u < NTW; ++u) sp[u] = sq[u];
    };
    auto stage = [&](auto qs) {
      constexpr int Qs = decltype(qs)::value;
      const int j = SPB * G + Qs;
      issue(j);
      group(std::integral_constant<int, GPS * Qs>{}, j);
      if constexpr (GPS == 2) group(std::integral_constant<int, GPS * Qs + 1>{}, j);
      wait_vm<big_wait<S, P>(Qs)>();
      __syncthreads();
      if constexpr (S::XW == 1) {   // the next stage's first fragments, now visible
#pragma unroll
        for (int i = 0; i < MT; ++i) a[0][i] = xl[((j + 1) % NBUF) * GPS * 16 * MP + 16 * i];
      }
    };
    stage(std::integral_constant<int, 0>{});
    if constexpr (SPB >= 2) stage(std::integral_constant<int, 1>{});
    if constexpr (SPB == 4) {
      stage(std::integral_constant<int, 2>{});
      stage(std::integral_constant<int, 3>{});
    }
  }
  // the last group's scale update (none after a kMode 2 group)
  if constexpr (!(kHalf && QPB == 4)) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][t][r] = __builtin_fmaf(sp[t], cgs[1][i][t][r], acc[i][t][r]);
  }
  wait_vm<0>();
  if constexpr (WPB == 1) {   // one wave holds the whole block: its lists from registers
    if (!blk_ok) return;
    block_select<MT, 4>([&](int i, int r, int t) { return acc[i][t][r]; }, A, b, hh, nn);
    return;
  }
  // every wave's DMA writes have landed and every wave is done with the ring:
  // its LDS now takes the workgroup's score keys (and the optional full rows
  // are written from the accumulators)
  __syncthreads();
  uint32_t* sk = reinterpret_cast<uint32_t*>(smem);
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int col = 16 * (T0 + t) + nn, n = 64 * b + col;
    const bool n_ok = blk_ok && n < A.N;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * hh + r;
        sk[(lb * MP + row) * kScStride + col] = f32_key_if(n_ok, acc[i][t][r]);   // -0 as +0
      }
  }
  if (wants_scores(A)) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int n = 64 * b + 16 * (T0 + t) + nn;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * hh + r;
          if (blk_ok && n < A.N && row < A.M) store_scores(A, row, n, acc[i][t][r]);
        }
    }
  }
  __syncthreads();
  if (A.kcand <= 8) lane_select8<MP, BPW>(sk, A, blockIdx.x * BPW, wave, W, lane);
  else big_select<MP, W, BPW>(sk, A, blockIdx.x * BPW, wave, hh, nn);
}

template <int MT, bool kHalf>
__global__ __launch_bounds__(64 * BigShape<MT>::W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void coarse_mfma_kernel(BigArgs BA) {
  extern __shared__ __align__(16) unsigned char smem[];
  if constexpr (BigShape<MT>::WPB == 2) {
    if (threadIdx.x >= 64 * BigShape<MT>::BPW) {
      big_wave<MT, 1, kHalf>(BA, smem);
      return;
    }
  }
  big_wave<MT, 0, kHalf>(BA, smem);
}

// ---------------------------------------------------------------------------
// Coarse kernel for more rows, scale folded into the weights (fp16 MFMA).
//
// Each group's contribution is x . (S/4) v, with v the 2-bit code and S the
// bf16 scale: (S/4) v has at most 10 significant bits (S has 8, v <= 3), so
// it is an exact fp16 value wherever |S| lies in [2^-15, 255] (below 2^-15 it
// rounds to the fp16 subnormal step, 2^-24), and x scaled by a power of two
// per row is an exact fp16 value for every element of at least 2^-31 times
// the row's largest magnitude (smaller ones round to that step as well).  The
// products are then exact in fp32, as with the page's bf16 decode, and the
// per-group scale needs neither its own
// accumulator nor an update per score: the MFMAs accumulate the whole row of
// K into one accumulator per tile, and the zero-point part, sum_g (S - ZS)
// X_g, joins it through one bf16 MFMA per byte group as in the many-row
// kernel.  The coarse score is the accumulator times 2^-f, f the row's scale.
//
// Decode of quarter q (code at bits 2q..2q+1 of each byte of a 16-bit half):
// OR-ing in the fp16 exponent of 1.0 gives 1 + v 2^(2q-10); a packed fp16
// fused multiply-add with T = (S/4) 2^(10-2q), d * T - T = v (S/4), rounds
// once, exactly.
//
// Workgroup = 8 waves = 8 blocks of 64 columns, one wave per block holding
// its 4 column tiles for all MT row tiles, so every x fragment read from LDS
// feeds 4 MFMAs, and 1940 blocks take 243 workgroups (one per CU).  Stage j
// = 4G + q is group q of byte group G.  Direct-to-LDS DMA ring:
//   x slabs (one group, 4 MT chunks of 1 KB) kH16XD stages ahead, in
//   kH16XD + 1 slots; every wave issues h16_xops(MT) ops per stage (chunk
//   wave + 8 k; chunks past the slab repeat chunk c - 4 MT into the same
//   place, the same bytes);
//   at stage 4G + 1 (after every wave took byte group G's codes into
//   registers): byte group G + 1's zero-point slab (chunk wave mod 4, again
//   issued twice) and its codes and scale pairs (each wave its own block, 9
//   chunks) into the single code slot.
// Every wave issues the same ops in the same order, so each wait is a
// constant: at the end of stage j it completes slab j + 1 and, at q = 3, the
// next byte group's codes and zero-point slab.
// (The schedule's shape, op addresses and wait counts: dh::h16_* in ring_plan.h.)
constexpr int kHBlocks = dh::kH16Blocks;
constexpr size_t h16_lds_bytes(int MT) {
  const size_t ring = dh::h16_ring_bytes(MT);
  const size_t keys = (size_t)kHBlocks * 16 * MT * 64 * 4;   // the epilogue's keys: 64 per (block, row)
  return ring > keys ? ring : keys;
}

// x for one launch of up to 80 rows in the workspace for the fp16 kernel,
// written by prep_xh_kernel: per row the scale exponent f (int), then slabs
// and zero-point slabs in the many-row kernel's layout, with x * 2^f as fp16
// and the group sums X * 2^f split in three bf16 parts.
struct HArgs {
  CoarseArgs c;
  const u32x4* xslab;
  const u32x4* zslab;
  const int* fexp;
};

// One workgroup (4 waves) per row m of a launch: wave w takes the byte groups
// G = w, w + 4, ...; lane q * 16 + p takes piece p (8 consecutive k) of group
// 4G + q.  The row's largest |x| (an exact max) gives f = 15 - e with
// max = m 2^e, 1/2 <= m < 1, so that every |x| 2^f < 2^15.
constexpr int kPrepHMaxG = 8;   // byte groups per wave held in registers: K <= 8 * 4 * 512
__global__ __launch_bounds__(256) void prep_xh_kernel(const uint16_t* __restrict__ x, int M, int MP, int K,
                                                      u32x4* __restrict__ xslab, u32x4* __restrict__ zslab,
                                                      int* __restrict__ fexp) {
  __shared__ float wmax[4];
  const int m = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NG4 = K >> 9, Q4 = K >> 2;
  const int q = lane >> 4, p = lane & 15;
  const int h = p >> 3, s = (p >> 1) & 3, e = p & 1, f = (h * 2 + e) * 4 + s;
  u32x4 v[kPrepHMaxG];
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < kPrepHMaxG; ++i) {
    const int G = wave + 4 * i;
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (G < NG4 && m < M) v[i] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + q * Q4 + 128 * G + 8 * p);
#pragma unroll
    for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fmaxf(fabsf(lo_bf16(v[i][c])), fabsf(hi_bf16(v[i][c]))));
  }
  mx = wave_max(mx);
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  int ex = 0;
  if (mx > 0.f) (void)__builtin_frexpf(mx, &ex);
  const int fx = mx > 0.f ? 15 - ex : 0;
  if (threadIdx.x == 0) fexp[m] = fx;
#pragma unroll
  for (int i = 0; i < kPrepHMaxG; ++i) {
    const int G = wave + 4 * i;
    if (G >= NG4) break;   // wave-uniform
    // fp16 x * 2^fx in the decode order {0,2,1,3,4,6,5,7}, and the unscaled sum
    float xs[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      xs[2 * c] = lo_bf16(v[i][c]);
      xs[2 * c + 1] = hi_bf16(v[i][c]);
    }
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) sum += xs[c];
    const int order[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    uint32_t hw[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const _Float16 hv = (_Float16)__builtin_ldexpf(xs[order[c]], fx);
      hw[c] = (uint32_t)__builtin_bit_cast(uint16_t, hv);
    }
    xslab[((size_t)(4 * G + q) * 16 + f) * MP + m] =
        u32x4{hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16, hw[6] | hw[7] << 16};
    sum = row16_sum(sum);
    float X[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) X[u] = __builtin_ldexpf(lane_value(sum, 16 * u), fx);
    if (lane < 2) {
      uint32_t part[3][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float r = X[u];
#pragma unroll
        for (int c = 0; c < 3; ++c) {   // r - bf16(r) is exact in fp32
          part[c][u] = f32_to_bf16_rne(r);
          r -= __uint_as_float(part[c][u] << 16);
        }
      }
      const u32x4 o = lane == 0 ? u32x4{part[0][0] | part[0][1] << 16, part[0][2] | part[0][3] << 16,
                                        part[1][0] | part[1][1] << 16, part[1][2] | part[1][3] << 16}
                                : u32x4{part[2][0] | part[2][1] << 16, part[2][2] | part[2][3] << 16, 0u, 0u};
      zslab[(size_t)G * kZpEntries + lane * MP + m] = o;
    }
  }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Quarter q's weights (S/4) v of one k-slice of a tile, as fp16 in the decode
// order: d = code bits | 1.0, then d * T - T per packed pair (one rounding).
// (d & mask) | one in one instruction (the compiler otherwise splits it in
// two, as its three-operand form takes no literal constants on this target).
__device__ __forceinline__ uint32_t and_or(uint32_t d, uint32_t mask, uint32_t one) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(d), "s"(mask), "v"(one));
  return r;
}
// mask (wave-uniform) and one: one AND-OR per pair.
__device__ __forceinline__ f16x8 decode_h16(uint32_t d0, uint32_t o0, uint32_t d1, uint32_t o1, uint32_t mask,
                                            uint32_t one, f16x2 tt) {
  const uint32_t w[4] = {and_or(d0, mask, one), and_or(o0, mask, one), and_or(d1, mask, one), and_or(o1, mask, one)};
  f16x8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 dv = __builtin_bit_cast(f16x2, w[i]);
    const f16x2 r = __builtin_elementwise_fma(dv, tt, -tt);
    out[2 * i] = r[0];
    out[2 * i + 1] = r[1];
  }
  return out;
}

template <int MT>
__global__ __launch_bounds__(64 * dh::h16_waves(MT))
__attribute__((amdgpu_waves_per_eu(dh::h16_waves(MT) / 4, dh::h16_waves(MT) / 4)))
void coarse_h16_kernel(HArgs HA) {
  constexpr int MP = 16 * MT, NX = dh::h16_xops(MT), SLOTS = dh::kH16Slots;
  constexpr int NTW = dh::h16_ntw(MT), WPB = 4 / NTW, W = dh::h16_waves(MT);   // tiles a wave, waves a block
  const CoarseArgs& A = HA.c;
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* xs = reinterpret_cast<u32x4*>(smem);                     // [SLOTS][16][MP]
  u32x4* cs = xs + SLOTS * 16 * MP;                                // [8 blocks][9 chunks][64]
  u32x4* zs = cs + kHBlocks * kCodeChunks * 64;                    // [2][256]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lb = wave / WPB, part = wave % WPB, T0 = NTW * part;   // block, and the wave's first column tile
  const int hh = lane >> 4, nn = lane & 15;
  const int b = blockIdx.x * kHBlocks + lb;
  const bool blk_ok = b < A.nblk;
  const int NG4 = A.K >> 9, NSTAGE = 4 * NG4;
  zero_counters(A);

  // A block past the last one streams block 0 (valid memory) and writes nothing.
  const u32x4* tp = A.tiled + (size_t)(blk_ok ? b : 0) * NG4 * 512;
  const u32x4* pp = A.pairs + (size_t)(blk_ok ? b : 0) * NG4 * 64;
  const uint32_t voff = lane * 16;
  const uint32_t xs_l = lds_addr(xs), zs_l = lds_addr(zs), cs_l = lds_addr(cs + lb * kCodeChunks * 64);

  auto issue_x = [&](int j) {   // slab of stage j (clamped to the last) into its slot
    const int slab = dh::h16_slab(j, NSTAGE);
    const uint32_t dst = xs_l + (uint32_t)((j % SLOTS) * 16 * MP * 16);
#pragma unroll
    for (int k = 0; k < NX; ++k) {
      const int c = dh::h16_xchunk(MT, wave, k);
      dma16(voff, HA.xslab + (size_t)slab * 256 * MT + c * 64, dst + c * 1024);
    }
  };
  auto issue_bytes = [&](int G) {   // zero-point slab and the wave's codes of byte group G (clamped)
    const int Gc = dh::h16_byte_group(G, NG4);
    const int c = wave & 3;
    dma16(voff, HA.zslab + (size_t)Gc * kZpEntries + c * 64, zs_l + (uint32_t)((Gc & 1) * 4096 + c * 1024));
#pragma unroll
    for (int k = 0; k < dh::h16_code_ops(MT); ++k) {
      const int ch = dh::h16_code_chunk(MT, part, k);
      dma16_nt(voff, ch < 8 ? tp + (Gc * 8 + ch) * 64 : pp + Gc * 64, cs_l + ch * 1024);
    }
  };

  // prologue: slabs of stages 0 .. kH16XD - 1, byte group 0
#pragma unroll
  for (int j = 0; j < dh::kH16XD; ++j) issue_x(j);
  issue_bytes(0);
  wait_vm<0>();
  __syncthreads();

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4* xl = xs + hh * MP + nn;   // this lane's fragment 0 (A row nn, k-slot hh) of slot 0
  const u32x4* cw = cs + lb * kCodeChunks * 64;
  for (int G = 0; G < NG4; ++G) {
    // byte group G's codes and scale pairs of the wave's tiles (the slot is
    // refilled at stage 4G + 1)
    u32x4 raw[2][NTW], raw8[2][NTW], sz[NTW];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < NTW; ++t) raw[h][t] = cw[(h * 4 + T0 + t) * 64 + lane];
#pragma unroll
    for (int t = 0; t < NTW; ++t) sz[t] = cw[512 + (T0 + t) * 16 + nn];
    shift_codes(raw, raw8);
    // zero-point part of byte group G: rows' X parts against S - ZS (exact in bf16)
    {
      const u32x4* zg = zs + (G & 1) * kZpEntries;
      u32x4 za[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) za[i] = hh < 2 ? zg[(hh & 1) * MP + 16 * i + nn] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        uint32_t d[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) d[qq] = __float_as_uint(lo_bf16(sz[t][qq]) - hi_bf16(sz[t][qq]));
        const uint32_t p01 = (d[0] >> 16) | (d[1] & 0xFFFF0000u);
        const uint32_t p23 = (d[2] >> 16) | (d[3] & 0xFFFF0000u);
        const u32x4 zb = u32x4{p01, p23, p01, p23};   // slots 8..15 meet zero x parts
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, za[i]),
                                                             __builtin_bit_cast(bf16x8, zb), acc[i][t], 0, 0, 0);
      }
    }
    auto stage = [&](auto qc) {
      constexpr int Q = decltype(qc)::value;
      const int j = 4 * G + Q;
      issue_x(j + dh::kH16XD);
      if constexpr (Q == 1) issue_bytes(G + 1);
      // the code bits of quarter Q, and the exponent field of 1.0 (disjoint from them)
      const uint32_t mask = __builtin_amdgcn_readfirstlane(0x00030003u << (2 * Q));
      const uint32_t one = 0x3C003C00u;
      f16x2 tt[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {   // T = (S/4) 2^(10 - 2Q) = S 2^(8 - 2Q), exact in fp16
        const _Float16 tv = (_Float16)__builtin_ldexpf(lo_bf16(sz[t][Q]), 8 - 2 * Q);
        tt[t] = f16x2{tv, tv};
      }
      const u32x4* xb = xl + (j % SLOTS) * 16 * MP;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int h = ks >> 1, e = ks & 1;
        u32x4 a[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) a[i] = xb[((h * 2 + e) * 4) * MP + 16 * i];
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const f16x8 bv = decode_h16(raw[h][t][2 * e], raw8[h][t][2 * e], raw[h][t][2 * e + 1],
                                      raw8[h][t][2 * e + 1], mask, one, tt[t]);
#pragma unroll
          for (int i = 0; i < MT; ++i)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[i]), bv, acc[i][t], 0,
                                                              0, 0);
        }
      }
      wait_vm<dh::h16_wait(MT, Q)>();
      __syncthreads();
    };
    stage(std::integral_constant<int, 0>{});
    stage(std::integral_constant<int, 1>{});
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 3>{});
  }
  wait_vm<0>();
  // Every wave's DMA writes have landed and every wave is done with the ring:
  // the LDS takes the keys of the workgroup's 8 blocks (of the accumulators:
  // a row's coarse scores are its accumulators times 2^-f, a power of two
  // that keeps their order and is applied to the values a list writes), row
  // rho = lb MP + m
  // (block lb, row m) in 16 pieces of 16 bytes, piece g holding columns g,
  // g + 16, g + 32, g + 48 (tiles 0..3 of column g: written by the block's
  // one wave, or its two waves 8 bytes each) at position g ^ (rho mod 16), so that
  // sixteen consecutive rows read piece by piece meet every bank once.  Then
  // thread q selects list q (list l: block l / M, row l % M).  (The fp16
  // kernel takes lists of at most eight.)
  u32x4* sk = reinterpret_cast<u32x4*>(smem);
  // the 2^-f of the rows of this thread's lists, requested now so that they
  // arrive during the key phase and the selection
  constexpr int kNL = (kHBlocks * MP + 64 * W - 1) / (64 * W);   // lists a thread takes, at most
  float lsc[kNL];
#pragma unroll
  for (int u = 0; u < kNL; ++u) {
    const int l = threadIdx.x + 64 * W * u;
    lsc[u] = __builtin_ldexpf(1.0f, -HA.fexp[l < kHBlocks * A.M ? l % A.M : 0]);
  }
  __syncthreads();
  // masks of the live columns and rows, as bits (conditions the compiler
  // would otherwise turn into branches around every key)
  uint32_t colm[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) colm[t] = 0u - (uint32_t)(blk_ok & (64 * b + 16 * (T0 + t) + nn < A.N));
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * i + 4 * hh + r, rho = lb * MP + row;
      const uint32_t rowm = 0u - (uint32_t)(row < A.M);
      uint32_t kk[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) kk[t] = f32_key(acc[i][t][r] + 0.0f) & colm[t] & rowm;   // -0 as +0
      u32x4* piece = sk + rho * 16 + (nn ^ (row & 15));
      if constexpr (NTW == 4) *piece = u32x4{kk[0], kk[1], kk[2], kk[3]};
      else reinterpret_cast<u32x2*>(piece)[part] = u32x2{kk[0], kk[1]};
    }
  if (wants_scores(A)) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rs = __builtin_ldexpf(1.0f, -HA.fexp[16 * i + 4 * hh + r]);
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const int row = 16 * i + 4 * hh + r, n = 64 * b + 16 * (T0 + t) + nn;
          if (blk_ok && n < A.N && row < A.M) store_scores(A, row, n, acc[i][t][r] * rs);
        }
      }
  }
  __syncthreads();
#pragma unroll 1
  for (int u = 0; u < kNL; ++u) {   // rolled, as the selection in it
    const int l = threadIdx.x + 64 * W * u;
    if (l >= kHBlocks * A.M) break;
    const int lbl = l / A.M, m = l - lbl * A.M, bq = blockIdx.x * kHBlocks + lbl;
    if (bq >= A.nblk) continue;
    float sc = lsc[0];
#pragma unroll
    for (int v = 1; v < kNL; ++v) sc = u == v ? lsc[v] : sc;
    const u32x4* row = sk + (lbl * MP + m) * 16;
    const int sw = m & 15;
    emit_list8(
        [&](int r, uint32_t(&raw)[8]) {   // run r: pieces 2r and 2r + 1 (columns g, g + 16, g + 32, g + 48)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 v = row[(2 * r + h) ^ sw];
#pragma unroll
            for (int t = 0; t < 4; ++t) raw[4 * h + t] = v[t];
          }
        },
        [](int r, int e) { return 63 - 16 * (e & 3) - 2 * r - (e >> 2); },
        [&](int c) { return reinterpret_cast<const uint32_t*>(row + ((c & 15) ^ sw))[c >> 4]; }, A, m, bq, sc);
  }
}

// ---------------------------------------------------------------------------
// Rerank: one workgroup per row.
//
// Selection (`bm.topk(RERANK)` + `bi.gather`): each candidate becomes a 64-bit
// key (ordered float bits << 32 | ~id), so "larger key" is "larger value, then
// lower id", and the keys of valid candidates are all distinct; invalid slots
// (id -1, or an id >= N that no coarse call writes) get key 0.
//   1. Thread t reads candidates t, t + 1024, ... (coalesced) and keeps them
//      and their maximum.
//   2. Wave 0 finds T, the R-th largest of the 1024 per-thread maxima, by a
//      radix select over 8-bit digits with no workgroup barrier.  R maxima
//      are >= T, so the R-th largest key overall is >= T.
//   3. The keys >= T (usually a few more than R) are gathered; wave 0 sorts
//      them with a shuffle bitonic network when there are at most 64, the
//      workgroup with an LDS bitonic network otherwise.
// Rows with more than 16384 candidates, R above the 1024 maxima, or more than
// DH_MAX_R survivors take T from a workgroup radix select over all keys.
//
// Exact logits (`_rerank_exact`, bf16 branch): the 16 waves then take the R
// selected rows of W in turn, one dot of length K each, fp32 products and sums,
// all loads of a row issued before any is used.
// Exact logit of one candidate row, x[m] . W[id], by one wave with every
// load of the row issued before any is used (fp32 products and sums).
//   bf16 rows (`_rerank_exact`, bf16 branch): lane l takes 8 consecutive k
//   per 512; e4m3 rows (FP8 branch): lane l takes 16 consecutive k per 1024,
//   each byte decoded by the page's bit arithmetic (e = (b >> 3) & 15,
//   mant = b & 7: mant * 2^-9 if e == 0, else (1 + mant/8) * 2^(e-7); bit 7
//   the sign) and multiplied by the row's scale, one fp32 rounding.
constexpr int kDotBf16 = 10;   // 16-byte W loads per lane in flight (5120 k)
constexpr int kDotE4m3 = 5;    // 16-byte W loads per lane in flight (5120 k)
constexpr int kDotNvfp4 = 3;   // 16-byte W loads per lane in flight (6144 k)

// e4m3 byte b as the page decodes it: magnitude mant * 2^-9 for e = 0, else
// (1 + mant/8) * 2^(e-7), bit 7 the sign (0x7F reads as 480).  Bits 6..0
// placed at fp32 bits 26..20 give 2^(e-127) (1 + mant/8), or the fp32
// denormal mant * 2^-129 for e = 0 (denormals are kept: the kernels run
// with fp32 denormal mode "preserve"); times 2^120, exactly, the values above.
__device__ __forceinline__ float e4m3_page(uint32_t b) {
  return __uint_as_float(((b & 127u) << 20) | ((b & 128u) << 24)) * 0x1p120f;
}

// e2m1 (FP4) nibble: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0;
// exponent 0 is the subnormal 0.5 * mantissa.  Bits 2..0 placed at fp32 bits
// 24..22 give 2^(e-127) (1 + mant/2), or the fp32 denormal mant * 2^-127 for
// e = 0; times 2^126, exactly, the e2m1 values.
__device__ __forceinline__ float e2m1_value(uint32_t n) {
  return __uint_as_float(((n & 7u) << 22) | ((n & 8u) << 28)) * 0x1p126f;
}

// NVFP4 block scale: an e4m3 byte as the format defines it (0x7F, 0xFF NaN).
__device__ __forceinline__ float e4m3_scale(uint32_t b) {
  return (b & 127u) == 127u ? __builtin_nanf("") : e4m3_page(b);
}

// fp32 -> bf16 -> fp32, round to nearest even (NaN kept).
__device__ __forceinline__ float round_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return f != f ? f : __uint_as_float(r);
}

// x.lo * w.lo + x.hi * w.hi + acc for two bf16 pairs (v_dot2c_f32_bf16): the
// products of bf16 values are exact in fp32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_dot2(uint32_t x, uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, w), acc, false);
}

// Sum over the wave, the same in every lane, in a fixed order: pairs, quads,
// eights and rows of 16 by DPP, then the four rows.  Every lane must be active.
template <int kCtrl>
__device__ __forceinline__ float dpp_plus(float s) {
  return s + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float s) {
  s = dpp_plus<0xB1>(s);    // quad_perm 1,0,3,2
  s = dpp_plus<0x4E>(s);    // quad_perm 2,3,0,1
  s = dpp_plus<0x141>(s);   // row_half_mirror: lane i and 7 - i of each eight
  s = dpp_plus<0x140>(s);   // row_mirror: lane i and 15 - i of each row
  const auto row = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), l)); };
  return (row(0) + row(16)) + (row(32) + row(48));
}

// x of one row in the lane layout of the rerank's dot for rows of kind kKind:
// one chunk of the row (K elements, K a multiple of 256), clamped loads
// (positions past K read the last valid piece and are masked in the dot).
//   bf16 rows:  lane l holds x[c0 + 512 j + 8 l .. +8) for j < kDotBf16
//   e4m3 rows:  lane l holds x[c0 + 1024 j + 16 l .. +16) for j < kDotE4m3
//   NVFP4 rows: lane l holds x[c0 + 2048 j + 32 l .. +32) for j < kDotNvfp4
template <int kKind>
struct XChunk {
  static constexpr int kPass = kKind == kRowsBf16 ? 512 : kKind == kRowsE4m3 ? 1024 : 2048;   // k per pass
  static constexpr int kPasses = kKind == kRowsBf16 ? kDotBf16 : kKind == kRowsE4m3 ? kDotE4m3 : kDotNvfp4;
  static constexpr int kPieces = kKind == kRowsBf16 ? 1 : kKind == kRowsE4m3 ? 2 : 4;   // 16-byte pieces per pass
  static constexpr int kLen = kPass * kPasses;                                             // k per chunk
  u32x4 v[kPasses][kPieces];
  __device__ __forceinline__ void load(const uint16_t* xr, int K, int c0, int lane) {
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const int k = min(c0 + kPass * j + lane * 8 * kPieces, K - 8 * kPieces);
#pragma unroll
      for (int q = 0; q < kPieces; ++q) v[j][q] = *reinterpret_cast<const u32x4*>(xr + k + 8 * q);
    }
  }
};

// The exact logits of NR candidate rows, one wave, fp32 accumulation: per
// chunk of k, every load of the NR rows and of x (from global memory, or from
// LDS where the caller staged the row) issued before any is used.  ids[i] < 0:
// no row (reads row 0, returns -inf).
//   bf16 rows (`_rerank_exact`, bf16 branch): x . W[id].
//   e4m3 rows (FP8 branch): each byte decoded by the page's bit arithmetic
//     (e = (b >> 3) & 15, mant = b & 7: mant * 2^-9 if e == 0, else
//     (1 + mant/8) * 2^(e-7); bit 7 the sign) and multiplied by the row's
//     scale, one fp32 rounding.
//   NVFP4 rows: e2m1 nibbles (low nibble first) times the e4m3 scale of their
//     16-element block times the global scale, rounded to bf16.
template <int kKind, int NR>
__device__ void wave_dots(const RowSrc& S, const int (&ids)[NR], const uint16_t* xr, int K, int lane,
                          float (&out)[NR]) {
  using XC = XChunk<kKind>;
  float s0[NR], s1[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) s0[i] = s1[i] = 0.f;
  // one chunk of k: the NR rows' loads, then their products with x
  auto chunk = [&](const XC& xc, int c0) {
    if constexpr (kKind == kRowsBf16) {
      u32x4 wv[NR][kDotBf16];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const uint16_t* wr = static_cast<const uint16_t*>(S.w) + (size_t)(ids[i] < 0 ? 0 : ids[i]) * S.ldw;
#pragma unroll
        for (int j = 0; j < kDotBf16; ++j)
          wv[i][j] = *reinterpret_cast<const u32x4*>(wr + min(c0 + 512 * j + lane * 8, K - 8));
      }
#pragma unroll
      for (int j = 0; j < kDotBf16; ++j) {
        if (c0 + 512 * j + lane * 8 < K) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int c = 0; c < 4; c += 2) {   // one dot2 per bf16 pair: products exact, fp32 sums
              s0[i] = bf16_dot2(xc.v[j][0][c], wv[i][j][c], s0[i]);
              s1[i] = bf16_dot2(xc.v[j][0][c + 1], wv[i][j][c + 1], s1[i]);
            }
        }
      }
    } else if constexpr (kKind == kRowsE4m3) {
      u32x4 wv[NR][kDotE4m3];
      float scale[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int id = ids[i] < 0 ? 0 : ids[i];
        const uint8_t* wr = static_cast<const uint8_t*>(S.w) + (size_t)id * S.ldw;
        scale[i] = S.wscale[id];
#pragma unroll
        for (int j = 0; j < kDotE4m3; ++j)
          wv[i][j] = *reinterpret_cast<const u32x4*>(wr + min(c0 + 1024 * j + lane * 16, K - 16));
      }
#pragma unroll
      for (int j = 0; j < kDotE4m3; ++j) {
        if (c0 + 1024 * j + lane * 16 < K) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {   // bytes 4c .. 4c+3 of the 16
              const uint32_t b4 = wv[i][j][c];
              const u32x4& xh = xc.v[j][c >> 1];
              const uint32_t x01 = xh[2 * (c & 1)], x23 = xh[2 * (c & 1) + 1];
              s0[i] = __builtin_fmaf(lo_bf16(x01), e4m3_page(b4 & 255u) * scale[i], s0[i]);
              s1[i] = __builtin_fmaf(hi_bf16(x01), e4m3_page((b4 >> 8) & 255u) * scale[i], s1[i]);
              s0[i] = __builtin_fmaf(lo_bf16(x23), e4m3_page((b4 >> 16) & 255u) * scale[i], s0[i]);
              s1[i] = __builtin_fmaf(hi_bf16(x23), e4m3_page(b4 >> 24) * scale[i], s1[i]);
            }
        }
      }
    } else {
      const float g = *S.gscale;
      u32x4 wv[NR][kDotNvfp4];
      uint32_t bv[NR][kDotNvfp4];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int id = ids[i] < 0 ? 0 : ids[i];
        const uint8_t* wr = static_cast<const uint8_t*>(S.w) + (size_t)id * S.ldw;
        const uint8_t* br = S.bscale + (size_t)id * S.lds;
#pragma unroll
        for (int j = 0; j < kDotNvfp4; ++j) {
          const int k = min(c0 + 2048 * j + lane * 32, K - 32);
          wv[i][j] = *reinterpret_cast<const u32x4*>(wr + k / 2);
          bv[i][j] = *reinterpret_cast<const uint16_t*>(br + k / 16);
        }
      }
#pragma unroll
      for (int j = 0; j < kDotNvfp4; ++j) {
        if (c0 + 2048 * j + lane * 32 < K) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {   // scale block h: bytes 8h .. 8h+7, elements 16h .. 16h+15
              const float bs = e4m3_scale((bv[i][j] >> (8 * h)) & 255u);
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const uint32_t b4 = wv[i][j][2 * h + c];   // elements 16h + 8c .. +7, low nibble first
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const uint32_t xw = xc.v[j][2 * h + c][e];   // x of elements 2e, 2e+1 of this word
                  const float w0 = round_bf16(e2m1_value((b4 >> (8 * e)) & 15u) * bs * g);
                  const float w1 = round_bf16(e2m1_value((b4 >> (8 * e + 4)) & 15u) * bs * g);
                  s0[i] = __builtin_fmaf(lo_bf16(xw), w0, s0[i]);
                  s1[i] = __builtin_fmaf(hi_bf16(xw), w1, s1[i]);
                }
              }
            }
        }
      }
    }
  };
  for (int c0 = 0; c0 < K; c0 += XC::kLen) {
    XC xc;
    xc.load(xr, K, c0, lane);
    chunk(xc, c0);
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const float sum = wave_sum(s0[i] + s1[i]);
    out[i] = ids[i] < 0 ? -__builtin_inff() : sum;
  }
}

// The exact logit of one row (see wave_dots).
template <int kKind>
__device__ float wave_dot(const RowSrc& S, uint32_t id, const uint16_t* xr, int K, int lane) {
  const int ids[1] = {(int)id};
  float out[1];
  wave_dots<kKind, 1>(S, ids, xr, K, lane, out);
  return out[0];
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelCache = 16;

__device__ __forceinline__ unsigned long long cand_key(float v, int id, int N) {
  if (id < 0 || id >= N) return 0ull;
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ uint32_t key_id(unsigned long long k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull);
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long umin64(unsigned long long a, unsigned long long b) {
  return a < b ? a : b;
}

struct SelectShared {
  unsigned int whist[kSelWaves][256];
  unsigned long long tmax[kSelThreads];
  unsigned long long keys[DH_MAX_R];
  unsigned long long wmax[kSelWaves], wmin[kSelWaves];
  unsigned int wcnt[kSelWaves];
  unsigned long long prefix, thresh;
  int need, done;
  unsigned int count;
};

// Block-wide count, max and min of per-thread values.
__device__ void block_stats(unsigned int cnt, unsigned long long vmax, unsigned long long vmin,
                            SelectShared& sh, unsigned int& total, unsigned long long& gmax,
                            unsigned long long& gmin) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off, 64);
    vmax = umax64(vmax, __shfl_xor(vmax, off, 64));
    vmin = umin64(vmin, __shfl_xor(vmin, off, 64));
  }
  if (lane == 0) {
    sh.wcnt[wave] = cnt;
    sh.wmax[wave] = vmax;
    sh.wmin[wave] = vmin;
  }
  __syncthreads();
  total = 0;
  gmax = 0ull;
  gmin = ~0ull;
  for (int i = 0; i < kSelWaves; ++i) {
    total += sh.wcnt[i];
    gmax = umax64(gmax, sh.wmax[i]);
    gmin = umin64(gmin, sh.wmin[i]);
  }
  __syncthreads();
}

// One radix pass decision: given the 256 digit counts c[4 * lane + d] of the
// keys matching the current prefix, find the digit holding the need-th largest
// key.  Returns (in all lanes) the digit, the rank within it and whether the
// bucket is taken whole.
__device__ __forceinline__ void pick_digit(const unsigned int (&c)[4], int need, int& digit,
                                           int& need_out, bool& whole) {
  const int lane = threadIdx.x & 63;
  const unsigned int mine = c[0] + c[1] + c[2] + c[3];
  unsigned int incl = mine;  // sum over lanes >= l
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned int o = __shfl_down(incl, off, 64);
    if (lane + off < 64) incl += o;
  }
  unsigned int above = incl - mine;
  int my_digit = -1, my_need = 0, my_whole = 0;
#pragma unroll
  for (int d = 3; d >= 0; --d) {
    if (above < (unsigned)need && above + c[d] >= (unsigned)need) {
      my_digit = 4 * lane + d;
      my_need = need - (int)above;
      my_whole = above + c[d] == (unsigned)need;
    }
    above += c[d];
  }
  const unsigned long long who = __ballot(my_digit >= 0);
  const int src = __ffsll((long long)who) - 1;
  digit = __shfl(my_digit, src, 64);
  need_out = __shfl(my_need, src, 64);
  whole = __shfl(my_whole, src, 64) != 0;
}

// k-th largest (1 <= k <= count of non-zero keys) of the non-zero keys the
// calling wave's lanes hold in v[0..NV) (wave-level, no workgroup barrier;
// hist: 256 words of LDS private to the wave).  Skips the leading bytes all
// keys share; stops once the bucket holding the k-th key is taken whole.
// Returns the smallest key of that bucket: exactly k keys are >= it.
// The keys are presented by key(j), j < NV, computed on demand; loops over j
// are unrolled U times (1 for keys read from memory, so that few are live).
template <int NV, int U, class Key>
__device__ unsigned long long wave_kth_largest_of(Key key_of, int k, unsigned int* hist) {
  const int lane = threadIdx.x & 63;
  unsigned long long vmax = 0ull, vmin = ~0ull;
#pragma unroll U
  for (int j = 0; j < NV; ++j) {
    const unsigned long long v = key_of(j);
    if (v) {
      vmax = umax64(vmax, v);
      vmin = umin64(vmin, v);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    vmax = umax64(vmax, __shfl_xor(vmax, off, 64));
    vmin = umin64(vmin, __shfl_xor(vmin, off, 64));
  }
  if (vmax == vmin) return vmax;
  const int common = __builtin_clzll(vmax ^ vmin) & ~7;
  unsigned long long pre = common ? (vmax >> (64 - common)) : 0ull;
  int need = k, shift = 64 - common;
  for (;;) {
    shift -= 8;
#pragma unroll
    for (int d = 0; d < 4; ++d) hist[4 * lane + d] = 0u;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the clears land before the adds
#pragma unroll U
    for (int j = 0; j < NV; ++j) {
      const unsigned long long key = key_of(j);
      if (key && (shift + 8 == 64 || (key >> (shift + 8)) == pre))
        atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    unsigned int c[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) c[d] = hist[4 * lane + d];
    int digit, nneed;
    bool whole;
    pick_digit(c, need, digit, nneed, whole);
    pre = (pre << 8) | (unsigned long long)digit;
    need = nneed;
    if (whole || shift == 0) break;
  }
  return pre << shift;
}

template <int NV>
__device__ unsigned long long wave_kth_largest(const unsigned long long (&v)[NV], int k,
                                               unsigned int* hist) {
  return wave_kth_largest_of<NV, NV>([&](int j) { return v[j]; }, k, hist);
}

// Same, over the whole workgroup: keys presented by for_each_key(f).
template <class ForEach>
__device__ unsigned long long block_kth_largest(ForEach for_each_key, int k, unsigned long long gmax,
                                                unsigned long long gmin, SelectShared& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (gmax == gmin) return gmax;
  const int common = __builtin_clzll(gmax ^ gmin) & ~7;
  unsigned long long pre = common ? (gmax >> (64 - common)) : 0ull;
  int need = k, shift = 64 - common;
  for (;;) {
    shift -= 8;
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&sh.whist[0][0])[i] = 0u;
    __syncthreads();
    for_each_key([&](unsigned long long key) {
      if (key && (shift + 8 == 64 || (key >> (shift + 8)) == pre))
        atomicAdd(&sh.whist[wave][(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (tid < 64) {
      unsigned int c[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        unsigned int t = 0;
#pragma unroll
        for (int w = 0; w < kSelWaves; ++w) t += sh.whist[w][4 * lane + d];
        c[d] = t;
      }
      int digit, nneed;
      bool whole;
      pick_digit(c, need, digit, nneed, whole);
      if (lane == 0) {
        sh.prefix = (pre << 8) | (unsigned long long)digit;
        sh.need = nneed;
        sh.done = whole || shift == 0;
      }
    }
    __syncthreads();
    pre = sh.prefix;
    need = sh.need;
    const int done = sh.done;
    __syncthreads();
    if (done) break;
  }
  return pre << shift;
}

template <int kKind>
__global__ __launch_bounds__(kSelThreads) void rerank_kernel(
    const uint16_t* __restrict__ x, RowSrc src, int K, int N, const float* __restrict__ cand_val, const int32_t* __restrict__ cand_id, int ncand, int R,
    int32_t* __restrict__ rr_id, float* __restrict__ rr_val) {
  __shared__ SelectShared sh;
  const int m = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* cv = cand_val + (size_t)m * ncand;
  const int32_t* ci = cand_id + (size_t)m * ncand;
  const bool cached = ncand <= kSelThreads * kSelCache;

  // 1. keys (thread t: candidates t + 1024 j), their count, max and min
  unsigned long long kc[kSelCache];
  unsigned long long tmax = 0ull, tmin = ~0ull;
  unsigned int tcnt = 0;
  if (cached) {
    float vv[kSelCache];
    int iv[kSelCache];
#pragma unroll
    for (int j = 0; j < kSelCache; ++j) {   // clamped, unconditional loads
      const int i = min(tid + j * kSelThreads, ncand - 1);
      vv[j] = cv[i];
      iv[j] = ci[i];
    }
#pragma unroll
    for (int j = 0; j < kSelCache; ++j)
      kc[j] = tid + j * kSelThreads < ncand ? cand_key(vv[j], iv[j], N) : 0ull;
#pragma unroll
    for (int j = 0; j < kSelCache; ++j)
      if (kc[j]) {
        ++tcnt;
        tmax = umax64(tmax, kc[j]);
        tmin = umin64(tmin, kc[j]);
      }
  } else {
    for (int i = tid; i < ncand; i += kSelThreads) {
      const unsigned long long key = cand_key(cv[i], ci[i], N);
      if (key) {
        ++tcnt;
        tmax = umax64(tmax, key);
        tmin = umin64(tmin, key);
      }
    }
  }
  sh.tmax[tid] = tmax;
  unsigned int nvalid;
  unsigned long long gmax, gmin;
  block_stats(tcnt, tmax, tmin, sh, nvalid, gmax, gmin);   // (its barriers publish tmax too)

  auto each_key = [&](auto&& f) {
    if (cached) {
#pragma unroll
      for (int j = 0; j < kSelCache; ++j) f(kc[j]);
    } else {
      for (int i = tid; i < ncand; i += kSelThreads) f(cand_key(cv[i], ci[i], N));
    }
  };
  auto gather = [&](unsigned long long t) {
    __syncthreads();   // earlier readers of sh.count are done
    if (tid == 0) sh.count = 0;
    __syncthreads();
    each_key([&](unsigned long long key) {
      if (key && key >= t) {
        const unsigned int pos = atomicAdd(&sh.count, 1u);
        if (pos < (unsigned)DH_MAX_R) sh.keys[pos] = key;
      }
    });
    __syncthreads();
    return sh.count;
  };

  // 2. threshold; 3. survivors
  unsigned int got;
  if (nvalid <= (unsigned)R) {
    got = gather(1ull);                  // every valid key
  } else {
    bool exact = !cached;
    if (cached) {
      if (wave == 0) {
        unsigned long long mv[kSelCache];
        unsigned int nm = 0;
#pragma unroll
        for (int j = 0; j < kSelCache; ++j) {
          mv[j] = sh.tmax[lane + 64 * j];
          nm += mv[j] != 0ull;
        }
        for (int off = 32; off > 0; off >>= 1) nm += __shfl_xor(nm, off, 64);
        // with at most R non-empty threads every valid key is a survivor
        const unsigned long long t = nm > (unsigned)R ? wave_kth_largest(mv, R, &sh.whist[0][0]) : 1ull;
        if (lane == 0) sh.thresh = t;
      }
      __syncthreads();
      got = gather(sh.thresh);
      exact = got > (unsigned)DH_MAX_R;
    }
    if (exact) got = gather(block_kth_largest(each_key, R, gmax, gmin, sh));
  }
  const int cnt = (int)min(got, (unsigned)R);
  const int ns = (int)min(got, (unsigned)DH_MAX_R);

  // sort the survivors, descending
  if (ns <= 64) {
    if (wave == 0) {
      unsigned long long v = lane < ns ? sh.keys[lane] : 0ull;
      for (int size = 2; size <= 64; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          const unsigned long long o = __shfl_xor(v, stride, 64);
          const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
          v = keep_max ? umax64(v, o) : umin64(v, o);
        }
      if (lane < ns) sh.keys[lane] = v;
    }
    __syncthreads();
  } else {
    int P = 1;
    while (P < ns) P <<= 1;
    for (int i = ns + tid; i < P; i += kSelThreads) sh.keys[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < P; i += kSelThreads) {
          const int j = i ^ stride;
          if (j > i) {
            const bool desc = (i & size) == 0;
            const unsigned long long a = sh.keys[i], c = sh.keys[j];
            if (desc ? (a < c) : (a > c)) {
              sh.keys[i] = c;
              sh.keys[j] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  for (int r = tid; r < R; r += kSelThreads)
    rr_id[(size_t)m * R + r] = (r < cnt) ? (int32_t)key_id(sh.keys[r]) : -1;

  // exact logits of the selected rows, one wave per row
  const uint16_t* xr = x + (size_t)m * K;
  for (int r = wave; r < R; r += kSelWaves) {
    const bool valid = r < cnt;
    float sum = 0.f;
    if (valid) {
      const uint32_t id = key_id(sh.keys[r]);
      sum = wave_dot<kKind>(src, id, xr, K, lane);
    }
    if (lane == 0) rr_val[(size_t)m * R + r] = valid ? sum : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// Rerank, block-maximum path (rerank_list below).  It relies on the candidate
// arrays being the ones draft_head_coarse writes: block b owns slots
// b*kcand .. b*kcand+kcand-1 in (value desc, column asc) order, so slot
// b*kcand holds the block maximum, and among equal values slot order is
// column order.  Keys built from (value, ~slot) therefore order the
// candidates exactly as (value, ~id) does.
constexpr int kFastNV = 32;        // block maxima per lane (over all waves): nblk <= 2048

__device__ __forceinline__ unsigned long long slot_key(float v, int slot) {
  if (v == -__builtin_inff()) return 0ull;   // padding slot
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)slot);
}

__device__ __forceinline__ int lane_prefix(unsigned long long bal) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// Rerank of one row split over `nparts` workgroups of NTHR threads (NW = NTHR/64
// waves each).  Every part of row m computes the row's top-R list (the same
// list in every part), then each of its waves computes the exact logits of
// ranks r = NW (part + nparts i) + wave, so the R rows of W are read by up to
// NW * nparts waves at once.  With kArgmax each part takes the best of its
// ranks, and the last part of the row to finish (a per-row arrival counter,
// zeroed by the coarse kernel of the same call and reset here) takes the best
// of the parts' bests.
//
// The list (block-maximum selection; the candidates are the ones
// draft_head_coarse writes, so slot b*kcand holds block b's maximum and slot
// order is column order among equal values):
//   1. The waves read the block maxima (block lane + 64 j: 32 per lane over
//      all waves; from the contiguous copy the coarse kernels write for the
//      one-call path, else at slot b*kcand) as (value, slot) keys.
//      With R <= 64, T' = the R-th largest of the 64 lane maxima (their
//      value halves cut to 16 bits, by bisection with ballots) is at most the
//      R-th largest block maximum, so every one of the row's R best
//      candidates is >= T'; the blocks at or above it are compacted in the
//      same pass that counts them.  If T' lets more than DH_MAX_R / kcand
//      blocks through (or R > 64), T' = the exact R-th largest block maximum
//      (radix select by wave 0) and the blocks are compacted again.
//   2. The candidates >= T' of those blocks survive (at least R, at most
//      DH_MAX_R); each is ranked by counting the survivors above it (eight
//      lanes per key up to 64 survivors), and the first R ranks are the
//      list.
// Eight waves per workgroup, four workgroups per row at R = 32: measured per
// call (K = 5120, N = 124160) against four waves in eight parts, sixteen in
// two and sixteen in one: 41.2 / 42.5 / 42.9 / 45.3 us at M = 1, 46.4 / 48.2
// / 48.3 / 50.0 us at M = 8, within 0.3 us of each other at M = 72 except
// four waves (+3 us): fewer parts repeat the list less, but load the R rows
// of W through fewer CUs.
constexpr int kWideThreads = 512;
// From this many rows on, the one-call path takes each row in two
// workgroups, each wave holding the loads of kRerankRows candidate rows at
// once (16 rows in flight per workgroup at R = 32): with this many rows the
// R rows of W still arrive through enough CUs, and one hand-off between two
// parts costs less than four parts' (per call, one part against four:
// 132.4 / 133.5 us at M = 72, 99.4 / 99.1 at 48, 73.8 / 71.5 at 32, 50.2 /
// 47.8 at 8: with few rows, a row's 320 KB of W through one CU takes longer
// than the hand-off; two parts against one, on another box: 118.7-119.2 /
// 119.7 us at M = 72, 105.7-105.8 / 106.2-107.2 at 64; two against four:
// 90.8-91.0 / 91.5-92.2 us at M = 48, equal at 16 and 32).
constexpr int kRerankManyRowsM = 48;
constexpr int kRerankRows = 2;
// Dynamic LDS of the block-maximum rerank: x of one row (K <= DH_MAX_K).
constexpr size_t kWideMaxLds = (size_t)2 * DH_MAX_K;

struct WideShared {
  unsigned int hist[256];
  unsigned int bmax[16][64];   // per wave, each lane's largest block maximum
  int qual[DH_MAX_R];
  unsigned long long keys[DH_MAX_R];
  unsigned long long list[DH_MAX_R];
  unsigned long long T;
  int ns, qcur;
  uint32_t wbest[16][2];   // per wave: its best exact logit (value bits, id)
};

static_assert(64 * kFastNV * sizeof(uint32_t) <= sizeof(WideShared::keys), "block maxima staged in keys");

// Row m's top-R list into sh.list[0..R); called by the whole workgroup, ends
// with a barrier.
template <int NTHR>
__device__ void rerank_list(WideShared& sh, const RerankArgs& A, int m) {
  constexpr int kGather = DH_MAX_R / NTHR;   // candidate loads per thread in flight
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nblk = A.nblk, kcand = A.kcand, R = A.R, N = A.N;
  const int ncand = nblk * kcand;
  const float* cv = A.cand_val + (size_t)m * ncand;
  const int32_t* ci = A.cand_id + (size_t)m * ncand;

  // Block b = lane + 64 j, j = JW * wave + jj: its maximum's key is
  // slot_key(value, b * kcand), held as the upper half alone (0: no such
  // block); the lower half is ~(b * kcand), so keys compare as (upper, then
  // lower j first).  Each wave holds JW of every lane's kFastNV maxima.
  constexpr int NW = NTHR / 64, JW = kFastNV / NW;
  static_assert(kFastNV % NW == 0 && NW <= 16, "maxima split over the waves");
  // the maxima: contiguous where the coarse kernel wrote them so, else slot
  // b*kcand of the candidate array (the same value)
  const float* mx = A.bmax ? A.bmax + (size_t)m * nblk : cv;
  const int mstride = A.bmax ? 1 : kcand;
  uint32_t mo[JW];
#pragma unroll
  for (int jj = 0; jj < JW; ++jj)
    mo[jj] = __float_as_uint(mx[min(lane + 64 * (JW * wave + jj), nblk - 1) * mstride]);   // clamped loads
#pragma unroll
  for (int jj = 0; jj < JW; ++jj)
    mo[jj] = lane + 64 * (JW * wave + jj) < nblk ? (uint32_t)(slot_key(__uint_as_float(mo[jj]), 0) >> 32) : 0u;
  auto lower = [&](int j) { return 0xFFFFFFFFu - (uint32_t)((lane + 64 * j) * kcand); };
  // key of (lane, JW wave + jj) >= (to, tl), for a block that exists and has
  // a maximum (o != 0: so at most R blocks qualify against an exact T, even
  // where fewer than R blocks have a maximum and T is 0)
  auto at_least = [&](int jj, uint32_t to, uint32_t tl) {
    const uint32_t o = mo[jj];
    return (o != 0u) & ((o > to) | ((o == to) & (lower(JW * wave + jj) >= tl)));
  };
  uint32_t* so = reinterpret_cast<uint32_t*>(sh.keys);   // every maximum, for the exact fallback
  uint32_t bw = 0u;
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    bw = max(bw, mo[jj]);
    so[64 * (JW * wave + jj) + lane] = mo[jj];
  }
  sh.bmax[wave][lane] = bw;
  if (tid == 0) {
    sh.qcur = 0;
    sh.ns = 0;
  }
  // The blocks whose maximum is >= (to, tl), compacted into sh.qual (their
  // order does not matter; entries past its capacity are dropped, and then
  // the count rules this threshold out).
  auto compact = [&](uint32_t to, uint32_t tl) {
    unsigned long long bal[JW];
    int nw = 0;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      bal[jj] = __ballot(at_least(jj, to, tl));
      nw += __popcll(bal[jj]);
    }
    int base = 0;
    if (lane == 0) base = atomicAdd(&sh.qcur, nw);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int q = base + lane_prefix(bal[jj]);
      if (((bal[jj] >> lane) & 1ull) && q < DH_MAX_R) sh.qual[q] = lane + 64 * (JW * wave + jj);
      base += __popcll(bal[jj]);
    }
  };
  __syncthreads();
  // T' = (to, 0) with to the R-th largest of the 64 lane maxima's upper
  // halves cut to their top 16 bits (bisection over those bits, counting
  // lanes by ballot; every wave finds the same value): at least R lanes hold
  // a block maximum >= T', so T' is at most the R-th largest block maximum
  // (the cut lowers it by less than one bf16 step, letting a few more blocks
  // through for half the steps).  Its blocks are compacted at once; the
  // count decides after one barrier whether T' stands.
  uint32_t to = 0u;
  if (R <= 64) {
    uint32_t bo = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) bo = max(bo, sh.bmax[w][lane]);
    for (int bit = 31; bit >= 16; --bit) {
      const uint32_t t = to | (1u << bit);
      if (__popcll(__ballot(bo >= t)) >= R) to = t;
    }
    compact(to, 0u);
  }
  __syncthreads();
  int nq = sh.qcur;
  unsigned long long T = (unsigned long long)to << 32;
  if (R > 64 || to == 0u || nq * kcand > DH_MAX_R) {   // uniform: the exact R-th largest maximum
    __syncthreads();   // every thread has read qcur
    if (wave == 0) {
      T = wave_kth_largest_of<kFastNV, 1>(
          [&](int j) -> unsigned long long {
            const uint32_t o = *reinterpret_cast<volatile uint32_t*>(so + 64 * j + lane);
            return o ? ((unsigned long long)o << 32) | lower(j) : 0ull;
          },
          R, sh.hist);
      if (lane == 0) {
        sh.T = T;
        sh.qcur = 0;
      }
    }
    __syncthreads();
    T = sh.T;
    compact((uint32_t)(T >> 32), (uint32_t)T);
    __syncthreads();
    nq = sh.qcur;
  }
  for (int i = tid; i < R; i += NTHR) sh.list[i] = 0ull;   // a rank no survivor takes stays empty
  if (nq > 0) {   // the survivors, gathered by the whole workgroup (their order does not matter)
    const int items = nq * kcand;   // <= DH_MAX_R; no block qualifies only where none has a maximum
    float v[kGather];
    int id[kGather], slot[kGather];
#pragma unroll
    for (int j = 0; j < kGather; ++j) {   // clamped loads
      const int i = min(tid + NTHR * j, items - 1);
      slot[j] = sh.qual[i / kcand] * kcand + i % kcand;
      v[j] = cv[slot[j]];
      id[j] = ci[slot[j]];
    }
#pragma unroll
    for (int j = 0; j < kGather; ++j) {
      const bool in = tid + NTHR * j < items;
      const unsigned long long k = in ? slot_key(v[j], slot[j]) : 0ull;
      if (k != 0ull && k >= T && id[j] >= 0 && id[j] < N) sh.keys[atomicAdd(&sh.ns, 1)] = cand_key(v[j], id[j], N);
    }
  }
  __syncthreads();
  // Rank the survivors (distinct keys): list[rank] for rank < R, a key's
  // rank being the number of survivors above it.  Up to 64 survivors (NTHR
  // >= 512): eight lanes per key, each counting every eighth survivor, summed
  // over the eight by DPP; more: one thread per key.
  const int ns = sh.ns;   // R <= ns <= DH_MAX_R
  if (NTHR >= 512 && ns <= 64) {   // uniform
    const int i = tid >> 3, c = tid & 7;
    const unsigned long long key = i < ns ? sh.keys[i] : 0ull;
    int above = 0;
    for (int j = c; j < ns; j += 8) above += sh.keys[j] > key;
    above += __builtin_amdgcn_update_dpp(0, above, 0xB1, 0xF, 0xF, false);    // quad_perm 1,0,3,2
    above += __builtin_amdgcn_update_dpp(0, above, 0x4E, 0xF, 0xF, false);    // quad_perm 2,3,0,1
    above += __builtin_amdgcn_update_dpp(0, above, 0x141, 0xF, 0xF, false);   // row_half_mirror
    if (c == 0 && i < ns && above < R) sh.list[above] = key;
  } else {
    for (int i = tid; i < ns; i += NTHR) {
      const unsigned long long key = sh.keys[i];
      int above = 0;
      for (int j = 0; j < ns; ++j) above += sh.keys[j] > key;
      if (above < R) sh.list[above] = key;
    }
  }
  __syncthreads();
}

// A row's hand-off word between the parts of its rerank: bits 63..4 the best
// (value, id) seen so far as a 60-bit key that orders exactly as ranks_above
// does, bits 3..0 the number of parts counted.  Key: the value's
// order-preserving 32 bits (-0 taken as +0; a NaN as 0, below -inf's key),
// then 2^28 - 1 - id (a lower id above), so that 0 is "nothing yet" and no
// candidate's key is 0 (ids are below 2^28 - 1).
constexpr int kHandIdBits = 28;
__device__ __forceinline__ unsigned long long hand_key(float v, int id) {
  if (id < 0) return 0ull;
  const uint32_t vk = v != v ? 0u : f32_key(v + 0.0f);
  return ((unsigned long long)vk << kHandIdBits) | (unsigned long long)((1u << kHandIdBits) - 1u - (uint32_t)id);
}
__device__ __forceinline__ void hand_decode(unsigned long long key, float& v, int& id) {
  if (key == 0ull) {
    v = -__builtin_inff();
    id = -1;
    return;
  }
  const uint32_t vk = (uint32_t)(key >> kHandIdBits);
  v = vk == 0u ? __builtin_nanf("") : key_f32(vk);
  id = (int)((1u << kHandIdBits) - 1u - (uint32_t)(key & ((1u << kHandIdBits) - 1u)));
}

// (v, id) ranks above (bv, bi) in the final argmax: a larger value, or an
// equal one with a lower id.  A NaN value (an NVFP4 row with a NaN block
// scale) ranks below every number, -inf included; id < 0 is an empty slot
// and never ranks above anything, bi < 0 (nothing yet) is below everything.
__device__ __forceinline__ bool ranks_above(float v, int id, float bv, int bi) {
  if (id < 0) return false;
  if (bi < 0) return true;
  const bool vn = v != v, bn = bv != bv;
  if (vn != bn) return bn;
  if (vn) return id < bi;
  return v > bv || (v == bv && id < bi);
}

constexpr int kMaxParts = 8;   // workgroups one row's exact logits are split over, at most

// Ranks r = NW (part + nparts i) + wave of row m: this part's share of the
// exact logits.  With kArgmax the part also takes the best of its ranks; a
// row split over several parts hands the parts' bests to the part that
// arrives last.
template <int NTHR, bool kArgmax, int kKind, int NR>
__device__ void rerank_part(WideShared& sh, u32x4* xlds, const RerankArgs& A, int m, int part, int nparts) {
  constexpr int NW = NTHR / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = A.R, K = A.K;
  // x[m] into LDS by DMA while the list is selected: op o of wave w (o = w,
  // w + NW, ...) moves bytes 1024 o .. 1024 o + 1023 of the row, lanes past
  // the row's end re-reading its last 16 bytes into the padding
  {
    const uint16_t* xg = A.x + (size_t)m * K;
    const int bytes = 2 * K, ops = (bytes + 1023) / 1024;
    const int w0 = __builtin_amdgcn_readfirstlane(wave);
    for (int o = w0; o < ops; o += NW) {   // wave-uniform
      const uint32_t voff = (uint32_t)min(1024 * o + 16 * lane, bytes - 16);
      dma16(voff, xg, __builtin_amdgcn_readfirstlane(lds_addr(xlds) + 1024 * o));
    }
  }
  rerank_list<NTHR>(sh, A, m);
  wait_vm<0>();   // this wave's DMA has landed; after the barrier, every wave's
  __syncthreads();
  const uint16_t* xr = reinterpret_cast<const uint16_t*>(xlds);

  // The exact logits of ranks NR s .. NR s + NR - 1, slot s = NW (part +
  // nparts i) + wave: this wave reads the NR rows of W once, all loads in
  // flight.  An empty rank (key 0: fewer survivors than R, which candidates
  // written by the coarse pass never leave) is (-1, -inf).
  float bv = -__builtin_inff();
  int bi = -1;
  for (int sl = NW * part + wave; NR * sl < R; sl += NW * nparts) {   // wave-uniform
    int ids[NR];
    float sums[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = NR * sl + i;
      const unsigned long long key = r < R ? sh.list[r] : 0ull;
      ids[i] = key ? (int)key_id(key) : -1;
    }
    wave_dots<kKind, NR>(A.src, ids, xr, K, lane, sums);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = NR * sl + i;
      if (r >= R) break;
      if (lane == 0) {
        A.rr_id[(size_t)m * R + r] = ids[i];
        A.rr_val[(size_t)m * R + r] = sums[i];
        // `y.scatter_(1, idx, ex.to(bfloat16))`: ids of one row are distinct
        if (A.row_out && ids[i] >= 0) A.row_out[(size_t)m * A.N + ids[i]] = (uint16_t)f32_to_bf16_rne(sums[i]);
      }
      if (ranks_above(sums[i], ids[i], bv, bi)) {
        bv = sums[i];
        bi = ids[i];
      }
    }
  }
  if constexpr (kArgmax) {
    // the part's best: each wave's, then thread 0 over the NW waves
    if (lane == 0) {
      sh.wbest[wave][0] = __float_as_uint(bv);
      sh.wbest[wave][1] = (uint32_t)bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NW; ++w) {
        const float v = __uint_as_float(sh.wbest[w][0]);
        const int id = (int)sh.wbest[w][1];
        if (ranks_above(v, id, bv, bi)) {
          bv = v;
          bi = id;
        }
      }
      if (nparts == 1) {
        A.out_id[m] = bi;
        A.out_val[m] = bv;
      } else {
        // Several parts: each folds its best into the row's hand-off word
        // with one compare-and-swap, which also counts the part; the part
        // that brings the count to nparts holds the row's best and writes it.
        // Everything handed over travels in that one atomic word, so no
        // other memory has to be made visible between the workgroups.
        unsigned long long* word = A.hand + m;
        const unsigned long long mine = hand_key(bv, bi);
        unsigned long long old = 0ull, next;
        for (;;) {
          const unsigned long long best = (old >> 4) > mine ? old >> 4 : mine;
          next = (best << 4) | ((old & 15ull) + 1ull);
          unsigned long long seen = old;
          if (__hip_atomic_compare_exchange_strong(word, &seen, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT))
            break;
          old = seen;
        }
        if ((int)(next & 15ull) == nparts) {
          hand_decode(next >> 4, bv, bi);
          A.out_id[m] = bi;
          A.out_val[m] = bv;
          // ready for the next call (ordered before it by the kernel boundary)
          __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// Rerank kernel: grid (nparts, M), one part of one row per workgroup, NR
// candidate rows per wave at a time.
template <bool kArgmax, int kKind, int NTHR, int NR>
__global__ __launch_bounds__(NTHR) void rerank_wide_kernel(RerankArgs A) {
  __shared__ WideShared sh;
  extern __shared__ __align__(16) u32x4 xlds[];   // x[m], rounded up to 1 KB
  rerank_part<NTHR, kArgmax, kKind, NR>(sh, xlds, A, blockIdx.y, blockIdx.x, gridDim.x);
}


// Final token: one wave per row; largest value, ties to the lower id, id -1 skipped.
__global__ __launch_bounds__(256) void argmax_kernel(const int32_t* __restrict__ rr_id,
                                                     const float* __restrict__ rr_val, int M, int R,
                                                     int32_t* __restrict__ out_id,
                                                     float* __restrict__ out_val) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  float bv = -__builtin_inff();
  int bi = -1;
  for (int r = lane; r < R; r += 64) {
    const int id = rr_id[(size_t)m * R + r];
    const float v = rr_val[(size_t)m * R + r];
    if (ranks_above(v, id, bv, bi)) {
      bv = v;
      bi = id;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (ranks_above(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    out_id[m] = bi;
    out_val[m] = bv;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_k(int K) {
  if (K < 512 || K % 512 != 0 || K > DH_MAX_K)
    return dh::fail(DH_ESHAPE, "K must be a positive multiple of 512 up to %d (got %d)", DH_MAX_K, K);
  return DH_OK;
}

// A 4-bit head runs as a 2-bit head of length 2K.
int check_k4(int K) {
  if (K < 256 || K % 256 != 0 || 2 * K > DH_MAX_K)
    return dh::fail(DH_ESHAPE, "K must be a positive multiple of 256 up to %d for a 4-bit head (got %d)",
                    DH_MAX_K / 2, K);
  return DH_OK;
}

// The rerank reads whole rows of K elements: any multiple of 256.
int check_k_rerank(int K) {
  if (K < 256 || K % 256 != 0 || K > DH_MAX_K)
    return dh::fail(DH_ESHAPE, "K must be a positive multiple of 256 up to %d (got %d)", DH_MAX_K, K);
  return DH_OK;
}

int check_m(int M) {
  if (M < 1) return dh::fail(DH_EINVAL, "M must be >= 1 (got %d)", M);
  if (M > DH_MAX_M) return dh::fail(DH_EUNSUP, "M must be <= %d (got %d)", DH_MAX_M, M);
  return DH_OK;
}

int launch_error(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return dh::fail(DH_EHIP, "%s: %s", what, hipGetErrorString(e));
  return dh::ok();
}

constexpr size_t kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950

size_t resident_lds_bytes(int K, int MP) {
  const size_t groups = (size_t)K / DH_GROUP;
  const size_t blocks = (size_t)res_waves_of(MP) * res_nt(MP) / 4;   // 4 / res_nt waves per block
  return groups * 16 * MP * 16 + groups * MP * sizeof(float) + blocks * MP * 64 * sizeof(float);
}

template <int MP, bool kHalf>
hipError_t launch_resident_k(const CoarseArgs& A, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const size_t lds = resident_lds_bytes(A.kx, MP);
  static bool attr_set = false;   // the attribute only ever grows to kMaxLds
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&coarse_resident_kernel<MP, kHalf>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  constexpr int waves = res_waves<MP>();
  constexpr int blocks = waves * res_nt(MP) / 4;   // 4 / res_nt waves per 64-column block
  dim3 grid((A.nblk + blocks - 1) / blocks);
  hipExtLaunchKernelGGL(coarse_resident_kernel<MP, kHalf>, grid, dim3(64 * waves), lds, s, e0, e1, 0, A);
  return hipGetLastError();
}
template <int MP>
hipError_t launch_resident(const CoarseArgs& A, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return A.half_pairs ? launch_resident_k<MP, true>(A, s, e0, e1) : launch_resident_k<MP, false>(A, s, e0, e1);
}

template <int MT>
hipError_t launch_h16(const HArgs& A, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr size_t lds = h16_lds_bytes(MT);
  static_assert(lds <= kMaxLds, "LDS budget of the fp16 many-row kernel");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&coarse_h16_kernel<MT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((A.c.nblk + kHBlocks - 1) / kHBlocks);
  hipExtLaunchKernelGGL(coarse_h16_kernel<MT>, grid, dim3(64 * dh::h16_waves(MT)), lds, s, e0, e1, 0, A);
  return hipGetLastError();
}

template <int MT, bool kHalf>
hipError_t launch_big_k(const BigArgs& A, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  using S = BigShape<MT, dh::big_qpb(kHalf, MT)>;
  constexpr size_t lds = big_lds_bytes<S>();
  static_assert(lds <= kMaxLds, "LDS budget of the many-row kernel");
  static_assert((size_t)S::BPW * 16 * MT * kScStride * sizeof(float) <= lds, "the score area reuses the ring's LDS");
  static_assert(lds <= kMaxLds, "LDS of one workgroup");
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&coarse_mfma_kernel<MT, kHalf>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((A.c.nblk + S::BPW - 1) / S::BPW);
  hipExtLaunchKernelGGL(coarse_mfma_kernel<MT, kHalf>, grid, dim3(64 * S::W), lds, s, e0, e1, 0, A);
  return hipGetLastError();
}
template <int MT>
hipError_t launch_big(const BigArgs& A, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return A.c.half_pairs ? launch_big_k<MT, true>(A, s, e0, e1) : launch_big_k<MT, false>(A, s, e0, e1);
}

// Rows the resident kernel is instantiated for (M padded up).  One row runs
// the two-row kernel, whose ring keeps two byte groups in flight (1.7 us
// faster at K = 5120; the one-row form cannot within 128 registers), unless
// x of two rows would not fit the LDS.
int resident_rows(int M, int K) {
  if (M <= 1) return resident_lds_bytes(K, 2) <= kMaxLds ? 2 : 1;
  return M <= 2 ? 2 : M <= 4 ? 4 : 8;
}


// The many-row path of a 2-bit head with rows of up to 16384 runs the fp16
// kernel (its x preparation holds a row's pieces in registers); a 4-bit head
// (x read modulo kx < K) and longer rows run the bf16 kernel.
// The fp16 many-row kernel from three row tiles on (one or two tiles: the
// bf16 kernel, faster there on the same box: M = 16 54.7 against 68.0 us, M =
// 32 70.6 against 78.3 us per call; M = 48, 64, 72: 92.7, 106.0, 120.1 us
// against 98.4, 113.4, 130.8 us).
bool use_h16(int K, int kx, int mt, int kcand) {
  return mt >= 3 && kx == K && K <= kPrepHMaxG * 4 * 512 && kcand <= 8;
}

// Up to 8 rows whose x fits the workgroup's LDS take the resident kernel (no
// workspace); every other M the many-row kernel, in launches of up to 80 rows.
// ks: the staged row length of x (K, or K/2 for a 4-bit head in the tiles of a 2-bit head of length K).
bool use_resident(int M, int ks) { return M <= 8 && resident_lds_bytes(ks, resident_rows(M, ks)) <= kMaxLds; }

// Workspace: the rerank's per-row hand-off words; then for the resident
// kernel the block maxima of up to 8 rows, or for the many-row kernels the x
// of one launch followed by the block maxima of all M rows.  The maxima (up
// to 64 kFastNV blocks a row, fp32) are a contiguous copy of each block's
// slot 0 that the one-call path's coarse pass writes for its block-maximum
// rerank.
constexpr size_t kHeaderBytes = DH_MAX_M * sizeof(unsigned long long);
constexpr size_t kMaximaRowBytes = (size_t)64 * kFastNV * sizeof(float);
constexpr size_t kMaximaBytes = 8 * kMaximaRowBytes;

// ks: the staged row length of x when it differs from K (0: K).
size_t coarse_workspace_bytes(int M, int K, int ks = 0) {
  if (use_resident(M, ks ? ks : K)) return kHeaderBytes + kMaximaBytes;
  return kHeaderBytes + big_workspace_bytes(std::min((M + 15) / 16, kMaxMT), K) + (size_t)M * kMaximaRowBytes;
}

// Where the block maxima go in a workspace laid out for (M, K, ks).
float* workspace_maxima(void* workspace, int M, int K, int ks) {
  unsigned char* w = static_cast<unsigned char*>(workspace) + kHeaderBytes;
  if (!use_resident(M, ks ? ks : K)) w += big_workspace_bytes(std::min((M + 15) / 16, kMaxMT), K);
  return reinterpret_cast<float*>(w);
}

int validate_coarse(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                    int kcand, const float* cand_val, const int32_t* cand_id, const void* workspace,
                    size_t workspace_bytes, int ks = 0) {
  if (!x || !tiled || !pairs || !cand_val || !cand_id)
    return dh::fail(DH_EINVAL, "coarse: null pointer");
  int rc = check_m(M);
  if (rc) return rc;
  if ((rc = check_k(K))) return rc;
  if (N < 1) return dh::fail(DH_ESHAPE, "coarse: N must be >= 1 (got %d)", N);
  if (kcand < 1 || kcand > DH_MAX_KCAND)
    return dh::fail(DH_EUNSUP, "coarse: kcand must be in 1..%d (got %d)", DH_MAX_KCAND, kcand);
  if (!aligned16(x) || !aligned16(tiled) || !aligned16(pairs))
    return dh::fail(DH_EINVAL, "coarse: x, tiled and pairs must be 16-byte aligned");
  const size_t need = coarse_workspace_bytes(M, K, ks);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need)
    return dh::fail(DH_EINVAL, "coarse: M=%d, K=%d needs a 16-byte aligned workspace of %zu bytes (got %p, %zu)",
                    M, K, need, workspace, workspace_bytes);
  return DH_OK;
}

// Rows: bf16 (ldw elements, ldw % 8 == 0), e4m3 (ldw bytes, ldw % 16 == 0,
// per-row scales) or NVFP4 (ldw bytes >= K/2, ldw % 16 == 0; block scales in
// rows of lds bytes >= K/16, lds even; the global scale).  A row starts
// 16-byte aligned in each case.
int validate_rerank(const void* x, const RowSrc& src, int M, int K, int N, const float* cand_val,
                    const int32_t* cand_id, int ncand, int R, const int32_t* rr_id, const float* rr_val) {
  const bool nv = src.kind == kRowsNvfp4;
  if (!x || !src.w || !cand_val || !cand_id || !rr_id || !rr_val || (src.kind == kRowsE4m3 && !src.wscale) ||
      (nv && (!src.bscale || !src.gscale)))
    return dh::fail(DH_EINVAL, "rerank: null pointer");
  int rc = check_m(M);
  if (rc) return rc;
  if ((rc = check_k_rerank(K))) return rc;
  if (N < 1) return dh::fail(DH_ESHAPE, "rerank: N must be >= 1 (got %d)", N);
  const int align = src.kind == kRowsBf16 ? 8 : 16;
  const int64_t row = nv ? K / 2 : K;
  if (src.ldw < row || src.ldw % align != 0)
    return dh::fail(DH_EINVAL, "rerank: ldw must be >= %lld and a multiple of %d (got %lld)", (long long)row, align,
                    (long long)src.ldw);
  if (nv && (src.lds < K / 16 || src.lds % 2 != 0))
    return dh::fail(DH_EINVAL, "rerank: lds must be >= K/16 and even (got %lld)", (long long)src.lds);
  if (ncand < 1) return dh::fail(DH_EINVAL, "rerank: ncand must be >= 1 (got %d)", ncand);
  if (R < 1 || R > ncand || R > DH_MAX_R)
    return dh::fail(DH_EUNSUP, "rerank: R must be in 1..min(ncand=%d, %d) (got %d)", ncand, DH_MAX_R, R);
  if (!aligned16(x) || !aligned16(src.w))
    return dh::fail(DH_EINVAL, "rerank: x and w must be 16-byte aligned");
  if (nv && (reinterpret_cast<uintptr_t>(src.bscale) & 1u))
    return dh::fail(DH_EINVAL, "rerank: the block scales must be 2-byte aligned");
  return DH_OK;
}

int validate_argmax(const int32_t* rr_id, const float* rr_val, int M, int R, const int32_t* out_id,
                    const float* out_val) {
  if (!rr_id || !rr_val || !out_id || !out_val) return dh::fail(DH_EINVAL, "argmax: null pointer");
  int rc = check_m(M);
  if (rc) return rc;
  if (R < 1 || R > DH_MAX_R) return dh::fail(DH_EUNSUP, "argmax: R must be in 1..%d (got %d)", DH_MAX_R, R);
  return DH_OK;
}

// Launches only; arguments were validated.
// kx: row length of x (K, or K/2 for a 4-bit head run at length K).
int launch_coarse(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs, int kcand,
                  float* cand_val, int32_t* cand_id, float* coarse_out, void* workspace, hipStream_t s,
                  hipEvent_t ev0, hipEvent_t ev1, int kx = 0, uint16_t* row_out = nullptr, int topk_only = 0,
                  float* bmax = nullptr) {
  const int nblk = (N + DH_BLOCK_N - 1) / DH_BLOCK_N;
  const int ncand = nblk * kcand;
  CoarseArgs A{static_cast<const uint16_t*>(x), M, K, N, nblk, reinterpret_cast<const u32x4*>(tiled),
               reinterpret_cast<const u32x4*>(pairs), kcand, cand_val, cand_id, coarse_out, row_out, topk_only,
               static_cast<unsigned long long*>(workspace), M, kx ? kx : K};
  A.half_pairs = A.kx < A.K;   // a 4-bit head as draft_head_tile_int4 lays it out
  A.bmax = bmax;
  hipError_t e = hipSuccess;
  const int ks = A.kx;   // the row length of x the resident kernel stages
  if (use_resident(M, ks)) {
    switch (resident_rows(M, ks)) {
      case 1: e = launch_resident<1>(A, s, ev0, ev1); break;
      case 2: e = launch_resident<2>(A, s, ev0, ev1); break;
      case 4: e = launch_resident<4>(A, s, ev0, ev1); break;
      default: e = launch_resident<8>(A, s, ev0, ev1); break;
    }
    if (e != hipSuccess) return dh::fail(DH_EHIP, "coarse_resident_kernel: %s", hipGetErrorString(e));
    return dh::ok();
  }
  // Rows beyond one launch's 80 take further launches over the same weights;
  // they reuse the workspace (the launches are ordered on the stream).
  const int NG4 = K / 512;
  for (int m0 = 0; m0 < M; m0 += 16 * kMaxMT) {
    CoarseArgs B = A;
    B.M = std::min(M - m0, 16 * kMaxMT);
    B.x = A.x + (size_t)m0 * A.kx;
    B.cand_val = cand_val + (size_t)m0 * ncand;
    B.cand_id = cand_id + (size_t)m0 * ncand;
    B.coarse_out = coarse_out ? coarse_out + (size_t)m0 * N : nullptr;
    B.row_out = row_out ? row_out + (size_t)m0 * N : nullptr;
    B.bmax = bmax ? bmax + (size_t)m0 * nblk : nullptr;
    B.ncnt = m0 == 0 ? M : 0;
    const int mt = (B.M + 15) / 16, mp = 16 * mt;
    u32x4* xslab = reinterpret_cast<u32x4*>(static_cast<unsigned char*>(workspace) + kHeaderBytes);
    u32x4* zslab = xslab + (size_t)(K / DH_GROUP) * 256 * mt;
    int* fexp = reinterpret_cast<int*>(zslab + (size_t)NG4 * kZpEntries);
    hipEvent_t b0 = m0 == 0 ? ev0 : nullptr;
    hipEvent_t b1 = m0 + 16 * kMaxMT >= M ? ev1 : nullptr;
    if (use_h16(K, A.kx, mt, A.kcand)) {
      hipLaunchKernelGGL(prep_xh_kernel, dim3(mp), dim3(256), 0, s, B.x, B.M, mp, K, xslab, zslab, fexp);
      if ((e = hipGetLastError()) != hipSuccess)
        return dh::fail(DH_EHIP, "prep_xh_kernel: %s", hipGetErrorString(e));
      const HArgs HA{B, xslab, zslab, fexp};
      switch (mt) {
        case 3: e = launch_h16<3>(HA, s, b0, b1); break;
        case 4: e = launch_h16<4>(HA, s, b0, b1); break;
        default: e = launch_h16<5>(HA, s, b0, b1); break;
      }
      if (e != hipSuccess) return dh::fail(DH_EHIP, "coarse_h16_kernel: %s", hipGetErrorString(e));
      continue;
    }
    hipLaunchKernelGGL(prep_x_kernel, dim3((mp * NG4 + 3) / 4), dim3(256), 0, s, B.x, B.M, mp, K, A.kx,
                       dh::big_qpb(A.half_pairs, mt), xslab, zslab);
    if ((e = hipGetLastError()) != hipSuccess)
      return dh::fail(DH_EHIP, "prep_x_kernel: %s", hipGetErrorString(e));
    const BigArgs BA{B, xslab, zslab};
    switch (mt) {
      case 1: e = launch_big<1>(BA, s, b0, b1); break;
      case 2: e = launch_big<2>(BA, s, b0, b1); break;
      case 3: e = launch_big<3>(BA, s, b0, b1); break;
      case 4: e = launch_big<4>(BA, s, b0, b1); break;
      default: e = launch_big<5>(BA, s, b0, b1); break;
    }
    if (e != hipSuccess) return dh::fail(DH_EHIP, "coarse_mfma_kernel: %s", hipGetErrorString(e));
  }
  return dh::ok();
}

// The block-maximum rerank applies when the candidates are NBLK blocks of
// kcand slots, there are more blocks than R, wave 0 can hold every block
// maximum, and the R blocks' slots fit the survivor buffer.
bool fast_rerank(int N, int ncand, int R, int& nblk, int& kcand) {
  nblk = (N + DH_BLOCK_N - 1) / DH_BLOCK_N;
  if (ncand % nblk) return false;
  kcand = ncand / nblk;
  return kcand >= 1 && kcand <= DH_MAX_KCAND && nblk > R && nblk <= 64 * kFastNV &&
         (int64_t)R * kcand <= DH_MAX_R;
}

template <bool kArgmax>
hipError_t launch_wide(const void* x, const RowSrc& src, int M, int K, int N, const float* cand_val,
                       const int32_t* cand_id, int nblk, int kcand, int R, int32_t* rr_id, float* rr_val,
                       int32_t* out_id, float* out_val, unsigned long long* hand, hipStream_t s,
                       uint16_t* row_out = nullptr, const float* bmax = nullptr) {
  const RerankArgs A{static_cast<const uint16_t*>(x), src, K, N, cand_val,
                     cand_id, nblk, kcand, R, rr_id, rr_val, out_id, out_val, hand, row_out, bmax};
  auto go = [&](auto nthr, auto nr) {
    constexpr int NTHR = decltype(nthr)::value, NW = NTHR / 64, NR = decltype(nr)::value;
    // ids must fit the hand-off key to split a row; otherwise one part per row
    const int parts = (!kArgmax || N < (1 << kHandIdBits) - 1)
                          ? std::max(1, std::min((R + NW * NR - 1) / (NW * NR), kMaxParts)) : 1;
    const dim3 grid(parts, M);
    const size_t lds = ((size_t)2 * K + 1023) / 1024 * 1024;   // x[m] in LDS
    auto launch = [&](auto kernel) -> hipError_t {
      static bool attr_set = false;   // per instantiation; the attribute only ever grows to kWideMaxLds
      if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWideMaxLds);
        if (e != hipSuccess) return e;
        attr_set = true;
      }
      hipLaunchKernelGGL(kernel, grid, dim3(NTHR), lds, s, A);
      return hipGetLastError();
    };
    if (src.kind == kRowsE4m3) return launch(rerank_wide_kernel<kArgmax, kRowsE4m3, NTHR, NR>);
    if (src.kind == kRowsNvfp4) return launch(rerank_wide_kernel<kArgmax, kRowsNvfp4, NTHR, NR>);
    return launch(rerank_wide_kernel<kArgmax, kRowsBf16, NTHR, NR>);
  };
  if (kArgmax && M >= kRerankManyRowsM)
    return go(std::integral_constant<int, kWideThreads>{}, std::integral_constant<int, kRerankRows>{});
  return go(std::integral_constant<int, kWideThreads>{}, std::integral_constant<int, 1>{});
}

int launch_rerank(const void* x, const RowSrc& src, int M, int K, int N, const float* cand_val,
                  const int32_t* cand_id, int ncand, int R, int32_t* rr_id, float* rr_val, hipStream_t s) {
  int nblk, kcand;
  if (fast_rerank(N, ncand, R, nblk, kcand)) {
    hipError_t e = launch_wide<false>(x, src, M, K, N, cand_val, cand_id, nblk, kcand, R, rr_id, rr_val, nullptr,
                                      nullptr, nullptr, s);
    if (e != hipSuccess) return dh::fail(DH_EHIP, "rerank_wide_kernel: %s", hipGetErrorString(e));
    return dh::ok();
  }
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (src.kind == kRowsE4m3)
    hipLaunchKernelGGL(rerank_kernel<kRowsE4m3>, dim3(M), dim3(kSelThreads), 0, s, xb, src, K, N, cand_val, cand_id,
                       ncand, R, rr_id, rr_val);
  else if (src.kind == kRowsNvfp4)
    hipLaunchKernelGGL(rerank_kernel<kRowsNvfp4>, dim3(M), dim3(kSelThreads), 0, s, xb, src, K, N, cand_val,
                       cand_id, ncand, R, rr_id, rr_val);
  else
    hipLaunchKernelGGL(rerank_kernel<kRowsBf16>, dim3(M), dim3(kSelThreads), 0, s, xb, src, K, N, cand_val, cand_id,
                       ncand, R, rr_id, rr_val);
  return launch_error("rerank_kernel");
}

int launch_argmax(const int32_t* rr_id, const float* rr_val, int M, int R, int32_t* out_id, float* out_val,
                  hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3((M + 3) / 4), dim3(256), 0, s, rr_id, rr_val, M, R, out_id, out_val);
  return launch_error("argmax_kernel");
}

hipStream_t as_stream(void* p) { return reinterpret_cast<hipStream_t>(p); }

// The bf16 row handed to the caller (`_apply_head_int2` after the rerank):
// bf16(coarse), or -inf for a top-k caller, with each reranked id's exact
// value (bf16) in its entry.  Grid (ceil(N / kRowChunk), M): a workgroup
// first marks which entries of its chunk are reranked (LDS: rank, or -1),
// then writes every entry of the chunk once.
constexpr int kRowChunk = 4096;

__global__ __launch_bounds__(256) void logits_row_kernel(const float* __restrict__ coarse,
                                                         const int32_t* __restrict__ rr_id,
                                                         const float* __restrict__ rr_val, int N, int R,
                                                         int topk_only, uint16_t* __restrict__ row_out) {
  __shared__ int16_t rank[kRowChunk];
  const int m = blockIdx.y, n0 = blockIdx.x * kRowChunk, tid = threadIdx.x;
  const int len = min(kRowChunk, N - n0);
  for (int i = tid; i < kRowChunk; i += 256) rank[i] = -1;
  __syncthreads();
  for (int r = tid; r < R; r += 256) {
    const int id = rr_id[(size_t)m * R + r];
    if (id >= n0 && id < n0 + len) rank[id - n0] = (int16_t)r;
  }
  __syncthreads();
  const float* cr = coarse ? coarse + (size_t)m * N + n0 : nullptr;
  const float* vr = rr_val + (size_t)m * R;
  uint16_t* out = row_out + (size_t)m * N + n0;
  for (int i = tid; i < len; i += 256) {
    const int r = rank[i];
    uint32_t b;
    if (r >= 0) b = f32_to_bf16_rne(vr[r]);
    else b = topk_only ? 0xFF80u : f32_to_bf16_rne(cr[i]);
    out[i] = (uint16_t)b;
  }
}

// The exact values written over the bf16 row (the general rerank path; the
// block-maximum rerank writes them itself): one thread per (row, rank).
__global__ __launch_bounds__(256) void scatter_row_kernel(const int32_t* __restrict__ rr_id,
                                                          const float* __restrict__ rr_val, int M, int N, int R,
                                                          uint16_t* __restrict__ row_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * R) return;
  const int m = i / R, id = rr_id[i];
  if (id >= 0 && id < N) row_out[(size_t)m * N + id] = (uint16_t)f32_to_bf16_rne(rr_val[i]);
}

// Streaming-read reference: the achievable HBM read rate on this device, read
// the way the coarse kernel reads its codes (16-byte nontemporal loads, each
// workgroup a contiguous span, eight loads per lane in flight).  Workgroup b
// folds its span with XOR into out[b].
constexpr int kReadBlocks = DH_READ_BLOCKS;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ out) {
  const size_t per = (n16 + kReadBlocks - 1) / kReadBlocks;
  const size_t lo = (size_t)blockIdx.x * per, hi = std::min(n16, lo + per);
  uint32_t acc = 0u;
  for (size_t i = lo + threadIdx.x; i < hi; i += 256 * kReadUnroll) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const size_t k = i + 256 * u;
      v[u] = k < hi ? __builtin_nontemporal_load(p + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t wx[4];
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = wx[0] ^ wx[1] ^ wx[2] ^ wx[3];
}

}  // namespace

extern "C" {

int draft_head_workspace_bytes(int M, int K, size_t* bytes) {
  int rc = check_m(M);
  if (rc) return rc;
  if ((rc = check_k(K))) return rc;
  if (!bytes) return dh::fail(DH_EINVAL, "workspace_bytes: null pointer");
  *bytes = coarse_workspace_bytes(M, K);
  return dh::ok();
}

int draft_head_coarse(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                      int kcand, float* cand_val, int32_t* cand_id, float* coarse_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int rc = validate_coarse(x, M, K, N, tiled, pairs, kcand, cand_val, cand_id, workspace, workspace_bytes);
  if (rc) return rc;
  return launch_coarse(x, M, K, N, tiled, pairs, kcand, cand_val, cand_id, coarse_out, workspace,
                       as_stream(stream), nullptr, nullptr);
}

int draft_head_coarse_int4(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                           int kcand, float* cand_val, int32_t* cand_id, float* coarse_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int rc = check_k4(K);
  if (rc) return rc;
  if ((rc = validate_coarse(x, M, 2 * K, N, tiled, pairs, kcand, cand_val, cand_id, workspace, workspace_bytes,
                            K)))
    return rc;
  return launch_coarse(x, M, 2 * K, N, tiled, pairs, kcand, cand_val, cand_id, coarse_out, workspace,
                       as_stream(stream), nullptr, nullptr, K);
}

int draft_head_rerank(const void* x, const void* w, int64_t ldw, int M, int K, int N,
                      const float* cand_val, const int32_t* cand_id, int ncand, int R,
                      int32_t* rr_id, float* rr_val, void* stream) {
  const RowSrc src{w, ldw, nullptr, nullptr, 0, nullptr, kRowsBf16};
  int rc = validate_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val);
  if (rc) return rc;
  return launch_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val, as_stream(stream));
}

int draft_head_rerank_e4m3(const void* x, const uint8_t* w8, const float* wscale, int64_t ldw, int M, int K,
                           int N, const float* cand_val, const int32_t* cand_id, int ncand, int R,
                           int32_t* rr_id, float* rr_val, void* stream) {
  const RowSrc src{w8, ldw, wscale, nullptr, 0, nullptr, kRowsE4m3};
  int rc = validate_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val);
  if (rc) return rc;
  return launch_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val, as_stream(stream));
}

int draft_head_rerank_nvfp4(const void* x, const uint8_t* w4, int64_t ldw, const uint8_t* bscale, int64_t lds,
                            const float* gscale, int M, int K, int N, const float* cand_val, const int32_t* cand_id,
                            int ncand, int R, int32_t* rr_id, float* rr_val, void* stream) {
  const RowSrc src{w4, ldw, nullptr, bscale, lds, gscale, kRowsNvfp4};
  int rc = validate_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val);
  if (rc) return rc;
  return launch_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val, as_stream(stream));
}

int draft_head_logits_row(const float* coarse, const int32_t* rr_id, const float* rr_val, int M, int N, int R,
                          int topk_only, uint16_t* row_out, void* stream) {
  if (!rr_id || !rr_val || !row_out) return dh::fail(DH_EINVAL, "logits_row: null pointer");
  if (!coarse && !topk_only) return dh::fail(DH_EINVAL, "logits_row: coarse is needed unless topk_only");
  int rc = check_m(M);
  if (rc) return rc;
  if (N < 1) return dh::fail(DH_ESHAPE, "logits_row: N must be >= 1 (got %d)", N);
  if (R < 1 || R > DH_MAX_R) return dh::fail(DH_EUNSUP, "logits_row: R must be in 1..%d (got %d)", DH_MAX_R, R);
  hipLaunchKernelGGL(logits_row_kernel, dim3((N + kRowChunk - 1) / kRowChunk, M), dim3(256), 0, as_stream(stream),
                     coarse, rr_id, rr_val, N, R, topk_only ? 1 : 0, row_out);
  return launch_error("logits_row_kernel");
}

int draft_head_stream_read(const void* p, size_t bytes, uint32_t* out, void* stream) {
  if (!p || !out) return dh::fail(DH_EINVAL, "stream_read: null pointer");
  if (!aligned16(p) || bytes % 16 != 0 || bytes == 0)
    return dh::fail(DH_EINVAL, "stream_read: p must be 16-byte aligned and bytes a positive multiple of 16");
  hipLaunchKernelGGL(stream_read_kernel, dim3(kReadBlocks), dim3(256), 0, as_stream(stream),
                     static_cast<const u32x4*>(p), bytes / 16, out);
  return launch_error("stream_read_kernel");
}

int draft_head_argmax(const int32_t* rr_id, const float* rr_val, int M, int R, int32_t* out_id,
                      float* out_val, void* stream) {
  int rc = validate_argmax(rr_id, rr_val, M, R, out_id, out_val);
  if (rc) return rc;
  return launch_argmax(rr_id, rr_val, M, R, out_id, out_val, as_stream(stream));
}

}  // extern "C"

namespace {

// One call: coarse launch(es), then rerank + argmax on the rows src describes.
// int4: the coarse head is a 4-bit one in the tiles of a 2-bit head of
// length 2K (draft_head_tile_int4); the rerank reads rows of length K as always.
int validate_forward(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                     const RowSrc& src, int kcand, int R, const float* cand_val, const int32_t* cand_id,
                     const int32_t* rr_id, const float* rr_val, const int32_t* out_id, const float* out_val,
                     const void* workspace, size_t workspace_bytes, bool int4) {
  const int ncand = (N > 0 && kcand > 0) ? ((N + DH_BLOCK_N - 1) / DH_BLOCK_N) * kcand : 0;
  int rc = int4 ? check_k4(K) : DH_OK;
  if (rc) return rc;
  const int Kc = int4 ? 2 * K : K;
  if ((rc = validate_coarse(x, M, Kc, N, tiled, pairs, kcand, cand_val, cand_id, workspace, workspace_bytes,
                            int4 ? K : 0)))
    return rc;
  if ((rc = validate_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val))) return rc;
  return validate_argmax(rr_id, rr_val, M, R, out_id, out_val);
}

// Launches of one validated call.
// row_out (optional): the bf16 row for the caller, filled by the coarse
// kernel (coarse scores, or -inf with topk_only) and overwritten at the
// reranked ids with their exact values.
int launch_forward(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                   const RowSrc& src, int kcand, int R, float* cand_val, int32_t* cand_id, int32_t* rr_id,
                   float* rr_val, int32_t* out_id, float* out_val, float* coarse_out, void* workspace,
                   hipStream_t s, void* coarse_start_event, void* coarse_stop_event, bool int4,
                   uint16_t* row_out = nullptr, int topk_only = 0) {
  const int ncand = ((N + DH_BLOCK_N - 1) / DH_BLOCK_N) * kcand;
  const int Kc = int4 ? 2 * K : K;
  int nblk, kc;
  const bool fast = fast_rerank(N, ncand, R, nblk, kc);
  // the coarse pass also writes the block maxima contiguously for the
  // block-maximum rerank (nblk <= 64 kFastNV there)
  float* bmax = fast ? workspace_maxima(workspace, M, Kc, K) : nullptr;
  int rc = launch_coarse(x, M, Kc, N, tiled, pairs, kcand, cand_val, cand_id, coarse_out, workspace, s,
                         reinterpret_cast<hipEvent_t>(coarse_start_event),
                         reinterpret_cast<hipEvent_t>(coarse_stop_event), K, row_out, topk_only, bmax);
  if (rc) return rc;
  if (fast) {   // rerank and argmax in one kernel
    hipError_t e = launch_wide<true>(x, src, M, K, N, cand_val, cand_id, nblk, kc, R, rr_id, rr_val, out_id, out_val,
                                     static_cast<unsigned long long*>(workspace), s, row_out, bmax);
    if (e != hipSuccess) return dh::fail(DH_EHIP, "rerank_wide_kernel: %s", hipGetErrorString(e));
    return dh::ok();
  }
  if ((rc = launch_rerank(x, src, M, K, N, cand_val, cand_id, ncand, R, rr_id, rr_val, s))) return rc;
  if (row_out) {
    hipLaunchKernelGGL(scatter_row_kernel, dim3((M * R + 255) / 256), dim3(256), 0, s, rr_id, rr_val, M, N, R,
                       row_out);
    if ((rc = launch_error("scatter_row_kernel"))) return rc;
  }
  return launch_argmax(rr_id, rr_val, M, R, out_id, out_val, s);
}

int forward_impl(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs, const RowSrc& src,
                 int kcand, int R, float* cand_val, int32_t* cand_id,
                 int32_t* rr_id, float* rr_val, int32_t* out_id, float* out_val, float* coarse_out,
                 void* workspace, size_t workspace_bytes, void* stream, void* coarse_start_event,
                 void* coarse_stop_event, bool int4 = false) {
  int rc = validate_forward(x, M, K, N, tiled, pairs, src, kcand, R, cand_val, cand_id, rr_id, rr_val, out_id,
                            out_val, workspace, workspace_bytes, int4);
  if (rc) return rc;
  return launch_forward(x, M, K, N, tiled, pairs, src, kcand, R, cand_val, cand_id, rr_id, rr_val, out_id, out_val,
                        coarse_out, workspace, as_stream(stream), coarse_start_event, coarse_stop_event, int4);
}

// ---------------------------------------------------------------------------
// The one-call path for callers that cannot allocate (code under graph
// capture, serving loops or harnesses that forbid allocation): its workspace
// is `scratch`, a static device array that every GPU the library runs on
// holds until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the memory is reached only through the
// address hipGetSymbolAddress gives, once per device, kept in scratch_ptr.
// Every call on a GPU shares that GPU's array (calls that overlap on one GPU
// race); the kernels clear what must start at zero themselves (the coarse
// kernel zeroes the rerank's hand-off words of every call).
constexpr size_t kScratchBytes = DH_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The scratch address on the stream's device, which must be the current one.
int scratch_for(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dh::fail(DH_EHIP, "forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (s) {
    hipDevice_t sdev = -1;
    if ((e = hipStreamGetDevice(s, &sdev)) != hipSuccess)
      return dh::fail(DH_EHIP, "forward_noalloc: hipStreamGetDevice: %s", hipGetErrorString(e));
    if ((int)sdev != dev)
      return dh::fail(DH_EINVAL, "forward_noalloc: the stream belongs to device %d but device %d is current",
                      (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return dh::fail(DH_EUNSUP, "forward_noalloc: device %d beyond the %d the library keeps scratch for", dev,
                    kMaxDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess || !p)
      return dh::fail(DH_EHIP, "forward_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                      hipGetErrorString(e));
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return DH_OK;
}

}  // namespace

extern "C" {

int draft_head_forward(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                       const void* w, int64_t ldw, int kcand, int R, float* cand_val, int32_t* cand_id,
                       int32_t* rr_id, float* rr_val, int32_t* out_id, float* out_val, float* coarse_out,
                       void* workspace, size_t workspace_bytes, void* stream, void* coarse_start_event,
                       void* coarse_stop_event) {
  return forward_impl(x, M, K, N, tiled, pairs, RowSrc{w, ldw, nullptr, nullptr, 0, nullptr, kRowsBf16}, kcand, R,
                      cand_val, cand_id, rr_id, rr_val, out_id, out_val, coarse_out, workspace, workspace_bytes,
                      stream, coarse_start_event, coarse_stop_event);
}

int draft_head_forward_int4(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                            const void* w, int64_t ldw, int kcand, int R, float* cand_val, int32_t* cand_id,
                            int32_t* rr_id, float* rr_val, int32_t* out_id, float* out_val, float* coarse_out,
                            void* workspace, size_t workspace_bytes, void* stream, void* coarse_start_event,
                            void* coarse_stop_event) {
  return forward_impl(x, M, K, N, tiled, pairs, RowSrc{w, ldw, nullptr, nullptr, 0, nullptr, kRowsBf16}, kcand, R,
                      cand_val, cand_id, rr_id, rr_val, out_id, out_val, coarse_out, workspace, workspace_bytes,
                      stream, coarse_start_event, coarse_stop_event, true);
}

int draft_head_forward_e4m3(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                            const uint8_t* w8, const float* wscale, int64_t ldw, int kcand, int R, float* cand_val,
                            int32_t* cand_id, int32_t* rr_id, float* rr_val, int32_t* out_id, float* out_val,
                            float* coarse_out, void* workspace, size_t workspace_bytes, void* stream,
                            void* coarse_start_event, void* coarse_stop_event) {
  return forward_impl(x, M, K, N, tiled, pairs, RowSrc{w8, ldw, wscale, nullptr, 0, nullptr, kRowsE4m3}, kcand, R,
                      cand_val, cand_id, rr_id, rr_val, out_id, out_val, coarse_out, workspace, workspace_bytes,
                      stream, coarse_start_event, coarse_stop_event);
}

int draft_head_forward_row(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                           const void* w, int64_t ldw, int kcand, int R, float* cand_val, int32_t* cand_id,
                           int32_t* rr_id, float* rr_val, int32_t* out_id, float* out_val, uint16_t* row_out,
                           int topk_only, void* workspace, size_t workspace_bytes, void* stream) {
  const RowSrc src{w, ldw, nullptr, nullptr, 0, nullptr, kRowsBf16};
  if (!row_out) return dh::fail(DH_EINVAL, "forward_row: null row_out");
  int rc = validate_forward(x, M, K, N, tiled, pairs, src, kcand, R, cand_val, cand_id, rr_id, rr_val, out_id,
                            out_val, workspace, workspace_bytes, false);
  if (rc) return rc;
  return launch_forward(x, M, K, N, tiled, pairs, src, kcand, R, cand_val, cand_id, rr_id, rr_val, out_id, out_val,
                        nullptr, workspace, as_stream(stream), nullptr, nullptr, false, row_out, topk_only ? 1 : 0);
}

int draft_head_forward_noalloc(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                               const void* w, int64_t ldw, int kcand, int R, float* cand_val, int32_t* cand_id,
                               int32_t* rr_id, float* rr_val, int32_t* out_id, float* out_val, float* coarse_out,
                               void* stream, void* coarse_start_event, void* coarse_stop_event) {
  const RowSrc src{w, ldw, nullptr, nullptr, 0, nullptr, kRowsBf16};
  // Validated as draft_head_forward with a workspace of the scratch's size,
  // before any HIP call: a call that needs more is rejected here.
  if (M >= 1 && M <= DH_MAX_M && check_k(K) == DH_OK && coarse_workspace_bytes(M, K) > kScratchBytes)
    return dh::fail(DH_EUNSUP,
                    "forward_noalloc: M=%d, K=%d needs %zu bytes of scratch; the static scratch holds %zu",
                    M, K, coarse_workspace_bytes(M, K), kScratchBytes);
  int rc = validate_forward(x, M, K, N, tiled, pairs, src, kcand, R, cand_val, cand_id, rr_id, rr_val, out_id,
                            out_val, reinterpret_cast<const void*>(uintptr_t{256}), kScratchBytes, false);
  if (rc) return rc;
  const hipStream_t s = as_stream(stream);
  void* ws = nullptr;
  if ((rc = scratch_for(s, &ws))) return rc;
  return launch_forward(x, M, K, N, tiled, pairs, src, kcand, R, cand_val, cand_id, rr_id, rr_val, out_id, out_val,
                        coarse_out, ws, s, coarse_start_event, coarse_stop_event, false);
}

int draft_head_forward_nvfp4(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                             const uint8_t* w4, int64_t ldw, const uint8_t* bscale, int64_t lds, const float* gscale,
                             int kcand, int R, float* cand_val, int32_t* cand_id, int32_t* rr_id, float* rr_val,
                             int32_t* out_id, float* out_val, float* coarse_out, void* workspace,
                             size_t workspace_bytes, void* stream, void* coarse_start_event,
                             void* coarse_stop_event) {
  return forward_impl(x, M, K, N, tiled, pairs, RowSrc{w4, ldw, nullptr, bscale, lds, gscale, kRowsNvfp4}, kcand, R,
                      cand_val, cand_id, rr_id, rr_val, out_id, out_val, coarse_out, workspace, workspace_bytes,
                      stream, coarse_start_event, coarse_stop_event);
}

}  // extern "C"
