// Device side of the draft-head library: HIP kernels for gfx950 (MI355X) and
// the validating C entry points that launch them.
//
// Per call (radiance_drafthead.py page, `_apply_head_int2`):
//   coarse_kernel   scores x against the 2-bit weight and keeps the top KCAND
//                   columns of every 64-column block (`_draft_head_int2` + `_emit`)
//   select_kernel   row top-R of the candidates (`bm.topk` + `bi.gather`)
//   dot_kernel      exact fp32 dot of x with each candidate's bf16 row (`_rerank_exact`)
//   argmax_kernel   best reranked candidate per row
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/drafthead.h"
#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;            // waves per coarse workgroup; one 64-column block each
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxMT = 5;            // 16-row M tiles per coarse launch (80 rows)

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Decode quarter q of two code dwords into four bf16 pairs of 1 + v/4.
// Code v sits in bits 2q..2q+1 of each byte; moving it to bits 5-6 of a
// halfword and OR-ing 0x3F80 gives the bf16 value 1 + v/4 (the bit-pattern
// dequant of the module docstring).  Even pairs hold bytes 0 and 2 of a dword
// (rotate left by 5 - 2q, which for q = 3 is a rotate right by 1), odd pairs
// bytes 1 and 3 (shift right by 3 + 2q), so the element order of the result
// is byte {0, 2, 1, 3} of d0 then {0, 2, 1, 3} of d1; the x fragments are
// staged in the same order.  Bits rotated around land in bits 0-4 or 31 and
// are masked off.
//
// `one` must hold 0x3F803F80 in a VGPR: gfx9-family VOP3 instructions take no
// literal operand, so with the mask in an SGPR and `one` in a VGPR each pair
// is one shift and one v_and_or_b32.
__device__ __forceinline__ bf16x8 decode_quarter(uint32_t d0, uint32_t d1, uint32_t rot,
                                                 uint32_t shr, uint32_t one) {
  constexpr uint32_t kMask = 0x00600060u;
  const uint32_t e0 = (__builtin_amdgcn_alignbit(d0, d0, rot) & kMask) | one;
  const uint32_t e1 = (__builtin_amdgcn_alignbit(d1, d1, rot) & kMask) | one;
  const uint32_t o0 = ((d0 >> shr) & kMask) | one;
  const uint32_t o1 = ((d1 >> shr) & kMask) | one;
  u32x4 v = {e0, o0, e1, o1};
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Coarse kernel.
//
// Workgroup = 4 waves, wave w owns 64-column block b = 4*blockIdx.x + w and
// computes its M x 64 coarse scores with bf16 MFMA 16x16x32: the A operand is
// x (rows), the B operand is the decoded weight (1 + v/4), one 16-column tile
// per MFMA, four tiles per block.  The K loop walks the 4*NG4 groups in the
// order (byte-group G, quarter q); the 128 x values of each group are staged in
// LDS (double buffered, one barrier per group) in the permuted order the
// decode produces, together with the group sum X = sum_k x in fp32.  After a
// group's four MFMAs per tile the accumulator is updated with the page's
// premultiplied pair: acc += S * p - ZS * X.
//
// LDS layout of one staged group: 16 fragments f = (h*2 + e)*4 + s of 8 bf16
// per row, fragment f of row m at [f*MP + m] (16 bytes), MP = 16*MT rows
// (rows >= M stay zero); then X[MP].  The fixed row count makes every LDS
// offset a compile-time immediate.
template <int MT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MT <= 2 ? 2 : 1, MT <= 2 ? 2 : 1))) void coarse_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, int nblk,
    const u32x4* __restrict__ tiled, const u32x4* __restrict__ pairs, int kcand,
    float* __restrict__ cand_val, int32_t* __restrict__ cand_id, float* __restrict__ coarse_out) {
  constexpr int MP = 16 * MT;
  __shared__ u32x4 xs[2 * 16 * MP];
  __shared__ float Xs[2 * MP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 4, nn = lane & 15;
  const int b = blockIdx.x * kWaves + wave;
  const bool blk_ok = b < nblk;
  const int NG4 = K >> 9, Q4 = K >> 2;
  const int ncand = nblk * kcand;
  // bf16 pair (1.0, 1.0), kept opaque so it stays in a VGPR (see decode_quarter)
  uint32_t one;
  asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(one));

  // Code tiles of this block: [G][h][t][64 lanes] u32x4; pairs: [G][t][16] u32x4.
  // A wave past the last block reads block 0 (valid memory) and writes nothing.
  const u32x4* tp = tiled + (size_t)(blk_ok ? b : 0) * NG4 * 512;
  const u32x4* pp = pairs + (size_t)(blk_ok ? b : 0) * NG4 * 64;

  // zero the staging buffers once: rows M..MP-1 must read as zero
  for (int i = tid; i < 2 * 16 * MP; i += kThreads) xs[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < 2 * MP; i += kThreads) Xs[i] = 0.f;
  __syncthreads();

  f32x4 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_codes = [&](int G, u32x4 (&raw)[2][4], u32x4 (&sz)[4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        raw[h][t] = tp[((G * 2 + h) * 4 + t) * 64 + lane];
#pragma unroll
    for (int t = 0; t < 4; ++t) sz[t] = pp[(G * 4 + t) * 16 + nn];
  };

  // Staging of group (G, q): thread i < 16*M loads natural piece p = i & 15 of row
  // m = i >> 4, i.e. x[m][q*K/4 + 128*G + 8p .. +8].
  constexpr int kMaxStage = (16 * MP + kThreads - 1) / kThreads;
  const int stage_n = 16 * M;
  auto stage_load = [&](int G, int q, u32x4 (&st)[kMaxStage]) {
    const int kbase = q * Q4 + 128 * G;
#pragma unroll
    for (int r = 0; r < kMaxStage; ++r) {
      int i = tid + r * kThreads;
      if (i < stage_n) {
        int m = i >> 4, p = i & 15;
        st[r] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + kbase + 8 * p);
      }
    }
  };
  auto stage_store = [&](int buf, const u32x4 (&st)[kMaxStage]) {
    u32x4* dst = xs + buf * 16 * MP;
#pragma unroll
    for (int r = 0; r < kMaxStage; ++r) {
      int i = tid + r * kThreads;
      if (i < stage_n) {
        int m = i >> 4, p = i & 15;
        u32x4 v = st[r];
        // natural [x0 x1 | x2 x3 | x4 x5 | x6 x7] -> [x0 x2 | x1 x3 | x4 x6 | x5 x7]
        u32x4 o;
        o[0] = (v[0] & 0xFFFFu) | (v[1] << 16);
        o[1] = (v[0] >> 16) | (v[1] & 0xFFFF0000u);
        o[2] = (v[2] & 0xFFFFu) | (v[3] << 16);
        o[3] = (v[2] >> 16) | (v[3] & 0xFFFF0000u);
        int h = p >> 3, s = (p >> 1) & 3, e = p & 1;
        dst[((h * 2 + e) * 4 + s) * MP + m] = o;
        float sum = lo_bf16(v[0]) + hi_bf16(v[0]) + lo_bf16(v[1]) + hi_bf16(v[1]) +
                    lo_bf16(v[2]) + hi_bf16(v[2]) + lo_bf16(v[3]) + hi_bf16(v[3]);
        sum += __shfl_xor(sum, 1, 16);
        sum += __shfl_xor(sum, 2, 16);
        sum += __shfl_xor(sum, 4, 16);
        sum += __shfl_xor(sum, 8, 16);
        if (p == 0) Xs[buf * MP + m] = sum;
      }
    }
  };

  u32x4 raw[2][4], sz[4];
  load_codes(0, raw, sz);
  {
    u32x4 st[kMaxStage];
    stage_load(0, 0, st);
    stage_store(0, st);
  }
  __syncthreads();

  for (int G = 0; G < NG4; ++G) {
    u32x4 rawn[2][4], szn[4];
    if (G + 1 < NG4) load_codes(G + 1, rawn, szn);

#pragma nounroll
    for (int q = 0; q < 4; ++q) {
      const int cur = q & 1;  // 4 groups per G, so the buffer parity is q's
      // prefetch the next group's x into registers
      const bool has_next = (q < 3) || (G + 1 < NG4);
      u32x4 st[kMaxStage];
      if (has_next) stage_load(q < 3 ? G : G + 1, q < 3 ? q + 1 : 0, st);

      // rotate-left amount 5 - 2q (mod 32) for even pairs, shift 3 + 2q for odd ones
      const uint32_t rot = (uint32_t)(32 - (5 - 2 * q)) & 31u;  // alignbit rotates right
      const uint32_t shr = 3u + 2u * (uint32_t)q;

      f32x4 cg[MT][4];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) cg[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

      const u32x4* xb = xs + cur * 16 * MP + hh * MP + nn;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          bf16x8 a[MT];
#pragma unroll
          for (int i = 0; i < MT; ++i)
            a[i] = __builtin_bit_cast(bf16x8, xb[(h * 2 + e) * 4 * MP + 16 * i]);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const bf16x8 bv = decode_quarter(raw[h][t][2 * e], raw[h][t][2 * e + 1], rot, shr, one);
#pragma unroll
            for (int i = 0; i < MT; ++i)
              cg[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bv, cg[i][t], 0, 0, 0);
          }
        }
      }
      // group (G, q) complete: acc += S * p - ZS * X for rows 4*hh + r of each tile
      float X[MT][4];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) X[i][r] = Xs[cur * MP + 16 * i + 4 * hh + r];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t pr = q == 0 ? sz[t][0] : q == 1 ? sz[t][1] : q == 2 ? sz[t][2] : sz[t][3];
        const float S = lo_bf16(pr), ZS = hi_bf16(pr);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] += S * cg[i][t][r] - ZS * X[i][r];
      }
      if (has_next) stage_store(cur ^ 1, st);
      __syncthreads();
    }
    if (G + 1 < NG4) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) raw[h][t] = rawn[h][t];
#pragma unroll
      for (int t = 0; t < 4; ++t) sz[t] = szn[t];
    }
  }

  if (!blk_ok) return;

  // Epilogue: optional full row, then top-kcand of the block by successive
  // max-and-mask (`_emit`).  Lane (hh, nn) holds columns 16t + nn of rows
  // 16i + 4hh + r; the four rows of one (i, r) are handled at once, one per
  // 16-lane row of the wave.
  const float NEG_INF = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (16 * i + r >= M) continue;  // no row of this (i, r) is live (wave-uniform)
      const int m = 16 * i + 4 * hh + r;
      const bool row_ok = m < M;
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = b * 64 + 16 * t + nn;
        const bool ok = row_ok && n < N;
        v[t] = ok ? acc[i][t][r] : NEG_INF;
        if (coarse_out && ok) coarse_out[(size_t)m * N + n] = acc[i][t][r];
      }
      float kv[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
      int ki[4] = {-1, -1, -1, -1};
      for (int c = 0; c < kcand; ++c) {
        float bv = v[0];
        int bn = nn;
#pragma unroll
        for (int t = 1; t < 4; ++t)
          if (v[t] > bv) {
            bv = v[t];
            bn = 16 * t + nn;
          }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          float ov = __shfl_xor(bv, off, 16);
          int on = __shfl_xor(bn, off, 16);
          if (ov > bv || (ov == bv && on < bn)) {
            bv = ov;
            bn = on;
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (bn == 16 * t + nn) v[t] = NEG_INF;
        if ((c & 15) == nn) {
          const int slot = c >> 4;
          const float val = bv;
          const int id = (bv == NEG_INF) ? -1 : b * 64 + bn;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (s == slot) {
              kv[s] = val;
              ki[s] = id;
            }
        }
      }
      if (row_ok) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int c = 16 * s + nn;
          if (c < kcand) {
            const size_t o = (size_t)m * ncand + (size_t)b * kcand + c;
            cand_val[o] = kv[s];
            cand_id[o] = ki[s];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row top-R: one workgroup per row.  Each candidate becomes a 64-bit key
// (ordered float bits << 32 | ~id), so "larger key" is "larger value, then
// lower id" and all keys of valid candidates are distinct; invalid slots
// (id -1, or an id >= N that no coarse call writes) get key 0.  An 8-bit radix select over the 64-bit keys finds the
// R-th largest key, the keys at or above it are gathered and bitonic-sorted.
constexpr int kSelThreads = 1024;

__device__ __forceinline__ unsigned long long cand_key(float v, int id, int N) {
  if (id < 0 || id >= N) return 0ull;
  uint32_t u = __float_as_uint(v);
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)id);
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ cand_val,
                                                             const int32_t* __restrict__ cand_id,
                                                             int ncand, int N, int R,
                                                             int32_t* __restrict__ rr_id) {
  __shared__ unsigned int hist[256];
  __shared__ unsigned long long keys[DH_MAX_R];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_need;
  __shared__ unsigned int s_valid;
  __shared__ unsigned int s_count;

  const int m = blockIdx.x, tid = threadIdx.x;
  const float* cv = cand_val + (size_t)m * ncand;
  const int32_t* ci = cand_id + (size_t)m * ncand;

  if (tid == 0) {
    s_valid = 0;
    s_count = 0;
    s_prefix = 0;
    s_need = R;
  }
  __syncthreads();
  unsigned int local = 0;
  for (int i = tid; i < ncand; i += kSelThreads) local += (ci[i] >= 0 && ci[i] < N) ? 1u : 0u;
  atomicAdd(&s_valid, local);
  __syncthreads();
  const unsigned int nvalid = s_valid;

  unsigned long long thresh = 1ull;  // all valid keys if there are at most R of them
  if (nvalid > (unsigned)R) {
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      const unsigned long long pre = s_prefix;
      for (int i = tid; i < ncand; i += kSelThreads) {
        unsigned long long k = cand_key(cv[i], ci[i], N);
        if (k == 0) continue;
        if (pass > 0 && (k >> (shift + 8)) != pre) continue;
        atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      // exact scan of the 256 bins from the top, by one thread
      if (tid == 0) {
        int need = s_need;
        unsigned int cum = 0;
        int digit = 0;
        for (int d = 255; d >= 0; --d) {
          if (cum + hist[d] >= (unsigned)need) {
            digit = d;
            break;
          }
          cum += hist[d];
        }
        s_need = need - (int)cum;
        s_prefix = (pre << 8) | (unsigned long long)digit;
      }
      __syncthreads();
    }
    thresh = s_prefix;
  }
  for (int i = tid; i < ncand; i += kSelThreads) {
    unsigned long long k = cand_key(cv[i], ci[i], N);
    if (k != 0 && k >= thresh) {
      unsigned int pos = atomicAdd(&s_count, 1u);
      if (pos < (unsigned)DH_MAX_R) keys[pos] = k;
    }
  }
  __syncthreads();
  const int cnt = (int)min(s_count, (unsigned)R);
  int P = 1;
  while (P < cnt) P <<= 1;
  for (int i = cnt + tid; i < P; i += kSelThreads) keys[i] = 0ull;
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kSelThreads) {
        int j = i ^ stride;
        if (j > i) {
          bool desc = (i & size) == 0;
          unsigned long long a = keys[i], c = keys[j];
          if (desc ? (a < c) : (a > c)) {
            keys[i] = c;
            keys[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < R; r += kSelThreads)
    rr_id[(size_t)m * R + r] = (r < cnt) ? (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[r] & 0xFFFFFFFFull)) : -1;
}

// Exact logits: one wave per (row, candidate); fp32 products and sums.
__global__ __launch_bounds__(256) void dot_kernel(const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ w, int64_t ldw,
                                                  int M, int K, int N, int R,
                                                  const int32_t* __restrict__ rr_id,
                                                  float* __restrict__ rr_val) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (gw >= M * R) return;
  const int m = gw / R;
  const int id = rr_id[gw];
  if (id < 0 || id >= N) {
    if (lane == 0) rr_val[gw] = -__builtin_inff();
    return;
  }
  const uint16_t* xr = x + (size_t)m * K;
  const uint16_t* wr = w + (size_t)id * ldw;
  float s0 = 0.f, s1 = 0.f;
  for (int k = lane * 8; k < K; k += 512) {
    u32x4 xv = *reinterpret_cast<const u32x4*>(xr + k);
    u32x4 wv = *reinterpret_cast<const u32x4*>(wr + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s0 += lo_bf16(xv[j]) * lo_bf16(wv[j]);
      s1 += hi_bf16(xv[j]) * hi_bf16(wv[j]);
    }
  }
  float s = s0 + s1;
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) rr_val[gw] = s;
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
    int id = rr_id[(size_t)m * R + r];
    if (id < 0) continue;
    float v = rr_val[(size_t)m * R + r];
    if (bi < 0 || v > bv || (v == bv && id < bi)) {
      bv = v;
      bi = id;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    float ov = __shfl_xor(bv, off, 64);
    int oi = __shfl_xor(bi, off, 64);
    bool take = (oi >= 0) && (bi < 0 || ov > bv || (ov == bv && oi < bi));
    if (take) {
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

template <int MT>
void launch_coarse(const uint16_t* x, int M, int K, int N, int nblk, const u32x4* tiled,
                   const u32x4* pairs, int kcand, float* cv, int32_t* ci, float* co,
                   hipStream_t s) {
  dim3 grid((nblk + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(coarse_kernel<MT>, grid, dim3(kThreads), 0, s, x, M, K, N, nblk, tiled,
                     pairs, kcand, cv, ci, co);
}

}  // namespace

extern "C" {

int draft_head_coarse(const void* x, int M, int K, int N, const uint8_t* tiled, const uint32_t* pairs,
                      int kcand, float* cand_val, int32_t* cand_id, float* coarse_out, void* stream) {
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
  const int nblk = (N + DH_BLOCK_N - 1) / DH_BLOCK_N;
  const int ncand = nblk * kcand;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const u32x4* tp = reinterpret_cast<const u32x4*>(tiled);
  const u32x4* pp = reinterpret_cast<const u32x4*>(pairs);
  // Rows beyond one launch's 80 are handled by further launches over the
  // same weights (only for M > 80).
  for (int m0 = 0; m0 < M; m0 += 16 * kMaxMT) {
    const int mm = std::min(M - m0, 16 * kMaxMT);
    const int mt = (mm + 15) / 16;
    const uint16_t* xm = xb + (size_t)m0 * K;
    float* cv = cand_val + (size_t)m0 * ncand;
    int32_t* ci = cand_id + (size_t)m0 * ncand;
    float* co = coarse_out ? coarse_out + (size_t)m0 * N : nullptr;
    switch (mt) {
      case 1: launch_coarse<1>(xm, mm, K, N, nblk, tp, pp, kcand, cv, ci, co, s); break;
      case 2: launch_coarse<2>(xm, mm, K, N, nblk, tp, pp, kcand, cv, ci, co, s); break;
      case 3: launch_coarse<3>(xm, mm, K, N, nblk, tp, pp, kcand, cv, ci, co, s); break;
      case 4: launch_coarse<4>(xm, mm, K, N, nblk, tp, pp, kcand, cv, ci, co, s); break;
      default: launch_coarse<5>(xm, mm, K, N, nblk, tp, pp, kcand, cv, ci, co, s); break;
    }
    if ((rc = launch_error("coarse_kernel"))) return rc;
  }
  return dh::ok();
}

int draft_head_rerank(const void* x, const void* w, int64_t ldw, int M, int K, int N,
                      const float* cand_val, const int32_t* cand_id, int ncand, int R,
                      int32_t* rr_id, float* rr_val, void* stream) {
  if (!x || !w || !cand_val || !cand_id || !rr_id || !rr_val)
    return dh::fail(DH_EINVAL, "rerank: null pointer");
  int rc = check_m(M);
  if (rc) return rc;
  if ((rc = check_k(K))) return rc;
  if (N < 1) return dh::fail(DH_ESHAPE, "rerank: N must be >= 1 (got %d)", N);
  if (ldw < K || ldw % 8 != 0)
    return dh::fail(DH_EINVAL, "rerank: ldw must be >= K and a multiple of 8 (got %lld)", (long long)ldw);
  if (ncand < 1) return dh::fail(DH_EINVAL, "rerank: ncand must be >= 1 (got %d)", ncand);
  if (R < 1 || R > ncand || R > DH_MAX_R)
    return dh::fail(DH_EUNSUP, "rerank: R must be in 1..min(ncand=%d, %d) (got %d)", ncand, DH_MAX_R, R);
  if (!aligned16(x) || !aligned16(w))
    return dh::fail(DH_EINVAL, "rerank: x and w must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(select_kernel, dim3(M), dim3(kSelThreads), 0, s, cand_val, cand_id, ncand, N, R,
                     rr_id);
  if ((rc = launch_error("select_kernel"))) return rc;
  const int waves = M * R;
  hipLaunchKernelGGL(dot_kernel, dim3((waves + 3) / 4), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), ldw, M, K, N, R,
                     rr_id, rr_val);
  if ((rc = launch_error("dot_kernel"))) return rc;
  return dh::ok();
}

int draft_head_argmax(const int32_t* rr_id, const float* rr_val, int M, int R, int32_t* out_id,
                      float* out_val, void* stream) {
  if (!rr_id || !rr_val || !out_id || !out_val) return dh::fail(DH_EINVAL, "argmax: null pointer");
  int rc = check_m(M);
  if (rc) return rc;
  if (R < 1 || R > DH_MAX_R) return dh::fail(DH_EUNSUP, "argmax: R must be in 1..%d (got %d)", DH_MAX_R, R);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(argmax_kernel, dim3((M + 3) / 4), dim3(256), 0, s, rr_id, rr_val, M, R, out_id, out_val);
  return launch_error("argmax_kernel");
}

}  // extern "C"
