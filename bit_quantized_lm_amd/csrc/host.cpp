// Host side of the draft-head library: error state, buffer sizes, the int2
// quantiser with quarter-split packing, and the device-layout tiler.
//
// Built with -ffp-contract=off: the quantiser must round every float32
// operation on its own, as the separate torch element-wise operations of
// `_quantize_head_now` on the radiance_drafthead.py page do.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/drafthead.h"
#include "common.h"

namespace dh {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DH_OK;
}

}  // namespace dh

namespace {

inline float bf16_to_f32(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// float32 -> bf16, round to nearest, ties to even; NaN -> quiet NaN.
inline uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(r >> 16);
}

// A 4-bit head of length K runs as a 2-bit head of length 2K.
int check_shape4(int64_t N, int64_t K) {
  if (N < 1) return dh::fail(DH_ESHAPE, "N must be >= 1 (got %lld)", (long long)N);
  if (K < 256 || K % 256 != 0 || 2 * K > DH_MAX_K)
    return dh::fail(DH_ESHAPE, "K must be a positive multiple of 256 up to %d for a 4-bit head (got %lld)",
                    DH_MAX_K / 2, (long long)K);
  return DH_OK;
}

int check_shape(int64_t N, int64_t K) {
  if (N < 1) return dh::fail(DH_ESHAPE, "N must be >= 1 (got %lld)", (long long)N);
  if (K < 512 || K % 512 != 0 || K > DH_MAX_K)
    return dh::fail(DH_ESHAPE, "K must be a positive multiple of 512 up to %d (got %lld)",
                    DH_MAX_K, (long long)K);
  return DH_OK;
}

// The many-row kernels take each group's zero-point term as the one bf16
// weight S - ZS against the group's x sum, and the fp16 one forms each weight
// (S/4) v as an fp16 value, exact for |S| <= 255.  The page's quantiser meets
// both: S = bf16(4 (hi - lo) / 3) (under 255 for a group range under about
// 191) and ZS = bf16((4 + z) (hi - lo) / 3), z in 0..3, within a factor 1.75
// of S, so that S - ZS has at most 8 significant bits.  (The 4-bit head's
// pairs, scaled by 16 instead of 4, meet the same bounds at a quarter of the
// range.)  NG: groups per row, for the message.
int check_pairs(const uint16_t* S, const uint16_t* ZS, int64_t count, int64_t NG) {
  for (int64_t i = 0; i < count; ++i) {
    const float s = bf16_to_f32(S[i]), zs = bf16_to_f32(ZS[i]);
    if (!(s >= -255.0f && s <= 255.0f))
      return dh::fail(DH_EUNSUP, "tile: scale S[%lld][%lld] = %g is outside [-255, 255], the range the device "
                      "kernels represent exactly", (long long)(i / NG), (long long)(i % NG), (double)s);
    const float d = s - zs;
    uint32_t db;
    std::memcpy(&db, &d, 4);
    if (!std::isfinite(zs) || (double)d != (double)s - (double)zs || (db & 0xFFFFu) != 0u)
      return dh::fail(DH_EUNSUP, "tile: S - ZS at [%lld][%lld] (%g - %g) is not a bf16 value, the form the device "
                      "kernels take the zero-point term in", (long long)(i / NG), (long long)(i % NG), (double)s,
                      (double)zs);
  }
  return DH_OK;
}


template <class F>
void parallel_rows(int64_t N, int nthreads, F&& body) {
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = nthreads > 0 ? nthreads : (hw ? hw : 1);
  if (nt > N) nt = N;
  if (nt <= 1) {
    body(0, N);
    return;
  }
  std::vector<std::thread> pool;
  int64_t per = (N + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    int64_t a = t * per, b = std::min<int64_t>(N, a + per);
    if (a >= b) break;
    pool.emplace_back([&body, a, b] { body(a, b); });
  }
  for (auto& th : pool) th.join();
}

// The quantiser's arithmetic, one float32 operation at a time (this file is
// built without contraction, so no multiply-add is fused): that order is what
// makes the stored bytes equal, bit for bit, to what the page's quantiser
// (float32 tensor operations, round half to even) writes.
struct Grid {
  float step, zero;   // the group's grid: level i sits at (i - zero) * step
};

// An asymmetric grid of levels + 1 points over [lo, hi]: the step (at least
// the floor that keeps a constant group finite) and the level nearest zero.
Grid group_grid(float lo, float hi, float levels) {
  float step = (hi - lo) / levels;
  if (step < 1e-8f) step = 1e-8f;
  float zero = std::nearbyint(-lo / step);   // the default rounding mode: to nearest, ties to even
  zero = std::min(std::max(zero, 0.0f), levels);
  return {step, zero};
}

// A weight's code: its position on the grid, rounded to the nearest level.
uint8_t grid_code(float w, const Grid& g, float levels) {
  float pos = w / g.step;
  pos = pos + g.zero;
  return static_cast<uint8_t>(std::min(std::max(std::nearbyint(pos), 0.0f), levels));
}

// One row of K weights: its codes (K bytes) and its groups' stored pairs,
// S = bf16(premul step) and ZS = bf16(premul step + zero step): the decode's
// bias 1 + v/premul folded in (premul = 4 at two bits, 16 at four).
void quantize_row(const uint16_t* w, int64_t K, uint8_t* codes, uint16_t* S, uint16_t* ZS, float levels = 3.0f,
                  float premul = 4.0f) {
  for (int64_t g = 0; g < K / DH_GROUP; ++g) {
    const uint16_t* wg = w + g * DH_GROUP;
    float lo = bf16_to_f32(wg[0]), hi = lo;
    for (int i = 1; i < DH_GROUP; ++i) {
      const float v = bf16_to_f32(wg[i]);
      lo = std::min(lo, v);
      hi = std::max(hi, v);
    }
    const Grid grid = group_grid(lo, hi, levels);
    for (int i = 0; i < DH_GROUP; ++i) codes[g * DH_GROUP + i] = grid_code(bf16_to_f32(wg[i]), grid, levels);
    const float s_f32 = premul * grid.step;
    const float zs_f32 = s_f32 + grid.zero * grid.step;
    S[g] = f32_to_bf16(s_f32);
    ZS[g] = f32_to_bf16(zs_f32);
  }
}

}  // namespace

extern "C" {

const char* draft_head_last_error(void) { return dh::g_last_error.c_str(); }

int draft_head_sizes(int64_t N, int64_t K, size_t* packed_bytes, size_t* scale_elems,
                     size_t* tiled_bytes, size_t* tiled_pairs) {
  int rc = check_shape(N, K);
  if (rc) return rc;
  int64_t nblk = (N + DH_BLOCK_N - 1) / DH_BLOCK_N;
  if (packed_bytes) *packed_bytes = static_cast<size_t>(N) * (K / 4);
  if (scale_elems) *scale_elems = static_cast<size_t>(N) * (K / DH_GROUP);
  if (tiled_bytes) *tiled_bytes = static_cast<size_t>(nblk) * DH_BLOCK_N * (K / 4);
  if (tiled_pairs) *tiled_pairs = static_cast<size_t>(nblk) * DH_BLOCK_N * (K / DH_GROUP);
  return dh::ok();
}

int draft_head_quantize_pack(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                             uint8_t* packed, uint16_t* S, uint16_t* ZS, int nthreads) {
  if (!w || !packed || !S || !ZS) return dh::fail(DH_EINVAL, "quantize_pack: null pointer");
  int rc = check_shape(N, K);
  if (rc) return rc;
  if (ldw < K) return dh::fail(DH_EINVAL, "quantize_pack: ldw (%lld) < K (%lld)", (long long)ldw, (long long)K);
  if (nthreads < 0) return dh::fail(DH_EINVAL, "quantize_pack: nthreads < 0");
  const int64_t Q = K / 4;
  parallel_rows(N, nthreads, [&](int64_t a, int64_t b) {
    std::vector<uint8_t> codes(K);
    for (int64_t n = a; n < b; ++n) {
      quantize_row(w + n * ldw, K, codes.data(), S + n * (K / DH_GROUP), ZS + n * (K / DH_GROUP));
      uint8_t* out = packed + n * Q;
      for (int64_t j = 0; j < Q; ++j)
        out[j] = static_cast<uint8_t>(codes[j] | (codes[Q + j] << 2) | (codes[2 * Q + j] << 4) |
                                      (codes[3 * Q + j] << 6));
    }
  });
  return dh::ok();
}

int draft_head_quantize_pack_int4(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed4,
                                  uint16_t* S, uint16_t* ZS, int nthreads) {
  if (!w || !packed4 || !S || !ZS) return dh::fail(DH_EINVAL, "quantize_pack_int4: null pointer");
  int rc = check_shape4(N, K);
  if (rc) return rc;
  if (ldw < K)
    return dh::fail(DH_EINVAL, "quantize_pack_int4: ldw (%lld) < K (%lld)", (long long)ldw, (long long)K);
  if (nthreads < 0) return dh::fail(DH_EINVAL, "quantize_pack_int4: nthreads < 0");
  const int64_t H = K / 2;
  parallel_rows(N, nthreads, [&](int64_t a, int64_t b) {
    std::vector<uint8_t> codes(K);
    for (int64_t n = a; n < b; ++n) {
      quantize_row(w + n * ldw, K, codes.data(), S + n * (K / DH_GROUP), ZS + n * (K / DH_GROUP), 15.0f, 16.0f);
      uint8_t* out = packed4 + n * H;
      for (int64_t j = 0; j < H; ++j) out[j] = static_cast<uint8_t>(codes[j] | (codes[H + j] << 4));
    }
  });
  return dh::ok();
}

int draft_head_int4_as_int2(const uint8_t* packed4, const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K,
                            uint8_t* packed2, uint16_t* S2, uint16_t* ZS2) {
  if (!packed4 || !S || !ZS || !packed2 || !S2 || !ZS2) return dh::fail(DH_EINVAL, "int4_as_int2: null pointer");
  int rc = check_shape4(N, K);
  if (rc) return rc;
  const int64_t H = K / 2, NG = K / DH_GROUP;
  parallel_rows(N, 0, [&](int64_t a, int64_t b) {
    for (int64_t n = a; n < b; ++n) {
      // byte j of the 2K-long quarter-split row carries k' = j, K/2+j (high
      // halves of codes j, K/2+j) and K+j, 3K/2+j (their low halves)
      for (int64_t j = 0; j < H; ++j) {
        const uint32_t b4 = packed4[n * H + j], lo = b4 & 15u, hi = b4 >> 4;
        packed2[n * H + j] = static_cast<uint8_t>((lo >> 2) | ((hi >> 2) << 2) | ((lo & 3u) << 4) | ((hi & 3u) << 6));
      }
      for (int64_t g = 0; g < NG; ++g) {
        const uint16_t s = S[n * NG + g];
        const uint16_t s4 = f32_to_bf16(bf16_to_f32(s) * 0.25f);   // exact: a power-of-two scaling
        S2[n * 2 * NG + g] = s;
        ZS2[n * 2 * NG + g] = ZS[n * NG + g];
        S2[n * 2 * NG + NG + g] = s4;
        ZS2[n * 2 * NG + NG + g] = s4;
      }
    }
  });
  return dh::ok();
}

int draft_head_tile(const uint8_t* packed, const uint16_t* S, const uint16_t* ZS, int64_t N,
                    int64_t K, uint8_t* tiled, uint32_t* pairs) {
  if (!packed || !S || !ZS || !tiled || !pairs) return dh::fail(DH_EINVAL, "tile: null pointer");
  int rc = check_shape(N, K);
  if (rc) return rc;
  const int64_t Q = K / 4, NG4 = K / 512, NG = K / DH_GROUP;
  rc = check_pairs(S, ZS, N * NG, NG);
  if (rc) return rc;
  const int64_t nblk = (N + DH_BLOCK_N - 1) / DH_BLOCK_N;
  parallel_rows(nblk, 0, [&](int64_t a, int64_t bend) {
    for (int64_t b = a; b < bend; ++b) {
      for (int64_t col = 0; col < DH_BLOCK_N; ++col) {
        const int64_t n = b * DH_BLOCK_N + col;
        const bool valid = n < N;
        const int64_t t = col / 16, c = col % 16;
        for (int64_t j = 0; j < Q; ++j) {
          const int64_t G = j / 128, h = (j % 128) / 64, s = (j % 64) / 16, wb = j % 16;
          const int64_t off = ((((b * NG4 + G) * 2 + h) * 4 + t) * 64 + s * 16 + c) * 16 + wb;
          tiled[off] = valid ? packed[n * Q + j] : 0;
        }
        for (int64_t g = 0; g < NG; ++g) {
          const int64_t q = g / NG4, G = g % NG4;
          const int64_t off = ((b * NG4 + G) * 4 + t) * 64 + c * 4 + q;
          pairs[off] = valid ? (static_cast<uint32_t>(S[n * NG + g]) |
                                (static_cast<uint32_t>(ZS[n * NG + g]) << 16))
                             : 0u;
        }
      }
    }
  });
  return dh::ok();
}

int draft_head_tile_int4(const uint8_t* packed4, const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K,
                         uint8_t* tiled, uint32_t* pairs) {
  if (!packed4 || !S || !ZS || !tiled || !pairs) return dh::fail(DH_EINVAL, "tile_int4: null pointer");
  int rc = check_shape4(N, K);
  if (rc) return rc;
  const int64_t H = K / 2, NG = K / DH_GROUP, NG4 = K / 256;   // NG4: byte groups of 128 bytes a row
  rc = check_pairs(S, ZS, N * NG, NG);
  if (rc) return rc;
  const int64_t nblk = (N + DH_BLOCK_N - 1) / DH_BLOCK_N;
  parallel_rows(nblk, 0, [&](int64_t a, int64_t bend) {
    for (int64_t b = a; b < bend; ++b) {
      for (int64_t col = 0; col < DH_BLOCK_N; ++col) {
        const int64_t n = b * DH_BLOCK_N + col;
        const bool valid = n < N;
        const int64_t t = col / 16, c = col % 16;
        // the head's own bytes, placed as draft_head_tile places a 2-bit head
        // of length 2K (the same byte count)
        for (int64_t j = 0; j < H; ++j) {
          const int64_t G = j / 128, h = (j % 128) / 64, s = (j % 64) / 16, wb = j % 16;
          tiled[((((b * NG4 + G) * 2 + h) * 4 + t) * 64 + s * 16 + c) * 16 + wb] = valid ? packed4[n * H + j] : 0;
        }
        // pairs of quarters 0 and 1 of each byte group: nibble q's groups
        for (int64_t g = 0; g < NG; ++g) {
          const int64_t q = g / NG4, G = g % NG4;
          pairs[((b * NG4 + G) * 4 + t) * 32 + c * 2 + q] =
              valid ? (static_cast<uint32_t>(S[n * NG + g]) | (static_cast<uint32_t>(ZS[n * NG + g]) << 16)) : 0u;
        }
      }
    }
  });
  return dh::ok();
}

}  // extern "C"
