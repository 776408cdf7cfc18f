"""Quantiser, packing and the effective weight (oracle).

Follows the quantiser `_quantize_head_now` on the radiance_drafthead.py page
(asymmetric min/max at 2 bits, group 128 along K, quarter-split packing,
premultiplied bf16 scale pair) and the module docstring's description of the
packing ("Quarter-split packing") and of the collapse of the 1.0 bias
("Bit-pattern dequant, hoisted").

Arithmetic precision: the page runs the quantiser as separate torch float32
element-wise operations, so every operation here is a separate float32
operation (numpy evaluates each one on its own and rounds it; there is no
fused multiply-add).  Reading: `torch.round` rounds half to even, and numpy's
`np.round` does the same.
"""
import numpy as np

from . import bf16

GROUP = 128          # quantisation group along K (module constant GROUP)
BITS = 2
LEVELS = (1 << BITS) - 1   # highest code, 3
PREMUL = 4.0         # bf16 1 + v/4 bias: the stored scales are premultiplied by 4
CHUNK_ROWS = 8192


def quantize(w_bits):
    """Per (row n, group g of 128 consecutive k): min/max asymmetric int2.

    Steps, as in `_quantize_head_now` (row chunk loop body):
      lo, hi = min and max of the group (float32)
      sc = max((hi - lo) / 3, 1e-8)
      zp = clamp(round(-lo / sc), 0, 3)
      q  = clamp(round(w / sc + zp), 0, 3)
      S  = bf16(4 * sc)
      ZS = bf16(4 * sc + zp * sc)
    Returns (codes uint8 [N][K], S bits uint16 [N][K/128], ZS bits uint16 [N][K/128]).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    n, k = w_bits.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of the group size 128")
    codes = np.empty((n, k), dtype=np.uint8)
    S = np.empty((n, k // GROUP), dtype=np.uint16)
    ZS = np.empty((n, k // GROUP), dtype=np.uint16)
    for i in range(0, n, CHUNK_ROWS):       # row chunks bound memory only
        j = min(i + CHUNK_ROWS, n)
        codes[i:j], S[i:j], ZS[i:j] = _quantize_rows(w_bits[i:j])
    return codes, S, ZS


def _quantize_rows(w_bits, levels=LEVELS, premul=PREMUL):
    n, k = w_bits.shape
    wf = bf16.to_f32(w_bits).reshape(n, k // GROUP, GROUP)
    lo = wf.min(axis=2)
    hi = wf.max(axis=2)
    sc = (hi - lo) / np.float32(levels)
    sc = np.maximum(sc, np.float32(1e-8))
    zp = np.clip(np.round(-lo / sc), np.float32(0), np.float32(levels))
    t = wf / sc[:, :, None]
    t = t + zp[:, :, None]
    q = np.clip(np.round(t), np.float32(0), np.float32(levels)).astype(np.uint8)
    s4 = np.float32(premul) * sc
    zpsc = zp * sc
    S = bf16.from_f32(s4)
    ZS = bf16.from_f32(s4 + zpsc)
    return q.reshape(n, k), S, ZS


# ------------------------------------------------------------------ 4 bits
LEVELS4 = 15         # highest 4-bit code
PREMUL4 = 16.0       # bf16 1 + v/16 bias: the 4-bit scales are premultiplied by 16


def quantize_int4(w_bits):
    """The page's quantiser at BITS = 4 (`_quantize_head_now` with lv = 15 and
    the bias 16): per (row n, group g of 128 consecutive k)
      sc = max((hi - lo) / 15, 1e-8);  zp = clamp(round(-lo / sc), 0, 15)
      q  = clamp(round(w / sc + zp), 0, 15)
      S  = bf16(16 * sc);  ZS = bf16(16 * sc + zp * sc)
    each a separate float32 operation.  Returns (codes, S bits, ZS bits).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    n, k = w_bits.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of the group size 128")
    codes = np.empty((n, k), dtype=np.uint8)
    S = np.empty((n, k // GROUP), dtype=np.uint16)
    ZS = np.empty((n, k // GROUP), dtype=np.uint16)
    for i in range(0, n, CHUNK_ROWS):
        j = min(i + CHUNK_ROWS, n)
        codes[i:j], S[i:j], ZS[i:j] = _quantize_rows(w_bits[i:j], LEVELS4, PREMUL4)
    return codes, S, ZS


def pack_half_split(codes):
    """Byte j of a row carries k = j (bits 0-3) and K/2 + j (bits 4-7): the
    BITS == 4 branch of the packing in `_quantize_head_now`.  uint8 [N][K/2]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    if k % 2:
        raise ValueError("K must be even")
    h = k // 2
    return ((codes[:, :h] & np.uint8(15)) | ((codes[:, h:] & np.uint8(15)) << np.uint8(4))).astype(np.uint8)


def unpack_half_split(packed):
    """Inverse of pack_half_split: codes uint8 [N][K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    return np.concatenate([packed & np.uint8(15), packed >> np.uint8(4)], axis=1)


def quantize_pack_int4(w_bits):
    """(packed uint8 [N][K/2], S bits, ZS bits), the stored form of a 4-bit head."""
    codes, S, ZS = quantize_int4(w_bits)
    return pack_half_split(codes), S, ZS


def effective_weight_int4(packed, S_bits, ZS_bits, rows=None):
    """The weight a 4-bit head's stored arrays define, float64 [n][K]: the
    kernel forms S * sum x (1 + v/16) - ZS * sum x per group (the comment on
    the premultiplier in `_quantize_head_now`), i.e. (S/16) v - (ZS - S)."""
    if rows is not None:
        packed = packed[rows]
        S_bits = S_bits[rows]
        ZS_bits = ZS_bits[rows]
    codes = unpack_half_split(packed).astype(np.float64)
    s = bf16.to_f64(S_bits)
    zs = bf16.to_f64(ZS_bits)
    return codes * np.repeat(s / 16.0, GROUP, axis=1) - np.repeat(zs - s, GROUP, axis=1)


def pack_quarter_split(codes):
    """Byte j of a row carries k = j, K/4+j, K/2+j, 3K/4+j at bits 0-1, 2-3, 4-5, 6-7.

    Module docstring, "Quarter-split packing", and the BITS == 2 branch of the
    packing in `_quantize_head_now`.  Returns uint8 [N][K/4].
    """
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    if k % 4:
        raise ValueError("K must be a multiple of 4")
    q4 = k // 4
    out = np.zeros((n, q4), dtype=np.uint8)
    for quarter in range(4):
        out |= (codes[:, quarter * q4:(quarter + 1) * q4] & np.uint8(3)) << np.uint8(2 * quarter)
    return out


def unpack_quarter_split(packed):
    """Inverse of pack_quarter_split: codes uint8 [N][K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, q4 = packed.shape
    out = np.empty((n, 4 * q4), dtype=np.uint8)
    for quarter in range(4):
        out[:, quarter * q4:(quarter + 1) * q4] = (packed >> np.uint8(2 * quarter)) & np.uint8(3)
    return out


def quantize_pack(w_bits):
    """(packed uint8 [N][K/4], S bits, ZS bits), the stored form of the head."""
    codes, S, ZS = quantize(w_bits)
    return pack_quarter_split(codes), S, ZS


def effective_weight(packed, S_bits, ZS_bits, rows=None):
    """The weight the stored arrays define, float64 [n][K].

    The kernel on the page computes, per group, S * sum_k x_k (1 + v_k/4) minus
    ZS * sum_k x_k (module docstring, "Bit-pattern dequant, hoisted"), which is
    sum_k x_k * ((S/4) v_k - (ZS - S)).  So the effective weight of code v is
    (S/4) v - (ZS - S).  Reading: the stored bf16 pair, not the float32 sc/zp
    of the quantiser, defines the weight.  Every value here is exact in float64.
    `rows` optionally selects a slice of rows.
    """
    if rows is not None:
        packed = packed[rows]
        S_bits = S_bits[rows]
        ZS_bits = ZS_bits[rows]
    codes = unpack_quarter_split(packed).astype(np.float64)
    n, k = codes.shape
    s = bf16.to_f64(S_bits)
    zs = bf16.to_f64(ZS_bits)
    step = np.repeat(s / 4.0, GROUP, axis=1)
    offset = np.repeat(zs - s, GROUP, axis=1)
    return codes * step - offset
