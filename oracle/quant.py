"""Quantiser, packing and the effective weight (oracle).

What the radiance_drafthead.py page quantises (its load-time quantiser and
the module docstring's "Quarter-split packing" and "Bit-pattern dequant,
hoisted" paragraphs): every group of 128 consecutive k of a head row gets an
asymmetric grid of 2^BITS levels spanning the group's range; each weight
becomes the index of its nearest grid level; the grid is stored as one bf16
pair premultiplied by the decode's bias (S = 4 step, ZS = S + zero * step at
two bits), and the codes are packed four to a byte in quarter-split order.

Precision: the page computes the grid and the codes with separate float32
tensor operations, so this oracle does the same, one float32 operation at a
time (numpy rounds each on its own; no fused multiply-add), and rounds half
to even where the page rounds (torch's rounding; the hand-derived worked
example in the tests tells the two rules apart).  Only that operation order
is kept from the page: it is what makes the stored bytes reproducible bit
for bit.
"""
import numpy as np

from . import bf16

GROUP = 128          # quantisation group along K
BITS = 2
LEVELS = (1 << BITS) - 1   # highest code, 3
PREMUL = 4.0         # the decode's bias 1 + v/4: the stored pair carries 4 x the grid step
STEP_FLOOR = 1e-8    # smallest grid step (a constant group)
GROUPS_PER_PASS = 1 << 17   # groups quantised per numpy pass (bounds the temporaries only)


def _grid(lo, hi, levels):
    """The group's grid in float32: step = max((hi - lo) / levels, floor) and
    the zero level, -lo / step rounded to nearest even and clamped to the
    codes."""
    step = np.maximum((hi - lo) / np.float32(levels), np.float32(STEP_FLOOR))
    zero = np.clip(np.round(-lo / step), np.float32(0), np.float32(levels))
    return step, zero


def _encode(w, step, zero, levels):
    """Codes of the weights w [groups][128] on their grids: w / step + zero,
    rounded to nearest even, clamped (two float32 operations, then the round)."""
    pos = w / step[:, None]
    pos = pos + zero[:, None]
    return np.clip(np.round(pos), np.float32(0), np.float32(levels)).astype(np.uint8)


def _stored_pair(step, zero, premul):
    """The pair the head stores: S = bf16(premul * step), ZS = bf16(S' +
    zero * step) with S' the float32 premul * step."""
    s_f32 = np.float32(premul) * step
    return bf16.from_f32(s_f32), bf16.from_f32(s_f32 + zero * step)


def _quantize_groups(w_bits, levels, premul):
    """Codes [N][K] and pairs [N][K/128] of a head, all groups at once."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    n, k = w_bits.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of the group size 128")
    flat = w_bits.reshape(-1, GROUP)          # one group per row, in (n, g) order
    codes = np.empty(flat.shape, dtype=np.uint8)
    S = np.empty(flat.shape[0], dtype=np.uint16)
    ZS = np.empty(flat.shape[0], dtype=np.uint16)
    for a in range(0, flat.shape[0], GROUPS_PER_PASS):
        b = min(a + GROUPS_PER_PASS, flat.shape[0])
        w = bf16.to_f32(flat[a:b])
        step, zero = _grid(w.min(axis=1), w.max(axis=1), levels)
        codes[a:b] = _encode(w, step, zero, levels)
        S[a:b], ZS[a:b] = _stored_pair(step, zero, premul)
    return codes.reshape(n, k), S.reshape(n, k // GROUP), ZS.reshape(n, k // GROUP)


def quantize(w_bits):
    """The 2-bit head: codes uint8 [N][K] (0..3), S and ZS bf16 bits
    uint16 [N][K/128]; the weight of code v is (S/4) v - (ZS - S)."""
    return _quantize_groups(w_bits, LEVELS, PREMUL)


# ------------------------------------------------------------------ 4 bits
LEVELS4 = 15         # highest 4-bit code
PREMUL4 = 16.0       # bf16 1 + v/16 bias: the 4-bit scales are premultiplied by 16


def quantize_int4(w_bits):
    """The 4-bit head (the page's BITS = 4 configuration): the same grid with
    16 levels and the stored pair premultiplied by 16 (the bias 1 + v/16), so
    the weight of code v is (S/16) v - (ZS - S).  Returns (codes, S, ZS)."""
    return _quantize_groups(w_bits, LEVELS4, PREMUL4)


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
