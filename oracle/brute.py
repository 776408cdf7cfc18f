"""Exact, loop-by-loop re-statement of the draft head for tiny shapes.

Pure Python: rational arithmetic (fractions.Fraction) wherever the page's
computation is exact, and an explicitly written round-to-nearest-even to
float32 / bf16 wherever the page's quantiser rounds.  It follows the same
passages as the vectorised oracle (the quantiser `_quantize_head_now`, the
packing statement of the module docstring, `_draft_head_int2`, `_emit`, the
row top-R, `_rerank_exact`), but uses the page's own per-group form
S * sum x(1 + v/4) - ZS * sum x for the coarse score, so it checks the
vectorised oracle's effective-weight form against the page's form as well.

Only usable for a few thousand weights; the tests use it to pin the
vectorised oracle.
"""
from fractions import Fraction
import math
import struct

GROUP = 128
BLOCK_N = 64


# ---------------------------------------------------------------- rounding
def round_to_binary(q, mant_bits, emin, emax):
    """Round a rational to the nearest binary float with `mant_bits` fraction
    bits, exponent range [emin, emax], ties to even; returns a Fraction or
    +-inf.  Subnormals are handled with the fixed minimum exponent."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits)
    t = a / ulp
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * r


def f32(q):
    """Exact rational -> float32 value (as a Fraction), RNE."""
    return round_to_binary(Fraction(q), 23, -126, 127)


def bf16(q):
    """Exact rational -> bf16 value (as a Fraction), RNE."""
    return round_to_binary(Fraction(q), 7, -126, 127)


def bf16_bits_value(bits):
    """bf16 bit pattern -> exact Fraction (finite values only)."""
    f = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    return Fraction(f)


def bf16_value_bits(v):
    """Finite bf16 value (Fraction) -> bit pattern."""
    f = float(v)
    return struct.unpack("<I", struct.pack("<f", f))[0] >> 16


def round_half_even(q):
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return Fraction(fl)


# ---------------------------------------------------------------- quantiser
def quantize_row(w_row_bits, levels=3, premul=4):
    """One row: (codes list, S bits list, ZS bits list), each op rounded to f32.
    levels / premul: 3 / 4 for the 2-bit head, 15 / 16 for the 4-bit one."""
    k = len(w_row_bits)
    vals = [bf16_bits_value(b) for b in w_row_bits]
    codes = [0] * k
    s_bits, zs_bits = [], []
    for g in range(k // GROUP):
        grp = vals[g * GROUP:(g + 1) * GROUP]
        lo, hi = min(grp), max(grp)
        sc = f32(f32(hi - lo) / levels)
        if sc < f32(Fraction(1, 10 ** 8)):
            sc = f32(Fraction(1, 10 ** 8))
        zp = round_half_even(f32(-lo / sc))
        zp = min(max(zp, Fraction(0)), Fraction(levels))
        for i, w in enumerate(grp):
            t = f32(f32(w / sc) + zp)
            qv = min(max(round_half_even(t), Fraction(0)), Fraction(levels))
            codes[g * GROUP + i] = int(qv)
        s4 = f32(premul * sc)
        s_bits.append(bf16_value_bits(bf16(s4)))
        zs_bits.append(bf16_value_bits(bf16(f32(s4 + f32(zp * sc)))))
    return codes, s_bits, zs_bits


def pack_row(codes):
    """Byte j holds the codes of k = j, K/4+j, K/2+j, 3K/4+j in bits 0-1 .. 6-7."""
    k = len(codes)
    q4 = k // 4
    return [codes[j] | (codes[q4 + j] << 2) | (codes[2 * q4 + j] << 4) | (codes[3 * q4 + j] << 6)
            for j in range(q4)]


def pack_row_int4(codes):
    """4-bit head: byte j holds the code of k = j in bits 0-3 and of K/2+j in bits 4-7."""
    h = len(codes) // 2
    return [codes[j] | (codes[h + j] << 4) for j in range(h)]


# ---------------------------------------------------------------- per call
def coarse_row_int4(x_vals, packed_row, s_bits, zs_bits):
    """Exact coarse logit of one column of a 4-bit head, in the page's form:
    per group S * sum x (1 + v/16) - ZS * sum x, the 1 + v/16 being what the
    page's 4-bit bit-pattern decode yields and S, ZS its pair premultiplied
    by 16 (`_quantize_head_now`, comment on the premultiplier)."""
    h = len(packed_row)
    k = 2 * h
    total = Fraction(0)
    for g in range(k // GROUP):
        p = Fraction(0)
        xs = Fraction(0)
        for kk in range(g * GROUP, (g + 1) * GROUP):
            half, j = divmod(kk, h)
            v = (packed_row[j] >> (4 * half)) & 15
            p += x_vals[kk] * (1 + Fraction(v, 16))
            xs += x_vals[kk]
        total += bf16_bits_value(s_bits[g]) * p - bf16_bits_value(zs_bits[g]) * xs
    return total


def coarse_row(x_vals, packed_row, s_bits, zs_bits):
    """Exact coarse logit of one column: sum over groups of S * p - ZS * X."""
    q4 = len(packed_row)
    k = 4 * q4
    total = Fraction(0)
    for g in range(k // GROUP):
        p = Fraction(0)
        xs = Fraction(0)
        for kk in range(g * GROUP, (g + 1) * GROUP):
            quarter, j = divmod(kk, q4)
            v = (packed_row[j] >> (2 * quarter)) & 3
            p += x_vals[kk] * (1 + Fraction(v, 4))
            xs += x_vals[kk]
        total += bf16_bits_value(s_bits[g]) * p - bf16_bits_value(zs_bits[g]) * xs
    return total


def run(x_bits, w_bits, kcand, r, bits=2):
    """Whole head, exact.  x_bits [M][K], w_bits [N][K] as nested lists of ints.
    bits = 4: the 4-bit head (15 levels, premultiplier 16, half-split bytes)."""
    m = len(x_bits)
    n = len(w_bits)
    xv = [[bf16_bits_value(b) for b in row] for row in x_bits]
    packed, S, ZS, codes = [], [], [], []
    for row in w_bits:
        if bits == 4:
            c, s, z = quantize_row(row, levels=15, premul=16)
            packed.append(pack_row_int4(c))
        else:
            c, s, z = quantize_row(row)
            packed.append(pack_row(c))
        codes.append(c)
        S.append(s)
        ZS.append(z)
    score = coarse_row_int4 if bits == 4 else coarse_row
    coarse = [[score(xv[i], packed[col], S[col], ZS[col]) for col in range(n)]
              for i in range(m)]
    nblk = (n + BLOCK_N - 1) // BLOCK_N
    cand = []
    for i in range(m):
        row = []
        for b in range(nblk):
            cols = list(range(b * BLOCK_N, min((b + 1) * BLOCK_N, n)))
            cols.sort(key=lambda col: (-coarse[i][col], col))
            for slot in range(kcand):
                if slot < len(cols):
                    row.append((coarse[i][cols[slot]], cols[slot]))
                else:
                    row.append((None, -1))
        cand.append(row)
    rr = []
    for i in range(m):
        valid = [(v, c) for v, c in cand[i] if c >= 0]
        valid.sort(key=lambda vc: (-vc[0], vc[1]))
        ids = [c for _, c in valid[:r]]
        ids += [-1] * (r - len(ids))
        rr.append(ids)
    exact = []
    out = []
    out_val = []
    for i in range(m):
        ev = []
        for c in rr[i]:
            if c < 0:
                ev.append(None)
            else:
                ev.append(sum(xv[i][kk] * bf16_bits_value(w_bits[c][kk]) for kk in range(len(xv[i]))))
        exact.append(ev)
        best = None
        for c, e in zip(rr[i], ev):
            if c < 0:
                continue
            e32 = f32(e)
            if best is None or e32 > best[1] or (e32 == best[1] and c < best[0]):
                best = (c, e32)
        out.append(best[0] if best else -1)
        out_val.append(best[1] if best else None)
    return {"codes": codes, "packed": packed, "S": S, "ZS": ZS, "coarse": coarse,
            "cand": cand, "rr_id": rr, "rr_val": exact, "out_id": out, "out_val": out_val}
