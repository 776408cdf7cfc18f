"""The arithmetic the fp16 many-row coarse kernel rests on, checked on the CPU.

The kernel folds each group's scale into the weights: for quarter q of a
packed byte it ORs the fp16 exponent of 1.0 into the 2-bit code at bits
2q..2q+1 of a 16-bit half (the value 1 + v 2^(2q-10)), and one fused
multiply-add d * T - T with T = S 2^(8-2q) gives the weight (S/4) v in fp16.
The x rows are scaled by a power of two per row, 2^f with f = 15 - e for the
row's largest magnitude m 2^e (1/2 <= m < 1), and taken as fp16.  With the
products exact in fp32 the scores are those of the page's decode
(radiance_drafthead.py, `_draft_head_int2`: the bit-pattern 1 + v/4 times
the group scale) up to the order of the fp32 sums.

These tests hold the claims to the mathematics: every intermediate is an
exactly representable fp16 value over the stated ranges, so the one rounding
of the fused multiply-add changes nothing.  Parity with the oracle on the GPU
is tested separately; nothing here calls the library.
"""
import numpy as np


def _bf16_values(lo_exp, hi_exp):
    """Every positive bf16 value with exponent in [lo_exp, hi_exp], as float64."""
    e = np.arange(lo_exp, hi_exp + 1, dtype=np.float64)[:, None]
    m = 1.0 + np.arange(128, dtype=np.float64)[None, :] / 128.0
    return (m * 2.0 ** e).ravel()


def _exact_fp16(v):
    """Whether each float64 value is exactly an fp16 value."""
    return np.float16(v).astype(np.float64) == v


def test_decode_bit_pattern_is_one_plus_scaled_code():
    for q in range(4):
        for v in range(4):
            bits = np.array([0x3C00 | (v << (2 * q))], np.uint16)
            d = bits.view(np.float16).astype(np.float64)[0]
            assert d == 1.0 + v * 2.0 ** (2 * q - 10), (q, v)


def test_scaled_weight_is_exact_over_the_scale_range():
    """For every bf16 S with 2^-15 <= |S| <= 255 (255 = the largest bf16 below
    256), every code and quarter: T is an fp16 value, d T - T equals (S/4) v
    exactly, and (S/4) v is an fp16 value, so the kernel's weight is exact."""
    s = _bf16_values(-15, 7)
    s = s[s <= 255.0]
    assert s.min() == 2.0 ** -15 and s.max() == 255.0
    s = np.concatenate([s, -s])
    for q in range(4):
        t = s * 2.0 ** (8 - 2 * q)
        assert _exact_fp16(t).all() and np.abs(t).max() <= 65504.0, q
        for v in range(4):
            d = 1.0 + v * 2.0 ** (2 * q - 10)
            w = d * t - t          # exact in float64: at most 19 significant bits
            assert np.array_equal(w, s * v / 4.0), (q, v)
            assert _exact_fp16(w).all(), (q, v)


def test_scaled_weight_range_is_tight():
    """Just outside the range the identity fails: S = 256 overflows T at
    q = 0 (2^16 > 65504), and the smallest S below 2^-15 loses a bit of (S/4) v."""
    assert 256.0 * 2.0 ** 8 > 65504.0
    s = (1.0 + 127.0 / 128.0) * 2.0 ** -16
    assert not _exact_fp16(np.array([s * 3 / 4.0]))[0]


def test_row_scaled_x_is_exact_within_the_dynamic_range():
    """x 2^f with f = 15 - e is below 2^15 for every element and an exact fp16
    value for every bf16 element of magnitude at least 2^(e - 32), which holds
    for every element within a factor 2^31 of the row's largest."""
    rng = np.random.default_rng(11)
    for scale in (1e-6, 0.02, 1.0, 8.0, 3e4):
        x = rng.standard_normal(5120) * scale
        x[::97] *= 8.0                                   # outlier channels
        x = np.float32(x).view(np.uint32) & 0xFFFF0000   # truncated to bf16
        x = x.view(np.float32).astype(np.float64)
        mx = np.abs(x).max()
        _, e = np.frexp(mx)
        f = 15 - e
        xs = x * 2.0 ** f
        assert np.abs(xs).max() < 2.0 ** 15
        keep = np.abs(x) >= 2.0 ** (e - 32)
        assert _exact_fp16(xs[keep]).all(), scale
    # the boundary: every bf16 magnitude with exponent e - 32 is exact; one
    # binade lower, the odd mantissas are not
    e = 3
    mant = 1.0 + np.arange(128) / 128.0
    assert _exact_fp16(mant * 2.0 ** (e - 32) * 2.0 ** (15 - e)).all()
    assert not _exact_fp16(mant[1::2] * 2.0 ** (e - 33) * 2.0 ** (15 - e)).any()


def test_products_are_exact_in_fp32():
    """An fp16 x (11 bits) times an fp16 weight (at most 10 bits) has at most
    21 significant bits: exact in fp32, as the page's bf16 products are."""
    rng = np.random.default_rng(3)
    a = np.float16(rng.standard_normal(100000) * 100).astype(np.float64)
    s = rng.choice(_bf16_values(-15, 7), 100000)
    v = rng.integers(0, 4, 100000)
    w = np.float16(s * v / 4.0).astype(np.float64)
    p = a * w
    assert np.array_equal(np.float32(p).astype(np.float64), p)
