"""Pins of the CPU oracle to what the radiance_drafthead.py page and arithmetic fix.

None of these retype the oracle's own formulas: each compares the oracle with
a page identity, a hand-derived fixture (tests/golden), a closed form, a
special case whose answer is known without the method, a library routine, or
an exact rational brute force (oracle/brute.py, which uses the page's own
per-group form of the coarse score rather than the oracle's effective weight).
"""
from fractions import Fraction
import struct

import numpy as np
import pytest

import oracle
from oracle import bf16 as obf
from oracle import brute
from bit_quantized_lm_amd import workload


def _bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def _hex(s):
    return int(s, 16)


# ------------------------------------------------------------ page identities
def test_bit_pattern_identity_exhaustive(golden):
    """0x3F80 | ((b << (5-2q)) & 0x60), or (b >> 1) & 0x60 for q = 3, reads as
    bf16 1 + v/4 where v is the code the oracle unpacks from quarter q of b."""
    table = golden("bit_pattern_dequant.txt")
    for v in range(4):
        bits, val = table[str(v)][0]
        assert _bf16_value(_hex(bits)) == float(val) == 1.0 + v / 4.0
    k = 512
    q4 = k // 4
    for b in range(256):
        packed = np.full((1, q4), b, dtype=np.uint8)
        codes = oracle.unpack_quarter_split(packed)[0]
        for q in range(4):
            if q < 3:
                bits = 0x3F80 | ((b << (5 - 2 * q)) & 0x60)
            else:
                bits = 0x3F80 | ((b >> 1) & 0x60)
            v = int(codes[q * q4])
            assert _bf16_value(bits) == 1.0 + v / 4.0, (b, q)


def test_collapse_identity_exact():
    """S * sum x(1 + v/4) - ZS * sum x == sum x * w_eff, in exact rationals,
    for the oracle's effective weight and stored pair (module docstring,
    "Bit-pattern dequant, hoisted")."""
    rng = np.random.default_rng(5)
    k = 512
    w = workload.f32_to_bf16_bits(rng.standard_normal((6, k), dtype=np.float32) * 0.03)
    x = workload.f32_to_bf16_bits(rng.standard_normal((2, k), dtype=np.float32))
    packed, S, ZS = oracle.quantize_pack(w)
    w_eff = oracle.effective_weight(packed, S, ZS)
    codes = oracle.unpack_quarter_split(packed)
    for m in range(2):
        xv = [Fraction(float(v)) for v in obf.to_f32(x[m])]
        for n in range(6):
            for g in range(k // 128):
                sl = range(g * 128, (g + 1) * 128)
                lhs = (Fraction(float(obf.to_f32(S[n, g]))) * sum(xv[i] * (1 + Fraction(int(codes[n, i]), 4)) for i in sl)
                       - Fraction(float(obf.to_f32(ZS[n, g]))) * sum(xv[i] for i in sl))
                rhs = sum(xv[i] * Fraction(float(w_eff[n, i])) for i in sl)
                assert lhs == rhs


def test_effective_weight_is_exact_in_float64():
    """(S/4) v - (ZS - S) is representable: recomputing it in Fractions gives the same."""
    w, _ = workload.gen_weight(64, 512, seed=9), None
    packed, S, ZS = oracle.quantize_pack(w)
    w_eff = oracle.effective_weight(packed, S, ZS)
    codes = oracle.unpack_quarter_split(packed)
    for n in range(0, 64, 7):
        for kk in range(0, 512, 37):
            g = kk // 128
            s = Fraction(float(obf.to_f32(S[n, g])))
            zs = Fraction(float(obf.to_f32(ZS[n, g])))
            assert Fraction(float(w_eff[n, kk])) == s / 4 * int(codes[n, kk]) - (zs - s)


# ------------------------------------------------------------ layout
def test_quarter_split_layout_fixture(golden):
    fx = golden("quarter_split_example.txt")
    k = 512
    codes = np.zeros((1, k), dtype=np.uint8)
    for kk in fx["A_nonzero_k"][0]:
        codes[0, int(kk)] = 3
    packed = oracle.pack_quarter_split(codes)[0]
    assert [int(v) for v in packed[:4]] == [_hex(s) for s in fx["A_bytes_0_to_3"][0]]
    assert np.all(packed[4:] == _hex(fx["A_other_bytes"][0][0]))
    codes_b = (np.arange(k) // 128).astype(np.uint8)[None, :]
    assert np.all(oracle.pack_quarter_split(codes_b) == _hex(fx["B_every_byte"][0][0]))


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 4, size=(5, 1024), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_quarter_split(oracle.pack_quarter_split(codes)), codes)


# ------------------------------------------------------------ quantiser
def test_quantizer_worked_example(golden):
    fx = golden("quantizer_worked_example.txt")
    k = int(fx["K"][0][0])
    w = np.zeros((1, k), dtype=np.uint16)
    w[0, :4] = [_hex(s) for s in fx["w_bits_k0_to_3"][0]]
    codes, S, ZS = oracle.quantize(w)
    assert [int(c) for c in codes[0, :4]] == [int(s) for s in fx["codes_k0_to_3"][0]]
    assert np.all(codes[0, 4:128] == int(fx["code_rest_of_group0"][0][0]))
    assert np.all(codes[0, 128:] == int(fx["code_zero_groups"][0][0]))
    assert int(S[0, 0]) == _hex(fx["S_group0"][0][0])
    assert int(ZS[0, 0]) == _hex(fx["ZS_group0"][0][0])
    w_eff = oracle.effective_weight(oracle.pack_quarter_split(codes), S, ZS)[0]
    want = {int(a): float(b) for a, b in fx["w_eff_for_code"]}
    for kk in range(128):
        assert w_eff[kk] == want[int(codes[0, kk])]
    # all-zero groups decode to exactly zero
    assert np.all(w_eff[128:] == 0.0)


def test_quantizer_matches_exact_brute_force():
    """numpy float32 quantiser == rational re-statement with explicit f32 rounding."""
    rng = np.random.default_rng(17)
    rows = [
        rng.standard_normal(512, dtype=np.float32) * 0.02,
        rng.standard_normal(512, dtype=np.float32) * 3.0,
        np.full(512, 0.7, dtype=np.float32),                      # constant group
        np.zeros(512, dtype=np.float32),                          # zero group
        np.where(rng.random(512) < 0.5, -1.0, 1.0).astype(np.float32) * 1e-3,
        rng.standard_normal(512, dtype=np.float32) * 1e-9,        # below the 1e-8 clamp
        np.abs(rng.standard_normal(512, dtype=np.float32)),       # all positive: zp clamps
        -np.abs(rng.standard_normal(512, dtype=np.float32)),      # all negative
    ]
    w = workload.f32_to_bf16_bits(np.stack(rows))
    codes, S, ZS = oracle.quantize(w)
    for i in range(w.shape[0]):
        bc, bs, bz = brute.quantize_row([int(v) for v in w[i]])
        assert [int(c) for c in codes[i]] == bc, i
        assert [int(v) for v in S[i]] == bs, i
        assert [int(v) for v in ZS[i]] == bz, i


def test_clamp_constant_matches_exact_rounding():
    assert Fraction(float(np.float32(1e-8))) == brute.f32(Fraction(1, 10 ** 8))


def test_bf16_rounding_matches_exact_rounding():
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                           np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float32)])
    bits = obf.from_f32(vals)
    for v, b in zip(vals, bits):
        assert brute.bf16_value_bits(brute.bf16(Fraction(float(v)))) == int(b)


# ------------------------------------------------------------ special cases
def _lossless_weight(n, k, rng):
    """W built from codes with power-of-two step s and integer zero point z,
    every group holding codes 0 and 3: the quantiser must reproduce it."""
    codes = rng.integers(0, 4, size=(n, k)).astype(np.int64)
    codes[:, ::128] = 0
    codes[:, 1::128] = 3
    s = 2.0 ** rng.integers(-9, -5, size=(n, k // 128))
    z = rng.integers(0, 4, size=(n, k // 128)).astype(np.float64)
    w = (codes - np.repeat(z, 128, axis=1)) * np.repeat(s, 128, axis=1)
    return workload.f32_to_bf16_bits(w.astype(np.float32)), w


def test_lossless_special_case():
    rng = np.random.default_rng(23)
    n, k = 300, 1024
    w_bits, w = _lossless_weight(n, k, rng)
    packed, S, ZS = oracle.quantize_pack(w_bits)
    assert np.array_equal(oracle.effective_weight(packed, S, ZS), w)
    x = workload.gen_x(4, k, seed=31, outliers=True)
    out = oracle.pipeline(x, w_bits, packed, S, ZS, kcand=8, r=32)
    E = oracle.exact_head(x, w_bits)
    assert np.array_equal(out["coarse"], E)
    assert np.array_equal(out["out_id"], oracle.head.argmax_lowest(E.astype(np.float32)))


def test_all_ties_fixture(golden):
    fx = golden("all_ties.txt")
    n, k = int(fx["N"][0][0]), int(fx["K"][0][0])
    kc, r = int(fx["KCAND"][0][0]), int(fx["R"][0][0])
    w = workload.gen_weight(n, k, seed=4)
    x = np.zeros((1, k), dtype=np.uint16)
    packed, S, ZS = oracle.quantize_pack(w)
    out = oracle.pipeline(x, w, packed, S, ZS, kcand=kc, r=r)
    want_blocks = []
    for span in fx["block_lists"][0]:
        a, b = (int(v) for v in span.split("-"))
        want_blocks += list(range(a, b + 1))
    assert [int(v) for v in out["cand_id"][0]] == want_blocks
    assert [int(v) for v in out["rr_id"][0]] == [int(v) for v in fx["row_top_r"][0]]
    assert int(out["out_id"][0]) == int(fx["argmax"][0][0])


def test_degenerate_selection_is_plain_argmax():
    """KCAND = 64 and R >= N rerank every column: the result is the plain argmax
    of the exact head; KCAND = 64, R = 32 gives the full-row top-32 of the
    coarse scores (a library sort)."""
    n, k = 200, 512
    w = workload.gen_weight(n, k, seed=41)
    x = workload.gen_x(3, k, seed=42)
    packed, S, ZS = oracle.quantize_pack(w)
    out = oracle.pipeline(x, w, packed, S, ZS, kcand=64, r=256)
    E = oracle.exact_head(x, w).astype(np.float32)
    assert np.array_equal(out["out_id"], np.argmax(E, axis=1))
    out32 = oracle.pipeline(x, w, packed, S, ZS, kcand=64, r=32)
    c = out32["coarse"]
    for m in range(3):
        order = np.lexsort((np.arange(n), -c[m]))[:32]
        assert np.array_equal(out32["rr_id"][m], order)


def test_partial_block_padding():
    n, k = 70, 512                      # second block holds 6 valid columns
    w = workload.gen_weight(n, k, seed=43)
    x = workload.gen_x(1, k, seed=44)
    packed, S, ZS = oracle.quantize_pack(w)
    out = oracle.pipeline(x, w, packed, S, ZS, kcand=8, r=16)
    ids = out["cand_id"][0].reshape(2, 8)
    assert np.all(ids[0] >= 0) and np.all(ids[0] < 64)
    assert np.all(ids[1][:6] >= 64) and np.all(ids[1][6:] == -1)
    assert np.all(np.isneginf(out["cand_val"][0].reshape(2, 8)[1][6:]))
    assert np.sum(out["rr_id"][0] >= 0) == 14 and np.all(out["rr_id"][0][14:] == -1)


# ------------------------------------------------------------ brute force
@pytest.mark.parametrize("m,n,kc,r", [(1, 64, 8, 32), (2, 150, 4, 8), (3, 130, 2, 5)])
def test_pipeline_matches_exact_brute_force(m, n, kc, r):
    k = 512
    w = workload.gen_weight(n, k, seed=100 + n)
    x = workload.gen_x(m, k, seed=200 + n)
    ref = brute.run([[int(v) for v in row] for row in x], [[int(v) for v in row] for row in w], kc, r)
    packed, S, ZS = oracle.quantize_pack(w)
    assert [[int(v) for v in row] for row in packed] == ref["packed"]
    assert [[int(v) for v in row] for row in S] == ref["S"]
    assert [[int(v) for v in row] for row in ZS] == ref["ZS"]
    out = oracle.pipeline(x, w, packed, S, ZS, kcand=kc, r=r)
    exact = np.array([[float(v) for v in row] for row in ref["coarse"]])
    assert np.allclose(out["coarse"], exact, rtol=1e-12, atol=1e-12)
    cand_ids = np.array([[c for _, c in row] for row in ref["cand"]])
    assert np.array_equal(out["cand_id"], cand_ids)
    assert np.array_equal(out["rr_id"], np.array(ref["rr_id"]))
    ev = np.array([[float(v) if v is not None else -np.inf for v in row] for row in ref["rr_val"]])
    assert np.allclose(out["rr_val"], ev, rtol=1e-12, atol=1e-12)
    assert list(out["out_id"]) == ref["out_id"]


def test_coarse_matches_page_collapse_form():
    """The effective-weight form and the page's S*p - ZS*X form agree in float64."""
    w = workload.gen_weight(500, 1024, seed=50)
    x = workload.gen_x(3, 1024, seed=51)
    packed, S, ZS = oracle.quantize_pack(w)
    a = oracle.coarse(x, packed, S, ZS)
    b = oracle.coarse_collapse(x, packed, S, ZS)
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)


# ------------------------------------------------------------ sizes
def test_closed_form_sizes(golden):
    fx = golden("stored_sizes.txt")
    k = int(fx["hidden"][0][0])
    n = int(fx["vocab_shard"][0][0])
    packed_bytes = n * (k // 4)
    pair_bytes = 2 * n * (k // oracle.GROUP) * 2
    assert packed_bytes + pair_bytes == 178_790_400
    assert round((packed_bytes + pair_bytes) / 2 ** 30, 3) == float(fx["int2_head_gib"][0][0])
    assert round(packed_bytes / 2 ** 20) == int(fx["int2_codes_mib"][0][0])
    assert round(n * k * 2 / 2 ** 30, 2) == float(fx["bf16_head_gib"][0][0])


# ------------------------------------------------------------ recall lever
def test_kcand_is_the_recall_lever():
    """Module docstring: at KCAND = 1 a winner that shares its block with a
    stronger token is never a candidate; KCAND = 8 recovers it.  Planted
    near-tie pairs (gap 0.01, far below the 2-bit coarse error) in one block."""
    n, k, m = 4096, 512, 12
    w = workload.gen_weight(n, k, seed=60)
    x = workload.gen_x(m, k, seed=61)
    w, pairs = workload.plant_recall_pairs(x, w, target=12.0, gap=0.01, seed=62)
    E = oracle.exact_head(x, w)
    winners = np.argmax(E, axis=1)
    assert [int(v) for v in winners] == [p[0] for p in pairs]
    packed, S, ZS = oracle.quantize_pack(w)
    hit8 = oracle.pipeline(x, w, packed, S, ZS, kcand=8, r=32)["out_id"]
    hit1 = oracle.pipeline(x, w, packed, S, ZS, kcand=1, r=32)["out_id"]
    assert np.array_equal(hit8, winners)
    assert np.sum(hit1 != winners) >= 2


# ------------------------------------------------------- row for the caller
def test_logits_row_fixture(golden):
    """The row handed to the caller, hand-derived (full and top-k only)."""
    fx = golden("logits_row_example.txt")
    n = int(fx["N"][0][0])
    coarse = np.array([float(v) for v in fx["coarse"][0]], dtype=np.float32)[None, :]
    rr_id = np.array([[int(v) for v in fx["rr_id"][0]]])
    rr_val = np.array([[float(v) for v in fx["rr_val"][0]]], dtype=np.float32)
    full = oracle.logits_row(rr_id, rr_val, n, coarse_f32=coarse)
    topk = oracle.logits_row(rr_id, rr_val, n, topk_only=True)
    assert [int(b) for b in full[0]] == [int(v, 16) for v in fx["full"][0]]
    assert [int(b) for b in topk[0]] == [int(v, 16) for v in fx["topk"][0]]


@pytest.mark.parametrize("topk_only", [False, True])
def test_logits_row_matches_exact_rounding(topk_only):
    """Every entry against exact rational rounding: a reranked id holds its exact
    value in bf16, every other entry the coarse value in bf16 (or -inf)."""
    rng = np.random.default_rng(7)
    m, n, r = 3, 300, 20
    coarse = (rng.standard_normal((m, n)) * 4).astype(np.float32)
    rr_id = np.stack([rng.choice(n, size=r, replace=False) for _ in range(m)])
    rr_id[2, 15:] = -1
    rr_val = (rng.standard_normal((m, r)) * 4).astype(np.float32)
    y = oracle.logits_row(rr_id, rr_val, n, coarse_f32=coarse, topk_only=topk_only)
    for row in range(m):
        exact = {int(i): j for j, i in enumerate(rr_id[row]) if i >= 0}
        for col in range(n):
            if col in exact:
                want = brute.bf16_value_bits(brute.bf16(Fraction(float(rr_val[row, exact[col]]))))
            elif topk_only:
                want = 0xFF80
            else:
                want = brute.bf16_value_bits(brute.bf16(Fraction(float(coarse[row, col]))))
            assert int(y[row, col]) == want, (row, col)


# ------------------------------------------------------ e4m3 rerank source
def test_e4m3_decode_fixture(golden):
    fx = golden("e4m3_decode_example.txt")
    for code, val in fx["code"]:
        got = float(oracle.e4m3_value(np.array([int(code, 16)]))[0])
        assert got == float(val) and np.signbit(got) == np.signbit(float(val)), code


def test_e4m3_decode_is_the_standard_format_except_its_nan():
    """The page's decode equals the e4m3 format's closed form (sign, 4-bit
    exponent biased by 7, 3-bit mantissa, subnormals at exponent 0) for every
    code but the two the format reserves for NaN, which the page reads as +-480."""
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        want = -mag if s else mag
        got = Fraction(float(oracle.e4m3_value(np.array([b]))[0]))
        if (b & 0x7F) == 0x7F:
            assert got == (-480 if s else 480)
        else:
            assert got == want, b


def test_e4m3_rerank_equals_bf16_rerank_on_representable_rows():
    """Rows that are e4m3 values times a power-of-two scale are exact in bf16
    too: both rerank sources then give the same logits exactly."""
    rng = np.random.default_rng(11)
    n, k, m, r = 40, 256, 2, 6
    codes = rng.integers(0, 256, size=(n, k)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                      # no +-480 (not a standard value)
    scale = (2.0 ** rng.integers(-8, -4, size=n)).astype(np.float32)
    wv = oracle.e4m3_value(codes) * scale[:, None]
    w_bits = workload.f32_to_bf16_bits(wv.astype(np.float32))
    assert np.array_equal(obf.to_f64(w_bits), wv)             # representable in bf16
    x = workload.gen_x(m, k, seed=5)
    rr_id = np.stack([rng.choice(n, size=r, replace=False) for _ in range(m)])
    rr_id[1, 4:] = -1
    a = oracle.rerank_exact_e4m3(x, codes, scale, rr_id)
    b = oracle.rerank_exact(x, w_bits, rr_id)
    assert np.array_equal(a, b)


def test_synthetic_e4m3_head_rounds_to_nearest():
    """The generator's codes are the nearest e4m3 value to w / scale (inputs only)."""
    w = workload.gen_weight(64, 512, seed=3)
    codes, scale = workload.e4m3_head(w)
    v = obf.to_f64(w) / scale[:, None].astype(np.float64)
    got = oracle.e4m3_value(codes)
    table = np.unique(np.abs(oracle.e4m3_value(np.arange(0, 127))))
    err = np.abs(got - v)
    best = np.min(np.abs(np.abs(v)[..., None] - table[None, None, :]), axis=-1)
    assert np.all(err <= best + 1e-12)
    assert np.max(np.abs(got)) == 448.0


# ------------------------------------------------------------- 4-bit head
def test_int4_quantizer_worked_example(golden):
    fx = golden("quantizer_int4_worked_example.txt")
    k = int(fx["K"][0][0])
    w = np.zeros((1, k), dtype=np.float32)
    w[0, :4] = np.array([float(v) for v in fx["values_group0"][0]], dtype=np.float32) * 2.0 ** -7
    bits = obf.from_f32(w)
    codes, S, ZS = oracle.quantize_int4(bits)
    assert [int(c) for c in codes[0, :5]] == [int(v) for v in fx["codes_group0"][0]]
    assert np.all(codes[0, 4:128] == 8) and np.all(codes[0, 128:] == 0)
    assert int(S[0, 0]) == int(fx["S0"][0][0], 16) and int(ZS[0, 0]) == int(fx["ZS0"][0][0], 16)
    packed = oracle.pack_half_split(codes)
    assert [int(b) for b in packed[0, :5]] == [int(v, 16) for v in fx["bytes"][0]]
    assert np.array_equal(oracle.unpack_half_split(packed), codes)
    wv = oracle.effective_weight_int4(packed, S, ZS)[0, :128]
    assert np.array_equal(wv, (codes[0, :128].astype(np.float64) - 8) * 2.0 ** -7)


def test_int4_quantizer_matches_exact_brute_force():
    rng = np.random.default_rng(41)
    w = workload.f32_to_bf16_bits((rng.standard_normal((6, 256)) * 0.02).astype(np.float32))
    w[5, :128] = w[5, 0]                       # a constant group: the 1e-8 clamp
    codes, S, ZS = oracle.quantize_int4(w)
    for i in range(w.shape[0]):
        c, s, z = brute.quantize_row([int(b) for b in w[i]], levels=15, premul=16)
        assert [int(v) for v in codes[i]] == c, i
        assert [int(v) for v in S[i]] == s and [int(v) for v in ZS[i]] == z, i


def test_int4_collapse_identity_exact():
    """S * sum x (1 + v/16) - ZS * sum x == sum x ((S/16) v - (ZS - S)), in fractions."""
    rng = np.random.default_rng(43)
    for _ in range(20):
        S = Fraction(int(rng.integers(1, 255)), 2 ** int(rng.integers(6, 12)))
        ZS = S + Fraction(int(rng.integers(0, 15)), 16) * S
        xs = [Fraction(int(rng.integers(-1000, 1000)), 1024) for _ in range(128)]
        vs = [int(rng.integers(0, 16)) for _ in range(128)]
        lhs = S * sum(x * (1 + Fraction(v, 16)) for x, v in zip(xs, vs)) - ZS * sum(xs)
        rhs = sum(x * (S / 16 * v - (ZS - S)) for x, v in zip(xs, vs))
        assert lhs == rhs


def test_int4_lossless_special_case():
    """Codes with a power-of-two step, an integer zero point and both extreme
    codes in every group come back exactly, and the effective weight is W."""
    rng = np.random.default_rng(47)
    n, k = 8, 256
    codes = rng.integers(0, 16, size=(n, k)).astype(np.int64)
    codes[:, ::128] = 0
    codes[:, 1::128] = 15
    s = 2.0 ** rng.integers(-10, -6, size=(n, k // 128))
    z = rng.integers(0, 16, size=(n, k // 128)).astype(np.float64)
    w = (codes - np.repeat(z, 128, axis=1)) * np.repeat(s, 128, axis=1)
    bits = workload.f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(obf.to_f64(bits), w)
    q, S, ZS = oracle.quantize_int4(bits)
    assert np.array_equal(q, codes)
    assert np.array_equal(oracle.effective_weight_int4(oracle.pack_half_split(q), S, ZS), w)


# ------------------------------------------------------- NVFP4 rerank source
def _nvfp4_fixture(golden):
    fx = golden("nvfp4_rows_example.txt")
    g = np.float32(float(fx["gscale"][0][0]))
    rows, scales = [], []
    for r in fx["row"]:
        bar = r.index("|")
        rows.append([_hex(v) for v in r[1:bar]])
        scales.append([_hex(v) for v in r[bar + 1:]])
    w4 = np.array(rows, dtype=np.uint8)
    bs = np.array(scales, dtype=np.uint8)
    want = np.array([[float(v) for v in r[1:]] for r in fx["weights"]])
    return fx, w4, bs, g, want


def test_e2m1_decode_table(golden):
    fx = golden("nvfp4_rows_example.txt")
    mags = [float(v) for v in fx["e2m1"][0]]
    got = oracle.e2m1_value(np.arange(16))
    assert list(got[:8]) == mags
    assert list(-got[8:]) == mags
    assert all(np.signbit(got[8:]))


def test_nvfp4_rows_fixture(golden):
    """Hand-derived weights: nibble order, block scales, the global scale, the
    float32 product and the bf16 rounding (two ties to even, four roundings up)."""
    fx, w4, bs, g, want = _nvfp4_fixture(golden)
    got = oracle.nvfp4_rows(w4, bs, g, [0, 1], 32)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))   # -0.0 kept
    x = np.full((1, 32), 0x3F80, dtype=np.uint16)                      # x = 1
    e = oracle.rerank_exact_nvfp4(x, w4, bs, g, np.array([[0, -1]]))
    assert e[0, 0] == float(fx["dot_ones"][0][1])
    assert e[0, 1] == -np.inf


def _bf16_rne_fraction(v):
    """bf16 value nearest to the Fraction v, ties to the even mantissa (brute force)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    lo = Fraction(int(a * 128), 128)                                 # 7 mantissa bits
    hi = lo + Fraction(1, 128)
    if a - lo < hi - a or (a - lo == hi - a and int(lo * 128) % 2 == 0):
        q = lo
    else:
        q = hi
    return sign * q * Fraction(2) ** e


def _e4m3fn_fraction(b):
    e, mant = (b >> 3) & 15, b & 7
    mag = Fraction(mant, 512) if e == 0 else (1 + Fraction(mant, 8)) * Fraction(2) ** (e - 7)
    return -mag if b & 128 else mag


def test_nvfp4_rows_brute_force():
    """Exact rationals: d * s is exact, times g rounded once to float32 (the
    product of a 6-bit and a 24-bit significand is exact in float64), then
    the bf16 value nearest to it found by search."""
    rng = np.random.default_rng(21)
    n, k = 3, 64
    w4 = rng.integers(0, 256, size=(n, k // 2)).astype(np.uint8)
    bs = rng.integers(0, 127, size=(n, k // 16)).astype(np.uint8)
    bs[bs == 0x7F] = 0x38
    g = np.float32(0.0123)
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
           Fraction(6)]
    got = oracle.nvfp4_rows(w4, bs, g, np.arange(n), k)
    for r in range(n):
        for j in range(k):
            byte = int(w4[r, j // 2])
            nib = byte & 15 if j % 2 == 0 else byte >> 4
            d = -mag[nib & 7] if nib & 8 else mag[nib & 7]
            prod = d * _e4m3fn_fraction(int(bs[r, j // 16])) * Fraction(float(g))
            f32 = Fraction(float(np.float32(float(prod))))
            assert got[r, j] == float(_bf16_rne_fraction(f32)), (r, j)


def test_nvfp4_rerank_equals_bf16_rerank_on_representable_rows():
    """With a global scale of 1 and power-of-two block scales every weight is
    an e2m1 value times a power of two, exact in bf16: the NVFP4 source then
    gives exactly the bf16 rerank of those rows."""
    rng = np.random.default_rng(12)
    n, k, m, r = 30, 256, 2, 5
    w4 = rng.integers(0, 256, size=(n, k // 2)).astype(np.uint8)
    bs = ((rng.integers(4, 10, size=(n, k // 16)) << 3)).astype(np.uint8)   # 2^-3 .. 2^2, mantissa 0
    codes = np.empty((n, k), dtype=np.int64)
    codes[:, 0::2] = w4 & 15
    codes[:, 1::2] = w4 >> 4
    wv = oracle.e2m1_value(codes) * np.repeat(2.0 ** ((bs.astype(np.int64) >> 3) - 7), 16, axis=1)
    w_bits = workload.f32_to_bf16_bits(wv.astype(np.float32))
    assert np.array_equal(obf.to_f64(w_bits), wv)
    x = workload.gen_x(m, k, seed=6)
    rr_id = np.stack([rng.choice(n, size=r, replace=False) for _ in range(m)])
    rr_id[0, 3:] = -1
    a = oracle.rerank_exact_nvfp4(x, w4, bs, np.float32(1.0), rr_id)
    b = oracle.rerank_exact(x, w_bits, rr_id)
    assert np.array_equal(a, b)


def test_synthetic_nvfp4_head_rounds_to_nearest():
    """The generator's block scales and nibbles are nearest grid values (inputs only)."""
    w = workload.gen_weight(32, 512, seed=4)
    w4, bs, g = workload.nvfp4_head(w)
    wf = obf.to_f64(w)
    s = oracle.e4m3fn_value(bs)
    amax = np.abs(wf.reshape(32, -1, 16)).max(axis=2)
    table = np.unique(np.abs(oracle.e4m3_value(np.arange(0, 127))))
    t = amax / (6.0 * float(g))
    assert np.all(np.abs(s - t) <= np.min(np.abs(t[..., None] - table), axis=-1) + 1e-12)
    codes = np.empty((32, 512), dtype=np.int64)
    codes[:, 0::2] = w4 & 15
    codes[:, 1::2] = w4 >> 4
    d = oracle.e2m1_value(codes)
    v = wf / (np.repeat(s, 16, axis=1) * float(g))
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    best = np.min(np.abs(np.abs(v)[..., None] - grid), axis=-1)
    assert np.all(np.abs(np.abs(d) - np.abs(v)) <= best + 1e-12)
    assert np.all((d == 0) | (np.sign(d) == np.sign(v)))


# ------------------------------------------------------------- tie rows
def _tie_cases(golden):
    fx = golden("tie_rows_example.txt")
    cases = []
    for ids, e, tie, tied in zip(fx["id"], fx["e"], fx["tie"], fx["tied"]):
        cases.append((np.array([int(v) for v in ids]), np.array([float(v) for v in e]),
                      bool(int(tie[0])), {int(v) for v in tied}))
    return cases


def test_tie_rows_fixture(golden):
    """tie_rows and tied_ids against hand-derived rows: gaps just inside and
    just outside 1e-4 |e1|, a negative best, unsorted values, -inf padding, a
    single candidate, a three-way tie, exact equality at and away from zero."""
    cases = _tie_cases(golden)
    assert len(cases) == 10
    for i, (ids, e, tie, tied) in enumerate(cases):
        assert bool(oracle.tie_rows(e[None, :])[0]) == tie, i
        assert oracle.tied_ids(ids[None, :], e[None, :])[0] == tied, i
        # the oracle's own final id is always in the tied set
        out_id, _ = oracle.final_argmax(ids[None, :], e[None, :])
        if tied:
            assert int(out_id[0]) in tied, i
        else:
            assert int(out_id[0]) == -1, i


def test_pipeline_tie_rows_are_over_the_reranked_set():
    """With weights the quantiser reproduces (coarse == exact), two columns of
    one block with identical rows tie exactly in the full row; at KCAND = 1
    only the lower one is a candidate, so the reranked set holds no tie: the
    pipeline's tie flag follows the reranked values, not the full row."""
    rng = np.random.default_rng(29)
    n, k = 256, 512
    w_bits, _ = _lossless_weight(n, k, rng)
    x = workload.gen_x(2, k, seed=30)
    E = oracle.exact_head(x, w_bits)
    top = [int(np.argmax(E[i])) for i in range(2)]
    for i in range(2):   # a twin of the row's winner in the same block
        twin = top[i] + 1 if top[i] % 64 < 63 else top[i] - 1
        w_bits[twin] = w_bits[top[i]]
    E = oracle.exact_head(x, w_bits)
    assert np.all(oracle.tie_rows(E))                        # full row: a tie in each row
    packed, S, ZS = oracle.quantize_pack(w_bits)
    out1 = oracle.pipeline(x, w_bits, packed, S, ZS, kcand=1, r=32)
    assert np.array_equal(out1["coarse"], E)
    assert not np.any(out1["tie_rows"])                      # reranked set: one of the twins only
    out8 = oracle.pipeline(x, w_bits, packed, S, ZS, kcand=8, r=32)
    assert np.all(out8["tie_rows"])                          # both twins reranked
    for i in range(2):
        twins = {int(v) for v in np.nonzero(E[i] == E[i].max())[0]}
        assert out8["tied_ids"][i] == twins and int(out8["out_id"][i]) == min(twins)


# ------------------------------------------------------- 4-bit pipeline pins
@pytest.mark.parametrize("m,n,kc,r", [(1, 64, 1, 8), (2, 130, 4, 8), (2, 100, 1, 3)])
def test_int4_pipeline_matches_exact_brute_force(m, n, kc, r):
    """The 4-bit head, every step, against exact rationals: the brute force
    scores each column in the page's form S sum x (1 + v/16) - ZS sum x from
    its own half-split bytes, independently of the oracle's effective weight."""
    k = 256
    w = workload.gen_weight(n, k, seed=300 + n)
    x = workload.gen_x(m, k, seed=400 + n)
    ref = brute.run([[int(v) for v in row] for row in x], [[int(v) for v in row] for row in w], kc, r, bits=4)
    packed4, S, ZS = oracle.quantize_pack_int4(w)
    assert [[int(v) for v in row] for row in packed4] == ref["packed"]
    assert [[int(v) for v in row] for row in S] == ref["S"]
    assert [[int(v) for v in row] for row in ZS] == ref["ZS"]
    c = oracle.coarse_int4(x, packed4, S, ZS)
    exact = np.array([[float(v) for v in row] for row in ref["coarse"]])
    assert np.allclose(c, exact, rtol=1e-12, atol=1e-12)
    out = oracle.pipeline(x, w, packed4, S, ZS, kcand=kc, r=r, bits=4)
    assert np.array_equal(out["coarse"], c)
    assert np.array_equal(out["cand_id"], np.array([[cc for _, cc in row] for row in ref["cand"]]))
    assert np.array_equal(out["rr_id"], np.array(ref["rr_id"]))
    assert list(out["out_id"]) == ref["out_id"]
    assert [float(v) for v in out["out_val"]] == [float(v) for v in ref["out_val"]]


def test_int4_lossless_pipeline_is_the_exact_head():
    """A weight already on a 16-level grid (power-of-two step, integer zero
    point, codes 0 and 15 in every group): the 4-bit coarse scores equal the
    exact head, and the pipeline's token is the exact argmax on every row."""
    rng = np.random.default_rng(53)
    n, k = 300, 512
    codes = rng.integers(0, 16, size=(n, k)).astype(np.int64)
    codes[:, ::128] = 0
    codes[:, 1::128] = 15
    s = 2.0 ** rng.integers(-10, -7, size=(n, k // 128))
    z = rng.integers(0, 16, size=(n, k // 128)).astype(np.float64)
    wf = (codes - np.repeat(z, 128, axis=1)) * np.repeat(s, 128, axis=1)
    w_bits = workload.f32_to_bf16_bits(wf.astype(np.float32))
    x = workload.gen_x(5, k, seed=54)
    out = oracle.pipeline(x, w_bits, *oracle.quantize_pack_int4(w_bits), kcand=1, r=32, bits=4)
    E = oracle.exact_head(x, w_bits)
    assert np.array_equal(out["coarse"], E)
    assert np.array_equal(out["out_id"], np.argmax(E.astype(np.float32), axis=1))


def test_int4_coarse_is_the_split_of_a_long_int2_head():
    """An exact identity of the 4-bit weight: code v = 4 vh + vl, so
    (S/16) v - (ZS - S) = [(S/4) vh - (ZS - S)] + [(S/16) vl].  The 4-bit
    coarse score equals the 2-bit oracle's score of the 2K-long head built
    from those halves (second pair (S/4, S/4): weight (S/16) vl), in x' = (x, x)."""
    n, k = 70, 512
    w = workload.gen_weight(n, k, seed=55)
    x = workload.gen_x(3, k, seed=56)
    packed4, S, ZS = oracle.quantize_pack_int4(w)
    v = oracle.unpack_half_split(packed4).astype(np.uint8)
    codes2 = np.concatenate([v >> 2, v & 3], axis=1)
    s_quarter = obf.from_f32((obf.to_f32(S) * np.float32(0.25)).astype(np.float32))
    S2 = np.concatenate([S, s_quarter], axis=1)
    ZS2 = np.concatenate([ZS, s_quarter], axis=1)
    long = oracle.coarse(np.concatenate([x, x], axis=1), oracle.pack_quarter_split(codes2), S2, ZS2)
    assert np.allclose(oracle.coarse_int4(x, packed4, S, ZS), long, rtol=1e-12, atol=1e-12)


def test_final_argmax_nan_reading():
    """The final argmax's reading for NaN exact values (hand-made rows): a NaN
    never beats a number, -inf included; an all-NaN row returns its lowest id;
    equal values go to the lower id; padding (-1) is skipped."""
    ids = np.array([[5, 3, 9, -1], [4, 2, -1, -1], [1, 2, 3, 4], [7, 6, -1, -1], [8, -1, -1, -1]])
    nan, inf = np.nan, np.inf
    e = np.array([[nan, 2.0, 2.0, -inf], [nan, nan, -inf, -inf], [-inf, nan, -inf, 1.0],
                  [nan, -inf, -inf, -inf], [-inf, -inf, -inf, -inf]])
    out_id, out_val = oracle.final_argmax(ids, e)
    assert [int(v) for v in out_id] == [3, 2, 4, 6, 8]
    assert out_val[0] == 2.0 and np.isnan(out_val[1]) and out_val[2] == 1.0
    assert np.isneginf(out_val[3]) and np.isneginf(out_val[4])
