"""CPU tests of the C ABI: symbols, the host quantiser and tiler, and argument
validation of every entry point (validation runs before any HIP call, so no
GPU is needed)."""
import ctypes

import numpy as np
import pytest

import oracle
from bit_quantized_lm_amd import _binding as B
from bit_quantized_lm_amd import workload


@pytest.fixture(scope="module")
def lib():
    try:
        return B.load_library()
    except FileNotFoundError:
        import __graft_entry__
        __graft_entry__.build()
        return B.load_library()


def test_library_exports_every_header_symbol(lib):
    names = B.header_functions()
    assert set(names) == {"draft_head_last_error", "draft_head_sizes", "draft_head_quantize_pack",
                          "draft_head_tile", "draft_head_workspace_bytes", "draft_head_coarse",
                          "draft_head_rerank", "draft_head_argmax", "draft_head_forward",
                          "draft_head_stream_read", "draft_head_logits_row", "draft_head_rerank_e4m3",
                          "draft_head_forward_e4m3", "draft_head_rerank_nvfp4", "draft_head_forward_nvfp4",
                          "draft_head_quantize_pack_int4",
                          "draft_head_int4_as_int2", "draft_head_tile_int4", "draft_head_coarse_int4",
                          "draft_head_forward_int4",
                          "draft_head_forward_noalloc", "draft_head_forward_row"}
    for name in names:
        assert hasattr(lib, name), name


def test_sizes(lib):
    s = B.draft_head_sizes(124160, 5120)
    assert s["packed_bytes"] + 4 * s["scale_elems"] == 178_790_400
    s = B.draft_head_sizes(70, 512)
    assert s["packed_bytes"] == 70 * 128 and s["tiled_bytes"] == 128 * 128
    assert s["scale_elems"] == 70 * 4 and s["tiled_pairs"] == 128 * 4
    for n, k in ((0, 512), (10, 256), (10, 1000), (10, 0)):
        with pytest.raises(ValueError):
            B.draft_head_sizes(n, k)


# ------------------------------------------------------------ quantiser parity
def _edge_rows(k, rng):
    rows = [
        np.zeros(k, np.float32),
        np.full(k, 0.37, np.float32),
        rng.standard_normal(k, dtype=np.float32) * 1e-9,
        np.abs(rng.standard_normal(k, dtype=np.float32)),
        -np.abs(rng.standard_normal(k, dtype=np.float32)),
        rng.standard_normal(k, dtype=np.float32) * 50,
        np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32) * 0.01,
    ]
    wk = np.zeros(k, np.float32)
    wk[:4] = np.array([-3, -1, 1, 3], np.float32) * 2 ** -7   # round-half-even cases
    rows.append(wk)
    return workload.f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("n,k", [(8, 512), (300, 1024), (4096, 5120)])
def test_quantize_pack_matches_oracle_bytes(lib, n, k):
    rng = np.random.default_rng(n + k)
    w = workload.gen_weight(n, k, seed=n)
    w[:8] = _edge_rows(k, rng)
    p, S, ZS = B.draft_head_quantize_pack(w, nthreads=4)
    op, oS, oZS = oracle.quantize_pack(w)
    assert np.array_equal(p, op)
    assert np.array_equal(S, oS)
    assert np.array_equal(ZS, oZS)


def test_quantize_pack_strided_input(lib):
    w = workload.gen_weight(64, 1536, seed=3)
    view = w[:, :1024]                      # ldw = 1536 > K
    p, S, ZS = B.draft_head_quantize_pack(view)
    op, oS, oZS = oracle.quantize_pack(np.ascontiguousarray(view))
    assert np.array_equal(p, op) and np.array_equal(S, oS) and np.array_equal(ZS, oZS)


def test_quantize_pack_thread_count_does_not_matter(lib):
    w = workload.gen_weight(333, 512, seed=8)
    a = B.draft_head_quantize_pack(w, nthreads=1)
    b = B.draft_head_quantize_pack(w, nthreads=7)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ------------------------------------------------------------ tiler
def test_tile_layout(lib):
    """Check the tiler against the layout documented in drafthead.h."""
    n, k = 150, 1024                       # 3 blocks, the last one partial
    w = workload.gen_weight(n, k, seed=12)
    packed, S, ZS = oracle.quantize_pack(w)
    tiled, pairs = B.draft_head_tile(packed, S, ZS)
    q4, ng, ng4 = k // 4, k // 128, k // 512
    nblk = (n + 63) // 64
    assert tiled.size == nblk * 64 * q4 and pairs.size == nblk * 64 * ng
    rng = np.random.default_rng(0)
    for _ in range(4000):
        col = int(rng.integers(0, nblk * 64))
        j = int(rng.integers(0, q4))
        b, t, c = col // 64, (col % 64) // 16, col % 16
        G, h, s, wb = j // 128, (j % 128) // 64, (j % 64) // 16, j % 16
        off = ((((b * ng4 + G) * 2 + h) * 4 + t) * 64 + s * 16 + c) * 16 + wb
        assert tiled[off] == (packed[col, j] if col < n else 0)
        g = int(rng.integers(0, ng))
        q, G = g // ng4, g % ng4
        off = ((b * ng4 + G) * 4 + t) * 64 + c * 4 + q
        want = (int(S[col, g]) | (int(ZS[col, g]) << 16)) if col < n else 0
        assert int(pairs[off]) == want
    # a permutation: every code byte of every valid column appears exactly once
    assert np.array_equal(np.sort(tiled[tiled != 0]), np.sort(packed.ravel()[packed.ravel() != 0]))


# ------------------------------------------------------------ validation
FAKE = ctypes.c_void_p(4096)      # aligned, never dereferenced: validation rejects first
MIS = ctypes.c_void_p(4098)       # misaligned


def _err(lib, rc, code):
    assert rc == code, (rc, lib.draft_head_last_error())
    assert lib.draft_head_last_error()


def test_quantize_pack_validation(lib):
    w = np.zeros((4, 512), np.uint16)
    out = np.zeros(4096, np.uint8)
    p = w.ctypes.data
    _err(lib, lib.draft_head_quantize_pack(None, 4, 512, 512, out.ctypes.data, p, p, 0), B.DH_EINVAL)
    _err(lib, lib.draft_head_quantize_pack(p, 4, 512, 256, out.ctypes.data, p, p, 0), B.DH_EINVAL)
    _err(lib, lib.draft_head_quantize_pack(p, 4, 384, 512, out.ctypes.data, p, p, 0), B.DH_ESHAPE)
    _err(lib, lib.draft_head_quantize_pack(p, 0, 512, 512, out.ctypes.data, p, p, 0), B.DH_ESHAPE)
    _err(lib, lib.draft_head_quantize_pack(p, 4, 512, 512, out.ctypes.data, p, p, -1), B.DH_EINVAL)
    _err(lib, lib.draft_head_tile(None, p, p, 4, 512, p, p), B.DH_EINVAL)
    _err(lib, lib.draft_head_tile(p, p, p, 4, 500, p, p), B.DH_ESHAPE)


def test_workspace_bytes(lib):
    # 1 KiB of per-row hand-off words (128 rows, 8 bytes); the resident
    # kernel (up to 8 rows while x fits its LDS: (K/128) * (256 MP + 4 MP) +
    # blocks * MP * 256 within 160 KB) adds 64 KiB of block maxima (8 rows of
    # up to 2048 blocks, fp32)
    head = 1024
    for m, k in ((1, 5120), (1, 65536), (2, 39424), (4, 19456), (8, 5120), (8, 8704)):
        assert B.draft_head_workspace_bytes(m, k) == head + 65536, (m, k)
    # many-row kernel: + (K/128) * 4096 * MT + (K/512) * 4096 + 512 with MT = min(ceil(M/16), 5),
    # then 8 KiB of block maxima per row
    for m, k in ((2, 39936), (4, 19968), (8, 9216), (9, 512), (16, 1024), (17, 1024), (72, 5120),
                 (80, 5120), (81, 5120), (128, 5120)):
        mt = min((m + 15) // 16, 5)
        assert B.draft_head_workspace_bytes(m, k) == \
            head + (k // 128) * 4096 * mt + (k // 512) * 4096 + 512 + 8192 * m, (m, k)
    assert B.draft_head_workspace_bytes(72, 5120) == 1_451_520
    out = ctypes.c_size_t()
    _err(lib, lib.draft_head_workspace_bytes(1, 512, None), B.DH_EINVAL)
    _err(lib, lib.draft_head_workspace_bytes(0, 512, ctypes.byref(out)), B.DH_EINVAL)
    _err(lib, lib.draft_head_workspace_bytes(129, 512, ctypes.byref(out)), B.DH_EUNSUP)
    _err(lib, lib.draft_head_workspace_bytes(1, 700, ctypes.byref(out)), B.DH_ESHAPE)


@pytest.mark.parametrize("via", ["coarse", "forward"])
def test_coarse_validation(lib, via):
    if via == "forward":    # the same checks, before any launch, in the one-call entry point
        f = lambda x, M, K, N, t, p, kc, cv, ci, co, ws, wsb, s: lib.draft_head_forward(  # noqa: E731
            x, M, K, N, t, p, FAKE, K, kc, 8, cv, ci, FAKE, FAKE, FAKE, FAKE, co, ws, wsb, s, None, None)
    else:
        f = lambda *a: lib.draft_head_coarse(*a)  # noqa: E731
    ok = dict(x=FAKE, M=1, K=512, N=64, tiled=FAKE, pairs=FAKE, kc=8, cv=FAKE, ci=FAKE, co=None, ws=FAKE,
              wsb=B.draft_head_workspace_bytes(1, 512), s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["M"], a["K"], a["N"], a["tiled"], a["pairs"], a["kc"], a["cv"], a["ci"],
                 a["co"], a["ws"], a["wsb"], a["s"])
    _err(lib, call(x=None), B.DH_EINVAL)
    _err(lib, call(cv=None), B.DH_EINVAL)
    _err(lib, call(ci=None), B.DH_EINVAL)
    _err(lib, call(tiled=None), B.DH_EINVAL)
    _err(lib, call(M=0), B.DH_EINVAL)
    _err(lib, call(M=129), B.DH_EUNSUP)
    _err(lib, call(K=256), B.DH_ESHAPE)
    _err(lib, call(K=768), B.DH_ESHAPE)
    _err(lib, call(K=131072), B.DH_ESHAPE)
    _err(lib, call(N=0), B.DH_ESHAPE)
    _err(lib, call(kc=0), B.DH_EUNSUP)
    _err(lib, call(kc=65), B.DH_EUNSUP)
    _err(lib, call(x=MIS), B.DH_EINVAL)
    _err(lib, call(pairs=MIS), B.DH_EINVAL)
    # the caller's workspace: present, aligned, large enough
    _err(lib, call(ws=None), B.DH_EINVAL)
    _err(lib, call(wsb=B.draft_head_workspace_bytes(1, 512) - 1), B.DH_EINVAL)
    _err(lib, call(ws=MIS), B.DH_EINVAL)
    need = B.draft_head_workspace_bytes(9, 512)
    _err(lib, call(M=9, K=4096), B.DH_EINVAL)   # one row's workspace at K = 512: too small for 9 x 4096
    _err(lib, call(M=9, ws=FAKE, wsb=need - 16), B.DH_EINVAL)
    _err(lib, call(M=9, ws=MIS, wsb=need), B.DH_EINVAL)
    _err(lib, call(M=9, ws=None, wsb=need), B.DH_EINVAL)


def test_rerank_validation(lib):
    ok = dict(x=FAKE, w=FAKE, ldw=512, M=2, K=512, N=100, cv=FAKE, ci=FAKE, nc=16, R=8, ri=FAKE,
              rv=FAKE, s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.draft_head_rerank(a["x"], a["w"], a["ldw"], a["M"], a["K"], a["N"], a["cv"], a["ci"],
                                     a["nc"], a["R"], a["ri"], a["rv"], a["s"])
    _err(lib, call(w=None), B.DH_EINVAL)
    _err(lib, call(ri=None), B.DH_EINVAL)
    _err(lib, call(M=0), B.DH_EINVAL)
    _err(lib, call(M=200), B.DH_EUNSUP)
    _err(lib, call(K=100), B.DH_ESHAPE)
    _err(lib, call(N=0), B.DH_ESHAPE)
    _err(lib, call(ldw=256), B.DH_EINVAL)
    _err(lib, call(ldw=515), B.DH_EINVAL)
    _err(lib, call(nc=0), B.DH_EINVAL)
    _err(lib, call(R=0), B.DH_EUNSUP)
    _err(lib, call(R=17), B.DH_EUNSUP)
    _err(lib, call(R=2000, nc=4000), B.DH_EUNSUP)
    _err(lib, call(w=MIS), B.DH_EINVAL)


def test_argmax_validation(lib):
    _err(lib, lib.draft_head_argmax(None, FAKE, 1, 8, FAKE, FAKE, None), B.DH_EINVAL)
    _err(lib, lib.draft_head_argmax(FAKE, FAKE, 0, 8, FAKE, FAKE, None), B.DH_EINVAL)
    _err(lib, lib.draft_head_argmax(FAKE, FAKE, 1, 0, FAKE, FAKE, None), B.DH_EUNSUP)
    _err(lib, lib.draft_head_argmax(FAKE, FAKE, 1, 1025, FAKE, FAKE, None), B.DH_EUNSUP)


def test_rerank_e4m3_validation(lib):
    ok = dict(x=FAKE, w=FAKE, sc=FAKE, ldw=512, M=2, K=512, N=100, cv=FAKE, ci=FAKE, nc=16, R=8, ri=FAKE,
              rv=FAKE, s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.draft_head_rerank_e4m3(a["x"], a["w"], a["sc"], a["ldw"], a["M"], a["K"], a["N"], a["cv"],
                                          a["ci"], a["nc"], a["R"], a["ri"], a["rv"], a["s"])
    _err(lib, call(sc=None), B.DH_EINVAL)          # the e4m3 rows need their scales
    _err(lib, call(w=None), B.DH_EINVAL)
    _err(lib, call(ldw=520), B.DH_EINVAL)          # rows of bytes: a multiple of 16
    _err(lib, call(ldw=256), B.DH_EINVAL)
    _err(lib, call(w=MIS), B.DH_EINVAL)
    _err(lib, call(M=0), B.DH_EINVAL)
    _err(lib, call(K=100), B.DH_ESHAPE)
    _err(lib, call(R=17), B.DH_EUNSUP)
    f = lib.draft_head_forward_e4m3              # the same checks before any launch
    _err(lib, f(FAKE, 1, 512, 64, FAKE, FAKE, FAKE, None, 512, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                FAKE, 512, None, None, None), B.DH_EINVAL)
    _err(lib, f(FAKE, 1, 512, 64, FAKE, FAKE, FAKE, FAKE, 520, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                FAKE, 512, None, None, None), B.DH_EINVAL)


def test_rerank_nvfp4_validation(lib):
    ok = dict(x=FAKE, w=FAKE, ldw=256, bs=FAKE, lds=32, g=FAKE, M=2, K=512, N=100, cv=FAKE, ci=FAKE, nc=16, R=8,
              ri=FAKE, rv=FAKE, s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.draft_head_rerank_nvfp4(a["x"], a["w"], a["ldw"], a["bs"], a["lds"], a["g"], a["M"], a["K"],
                                           a["N"], a["cv"], a["ci"], a["nc"], a["R"], a["ri"], a["rv"], a["s"])
    _err(lib, call(bs=None), B.DH_EINVAL)          # the block scales
    _err(lib, call(g=None), B.DH_EINVAL)           # the global scale
    _err(lib, call(w=None), B.DH_EINVAL)
    _err(lib, call(ldw=240), B.DH_EINVAL)          # a row holds K/2 bytes
    _err(lib, call(ldw=264), B.DH_EINVAL)          # rows of bytes: a multiple of 16
    _err(lib, call(lds=30), B.DH_EINVAL)           # K/16 scale bytes per row
    _err(lib, call(lds=33), B.DH_EINVAL)           # even, for 2-byte scale loads
    _err(lib, call(bs=ctypes.c_void_p(4097)), B.DH_EINVAL)   # 2-byte aligned
    _err(lib, call(w=MIS), B.DH_EINVAL)
    _err(lib, call(M=0), B.DH_EINVAL)
    _err(lib, call(K=100), B.DH_ESHAPE)
    _err(lib, call(R=17), B.DH_EUNSUP)
    f = lib.draft_head_forward_nvfp4             # the same checks before any launch
    _err(lib, f(FAKE, 1, 512, 64, FAKE, FAKE, FAKE, 256, None, 32, FAKE, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                None, FAKE, 512, None, None, None), B.DH_EINVAL)
    _err(lib, f(FAKE, 1, 512, 64, FAKE, FAKE, FAKE, 256, FAKE, 31, FAKE, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                None, FAKE, 512, None, None, None), B.DH_EINVAL)


def test_logits_row_validation(lib):
    f = lib.draft_head_logits_row
    _err(lib, f(FAKE, None, FAKE, 1, 64, 8, 0, FAKE, None), B.DH_EINVAL)
    _err(lib, f(FAKE, FAKE, None, 1, 64, 8, 0, FAKE, None), B.DH_EINVAL)
    _err(lib, f(FAKE, FAKE, FAKE, 1, 64, 8, 0, None, None), B.DH_EINVAL)
    _err(lib, f(None, FAKE, FAKE, 1, 64, 8, 0, FAKE, None), B.DH_EINVAL)   # coarse needed unless top-k only
    _err(lib, f(FAKE, FAKE, FAKE, 0, 64, 8, 0, FAKE, None), B.DH_EINVAL)
    _err(lib, f(FAKE, FAKE, FAKE, 129, 64, 8, 0, FAKE, None), B.DH_EUNSUP)
    _err(lib, f(FAKE, FAKE, FAKE, 1, 0, 8, 0, FAKE, None), B.DH_ESHAPE)
    _err(lib, f(FAKE, FAKE, FAKE, 1, 64, 0, 0, FAKE, None), B.DH_EUNSUP)
    _err(lib, f(FAKE, FAKE, FAKE, 1, 64, 1025, 0, FAKE, None), B.DH_EUNSUP)


def test_stream_read_validation(lib):
    _err(lib, lib.draft_head_stream_read(None, 4096, FAKE, None), B.DH_EINVAL)
    _err(lib, lib.draft_head_stream_read(FAKE, 4096, None, None), B.DH_EINVAL)
    _err(lib, lib.draft_head_stream_read(MIS, 4096, FAKE, None), B.DH_EINVAL)
    _err(lib, lib.draft_head_stream_read(FAKE, 4100, FAKE, None), B.DH_EINVAL)
    _err(lib, lib.draft_head_stream_read(FAKE, 0, FAKE, None), B.DH_EINVAL)


def test_python_errors_are_value_errors(lib):
    with pytest.raises(ValueError):
        B.draft_head_quantize_pack(np.zeros((2, 300), np.uint16))


def test_forward_validation(lib):
    ok = dict(x=FAKE, M=2, K=512, N=640, t=FAKE, p=FAKE, w=FAKE, ldw=512, kc=8, R=32, cv=FAKE, ci=FAKE,
              ri=FAKE, rv=FAKE, oi=FAKE, ov=FAKE, co=None, s=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.draft_head_forward(a["x"], a["M"], a["K"], a["N"], a["t"], a["p"], a["w"], a["ldw"],
                                      a["kc"], a["R"], a["cv"], a["ci"], a["ri"], a["rv"], a["oi"],
                                      a["ov"], a["co"], FAKE, 1 << 20, a["s"], None, None)
    _err(lib, call(w=None), B.DH_EINVAL)
    _err(lib, call(ri=None), B.DH_EINVAL)
    _err(lib, call(oi=None), B.DH_EINVAL)
    _err(lib, call(ov=None), B.DH_EINVAL)
    _err(lib, call(ldw=256), B.DH_EINVAL)
    _err(lib, call(R=81), B.DH_EUNSUP)          # ncand = 10 blocks * 8
    _err(lib, call(N=64, R=9), B.DH_EUNSUP)     # ncand = 8
    _err(lib, call(R=0), B.DH_EUNSUP)
    _err(lib, call(M=129), B.DH_EUNSUP)
    _err(lib, call(w=MIS), B.DH_EINVAL)


# ------------------------------------------------------------- 4-bit head
@pytest.mark.parametrize("n,k", [(8, 256), (300, 1024), (2048, 5120)])
def test_quantize_pack_int4_matches_oracle(lib, n, k):
    w = workload.gen_weight(n, k, seed=n + k)
    w[3, :128] = w[3, 0]                      # a constant group
    got = B.draft_head_quantize_pack_int4(w)
    want = oracle.quantize_pack_int4(w)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_int4_as_int2_is_the_same_head():
    """The 2K-long 2-bit form's weights, summed over its two halves, are the
    4-bit head's weights exactly (the oracle's definitions of both)."""
    n, k = 200, 1024
    w = workload.gen_weight(n, k, seed=5)
    packed4, S, ZS = B.draft_head_quantize_pack_int4(w)
    packed2, S2, ZS2 = B.draft_head_int4_as_int2(packed4, S, ZS)
    w2 = oracle.effective_weight(packed2, S2, ZS2)
    assert np.array_equal(w2[:, :k] + w2[:, k:], oracle.effective_weight_int4(packed4, S, ZS))


@pytest.mark.parametrize("n,k", [(64, 256), (100, 768), (129, 1536)])
def test_tile_int4_places_the_heads_own_bytes_and_pairs(lib, n, k):
    """draft_head_tile_int4's codes are the 4-bit head's own bytes placed as
    draft_head_tile places a 2-bit head of length 2K (same byte count), and
    its pairs are that form's quarters 0 and 1, the head's own (S, ZS) of the
    groups of nibbles 0 and 1: N K/2 code bytes and N K/128 pairs, the 4-bit
    head's own size."""
    rng = np.random.default_rng(n + k)
    w = oracle.bf16.from_f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    packed4, S, ZS = B.draft_head_quantize_pack_int4(w)
    tiled4, pairs4 = B.draft_head_tile_int4(packed4, S, ZS)
    # draft_head_tile on the same bytes read as a 2-bit head of length 2K, with
    # the 2K-long head's pairs (the head's own in groups < K/128)
    _, S2, ZS2 = B.draft_head_int4_as_int2(packed4, S, ZS)
    tiled2, pairs2 = B.draft_head_tile(packed4, S2, ZS2)
    assert np.array_equal(tiled4, tiled2)
    nblk = (n + 63) // 64
    assert tiled4.size == nblk * 64 * k // 2
    assert pairs4.size == nblk * 64 * (k // 128) and pairs2.size == 2 * pairs4.size
    full = pairs2.reshape(nblk, k // 256, 4, 16, 4)      # [block][byte group][t][c][quarter]
    half = pairs4.reshape(nblk, k // 256, 4, 16, 2)
    assert np.array_equal(half, full[..., :2])
    # quarter q < 2 of byte group G is group q K/256 + G: the code of k = j in
    # the low nibble, of K/2 + j in the high one, with the head's own pairs
    col = np.arange(n)
    b, t, c = col // 64, (col % 64) // 16, col % 16
    for q in range(2):
        for G in range(k // 256):
            got = half[b, G, t, c, q]
            assert np.array_equal(got & 0xFFFF, S[:, q * (k // 256) + G])
            assert np.array_equal(got >> 16, ZS[:, q * (k // 256) + G])


def test_int4_validation(lib):
    p = np.zeros(4096, np.uint8).ctypes.data
    _err(lib, lib.draft_head_quantize_pack_int4(None, 4, 256, 256, p, p, p, 0), B.DH_EINVAL)
    _err(lib, lib.draft_head_quantize_pack_int4(p, 4, 384, 384, p, p, p, 0), B.DH_ESHAPE)
    _err(lib, lib.draft_head_quantize_pack_int4(p, 4, 256, 128, p, p, p, 0), B.DH_EINVAL)
    _err(lib, lib.draft_head_quantize_pack_int4(p, 4, 65536, 65536, p, p, p, 0), B.DH_ESHAPE)
    _err(lib, lib.draft_head_int4_as_int2(p, p, None, 4, 256, p, p, p), B.DH_EINVAL)
    _err(lib, lib.draft_head_int4_as_int2(p, p, p, 0, 256, p, p, p), B.DH_ESHAPE)
    _err(lib, lib.draft_head_tile_int4(p, p, None, 4, 256, p, p), B.DH_EINVAL)
    _err(lib, lib.draft_head_tile_int4(p, p, p, 4, 384, p, p), B.DH_ESHAPE)


def test_int4_device_validation(lib):
    """The 4-bit calls check the head's own K (a multiple of 256) and size the
    workspace for its 2K-long form, before any launch."""
    need = B.draft_head_workspace_bytes(9, 1024)           # M = 9, K = 512: the 2K = 1024 form
    f = lib.draft_head_coarse_int4
    _err(lib, f(FAKE, 1, 384, 64, FAKE, FAKE, 8, FAKE, FAKE, None, FAKE, 512, None), B.DH_ESHAPE)
    _err(lib, f(FAKE, 1, 32768 + 256, 64, FAKE, FAKE, 8, FAKE, FAKE, None, FAKE, 512, None), B.DH_ESHAPE)
    _err(lib, f(FAKE, 9, 512, 64, FAKE, FAKE, 8, FAKE, FAKE, None, FAKE, need - 16, None), B.DH_EINVAL)
    g = lib.draft_head_forward_int4
    _err(lib, g(FAKE, 1, 384, 64, FAKE, FAKE, FAKE, 384, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 512,
                None, None, None), B.DH_ESHAPE)


def test_forward_noalloc_validation(lib):
    """The entry point without a workspace validates like draft_head_forward,
    and rejects a call that needs more than its static scratch, before any
    HIP call."""
    def call(**kw):
        a = dict(x=FAKE, M=2, K=512, N=640, t=FAKE, p=FAKE, w=FAKE, ldw=512, kc=8, R=32, cv=FAKE, ci=FAKE,
                 ri=FAKE, rv=FAKE, oi=FAKE, ov=FAKE)
        a.update(kw)
        return lib.draft_head_forward_noalloc(a["x"], a["M"], a["K"], a["N"], a["t"], a["p"], a["w"], a["ldw"],
                                              a["kc"], a["R"], a["cv"], a["ci"], a["ri"], a["rv"], a["oi"],
                                              a["ov"], None, None, None, None)
    _err(lib, call(x=None), B.DH_EINVAL)
    _err(lib, call(oi=None), B.DH_EINVAL)
    _err(lib, call(M=0), B.DH_EINVAL)
    _err(lib, call(M=129), B.DH_EUNSUP)
    _err(lib, call(K=768), B.DH_ESHAPE)
    _err(lib, call(R=81), B.DH_EUNSUP)
    # the largest K the scratch takes at 128 rows, and the next multiple of 512
    assert B.draft_head_workspace_bytes(128, 18432) <= B.DH_NOALLOC_SCRATCH_BYTES
    assert B.draft_head_workspace_bytes(128, 18944) > B.DH_NOALLOC_SCRATCH_BYTES
    _err(lib, call(M=128, K=18944, ldw=18944), B.DH_EUNSUP)
    assert b"scratch" in lib.draft_head_last_error()
    _err(lib, call(M=72, K=65536, ldw=65536), B.DH_EUNSUP)


def test_forward_row_validation(lib):
    """The call with the caller's bf16 row validates like draft_head_forward,
    plus the row pointer."""
    def call(**kw):
        a = dict(x=FAKE, M=2, K=512, N=640, t=FAKE, p=FAKE, w=FAKE, ldw=512, kc=8, R=32, row=FAKE, ws=FAKE,
                 wsb=B.draft_head_workspace_bytes(2, 512))
        a.update(kw)
        return lib.draft_head_forward_row(a["x"], a["M"], a["K"], a["N"], a["t"], a["p"], a["w"], a["ldw"], a["kc"],
                                          a["R"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["row"], 0, a["ws"], a["wsb"],
                                          None)
    _err(lib, call(row=None), B.DH_EINVAL)
    _err(lib, call(x=None), B.DH_EINVAL)
    _err(lib, call(ws=None), B.DH_EINVAL)
    _err(lib, call(K=768), B.DH_ESHAPE)
    _err(lib, call(R=81), B.DH_EUNSUP)


def test_tile_rejects_pairs_beyond_the_exact_range(lib):
    """Every |S| <= 255 (the fp16 many-row kernel's weights (S/4) v are exact
    there) and every S - ZS a bf16 value (the many-row kernels' zero-point
    weight); other pairs, or non-finite ones, are rejected."""
    n, k = 64, 512
    packed = np.zeros((n, k // 4), np.uint8)
    bits = lambda v: oracle.bf16.from_f32(np.array([v], np.float32))[0]
    cases = ((255.0, 0.0, None), (-255.0, 0.0, None), (256.0, 0.0, "outside"), (float("inf"), 0.0, "outside"),
             (float("nan"), 0.0, "outside"), (1.0, 1.75, None), (1.0, 2.0 ** -10, "not a bf16"),
             (1.0, float("inf"), "not a bf16"), (3.0e-8, 4.0e-8, None))
    for s_val, zs_val, err in cases:
        S = np.full((n, k // 128), bits(1.0), np.uint16)
        ZS = np.full((n, k // 128), bits(1.25), np.uint16)
        S[7, 2], ZS[7, 2] = bits(s_val), bits(zs_val)
        if err is None:
            B.draft_head_tile(packed, S, ZS)
        else:
            with pytest.raises(ValueError, match=err):
                B.draft_head_tile(packed, S, ZS)


def test_quantiser_pairs_meet_the_tile_limits(lib):
    """The quantiser's pairs pass the tile's limits for the workloads' weight
    scales, wide groups and constant groups alike."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((96, 1024)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[4] = 0.37
    w[5, :128] = 20.0 * rng.standard_normal(128)
    w[6, :128] = 1e-30
    packed, S, ZS = B.draft_head_quantize_pack(oracle.bf16.from_f32(w))
    B.draft_head_tile(packed, S, ZS)
