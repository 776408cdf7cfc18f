"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Cases span several 16-row M tiles, several 64-column blocks with a ragged
last block, K with 1..10 byte groups, KCAND 1..64, R 1..256 (including R
above the number of valid candidates), all-zero rows (pure ties), weights the
quantiser reproduces exactly, determinism, and the full per-rank shard
(K=5120, N=124160) at M = 1, 8, 72 plus the recall-stress case, in the same
launch configuration bench.py times.
"""
import sys
import time

import numpy as np
import pytest

import oracle
from bit_quantized_lm_amd import _binding as B
from bit_quantized_lm_amd import workload
from oracle.acceptance import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.load_library()          # fails loudly if the library is not built
    return torch.device("cuda:0")


def _to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def run_gpu(head, x, dev, want_coarse=True):
    m = x.shape[0]
    xt = _to_dev(x, dev)
    coarse = torch.empty((m, head.N), dtype=torch.float32, device=dev) if want_coarse else None
    out = head(xt, coarse_out=coarse)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["coarse"] = coarse.cpu().numpy() if want_coarse else None
    return res


def check_case(dev, m, k, n, kcand, r, seed, x=None, w=None, log=True):
    w = workload.gen_weight(n, k, seed=seed) if w is None else w
    x = workload.gen_x(m, k, seed=seed + 1) if x is None else x
    _log(f"case m={m} k={k} n={n} kcand={kcand} r={r} seed={seed}")
    head = B.DraftHead.from_weight(w, kcand=kcand, R=r, device=dev)
    got = run_gpu(head, x, dev)
    ref = oracle.pipeline(x, w, *oracle.quantize_pack(w), kcand=kcand, r=r)
    stats = compare(ref, got, n, kcand)
    if log:
        _log(f"  ok {stats}")
    return ref, got, stats


CASES = [
    # m, k, n, kcand, r
    (1, 512, 64, 8, 8),
    (3, 1024, 1000, 8, 32),
    (16, 512, 2048, 8, 32),
    (17, 1024, 777, 4, 20),
    (33, 512, 640, 8, 64),
    (72, 1536, 1500, 8, 32),
    (80, 512, 1100, 8, 32),
    (81, 512, 300, 2, 8),
    (128, 1024, 2100, 8, 32),
    (5, 2048, 5000, 1, 1),
    (2, 512, 200, 64, 100),
    (4, 512, 70, 64, 100),     # fewer valid candidates than R: padded rr
    (7, 1536, 3000, 16, 256),
    (1, 5120, 1000, 8, 32),
    # block-maximum rerank: survivors > 64 (LDS sort), kcand * R at the buffer
    # limit, ragged last block with padding slots, 2048 blocks (the limit) and
    # one more block (general path)
    (2, 512, 70000, 8, 100),
    (3, 512, 4000, 64, 16),
    (4, 1024, 5000, 16, 32),
    (2, 512, 131072, 8, 32),
    (8, 512, 131072, 8, 32),   # the one-call path's block-maxima copy full: 8 rows x 2048 blocks
    (17, 512, 5000, 16, 32),   # many rows, lists longer than eight, the block-maximum rerank
    (2, 512, 131100, 8, 32),
    # R > 64 (exact threshold by radix select) in the separate rerank kernel
    (20, 512, 70000, 8, 100),
    # the resident kernel at its largest LDS (x of the longest rows it takes),
    # and the many-row kernel just past it
    (1, 39424, 300, 8, 32),
    (1, 40960, 300, 8, 32),    # one row past the two-row instance's LDS: the one-row instance
    (2, 39424, 300, 8, 32),
    (4, 19456, 300, 8, 32),
    (4, 19968, 300, 8, 32),
    (8, 8704, 500, 8, 32),
    (8, 9216, 500, 8, 32),
    # the many-row kernel's selections: one list per thread (kcand <= 8) and
    # the 16-lane rounds for longer lists, with one and two waves per block
    (48, 1024, 5000, 1, 16),
    (20, 512, 3000, 16, 64),
    (40, 1024, 2000, 12, 32),
    (72, 512, 1000, 64, 100),
    # every row-tile count of the many-row kernel: 9 rows (one tile, just past
    # the resident kernel), 57 and 64 (four tiles, two-group stages)
    (9, 1024, 3000, 8, 32),
    (57, 1536, 2500, 8, 32),
    (64, 512, 700, 8, 32),
]


@pytest.mark.parametrize("m,k,n,kcand,r", CASES)
def test_parity_small(dev, m, k, n, kcand, r):
    check_case(dev, m, k, n, kcand, r, seed=1000 + 7 * m + n)


def test_parity_tiny_config(dev):
    cfg = workload.CONFIGS["tiny"]
    x, w = workload.make_inputs(cfg)
    check_case(dev, cfg.m, cfg.k, cfg.n, cfg.kcand, cfg.rerank, seed=0, x=x, w=w)


def test_all_zero_rows_are_pure_ties(dev, golden):
    fx = golden("all_ties.txt")
    n, k = int(fx["N"][0][0]), int(fx["K"][0][0])
    kc, r = int(fx["KCAND"][0][0]), int(fx["R"][0][0])
    w = workload.gen_weight(n, k, seed=4)
    x = workload.gen_x(3, k, seed=5)
    x[0] = 0
    x[2] = 0
    _, got, _ = check_case(dev, 3, k, n, kc, r, seed=0, x=x, w=w)
    assert [int(v) for v in got["rr_id"][0]] == [int(v) for v in fx["row_top_r"][0]]
    assert int(got["out_id"][0]) == int(fx["argmax"][0][0]) == int(got["out_id"][2])


def test_zero_row_many_survivors(dev):
    """A zero x row ties every candidate: the block-maximum rerank keeps 249
    survivors (blocks 0..31) and must return ids 0-7, 64-71, ... in order."""
    n, k = 5000, 512
    w = workload.gen_weight(n, k, seed=8)
    x = workload.gen_x(2, k, seed=9)
    x[1] = 0
    _, got, _ = check_case(dev, 2, k, n, 8, 32, seed=0, x=x, w=w)
    want = [64 * b + i for b in range(4) for i in range(8)]
    assert [int(v) for v in got["rr_id"][1]] == want
    assert int(got["out_id"][1]) == 0


@pytest.mark.parametrize("m", [40, 72])
def test_many_row_ties(dev, m):
    """The many-row kernel's per-thread lists over exact ties: duplicated head
    rows give bit-identical coarse scores (keys equal above bit 5, so the list
    is rebuilt from full keys and columns; ties go to the lower column), and
    zero x rows tie every column of every block."""
    n, k = 3000, 1024
    w = workload.gen_weight(n, k, seed=4400 + m)
    for b in range(n // 64):
        w[64 * b + 1] = w[64 * b]
        w[64 * b + 7] = w[64 * b + 3]
        w[64 * b + 8] = w[64 * b + 3]
    x = workload.gen_x(m, k, seed=4401 + m)
    x[5] = 0
    x[m - 1] = 0
    _, got, _ = check_case(dev, m, k, n, 8, 32, seed=0, x=x, w=w)
    assert [int(v) for v in got["rr_id"][5][:8]] == [0, 1, 2, 3, 4, 5, 6, 7]


def test_lossless_weights_give_exact_argmax(dev):
    rng = np.random.default_rng(23)
    n, k = 1000, 1024
    codes = rng.integers(0, 4, size=(n, k)).astype(np.int64)
    codes[:, ::128] = 0
    codes[:, 1::128] = 3
    s = 2.0 ** rng.integers(-9, -5, size=(n, k // 128))
    z = rng.integers(0, 4, size=(n, k // 128)).astype(np.float64)
    wf = (codes - np.repeat(z, 128, axis=1)) * np.repeat(s, 128, axis=1)
    w = workload.f32_to_bf16_bits(wf.astype(np.float32))
    x = workload.gen_x(9, k, seed=31)
    ref, got, _ = check_case(dev, 9, k, n, 8, 32, seed=0, x=x, w=w)
    E = oracle.exact_head(x, w).astype(np.float32)
    assert np.array_equal(got["out_id"], np.argmax(E, axis=1))


def test_determinism(dev):
    n, k, m = 3000, 1024, 20
    w = workload.gen_weight(n, k, seed=91)
    x = workload.gen_x(m, k, seed=92)
    head = B.DraftHead.from_weight(w, kcand=8, R=32, device=dev)
    a = run_gpu(head, x, dev)
    b = run_gpu(head, x, dev)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_library_quantizer_matches_oracle_full_shape(full):
    assert full["packed_equal"]


# ------------------------------------------------------------------ full shape
@pytest.fixture(scope="module")
def full(dev):
    cfg = workload.CONFIGS["m72"]
    t0 = time.time()
    _log("full shape: generating W and x")
    x, w = workload.make_inputs(cfg)
    _log(f"full shape: library quantize_pack ({time.time() - t0:.0f}s)")
    packed = B.draft_head_quantize_pack(w)
    _log(f"full shape: oracle quantize_pack ({time.time() - t0:.0f}s)")
    opacked = oracle.quantize_pack(w)
    equal = all(np.array_equal(a, b) for a, b in zip(packed, opacked))
    _log(f"full shape: upload ({time.time() - t0:.0f}s)")
    head = B.DraftHead.from_weight(w, kcand=cfg.kcand, R=cfg.rerank, device=dev, packed=packed)
    _log(f"full shape: oracle coarse for 72 rows ({time.time() - t0:.0f}s)")
    c = oracle.coarse(x, *opacked)
    _log(f"full shape: oracle selection and rerank ({time.time() - t0:.0f}s)")
    cv, ci = oracle.block_topk(c, cfg.kcand)
    rr_id, _ = oracle.row_topr(cv, ci, cfg.rerank)
    e = oracle.rerank_exact(x, w, rr_id)
    out_id, out_val = oracle.final_argmax(rr_id, e)
    ref = {"coarse": c, "cand_val": cv, "cand_id": ci, "rr_id": rr_id, "rr_val": e,
           "out_id": out_id, "out_val": out_val, "tie_rows": oracle.tie_rows(e)}
    _log(f"full shape: ready ({time.time() - t0:.0f}s)")
    return {"x": x, "w": w, "head": head, "ref": ref, "packed_equal": equal, "cfg": cfg}


def _prefix(ref, m):
    return {k: (v[:m] if isinstance(v, np.ndarray) and v.ndim >= 1 else v) for k, v in ref.items()}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("m", [1, 2, 8, 9, 16, 32, 48, 64, 72])
def test_parity_full_shape(dev, full, m):
    """The full shard (K = 5120, N = 124160) at the resident kernel's row
    counts (1, 2, 8) and at every row-tile count of the many-row kernel
    (9 and 16: one tile; 32, 48, 64, 72: two to five), coarse values
    included; the rows are a prefix of the 72 the oracle scored once."""
    cfg = full["cfg"]
    got = run_gpu(full["head"], full["x"][:m], dev)
    stats = compare(_prefix(full["ref"], m), got, cfg.n, cfg.kcand)
    E = None
    _log(f"full shape m={m}: {stats}")
    if m == 72:
        E = oracle.exact_head(full["x"], full["w"])
        agree = int(np.sum(got["out_id"] == np.argmax(E, axis=1)))
        _log(f"full shape m=72: argmax agreement with the exact bf16 head {agree}/72 (reported)")
        # a top-16 caller of the top-k-only row draws from the R reranked tokens only
        top = np.argsort(-got["rr_val"], axis=1, kind="stable")[:, :16]
        mine = np.take_along_axis(got["rr_id"], top, axis=1)
        exact16 = np.argsort(-E, axis=1, kind="stable")[:, :16]
        overlap = np.mean([len(set(mine[i]) & set(exact16[i])) / 16 for i in range(72)])
        _log(f"full shape m=72: top-16 of the top-k-only row vs the exact head's top-16: "
             f"{overlap:.3f} overlap (reported)")


@pytest.mark.timeout(900)
def test_recall_stress_full_shape(dev, full):
    """Planted same-block near-ties: parity at KCAND = 8 and 1; misses reported."""
    cfg = workload.CONFIGS["recall"]
    x = full["x"][:cfg.m]
    _log("recall: planting")
    w, pairs = workload.plant_recall_pairs(x, full["w"], target=12.0, gap=0.01)
    packed = B.draft_head_quantize_pack(w)
    opacked = oracle.quantize_pack(w)
    assert all(np.array_equal(a, b) for a, b in zip(packed, opacked))
    c = oracle.coarse(x, *opacked)
    winners = np.array([p[0] for p in pairs])
    misses = {}
    for kc in (8, 1):
        head = B.DraftHead.from_weight(w, kcand=kc, R=32, device=dev, packed=packed)
        got = run_gpu(head, x, dev, want_coarse=False)
        cv, ci = oracle.block_topk(c, kc)
        rr_id, _ = oracle.row_topr(cv, ci, 32)
        e = oracle.rerank_exact(x, w, rr_id)
        out_id, out_val = oracle.final_argmax(rr_id, e)
        ref = {"coarse": c, "cand_val": cv, "cand_id": ci, "rr_id": rr_id, "rr_val": e,
               "out_id": out_id, "out_val": out_val, "tie_rows": oracle.tie_rows(e)}
        compare(ref, got, cfg.n, kc, check_coarse=False)
        misses[kc] = int(np.sum(got["out_id"] != winners))
        del head
    _log(f"recall stress: argmax misses vs planted winner: KCAND=8 {misses[8]}/32, KCAND=1 {misses[1]}/32")
    assert misses[8] == 0


@pytest.mark.parametrize("n,m", [(3000, 5), (20000, 1), (70000, 8), (20000, 20)])
def test_forward_matches_staged_calls(dev, n, m):
    """The one-call entry point (rerank and argmax in one kernel) equals the
    three separate calls, and sets the coarse kernel's timing events."""
    k, kc, r = 1024, 8, 32
    w = workload.gen_weight(n, k, seed=93)
    x = _to_dev(workload.gen_x(m, k, seed=94), dev)
    head = B.DraftHead.from_weight(w, kcand=kc, R=r, device=dev)
    a = head.staged(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    b = head(x, coarse_events=(e0, e1))
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    assert e0.elapsed_time(e1) > 0


def test_workspace_reuse_leaves_counters_zero(dev):
    """One workspace serves calls of several row counts in a row (resident
    and many-row coarse kernels); each result equals a call with a fresh
    workspace, and the per-row hand-off words of the rerank end at zero."""
    n, k = 20000, 1024
    w = workload.gen_weight(n, k, seed=95)
    x = _to_dev(workload.gen_x(20, k, seed=96), dev)
    head = B.DraftHead.from_weight(w, kcand=8, R=32, device=dev)
    ws = B.workspace_for(20, k, dev)
    for m in (1, 8, 2, 20, 1, 8):
        got = head(x[:m], workspace=ws)
        want = head(x[:m])
        torch.cuda.synchronize()
        for key in want:
            assert torch.equal(got[key], want[key]), (m, key)
        assert int(torch.count_nonzero(ws[:1024])) == 0, m


@pytest.mark.parametrize("words", [4, 1000, 2048 * 4 * 3 + 4 * 5, (3 << 20) + 12])
def test_stream_read_folds_every_word(dev, words):
    """The read-rate reference reads every word once: each workgroup's XOR
    fold equals the fold of its span, computed on the host."""
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    out = B.draft_head_stream_read(buf).cpu().numpy().view(np.uint32)
    n16 = words // 4
    per = -(-n16 // B.DH_READ_BLOCKS)
    want = np.zeros(B.DH_READ_BLOCKS, np.uint32)
    for b in range(B.DH_READ_BLOCKS):
        lo, hi = b * per * 4, min(n16, (b + 1) * per) * 4
        if lo < hi:
            want[b] = np.bitwise_xor.reduce(host[lo:hi])
    assert np.array_equal(out, want)


@pytest.mark.parametrize("m,n,r", [(1, 1, 1), (1, 4095, 32), (2, 4096, 32), (3, 4097, 100),
                                   (4, 9000, 1024), (1, 124160, 32)])
@pytest.mark.parametrize("topk_only", [False, True])
def test_logits_row_bit_exact(dev, m, n, r, topk_only):
    """The row handed to the caller, on seeded inputs: bit-exact against the oracle."""
    rng = np.random.default_rng(1000 * m + n + r)
    coarse = (rng.standard_normal((m, n)) * 4).astype(np.float32)
    rr_id = np.stack([rng.choice(n, size=r, replace=False) for _ in range(m)]).astype(np.int32)
    if r > 1:
        rr_id[-1, r // 2:] = -1          # a padded row
    rr_val = (rng.standard_normal((m, r)) * 4).astype(np.float32)
    want = oracle.logits_row(rr_id, rr_val, n, coarse_f32=coarse, topk_only=topk_only)
    _log(f"logits_row m={m} n={n} r={r} topk_only={topk_only}")
    got = B.draft_head_logits_row(torch.from_numpy(rr_id).to(dev), torch.from_numpy(rr_val).to(dev), n,
                                  coarse=None if topk_only else torch.from_numpy(coarse).to(dev),
                                  topk_only=topk_only)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("m,k,n,kc,r", [(1, 1024, 5000, 8, 32), (9, 512, 3000, 8, 32), (3, 512, 200, 8, 32),
                                         (20, 512, 70000, 8, 100), (72, 1024, 2100, 8, 32)])
@pytest.mark.parametrize("topk_only", [False, True])
def test_forward_row_equals_the_row_of_its_own_call(dev, m, k, n, kc, r, topk_only):
    """The row built inside the call (bf16 from the coarse epilogue, exact
    values scattered by the rerank, or by its own small kernel on the general
    rerank path: n = 200 has fewer blocks than R, R = 100 exceeds the
    block-maximum rerank's limit) equals draft_head_logits_row applied to the
    same call's fp32 coarse row and reranked values, bit for bit; the other
    outputs equal the plain call's."""
    w = workload.gen_weight(n, k, seed=4600 + n)
    x = _to_dev(workload.gen_x(m, k, seed=4601 + n), dev)
    head = B.DraftHead.from_weight(w, kcand=kc, R=r, device=dev)
    got = head.logits_row(x, topk_only=topk_only)
    want = head.logits_row_staged(x, topk_only=topk_only)
    torch.cuda.synchronize()
    assert torch.equal(got["row"], want["row"])
    for key in ("cand_val", "cand_id", "rr_id", "rr_val", "out_id", "out_val"):
        assert torch.equal(got[key], want[key]), key


@pytest.mark.timeout(900)
@pytest.mark.parametrize("topk_only", [False, True])
def test_forward_row_full_shape(dev, full, topk_only):
    """The full shard at M = 1, 8, 72: the row built inside the call equals the
    staged row of the same call, and holds the oracle's values (exact values at
    the reranked ids, the coarse values or -inf elsewhere) within the value
    tolerance plus one bf16 step."""
    cfg = full["cfg"]
    head = full["head"]
    for m in (1, 8, 72):
        x = _to_dev(full["x"][:m], dev)
        got = head.logits_row(x, topk_only=topk_only)
        want = head.logits_row_staged(x, topk_only=topk_only)
        torch.cuda.synchronize()
        assert torch.equal(got["row"], want["row"]), m
        ref = _prefix(full["ref"], m)
        row = oracle.bf16.to_f64(got["row"].cpu().numpy().view(np.uint16))
        exp = oracle.bf16.to_f64(oracle.logits_row(ref["rr_id"], ref["rr_val"], cfg.n,
                                                    coarse_f32=ref["coarse"].astype(np.float32),
                                                    topk_only=topk_only))
        fin = np.isfinite(exp)
        if np.array_equal(got["rr_id"].cpu().numpy(), ref["rr_id"]):   # else a counted near-tie list
            assert np.array_equal(np.isfinite(row), fin), m
        rms = np.sqrt(np.mean(ref["coarse"] ** 2, axis=1))[:, None]
        lim = 2e-3 * np.abs(exp) + 2e-3 * rms + 2.0 ** -7 * np.abs(exp)
        both = fin & np.isfinite(row)
        assert np.all(np.abs(row - exp)[both] <= np.broadcast_to(lim, row.shape)[both]), m


@pytest.mark.parametrize("topk_only", [False, True])
def test_logits_row_end_to_end(dev, topk_only):
    """One call plus the row, against the oracle's own pipeline: the reranked
    ids hold their exact values, every other entry the coarse value (or -inf),
    within the value tolerance plus one bf16 step."""
    m, k, n = 3, 1024, 5000
    w = workload.gen_weight(n, k, seed=97)
    x = workload.gen_x(m, k, seed=98)
    head = B.DraftHead.from_weight(w, kcand=8, R=32, device=dev)
    got = head.logits_row(_to_dev(x, dev), topk_only=topk_only)
    torch.cuda.synchronize()
    ref = oracle.pipeline(x, w, *oracle.quantize_pack(w), kcand=8, r=32)
    assert np.array_equal(got["rr_id"].cpu().numpy(), ref["rr_id"])   # no near-ties at this seed
    row = got["row"].cpu().numpy().view(np.uint16)
    want = oracle.logits_row(ref["rr_id"], ref["rr_val"], n, coarse_f32=ref["coarse"].astype(np.float32),
                             topk_only=topk_only)
    gv = oracle.bf16.to_f64(row)
    wv = oracle.bf16.to_f64(want)
    fin = np.isfinite(wv)
    assert np.array_equal(np.isfinite(gv), fin)
    rms = np.sqrt(np.mean(ref["coarse"] ** 2, axis=1))[:, None]
    lim = 2e-3 * np.abs(wv) + 2e-3 * rms + 2.0 ** -7 * np.abs(wv)
    assert np.all(np.abs(gv - wv)[fin] <= lim[fin])


def _library_packed(w):
    """The library's quantiser output, checked byte for byte against the oracle's."""
    packed = B.draft_head_quantize_pack(w)
    assert all(np.array_equal(a, b) for a, b in zip(packed, oracle.quantize_pack(w)))
    return packed


# ------------------------------------------------------- e4m3 rerank source
def _e4m3_ref(x, w, packed, w8, wscale, kcand, r):
    """The oracle's pipeline with the rerank read from the e4m3 rows."""
    ref = oracle.pipeline(x, w, *packed, kcand=kcand, r=r)
    e = oracle.rerank_exact_e4m3(x, w8, wscale, ref["rr_id"])
    ref["rr_val"] = e
    ref["out_id"], ref["out_val"] = oracle.final_argmax(ref["rr_id"], e)
    ref["tie_rows"] = oracle.tie_rows(e)
    return ref


def _e4m3_head(w, kcand, r, dev, packed=None):
    w8, wscale = workload.e4m3_head(w)
    head = B.DraftHead.from_weight(w, kcand=kcand, R=r, device=dev, packed=packed)
    head.w = torch.from_numpy(w8).to(dev)
    head.wscale = torch.from_numpy(wscale).to(dev)
    return head, w8, wscale


@pytest.mark.parametrize("m,k,n,kcand,r", [(3, 1024, 5000, 8, 32), (1, 512, 200, 64, 100), (17, 1024, 777, 4, 20),
                                           (8, 5120, 20000, 8, 32), (20, 512, 70000, 8, 100)])
def test_e4m3_rerank_parity(dev, m, k, n, kcand, r):
    w = workload.gen_weight(n, k, seed=2000 + n)
    x = workload.gen_x(m, k, seed=2001 + n)
    _log(f"e4m3 case m={m} k={k} n={n} kcand={kcand} r={r}")
    packed = _library_packed(w)
    head, w8, wscale = _e4m3_head(w, kcand, r, dev, packed=packed)
    got = run_gpu(head, x, dev)
    stats = compare(_e4m3_ref(x, w, packed, w8, wscale, kcand, r), got, n, kcand)
    _log(f"  ok {stats}")


def test_e4m3_rerank_edge_codes(dev):
    """e4m3 rows holding the codes 0x7F / 0xFF (the page's decode reads them as
    +-480; the e4m3 format reserves them for NaN) in every head row, 2 % of
    each row's bytes, so every reranked row carries some."""
    m, k, n, kcand, r = 4, 1024, 5000, 8, 32
    w = workload.gen_weight(n, k, seed=2100)
    x = workload.gen_x(m, k, seed=2101)
    packed = _library_packed(w)
    w8, wscale = workload.e4m3_head(w)
    w8 = workload.plant_codes(w8, range(n), [0x7F, 0xFF], frac=0.02, seed=2102)
    assert np.any(w8 == 0x7F) and np.any(w8 == 0xFF)
    head = B.DraftHead.from_weight(w, kcand=kcand, R=r, device=dev, packed=packed)
    head.w = torch.from_numpy(w8).to(dev)
    head.wscale = torch.from_numpy(wscale).to(dev)
    got = run_gpu(head, x, dev)
    ref = _e4m3_ref(x, w, packed, w8, wscale, kcand, r)
    assert np.all(np.isfinite(ref["rr_val"]))
    stats = compare(ref, got, n, kcand)
    _log(f"e4m3 edge codes: {stats}")


def test_e4m3_forward_matches_staged_calls(dev):
    n, k, m = 20000, 1024, 5
    w = workload.gen_weight(n, k, seed=99)
    head, _, _ = _e4m3_head(w, 8, 32, dev)
    x = _to_dev(workload.gen_x(m, k, seed=100), dev)
    a = head.staged(x)
    b = head(x)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.timeout(900)
def test_e4m3_rerank_full_shape(dev, full):
    """The per-rank shard with an e4m3 head: parity at M = 1, 8, 72 and the
    argmax agreement with the exact bf16 head (reported)."""
    cfg = full["cfg"]
    w8, wscale = workload.e4m3_head(full["w"])
    head = full["head"]
    h8 = B.DraftHead(head.tiled, head.pairs, torch.from_numpy(w8).to(dev), cfg.n, cfg.k, cfg.kcand, cfg.rerank,
                     wscale=torch.from_numpy(wscale).to(dev))
    for m in (1, 8, 72):
        x = full["x"][:m]
        got = run_gpu(h8, x, dev, want_coarse=False)
        ref = _prefix(full["ref"], m)
        e = oracle.rerank_exact_e4m3(x, w8, wscale, ref["rr_id"])
        ref = dict(ref, rr_val=e, tie_rows=oracle.tie_rows(e))
        ref["out_id"], ref["out_val"] = oracle.final_argmax(ref["rr_id"], e)
        stats = compare(ref, got, cfg.n, cfg.kcand, check_coarse=False)
        _log(f"e4m3 full shape m={m}: {stats}")
    E = oracle.exact_head(full["x"], full["w"])
    agree = int(np.sum(got["out_id"] == np.argmax(E, axis=1)))
    _log(f"e4m3 full shape m=72: argmax agreement with the exact bf16 head {agree}/72 (reported)")


# ------------------------------------------------------------- graph capture
@pytest.mark.parametrize("m", [1, 4, 20])
def test_forward_graph_replay(dev, m):
    """The one-call forward captured in a HIP graph (torch.cuda.CUDAGraph):
    every replay, with eager calls and synchronisations between replays, gives
    the eager call's outputs on the same input bit for bit (the library
    records no memset; its counters are cleared by its own kernels)."""
    n, k = 20000, 1024
    w = workload.gen_weight(n, k, seed=105)
    head = B.DraftHead.from_weight(w, kcand=8, R=32, device=dev)
    xs = [_to_dev(workload.gen_x(m, k, seed=106 + i), dev) for i in range(3)]
    x_static = torch.empty_like(xs[0])
    out = B.forward_buffers(m, n, 8, 32, dev)
    ws = B.workspace_for(m, k, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        x_static.copy_(xs[0])
        head(x_static, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        head(x_static, out=out, workspace=ws)
    torch.cuda.synchronize()
    _log(f"graph replay m={m}")
    for rep in range(3):
        for i, x in enumerate(xs):
            eager = head(x)
            torch.cuda.synchronize()
            x_static.copy_(x)
            g.replay()
            torch.cuda.synchronize()
            for key in ("cand_val", "cand_id", "rr_id", "rr_val", "out_id", "out_val"):
                assert torch.equal(out[key], eager[key]), (rep, i, key)


# ------------------------------------------------------ NVFP4 rerank source
def _nvfp4_ref(x, w, packed, w4, bs, g, kcand, r):
    """The oracle's pipeline with the rerank read from the NVFP4 rows."""
    ref = oracle.pipeline(x, w, *packed, kcand=kcand, r=r)
    e = oracle.rerank_exact_nvfp4(x, w4, bs, g, ref["rr_id"])
    ref["rr_val"] = e
    ref["out_id"], ref["out_val"] = oracle.final_argmax(ref["rr_id"], e)
    ref["tie_rows"] = oracle.tie_rows(e)
    return ref


def _nvfp4_dev(w4, bs, g, dev):
    return (torch.from_numpy(w4).to(dev), torch.from_numpy(bs).to(dev),
            torch.tensor([g], dtype=torch.float32, device=dev))


def _nvfp4_head(w, kcand, r, dev, packed=None):
    w4, bs, g = workload.nvfp4_head(w)
    head = B.DraftHead.from_weight(w, kcand=kcand, R=r, device=dev, packed=packed)
    head.w, head.bscale, head.gscale = _nvfp4_dev(w4, bs, g, dev)
    return head, w4, bs, g


@pytest.mark.parametrize("m,k,n,kcand,r", [(3, 1024, 5000, 8, 32), (1, 512, 200, 64, 100), (17, 1536, 777, 4, 20),
                                           (8, 5120, 20000, 8, 32), (20, 512, 70000, 8, 100)])
def test_nvfp4_rerank_parity(dev, m, k, n, kcand, r):
    w = workload.gen_weight(n, k, seed=4000 + n)
    x = workload.gen_x(m, k, seed=4001 + n)
    _log(f"nvfp4 case m={m} k={k} n={n} kcand={kcand} r={r}")
    packed = _library_packed(w)
    head, w4, bs, g = _nvfp4_head(w, kcand, r, dev, packed=packed)
    got = run_gpu(head, x, dev)
    stats = compare(_nvfp4_ref(x, w, packed, w4, bs, g, kcand, r), got, n, kcand)
    _log(f"  ok {stats}")


@pytest.mark.parametrize("all_nan", [False, True])
def test_nvfp4_nan_block_scale(dev, all_nan):
    """NVFP4 rows with the block scale 0x7F (NaN through the e4m3 format):
    the exact value of every such candidate is NaN on both sides, and a NaN
    value never wins the final argmax (a number, -inf included, ranks above
    it).  The rows of every row's oracle winner get a NaN block scale, so the
    token must move to the next candidate; with all_nan, every block scale of
    every head row is NaN and each row returns its lowest reranked id with
    value NaN."""
    m, k, n, kcand, r = 5, 1024, 5000, 8, 32
    w = workload.gen_weight(n, k, seed=4200)
    x = workload.gen_x(m, k, seed=4201)
    packed = _library_packed(w)
    w4, bs, g = workload.nvfp4_head(w)
    if all_nan:
        bs = np.full_like(bs, 0x7F)
    else:
        first = oracle.pipeline(x, w, *packed, kcand=kcand, r=r)
        bs = workload.plant_codes(bs, sorted({int(v) for v in first["out_id"]}), [0x7F], frac=0.05, seed=4202)
    head = B.DraftHead.from_weight(w, kcand=kcand, R=r, device=dev, packed=packed)
    head.w, head.bscale, head.gscale = _nvfp4_dev(w4, bs, g, dev)
    got = run_gpu(head, x, dev)
    ref = _nvfp4_ref(x, w, packed, w4, bs, g, kcand, r)
    assert np.any(np.isnan(ref["rr_val"]))
    if all_nan:
        assert np.array_equal(ref["out_id"], ref["rr_id"].min(axis=1, where=ref["rr_id"] >= 0, initial=n))
    else:
        assert not np.any(np.isin(ref["out_id"], first["out_id"]))
    stats = compare(ref, got, n, kcand)
    _log(f"nvfp4 NaN block scales (all={all_nan}): {stats}")


def test_nvfp4_forward_matches_staged_calls(dev):
    n, k, m = 20000, 1024, 5
    w = workload.gen_weight(n, k, seed=103)
    head, _, _, _ = _nvfp4_head(w, 8, 32, dev)
    x = _to_dev(workload.gen_x(m, k, seed=104), dev)
    a = head.staged(x)
    b = head(x)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_rerank_degenerate_candidates(dev):
    """The block-maximum rerank on candidate arrays no coarse call writes:
    every slot the same (value 0, id 0), so the survivors share one key and
    ranks 1.. stay empty; and every slot padding (-inf, -1), so no block has
    a maximum.  Empty ranks come back as (-1, -inf) and read no row."""
    m, k, n, kcand, r = 3, 1024, 20000, 8, 32
    w = workload.gen_weight(n, k, seed=4300)
    x = workload.gen_x(m, k, seed=4301)
    nblk = (n + 63) // 64
    wt, xt = _to_dev(w, dev), _to_dev(x, dev)
    exact0 = oracle.bf16.to_f64(x) @ oracle.bf16.to_f64(w[0])
    for name, val, idv in (("duplicates", 0.0, 0), ("padding", -np.inf, -1)):
        _log(f"degenerate candidates: {name}")
        cv = torch.full((m, nblk * kcand), val, dtype=torch.float32, device=dev)
        ci = torch.full((m, nblk * kcand), idv, dtype=torch.int32, device=dev)
        got_id, got_val = B.draft_head_rerank(xt, wt, cv, ci, R=r)
        out_id, out_val = B.draft_head_argmax(got_id, got_val)
        torch.cuda.synchronize()
        gi, gv = got_id.cpu().numpy(), got_val.cpu().numpy().astype(np.float64)
        if name == "duplicates":
            assert np.all(gi[:, 0] == 0) and np.all(gi[:, 1:] == -1)
            assert np.all(np.abs(gv[:, 0] - exact0) <= 2e-3 * np.abs(exact0) + 1e-5)
            assert np.all(gv[:, 1:] == -np.inf)
            assert np.array_equal(out_id.cpu().numpy(), np.zeros(m, dtype=np.int32))
        else:
            assert np.all(gi == -1) and np.all(gv == -np.inf)
            assert np.all(out_id.cpu().numpy() == -1)


@pytest.mark.parametrize("k,n,r", [(256, 3000, 32), (768, 3000, 32), (2304, 200, 16)])
def test_nvfp4_rerank_alone(dev, k, n, r):
    """The NVFP4 rerank by itself at row lengths the 2-bit coarse pass does not
    take (K % 512 != 0, last 2048-element pass partly empty), on candidate
    lists with the coarse kernel's block structure drawn at random; n = 200
    (fewer blocks than R) takes the general rerank kernel."""
    m, kcand = 4, 8
    rng = np.random.default_rng(k + n)
    w = workload.gen_weight(n, k, seed=4100 + k)
    x = workload.gen_x(m, k, seed=4101 + k)
    w4, bs, g = workload.nvfp4_head(w)
    nblk = (n + 63) // 64
    cv = np.full((m, nblk * kcand), -np.inf, dtype=np.float32)
    ci = np.full((m, nblk * kcand), -1, dtype=np.int32)
    for row in range(m):
        for b in range(nblk):
            cols = np.arange(64 * b, min(64 * b + 64, n))
            pick = rng.choice(cols, size=min(kcand, len(cols)), replace=False)
            vals = np.sort(rng.standard_normal(len(pick)).astype(np.float32))[::-1]
            order = np.lexsort((pick, -vals.astype(np.float64)))
            cv[row, b * kcand:b * kcand + len(pick)] = vals[order]
            ci[row, b * kcand:b * kcand + len(pick)] = pick[order]
    _log(f"nvfp4 rerank alone k={k} n={n} r={r}")
    rr_id, _ = oracle.row_topr(cv, ci, r)
    e = oracle.rerank_exact_nvfp4(x, w4, bs, g, rr_id)
    t_w4, t_bs, t_g = _nvfp4_dev(w4, bs, g, dev)
    got_id, got_val = B.draft_head_rerank_nvfp4(_to_dev(x, dev), t_w4, t_bs, t_g, torch.from_numpy(cv).to(dev),
                                                torch.from_numpy(ci).to(dev), R=r, N=n)
    torch.cuda.synchronize()
    assert np.array_equal(got_id.cpu().numpy(), rr_id)
    gv = got_val.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gv - e) <= 2e-3 * np.abs(e) + 1e-5)


@pytest.mark.timeout(900)
def test_nvfp4_rerank_full_shape(dev, full):
    """The per-rank shard with an NVFP4 rerank source: parity at M = 1, 8, 72
    and the argmax agreement with the exact bf16 head (reported)."""
    cfg = full["cfg"]
    _log("nvfp4 full shape: synthetic NVFP4 head")
    w4, bs, g = workload.nvfp4_head(full["w"])
    head = full["head"]
    t_w4, t_bs, t_g = _nvfp4_dev(w4, bs, g, dev)
    h4 = B.DraftHead(head.tiled, head.pairs, t_w4, cfg.n, cfg.k, cfg.kcand, cfg.rerank, bscale=t_bs, gscale=t_g)
    for m in (1, 8, 72):
        x = full["x"][:m]
        got = run_gpu(h4, x, dev, want_coarse=False)
        ref = _prefix(full["ref"], m)
        e = oracle.rerank_exact_nvfp4(x, w4, bs, g, ref["rr_id"])
        ref = dict(ref, rr_val=e, tie_rows=oracle.tie_rows(e))
        ref["out_id"], ref["out_val"] = oracle.final_argmax(ref["rr_id"], e)
        stats = compare(ref, got, cfg.n, cfg.kcand, check_coarse=False)
        _log(f"nvfp4 full shape m={m}: {stats}")
    E = oracle.exact_head(full["x"], full["w"])
    agree = int(np.sum(got["out_id"] == np.argmax(E, axis=1)))
    _log(f"nvfp4 full shape m=72: argmax agreement with the exact bf16 head {agree}/72 (reported)")


# ------------------------------------------------------------ 4-bit head
@pytest.mark.parametrize("m,k,n,kcand,r", [(1, 256, 3000, 1, 32), (3, 768, 5000, 1, 32), (8, 1024, 20000, 8, 32),
                                           (20, 512, 3000, 1, 16), (5, 2048, 5000, 4, 32), (72, 1024, 2100, 1, 32),
                                           # every row-tile count of the many-row kernel's 4-bit form
                                           (9, 1024, 3000, 1, 32), (40, 512, 2000, 1, 32), (57, 1024, 2500, 4, 32),
                                           (64, 2560, 2600, 1, 32),
                                           # one byte group (K = 256) with two groups a byte group: three,
                                           # four and five row tiles (one stage a byte group at four and five)
                                           (33, 256, 1500, 1, 16), (49, 256, 1500, 2, 32), (80, 256, 1100, 1, 16),
                                           # two byte groups at five row tiles, ragged N
                                           (75, 512, 1333, 8, 32)])
def test_int4_parity(dev, m, k, n, kcand, r):
    """The 4-bit head (its own bytes, draft_head_tile_int4) against the
    oracle's own 4-bit definition."""
    w = workload.gen_weight(n, k, seed=3000 + n)
    x = workload.gen_x(m, k, seed=3001 + n)
    _log(f"int4 case m={m} k={k} n={n} kcand={kcand} r={r}")
    packed4 = B.draft_head_quantize_pack_int4(w)
    opacked4 = oracle.quantize_pack_int4(w)
    assert all(np.array_equal(a, b) for a, b in zip(packed4, opacked4))
    head = B.DraftHead.from_weight(w, kcand=kcand, R=r, device=dev, packed=packed4, bits=4)
    got = run_gpu(head, x, dev)
    stats = compare(oracle.pipeline(x, w, *opacked4, kcand=kcand, r=r, bits=4), got, n, kcand)
    _log(f"  ok {stats}")


def test_int4_forward_matches_staged_calls(dev):
    n, k, m = 20000, 1024, 5
    w = workload.gen_weight(n, k, seed=101)
    head = B.DraftHead.from_weight(w, kcand=1, R=32, device=dev, bits=4)
    x = _to_dev(workload.gen_x(m, k, seed=102), dev)
    a = head.staged(x)
    b = head(x)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.timeout(900)
def test_int4_full_shape(dev, full):
    """The per-rank shard as a 4-bit head at KCAND = 1 (the page's 4-bit
    configuration): the library quantiser against the oracle's, parity at
    M = 1, 8, 72, and the agreement with the exact bf16 head (reported)."""
    cfg = full["cfg"]
    x, w = full["x"], full["w"]
    _log("int4 full shape: quantize_pack_int4 (library and oracle)")
    packed4 = B.draft_head_quantize_pack_int4(w)
    opacked4 = oracle.quantize_pack_int4(w)
    assert all(np.array_equal(a, b) for a, b in zip(packed4, opacked4))
    head = B.DraftHead.from_weight(w, kcand=1, R=cfg.rerank, device=dev, packed=packed4, bits=4)
    _log("int4 full shape: oracle coarse for 72 rows")
    c = oracle.coarse_int4(x, *opacked4)
    cv, ci = oracle.block_topk(c, 1)
    rr_id, _ = oracle.row_topr(cv, ci, cfg.rerank)
    e = oracle.rerank_exact(x, w, rr_id)
    out_id, out_val = oracle.final_argmax(rr_id, e)
    ref = {"coarse": c, "cand_val": cv, "cand_id": ci, "rr_id": rr_id, "rr_val": e, "out_id": out_id,
           "out_val": out_val, "tie_rows": oracle.tie_rows(e)}
    for m in (1, 8, 72):
        got = run_gpu(head, x[:m], dev)
        stats = compare(_prefix(ref, m), got, cfg.n, 1)
        _log(f"int4 full shape m={m} kcand=1: {stats}")
    E = oracle.exact_head(x, w)
    agree = int(np.sum(got["out_id"] == np.argmax(E, axis=1)))
    _log(f"int4 full shape m=72 kcand=1: argmax agreement with the exact bf16 head {agree}/72 (reported)")


@pytest.mark.timeout(900)
def test_int4_recall_stress_full_shape(dev, full):
    """Planted same-block near-ties with a 4-bit head: parity at KCAND = 1, misses reported."""
    cfg = workload.CONFIGS["recall"]
    x = full["x"][:cfg.m]
    w, pairs = workload.plant_recall_pairs(x, full["w"], target=12.0, gap=0.01)
    packed4 = B.draft_head_quantize_pack_int4(w)
    opacked4 = oracle.quantize_pack_int4(w)
    assert all(np.array_equal(a, b) for a, b in zip(packed4, opacked4))
    head = B.DraftHead.from_weight(w, kcand=1, R=32, device=dev, packed=packed4, bits=4)
    got = run_gpu(head, x, dev, want_coarse=False)
    c = oracle.coarse_int4(x, *opacked4)
    cv, ci = oracle.block_topk(c, 1)
    rr_id, _ = oracle.row_topr(cv, ci, 32)
    e = oracle.rerank_exact(x, w, rr_id)
    out_id, out_val = oracle.final_argmax(rr_id, e)
    ref = {"coarse": c, "cand_val": cv, "cand_id": ci, "rr_id": rr_id, "rr_val": e, "out_id": out_id,
           "out_val": out_val, "tie_rows": oracle.tie_rows(e)}
    compare(ref, got, cfg.n, 1, check_coarse=False)
    winners = np.array([p[0] for p in pairs])
    _log(f"int4 recall stress: argmax misses vs planted winner at KCAND=1: "
         f"{int(np.sum(got['out_id'] != winners))}/32 (reported)")
