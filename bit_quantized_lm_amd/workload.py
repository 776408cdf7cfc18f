"""Seeded synthetic inputs for the 2-bit draft head.

This module only draws random numbers and rounds them to bf16 storage. It
holds none of the head's arithmetic (no quantisation, packing, scoring or
selection), so the HIP path and the CPU oracle can both be fed from it.

The workload it imitates is the one the radiance_drafthead.py page describes
in its module docstring: per tensor-parallel rank the draft head is
x[M, 5120] @ W[5120, 124160], run once per draft slot, with M from 1 to 72.
The page measured on hidden states captured from a live serve, which are not
available; the stand-ins are:

* W: bf16, N(0, 0.02), generated in 8192-row chunks in row order.
* x: bf16, N(0, 1), with 1% of the hidden channels (a fixed set shared by all
  rows) scaled by 8 to imitate activation outliers.  x is always generated as
  72 rows and the first M are used, so M = 1, 8 and 72 nest.

All arrays are returned as raw bf16 bit patterns (numpy uint16).
"""
from __future__ import annotations

import dataclasses

import numpy as np

# Shapes of one rank's vocabulary shard of the head (module docstring of the
# radiance_drafthead.py page).
HIDDEN = 5120
VOCAB_SHARD = 124160
X_ROWS_GENERATED = 72

SEED_W = 1
SEED_X = 2
SEED_OUTLIERS = 3
SEED_PLANT = 4


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = np.isnan(a)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gen_weight(n: int, k: int, seed: int = SEED_W, std: float = 0.02,
               chunk: int = 8192) -> np.ndarray:
    """bf16 weight [n][k] (row n = vocabulary token n), N(0, std)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((n, k), dtype=np.uint16)
    for i in range(0, n, chunk):
        j = min(i + chunk, n)
        blk = rng.standard_normal((j - i, k), dtype=np.float32)
        blk *= np.float32(std)
        out[i:j] = f32_to_bf16_bits(blk)
    return out


def _e4m3_round(v: np.ndarray):
    """Nearest e4m3 grid value to v (float64), ties to the even code, within
    +-448: (value, code uint8)."""
    a = np.minimum(np.abs(v), 448.0)
    # step of the e4m3 grid around a: 2^(e-3) for a in [2^e, 2^(e+1)), e >= -6; 2^-9 below 2^-6
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = np.exp2(e - 3)
    q = np.minimum(np.rint(a / step) * step, 448.0)          # ties to even step count = even code
    sub = q < 2.0 ** -6
    eq = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    code = np.where(sub, np.rint(q / 2.0 ** -9), (eq + 7) * 8 + np.rint(q / np.exp2(eq) * 8 - 8))
    code = (code.astype(np.int64) | np.where(v < 0, 128, 0)).astype(np.uint8)
    return np.where(v < 0, -q, q), code


def e4m3_head(w_bits: np.ndarray):
    """A synthetic e4m3 head (stand-in for a checkpoint's per-channel FP8
    lm_head): per row, scale = max |w| / 448 (float32) and codes = w / scale
    rounded to the nearest e4m3 value (ties to the even code), within +-448.
    Returns (codes uint8 [N][K], scale float32 [N])."""
    w = bf16_bits_to_f32(w_bits)
    amax = np.abs(w).max(axis=1).astype(np.float64)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    out = np.empty(w.shape, dtype=np.uint8)
    for i in range(0, w.shape[0], 512):
        v = w[i:i + 512].astype(np.float64) / scale[i:i + 512, None].astype(np.float64)
        out[i:i + 512] = _e4m3_round(v)[1]
    return out, scale


def plant_codes(a: np.ndarray, rows, codes, frac: float = 0.02, seed: int = 5) -> np.ndarray:
    """A copy of the byte array `a` [N][L] in which about `frac` of the bytes of
    each row in `rows` are replaced by values drawn from `codes` (seeded):
    the edge codes of a stored format (the e4m3 codes 0x7F / 0xFF, a NaN block
    scale) placed where a test will read them."""
    out = np.array(a, copy=True)
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = np.asarray(codes, dtype=out.dtype)
    for r in rows:
        cnt = max(1, int(round(frac * out.shape[1])))
        pos = rng.choice(out.shape[1], size=cnt, replace=False)
        out[r, pos] = rng.choice(codes, size=cnt)
    return out


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def nvfp4_head(w_bits: np.ndarray):
    """A synthetic NVFP4 head (stand-in for a checkpoint's NVFP4 weight, the
    two-level scaling such checkpoints use): global scale g = max |w| /
    (6 * 448) (float32); per 16 elements an e4m3 block scale, the nearest
    e4m3 value to the block's max |w| / (6 g); each element the nearest e2m1
    value to w / (block scale * g).  Bytes hold element 2j in the low nibble,
    2j+1 in the high one.
    Returns (w4 uint8 [N][K/2], bscale uint8 [N][K/16], gscale float32)."""
    w = bf16_bits_to_f32(w_bits)
    n, k = w.shape
    amax = float(np.abs(w).max())
    g = np.float32(amax / (6.0 * 448.0) if amax > 0 else 1.0)
    w4 = np.empty((n, k // 2), dtype=np.uint8)
    bscale = np.empty((n, k // 16), dtype=np.uint8)
    mids = (E2M1_GRID[1:] + E2M1_GRID[:-1]) / 2
    for i in range(0, n, 512):
        blk = w[i:i + 512].astype(np.float64).reshape(-1, k // 16, 16)
        bq, bcode = _e4m3_round(np.abs(blk).max(axis=2) / (6.0 * float(g)))
        bscale[i:i + 512] = bcode
        den = bq[..., None] * float(g)
        v = np.divide(blk, den, out=np.zeros_like(blk), where=den > 0)
        a = np.abs(v)
        idx = np.zeros(a.shape, dtype=np.int64)
        for t in mids:
            idx += a > t
        codes = (idx | np.where(v < 0, 8, 0)).reshape(-1, k)
        w4[i:i + 512] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return w4, bscale, g


def outlier_channels(k: int, frac: float = 0.01, seed: int = SEED_OUTLIERS) -> np.ndarray:
    cnt = int(round(frac * k))
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(k, size=cnt, replace=False))


def gen_x(m: int, k: int, seed: int = SEED_X, outliers: bool = True,
          outlier_scale: float = 8.0, rows_generated: int | None = None) -> np.ndarray:
    """bf16 activations [m][k]: N(0, 1), optionally 1% of channels scaled by 8."""
    rows = max(m, X_ROWS_GENERATED if rows_generated is None else rows_generated)
    rng = np.random.Generator(np.random.PCG64(seed))
    xf = rng.standard_normal((rows, k), dtype=np.float32)
    if outliers:
        xf[:, outlier_channels(k)] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(xf[:m])


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    m: int
    k: int
    n: int
    kcand: int = 8
    rerank: int = 32
    outliers: bool = True
    seed_w: int = SEED_W
    seed_x: int = SEED_X


# The tiny case, one rank's shard at M = 1, 8 and 72, and the recall stress
# case (planted near-ties, see plant_recall_pairs).
CONFIGS = {
    "tiny": Config("tiny", 1, 1024, 16384, outliers=False, seed_w=11, seed_x=12),
    "m1": Config("m1", 1, HIDDEN, VOCAB_SHARD),
    "m8": Config("m8", 8, HIDDEN, VOCAB_SHARD),
    "m72": Config("m72", 72, HIDDEN, VOCAB_SHARD),
    "recall": Config("recall", 32, HIDDEN, VOCAB_SHARD),
}


def make_inputs(cfg: Config):
    """(x bits [m][k], W bits [n][k]) for a config."""
    w = gen_weight(cfg.n, cfg.k, seed=cfg.seed_w)
    x = gen_x(cfg.m, cfg.k, seed=cfg.seed_x, outliers=cfg.outliers)
    return x, w


def plant_recall_pairs(x_bits: np.ndarray, w_bits: np.ndarray, target: float = 12.0,
                       gap: float = 0.01, seed: int = SEED_PLANT, block: int = 64):
    """Plant, for each row m of x, two columns of one 64-column block whose exact
    logits are `target` and `target - gap`, far above every other logit of the row.

    This builds the situation the module docstring of the radiance_drafthead.py
    page names as the reason KCAND is the recall lever: the winner shares its
    block with another strong token.  Returns (w_bits_planted, pairs) where
    pairs[m] = (c1, c2) is the planted (winner, runner-up).  W is modified on a
    copy: each planted row becomes base + alpha * x_m rounded to bf16, then a
    few single-channel corrections on large non-outlier channels of x_m bring
    its logit to within a small fraction of `gap` of the target.  Raises if a
    planted pair does not end up as its row's top two with a gap in
    [gap / 2, 2 * gap].
    """
    m, k = x_bits.shape
    n = w_bits.shape[0]
    full_blocks = n // block
    if m > full_blocks:
        raise ValueError("need at least one full block per planted row")
    rng = np.random.Generator(np.random.PCG64(seed))
    blocks = rng.choice(full_blocks, size=m, replace=False)
    w = w_bits.copy()
    xf = bf16_bits_to_f32(x_bits).astype(np.float64)
    outl = set(int(v) for v in outlier_channels(k))
    pairs = []
    for row in range(m):
        b = int(blocks[row])
        c1, c2 = (int(v) for v in rng.choice(block, size=2, replace=False))
        c1 += b * block
        c2 += b * block
        xm = xf[row]
        xx = float(xm @ xm)
        order = [int(i) for i in np.argsort(-np.abs(xm)) if int(i) not in outl]
        for col, tgt in ((c1, target), (c2, target - gap)):
            base = bf16_bits_to_f32(w[col]).astype(np.float64)
            alpha = (tgt - float(base @ xm)) / xx
            wf = bf16_bits_to_f32(f32_to_bf16_bits((base + alpha * xm).astype(np.float32))).astype(np.float64)
            for ch in order[:16]:
                resid = tgt - float(wf @ xm)
                if abs(resid) < 1e-3 * gap:
                    break
                wf[ch] = float(bf16_bits_to_f32(f32_to_bf16_bits(
                    np.array([wf[ch] + resid / xm[ch]], dtype=np.float32)))[0])
            w[col] = f32_to_bf16_bits(wf.astype(np.float32))
        pairs.append((c1, c2))
    # verify on the final weights
    logits = np.concatenate([bf16_bits_to_f32(w[i:i + 8192]).astype(np.float64) @ xf.T
                             for i in range(0, n, 8192)], axis=0)
    for row, (c1, c2) in enumerate(pairs):
        lg = logits[:, row]
        top = np.argsort(-lg, kind="stable")[:2]
        d = lg[c1] - lg[c2]
        if [int(top[0]), int(top[1])] != [c1, c2] or not (gap / 2 <= d <= 2 * gap):
            raise RuntimeError(f"planting failed for row {row}: top {top}, gap {d}")
    return w, pairs
