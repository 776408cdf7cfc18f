"""Per-call steps of the draft head (oracle).

Follows `_apply_head_int2` on the radiance_drafthead.py page and the kernels
it launches: `_draft_head_int2` (coarse scores), `_emit` (top-KCAND of each
64-column block by successive max-and-mask), the row top-R of the candidates
(`bm.topk(RERANK)` then `bi.gather`), `_rerank_exact` (exact dot of x with
the bf16 weight row of each candidate) and the final argmax the caller takes.

Precision: coarse scores and exact logits are accumulated in float64 and
reported both in float64 (for margins) and rounded to float32 (the page's
kernels accumulate in float32).

Readings where the page is silent (all also listed in the design notes):
* Ties rank the lower column id first, at every stage (Triton's argmax takes
  the first maximum; torch.topk's tie order is unspecified).
* A block with fewer than KCAND valid columns (the partial last block) pads
  its list with (-inf, id -1); a row with fewer than R valid candidates pads
  the same way.
* The final token is the argmax over the R exact values (the page writes the
  exact values back into a bf16 row and leaves the argmax to the caller).
  The decision is taken on the float32 values, ties to the lower id.
* M is the true number of rows (the page pads M to a power of two >= 16 only
  because its Triton dot needs it).
"""
import numpy as np

from . import bf16
from .quant import GROUP, effective_weight, effective_weight_int4, unpack_quarter_split

BLOCK_N = 64          # width of one selection block (module constant BLOCK_N)
CHUNK_ROWS = 8192     # rows of W handled at once (memory bound only)


def _x64(x_bits):
    return bf16.to_f64(np.asarray(x_bits, dtype=np.uint16))


def coarse(x_bits, packed, S_bits, ZS_bits):
    """c[m][n] = sum_k x[m][k] * w_eff[n][k], float64 [M][N].

    `_draft_head_int2` accumulates S * p - ZS * X per group into the fp32
    accumulator it later selects from; algebraically that is the dot of x
    with the effective weight (see quant.effective_weight).
    """
    x = _x64(x_bits)
    n = packed.shape[0]
    out = np.empty((x.shape[0], n), dtype=np.float64)
    for i in range(0, n, CHUNK_ROWS):
        j = min(i + CHUNK_ROWS, n)
        w = effective_weight(packed, S_bits, ZS_bits, rows=slice(i, j))
        out[:, i:j] = x @ w.T
    return out


def coarse_int4(x_bits, packed4, S_bits, ZS_bits):
    """c[m][n] = sum_k x[m][k] * w_eff[n][k] for a 4-bit head (half-split
    packing, weight (S/16) v - (ZS - S)), float64 [M][N]."""
    x = _x64(x_bits)
    n = np.asarray(packed4).shape[0]
    out = np.empty((x.shape[0], n), dtype=np.float64)
    for i in range(0, n, CHUNK_ROWS):
        j = min(i + CHUNK_ROWS, n)
        out[:, i:j] = x @ effective_weight_int4(packed4, S_bits, ZS_bits, rows=slice(i, j)).T
    return out


def coarse_collapse(x_bits, packed, S_bits, ZS_bits):
    """The page's own per-group form, in float64, for cross-checking `coarse`.

    p_g = sum_{k in g} x_k (1 + v_k / 4) (the value the bit-pattern dequant
    makes the dot return), X_g = sum_{k in g} x_k, and the group adds
    S * p_g - ZS * X_g (module docstring, "Bit-pattern dequant, hoisted";
    the scale and zero-point updates of `_draft_head_int2`).
    """
    x = _x64(x_bits)
    v = unpack_quarter_split(packed).astype(np.float64)
    S = bf16.to_f64(S_bits)
    ZS = bf16.to_f64(ZS_bits)
    m, k = x.shape
    out = np.zeros((m, packed.shape[0]), dtype=np.float64)
    for g in range(k // GROUP):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        p = x[:, sl] @ (1.0 + v[:, sl] / 4.0).T
        X = x[:, sl].sum(axis=1)
        out += S[:, g][None, :] * p - ZS[:, g][None, :] * X[:, None]
    return out


def block_topk(c, kcand):
    """Top-KCAND of each 64-column block, ordered (value desc, column asc).

    `_emit`: KCAND rounds of max / argmax / mask over the block's columns, with
    columns past N masked to -inf.  Returns (val64, ids) of shape
    [M][NBLK * kcand]; padding slots hold (-inf, -1).
    """
    c = np.asarray(c, dtype=np.float64)
    m, n = c.shape
    nblk = (n + BLOCK_N - 1) // BLOCK_N
    padded = np.full((m, nblk * BLOCK_N), -np.inf)
    padded[:, :n] = c
    blocks = padded.reshape(m, nblk, BLOCK_N)
    # stable sort of the negated values: equal values keep ascending column order
    order = np.argsort(-blocks, axis=2, kind="stable")
    take = min(kcand, BLOCK_N)
    top = order[:, :, :take]
    vals = np.take_along_axis(blocks, top, axis=2)
    ids = top + (np.arange(nblk) * BLOCK_N)[None, :, None]
    ids = np.where(ids < n, ids, -1)
    vals = np.where(ids >= 0, vals, -np.inf)
    if take < kcand:
        pad_v = np.full((m, nblk, kcand - take), -np.inf)
        pad_i = np.full((m, nblk, kcand - take), -1)
        vals = np.concatenate([vals, pad_v], axis=2)
        ids = np.concatenate([ids, pad_i], axis=2)
    return vals.reshape(m, nblk * kcand), ids.reshape(m, nblk * kcand).astype(np.int64)


def row_topr(cand_val, cand_id, r):
    """R best candidates of each row, ordered (value desc, id asc), id -1 skipped.

    `bm.topk(RERANK, dim=1)` followed by `bi.gather` in `_apply_head_int2`.
    Returns (ids int64 [M][R], vals float64 [M][R]); missing slots (-1, -inf).
    """
    cand_val = np.asarray(cand_val, dtype=np.float64)
    cand_id = np.asarray(cand_id)
    m = cand_val.shape[0]
    ids = np.full((m, r), -1, dtype=np.int64)
    vals = np.full((m, r), -np.inf)
    for row in range(m):
        ok = cand_id[row] >= 0
        v = cand_val[row][ok]
        i = cand_id[row][ok].astype(np.int64)
        order = np.lexsort((i, -v))[:r]
        ids[row, :len(order)] = i[order]
        vals[row, :len(order)] = v[order]
    return ids, vals


def rerank_exact(x_bits, w_bits, rr_id):
    """e[m][r] = sum_k x[m][k] * W[rr_id[m][r]][k], float64; -inf for id -1.

    `_rerank_exact` (bf16 branch): one dot per (row, candidate), straight off
    the head's own bf16 weight, accumulated in fp32 on the page (float64 here).
    """
    x = _x64(x_bits)
    rr_id = np.asarray(rr_id)
    out = np.full(rr_id.shape, -np.inf)
    for row in range(rr_id.shape[0]):
        ok = rr_id[row] >= 0
        rows = bf16.to_f64(np.asarray(w_bits)[rr_id[row][ok]])
        out[row, ok] = rows @ x[row]
    return out


def e4m3_value(codes):
    """Value of e4m3 bytes as `_rerank_exact` (FP8 branch) decodes them, float64.

    The page's bit arithmetic: e = (b >> 3) & 15, mant = b & 7; magnitude
    mant * 2^-9 when e == 0, else (1 + mant/8) * 2^(e-7); bit 7 is the sign.
    Every byte decodes to a number (codes 0x7F / 0xFF give +-480: the page
    does not treat them as NaN).
    """
    b = np.asarray(codes, dtype=np.int64)
    e = (b >> 3) & 15
    mant = (b & 7).astype(np.float64)
    mag = np.where(e == 0, mant * 2.0 ** -9, (1.0 + mant / 8.0) * np.exp2(e - 7.0))
    return np.where((b & 128) != 0, -mag, mag)


def rerank_exact_e4m3(x_bits, w8, scale, rr_id):
    """e[m][r] = sum_k x[m][k] * wv[k], wv = float32(decode(W8[id][k]) * scale[id]).

    `_rerank_exact` (FP8 branch): the head's own e4m3 rows, decoded by bit
    arithmetic and multiplied by the row's float32 scale (one float32
    rounding), accumulated in fp32 on the page (float64 here); -inf for id -1.
    """
    x = _x64(x_bits)
    rr_id = np.asarray(rr_id)
    w8 = np.asarray(w8)
    scale = np.asarray(scale, dtype=np.float32)
    out = np.full(rr_id.shape, -np.inf)
    for row in range(rr_id.shape[0]):
        ok = rr_id[row] >= 0
        ids = rr_id[row][ok]
        wv = (e4m3_value(w8[ids]).astype(np.float32) * scale[ids][:, None]).astype(np.float64)
        out[row, ok] = wv @ x[row]
    return out


def e2m1_value(nibbles):
    """Value of e2m1 (FP4) codes, float64, as the format defines them: sign
    bit 3, exponent bits 2-1 with bias 1, mantissa bit 0; exponent 0 is
    subnormal (magnitude 0.5 * mantissa), otherwise the magnitude is
    (1 + mantissa/2) * 2^(exponent - 1).  The NVFP4 rows of the page for vLLM
    pull request 55713 hold these codes (its kernel decodes them with
    `_e2m1_inline`, whose body the page does not show).
    """
    n = np.asarray(nibbles, dtype=np.int64) & 15
    e = (n >> 1) & 3
    mant = (n & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * mant, (1.0 + mant / 2.0) * np.exp2(e - 1.0))
    return np.where((n & 8) != 0, -mag, mag)


def e4m3fn_value(codes):
    """e4m3 bytes as the format defines them (the page for pull request 55713
    converts its block scales through Triton's float8e4nv type): as
    e4m3_value, except that 0x7F and 0xFF are NaN."""
    b = np.asarray(codes, dtype=np.int64)
    return np.where((b & 127) == 127, np.nan, e4m3_value(b))


def nvfp4_rows(w4, bscale, gscale, ids, k):
    """The weights of NVFP4 rows ids, float64 [len(ids)][k].

    `_nvfp4_gathered_bias_kernel` (page for vLLM pull request 55713): byte j
    of a row holds element 2j in its low nibble and 2j+1 in its high nibble
    (`tl.interleave(low, high)`); element k is scaled by the e4m3 scale of
    its 16-element block and by the global scale, in float32, left to right,
    then rounded to bf16 (`.to(tl.bfloat16)`, nearest even).
    """
    ids = np.asarray(ids, dtype=np.int64)
    rows = np.asarray(w4)[ids][:, : k // 2].astype(np.int64)
    codes = np.empty((len(ids), k), dtype=np.int64)
    codes[:, 0::2] = rows & 15
    codes[:, 1::2] = rows >> 4
    d = e2m1_value(codes).astype(np.float32)
    s = e4m3fn_value(np.asarray(bscale)[ids][:, : k // 16]).astype(np.float32)
    t = (d * np.repeat(s, 16, axis=1)).astype(np.float32)
    t = (t * np.float32(gscale)).astype(np.float32)
    return bf16.to_f64(bf16.from_f32(t))


def rerank_exact_nvfp4(x_bits, w4, bscale, gscale, rr_id):
    """e[m][r] = sum_k x[m][k] * nvfp4_rows(...)[r][k], float64; -inf for id -1.

    The dot of `_nvfp4_gathered_bias_kernel` (page for vLLM pull request
    55713): float32 products of the bf16 weight and x, summed in float32 on
    the page (float64 here).
    """
    x = _x64(x_bits)
    rr_id = np.asarray(rr_id)
    k = x.shape[1]
    out = np.full(rr_id.shape, -np.inf)
    for row in range(rr_id.shape[0]):
        ok = rr_id[row] >= 0
        out[row, ok] = nvfp4_rows(w4, bscale, gscale, rr_id[row][ok], k) @ x[row]
    return out


def final_argmax(rr_id, e):
    """Argmax over the R exact values of each row, float32 decision, ties -> lower id.

    Reading (the page leaves the caller's argmax unshown): a NaN exact value
    (an NVFP4 row whose block scale is the e4m3 NaN code) ranks below every
    number, -inf included, so it is returned only when every reranked value
    of the row is NaN (then the lowest such id, with value NaN).
    Returns (out_id int64 [M], out_val float32 [M]); (-1, -inf) for a row with
    no valid candidate.
    """
    e32 = np.asarray(e, dtype=np.float64).astype(np.float32)
    rr_id = np.asarray(rr_id)
    m = rr_id.shape[0]
    out_id = np.full(m, -1, dtype=np.int64)
    out_val = np.full(m, -np.inf, dtype=np.float32)
    for row in range(m):
        best = None
        for r in range(rr_id.shape[1]):
            i = int(rr_id[row, r])
            if i < 0:
                continue
            v = e32[row, r]
            # order key: (is a number, value, lower id first)
            key = (not np.isnan(v), v if not np.isnan(v) else 0.0, -i)
            if best is None or key > best[0]:
                best = (key, i, v)
        if best is not None:
            out_id[row], out_val[row] = best[1], best[2]
    return out_id, out_val


def logits_row(rr_id, rr_val, n, coarse_f32=None, topk_only=False):
    """The bf16 row `_apply_head_int2` hands to its caller after the rerank.

    The coarse scores rounded to bf16 (the row `_draft_head_int2` writes), or,
    for a top-k caller (`_radiance_topk_only`), -inf in every entry; then each
    reranked id's exact value, rounded to bf16, is written over its entry
    (`y.scatter_(1, idx, ex.to(bfloat16))`).  Reading: entries of rr_id that
    are -1 (a row with fewer than R candidates) are skipped.  `coarse_f32`:
    float32 [M][N] (not used when topk_only); returns bf16 bit patterns [M][N].
    """
    rr_id = np.asarray(rr_id)
    rr_val = np.asarray(rr_val, dtype=np.float32)
    m, r = rr_id.shape
    if topk_only:
        y = np.full((m, n), 0xFF80, dtype=np.uint16)        # bf16 -inf
    else:
        y = bf16.from_f32(np.asarray(coarse_f32, dtype=np.float32)).reshape(m, n).copy()
    for row in range(m):
        for j in range(r):
            i = int(rr_id[row, j])
            if i >= 0:
                y[row, i] = bf16.from_f32(rr_val[row, j:j + 1])[0]
    return y


def exact_head(x_bits, w_bits):
    """E[m][n] = x . W_bf16[n] in float64 (the bf16 head the method stands in for).

    Used only to report agreement; not part of the method.
    """
    x = _x64(x_bits)
    w_bits = np.asarray(w_bits)
    n = w_bits.shape[0]
    out = np.empty((x.shape[0], n), dtype=np.float64)
    for i in range(0, n, CHUNK_ROWS):
        j = min(i + CHUNK_ROWS, n)
        out[:, i:j] = x @ bf16.to_f64(w_bits[i:j]).T
    return out


def argmax_lowest(E):
    """Row argmax of a float64 matrix with ties to the lower column."""
    return np.argmax(E, axis=1)   # numpy returns the first maximum


def tie_rows(e, rel=1e-4):
    """Rows whose two best exact values differ by less than rel * |best|.

    `e` holds the reranked exact values of each row (the values the final
    argmax decides between), -inf for padding; a row with fewer than two
    finite values is never a tie row.  Reading of the acceptance rule "the
    top two exact logits differ by less than 1e-4 relative".
    """
    e = np.asarray(e, dtype=np.float64)
    flags = np.zeros(e.shape[0], dtype=bool)
    for row in range(e.shape[0]):
        v = np.sort(e[row][np.isfinite(e[row])])[::-1]
        if len(v) >= 2 and (v[0] - v[1]) < rel * abs(v[0]):
            flags[row] = True
    return flags


def tied_ids(rr_id, e, rel=1e-4):
    """Per row, the set of reranked ids a tie row may return: every valid id
    whose exact value equals the row's best or lies within rel * |best| below
    it.  On a tie row the final token is any one of these (the float32 order
    of the summation decides between them); on other rows only the oracle's
    own out_id is accepted.  Returns a list of sets of ints.
    """
    rr_id = np.asarray(rr_id)
    e = np.asarray(e, dtype=np.float64)
    out = []
    for row in range(rr_id.shape[0]):
        ok = (rr_id[row] >= 0) & np.isfinite(e[row])
        if not np.any(ok):
            out.append(set())
            continue
        best = np.max(e[row][ok])
        near = ok & ((e[row] == best) | ((best - e[row]) < rel * abs(best)))
        out.append({int(i) for i in rr_id[row][near]})
    return out


def pipeline(x_bits, w_bits, packed, S_bits, ZS_bits, kcand=8, r=32, bits=2):
    """All per-call steps in order; returns a dict of every intermediate.
    bits = 4: the head is a 4-bit one (quantize_pack_int4's arrays)."""
    c = (coarse_int4 if bits == 4 else coarse)(x_bits, packed, S_bits, ZS_bits)
    cv, ci = block_topk(c, kcand)
    rr_id, rr_cv = row_topr(cv, ci, r)
    e = rerank_exact(x_bits, w_bits, rr_id)
    out_id, out_val = final_argmax(rr_id, e)
    return {
        "coarse": c, "cand_val": cv, "cand_id": ci, "rr_id": rr_id,
        "rr_coarse": rr_cv, "rr_val": e, "out_id": out_id, "out_val": out_val,
        "tie_rows": tie_rows(e), "tied_ids": tied_ids(rr_id, e),
    }
