"""The parity comparator accepts the oracle against itself and rejects planted
mistakes (planted in copies of the oracle's own outputs, on the CPU)."""
import copy

import numpy as np
import pytest

import oracle
from bit_quantized_lm_amd import workload
from oracle.acceptance import compare


@pytest.fixture(scope="module")
def case():
    n, k, m = 1000, 1024, 4
    w = workload.gen_weight(n, k, seed=5)
    x = workload.gen_x(m, k, seed=6)
    ref = oracle.pipeline(x, w, *oracle.quantize_pack(w), kcand=8, r=32)
    as_gpu = {
        "coarse": ref["coarse"].astype(np.float32), "cand_val": ref["cand_val"].astype(np.float32),
        "cand_id": ref["cand_id"].astype(np.int32), "rr_id": ref["rr_id"].astype(np.int32),
        "rr_val": ref["rr_val"].astype(np.float32), "out_id": ref["out_id"].astype(np.int32),
        "out_val": ref["out_val"].astype(np.float32),
    }
    return n, ref, as_gpu


@pytest.fixture(scope="module")
def tie_case():
    """Row 0's winning token gets a twin (an identical head row) in another
    block: both are reranked with the same exact value, so row 0 is a tie row
    whose tied set is exactly the two twins."""
    n, k, m = 1000, 1024, 2
    w = workload.gen_weight(n, k, seed=7)
    x = workload.gen_x(m, k, seed=8)
    win = int(oracle.pipeline(x, w, *oracle.quantize_pack(w), kcand=8, r=32)["out_id"][0])
    twin = (win + 64 * 3) % n
    w[twin] = w[win]
    ref = oracle.pipeline(x, w, *oracle.quantize_pack(w), kcand=8, r=32)
    assert ref["tie_rows"][0] and ref["tied_ids"][0] == {win, twin}
    g = {key: np.array(ref[key], dtype=np.float32 if key in ("coarse", "cand_val", "rr_val", "out_val")
                       else np.int32) for key in ("coarse", "cand_val", "cand_id", "rr_id", "rr_val", "out_id",
                                                  "out_val")}
    return n, ref, g, win, twin


def test_tie_row_accepts_the_twin(tie_case):
    n, ref, g, win, twin = tie_case
    g = copy.deepcopy(g)
    other = twin if int(ref["out_id"][0]) == win else win
    g["out_id"][0] = other
    stats = compare(ref, g, n, 8)
    assert stats["final_mismatch_on_tie_rows"] == 1 and stats["tie_rows"] >= 1


@pytest.mark.parametrize("mutation", ["outside_tied_set", "out_val_of_the_other_id"])
def test_tie_row_rejects(tie_case, mutation):
    n, ref, g, win, twin = tie_case
    g = copy.deepcopy(g)
    if mutation == "outside_tied_set":     # another reranked id of the tie row
        g["out_id"][0] = next(int(i) for i in ref["rr_id"][0] if int(i) not in (win, twin))
    else:                                  # the token's value taken from a different reranked id
        g["out_val"][0] = np.float32(ref["rr_val"][0][5])
    with pytest.raises(AssertionError):
        compare(ref, g, n, 8)


def test_oracle_against_itself(case):
    n, ref, g = case
    stats = compare(ref, g, n, 8)
    assert stats["blocks_excused"] == 0


@pytest.mark.parametrize("mutation", ["swap_cand", "wrong_block", "cand_value", "rr_swap",
                                      "rr_value", "final", "coarse", "pad_value", "out_val",
                                      "out_val_missing_token"])
def test_planted_mistakes_are_caught(case, mutation):
    n, ref, g = case
    g = copy.deepcopy(g)
    if mutation == "swap_cand":          # positions 0 and 5 of block 3 (not a near-tie)
        ids = g["cand_id"][0].reshape(-1, 8)
        ids[3, [0, 5]] = ids[3, [5, 0]]
    elif mutation == "wrong_block":
        g["cand_id"][1, 8 * 2] = g["cand_id"][1, 8 * 2] + 64
    elif mutation == "cand_value":
        g["cand_val"][2, 17] += 0.05 * (1 + abs(g["cand_val"][2, 17]))
    elif mutation == "rr_swap":
        g["rr_id"][0, [0, 3]] = g["rr_id"][0, [3, 0]]
    elif mutation == "rr_value":
        g["rr_val"][1, 2] *= 1.01
    elif mutation == "final":
        g["out_id"][3] = g["rr_id"][3, 5]
    elif mutation == "coarse":
        g["coarse"][0, 123] += 0.1
    elif mutation == "out_val":
        g["out_val"][2] += np.float32(0.01 * (1 + abs(g["out_val"][2])))
    elif mutation == "out_val_missing_token":
        g["out_val"][1] = np.float32(-np.inf)
    elif mutation == "pad_value":
        g["cand_val"][0, -1] = np.float32(np.nan)
        g["cand_id"][0, -1] = -1
    with pytest.raises(AssertionError):
        compare(ref, g, n, 8)
