"""The parity comparator accepts the oracle against itself and rejects planted
mistakes (planted in copies of the oracle's own outputs, on the CPU)."""
import copy

import numpy as np
import pytest

import oracle
from bit_quantized_lm_amd import workload
from parity_util import compare


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
    }
    return n, ref, as_gpu


def test_oracle_against_itself(case):
    n, ref, g = case
    stats = compare(ref, g, n, 8)
    assert stats["blocks_excused"] == 0


@pytest.mark.parametrize("mutation", ["swap_cand", "wrong_block", "cand_value", "rr_swap",
                                      "rr_value", "final", "coarse", "pad_value"])
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
    elif mutation == "pad_value":
        g["cand_val"][0, -1] = np.float32(np.nan)
        g["cand_id"][0, -1] = -1
    with pytest.raises(AssertionError):
        compare(ref, g, n, 8)
