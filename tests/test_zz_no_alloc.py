"""The entry point that allocates nothing (draft_head_forward_noalloc), called
through the C ABI: on two calls in a row, the second with a smaller input
(the many-row kernel, then the resident one), its outputs equal those of
draft_head_forward with a caller workspace bit for bit (the same kernels),
and the rerank's per-row counters in the library's static scratch end at
zero (the next call's coarse kernel would clear them anyway).  Sizes beyond
the static array are rejected before any launch."""
import ctypes

import numpy as np
import pytest

from bit_quantized_lm_amd import _binding as B
from bit_quantized_lm_amd import workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.load_library()
    return torch.device("cuda:0")


def _forward_pair(head, x, dev):
    m = x.shape[0]
    want = head(x, coarse_out=torch.empty((m, head.N), dtype=torch.float32, device=dev))
    got_coarse = torch.empty((m, head.N), dtype=torch.float32, device=dev)
    got = B.draft_head_forward_noalloc(x, head.tiled, head.pairs, head.w, head.N, head.kcand, head.R,
                                       coarse_out=got_coarse)
    torch.cuda.synchronize()
    return want, got, got_coarse


def test_noalloc_matches_forward_two_calls(dev):
    n, k = 20000, 1024
    w = workload.gen_weight(n, k, seed=4500)
    head = B.DraftHead.from_weight(w, kcand=8, R=32, device=dev)
    xs = workload.gen_x(72, k, seed=4501)
    for m in (72, 3):      # the second call smaller: many-row kernel, then the resident kernel
        x = torch.from_numpy(xs[:m].view(np.int16)).to(dev)
        want, got, _ = _forward_pair(head, x, dev)
        for key in ("cand_val", "cand_id", "rr_id", "rr_val", "out_id", "out_val"):
            assert torch.equal(got[key], want[key]), (m, key)


def test_noalloc_full_shape_then_one_row(dev):
    cfg = workload.CONFIGS["m72"]
    x_host, w = workload.make_inputs(cfg)
    head = B.DraftHead.from_weight(w, kcand=cfg.kcand, R=cfg.rerank, device=dev)
    for m in (72, 1):
        x = torch.from_numpy(x_host[:m].view(np.int16)).to(dev)
        want, got, coarse = _forward_pair(head, x, dev)
        for key in ("cand_val", "cand_id", "rr_id", "rr_val", "out_id", "out_val"):
            assert torch.equal(got[key], want[key]), (m, key)


def test_noalloc_rejects_sizes_beyond_its_scratch(dev):
    lib = B.load_library()
    K = 65536            # M = 72 at this K needs far more than the static scratch
    need = B.draft_head_workspace_bytes(72, K)
    assert need > B.DH_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(4096)
    rc = lib.draft_head_forward_noalloc(fake, 72, K, 64, fake, fake, fake, K, 8, 8, fake, fake, fake, fake,
                                        fake, fake, None, None, None, None)
    assert rc == B.DH_EUNSUP, (rc, lib.draft_head_last_error())
    assert b"scratch" in lib.draft_head_last_error()
