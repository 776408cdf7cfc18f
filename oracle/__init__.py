"""CPU oracle for the 2-bit speculative-draft LM head.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, step-by-step CPU
implementation of what the draft head computes, written from the page
"radiance_drafthead.py" (a vLLM plug-in module; its module docstring, the
quantiser `_quantize_head_now`, the kernels `_draft_head_int2`, `_emit`,
`_rerank_exact` and the per-call glue `_apply_head_int2`), and, for one
optional rerank source, the page on vLLM pull request 55713 (the NVFP4
gathered projection `_nvfp4_gathered_bias_kernel`).  Only the tests,
`__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py` may use it.
The product library never imports it and it imports nothing from the product
library.

Modules
-------
bf16     bf16 <-> float conversions (round to nearest even), own code.
quant    min/max asymmetric int2 quantiser, quarter-split packing, unpacking
         and the effective weight defined by the stored scale pair; the same
         at 4 bits (half-split packing, bias 16).
head     coarse scores, block top-KCAND, row top-R, exact rerank (bf16 rows,
         e4m3 rows with a per-row scale, or NVFP4 rows), argmax, the
         bf16 row handed to the caller (full or top-k only), and the exact
         bf16 head (for agreement reports only).
brute    pure-Python, exact-rational re-statement of every step for tiny
         shapes; pins the vectorised code.
acceptance
         the acceptance rules: a HIP result against the oracle's (ids exact
         up to counted near-ties and tie rows, values within tolerance).

Every function cites the passage it follows.  Where the page is silent the
reading taken is stated in the docstring; all readings are listed in the
design notes of the repository.

Parity status: every function here is pinned by a `-m "not gpu"` test
(tests/test_oracle_pins.py) against a page identity, a closed form, a
hand-derived fixture under tests/golden/, a special case or exact brute force.
The page's real-data claims (argmax agreement on 8192 captured serve inputs,
the ~5% top-1 change of the unreranked head) are parity unpinned: the captured
inputs and the real weights are not available.
"""
from . import bf16, quant, head, brute, acceptance  # noqa: F401
from .quant import (GROUP, quantize, pack_quarter_split, unpack_quarter_split,  # noqa: F401
                    effective_weight, quantize_pack, quantize_int4, pack_half_split, unpack_half_split,
                    quantize_pack_int4, effective_weight_int4)
from .head import (BLOCK_N, coarse, coarse_int4, coarse_collapse, block_topk, row_topr,  # noqa: F401
                   rerank_exact, final_argmax, logits_row, exact_head, pipeline, tie_rows, tied_ids,
                   e4m3_value, rerank_exact_e4m3, e2m1_value, e4m3fn_value, nvfp4_rows,
                   rerank_exact_nvfp4)
