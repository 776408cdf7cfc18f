"""2-bit speculative-draft LM head for MI355X (gfx950).

The head computes x[M, K] @ W[K, N] for one tensor-parallel rank's vocabulary
shard with int2 weights, keeps the top KCAND columns of every 64-column block,
reranks the best R candidates exactly against the bf16 weight and returns the
argmax token.  All per-call steps run in hand-written HIP kernels behind a
C ABI (include/drafthead.h); `_binding` is a thin ctypes layer over it.

Importing the package loads nothing native: the binding's names are resolved
on first attribute access, and the native library is loaded on first call
(raising if it has not been built).
"""
_BINDING_NAMES = (
    "DraftHeadError", "draft_head_sizes", "draft_head_quantize_pack", "draft_head_tile",
    "draft_head_coarse", "draft_head_rerank", "draft_head_argmax", "draft_head_last_error",
    "DraftHead", "library_path", "load_library",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
