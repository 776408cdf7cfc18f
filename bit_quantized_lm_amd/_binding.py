"""ctypes binding of libdrafthead.so (include/drafthead.h), same names as the C ABI.

Argument marshalling only: host functions take and return numpy arrays, device
functions take torch CUDA tensors (torch is used for device memory and the
current stream, nothing else) and allocate their outputs with torch.empty when
the caller passes none.  Every step of the draft head runs in the library.

Error mapping: DH_EINVAL / DH_ESHAPE / DH_EUNSUP raise ValueError, DH_EHIP
raises DraftHeadError (a RuntimeError); the message is the library's own.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "drafthead.h")

DH_OK, DH_EINVAL, DH_ESHAPE, DH_EUNSUP, DH_EHIP = 0, -1, -2, -3, -4
DH_NOALLOC_SCRATCH_BYTES = 4 << 20
BLOCK_N = 64
GROUP = 128

_lib = None


class DraftHeadError(RuntimeError):
    """A HIP runtime or launch error reported by the library."""


def library_path() -> str:
    return os.environ.get("DRAFTHEAD_LIB", os.path.join(_PKG, "libdrafthead.so"))


def load_library() -> ctypes.CDLL:
    """Load the in-tree library (raises FileNotFoundError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m bit_quantized_lm_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.draft_head_last_error.restype = ctypes.c_char_p
    lib.draft_head_last_error.argtypes = []
    lib.draft_head_sizes.restype = i32
    lib.draft_head_sizes.argtypes = [i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz),
                                     ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.draft_head_quantize_pack.restype = i32
    lib.draft_head_quantize_pack.argtypes = [P, i64, i64, i64, P, P, P, i32]
    lib.draft_head_quantize_pack_int4.restype = i32
    lib.draft_head_quantize_pack_int4.argtypes = [P, i64, i64, i64, P, P, P, i32]
    lib.draft_head_int4_as_int2.restype = i32
    lib.draft_head_int4_as_int2.argtypes = [P, P, P, i64, i64, P, P, P]
    lib.draft_head_tile_int4.restype = i32
    lib.draft_head_tile_int4.argtypes = [P, P, P, i64, i64, P, P]
    lib.draft_head_tile.restype = i32
    lib.draft_head_tile.argtypes = [P, P, P, i64, i64, P, P]
    lib.draft_head_workspace_bytes.restype = i32
    lib.draft_head_workspace_bytes.argtypes = [i32, i32, ctypes.POINTER(sz)]
    lib.draft_head_coarse.restype = i32
    lib.draft_head_coarse.argtypes = [P, i32, i32, i32, P, P, i32, P, P, P, P, sz, P]
    lib.draft_head_forward.restype = i32
    lib.draft_head_forward.argtypes = [P, i32, i32, i32, P, P, P, i64, i32, i32, P, P, P, P, P, P, P, P, sz,
                                       P, P, P]
    lib.draft_head_rerank.restype = i32
    lib.draft_head_rerank.argtypes = [P, P, i64, i32, i32, i32, P, P, i32, i32, P, P, P]
    lib.draft_head_argmax.restype = i32
    lib.draft_head_argmax.argtypes = [P, P, i32, i32, P, P, P]
    lib.draft_head_coarse_int4.restype = i32
    lib.draft_head_coarse_int4.argtypes = [P, i32, i32, i32, P, P, i32, P, P, P, P, sz, P]
    lib.draft_head_forward_row.restype = i32
    lib.draft_head_forward_row.argtypes = [P, i32, i32, i32, P, P, P, i64, i32, i32, P, P, P, P, P, P, P, i32, P, sz,
                                           P]
    lib.draft_head_forward_noalloc.restype = i32
    lib.draft_head_forward_noalloc.argtypes = [P, i32, i32, i32, P, P, P, i64, i32, i32, P, P, P, P, P, P, P, P,
                                               P, P]
    lib.draft_head_forward_int4.restype = i32
    lib.draft_head_forward_int4.argtypes = [P, i32, i32, i32, P, P, P, i64, i32, i32, P, P, P, P, P, P, P, P, sz,
                                            P, P, P]
    lib.draft_head_rerank_e4m3.restype = i32
    lib.draft_head_rerank_e4m3.argtypes = [P, P, P, i64, i32, i32, i32, P, P, i32, i32, P, P, P]
    lib.draft_head_forward_e4m3.restype = i32
    lib.draft_head_forward_e4m3.argtypes = [P, i32, i32, i32, P, P, P, P, i64, i32, i32, P, P, P, P, P, P, P, P,
                                            sz, P, P, P]
    lib.draft_head_rerank_nvfp4.restype = i32
    lib.draft_head_rerank_nvfp4.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, P, P, i32, i32, P, P, P]
    lib.draft_head_forward_nvfp4.restype = i32
    lib.draft_head_forward_nvfp4.argtypes = [P, i32, i32, i32, P, P, P, i64, P, i64, P, i32, i32, P, P, P, P, P,
                                             P, P, P, sz, P, P, P]
    lib.draft_head_logits_row.restype = i32
    lib.draft_head_logits_row.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
    lib.draft_head_stream_read.restype = i32
    lib.draft_head_stream_read.argtypes = [P, sz, P, P]
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/drafthead.h declares."""
    with open(_HEADER) as f:
        text = f.read()
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(draft_head_\w+)\s*\(", text, flags=re.M)


def draft_head_last_error() -> str:
    return load_library().draft_head_last_error().decode()


def _check(rc: int):
    if rc == DH_OK:
        return
    msg = draft_head_last_error()
    if rc in (DH_EINVAL, DH_ESHAPE, DH_EUNSUP):
        raise ValueError(f"drafthead error {rc}: {msg}")
    raise DraftHeadError(f"drafthead error {rc}: {msg}")


def _ptr(a) -> int | None:
    """Address of a numpy array or torch tensor (None -> NULL)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


# ------------------------------------------------------------------ host side
def draft_head_sizes(N: int, K: int) -> dict:
    lib = load_library()
    vals = [ctypes.c_size_t() for _ in range(4)]
    _check(lib.draft_head_sizes(N, K, *[ctypes.byref(v) for v in vals]))
    keys = ("packed_bytes", "scale_elems", "tiled_bytes", "tiled_pairs")
    return {k: v.value for k, v in zip(keys, vals)}


def draft_head_quantize_pack(w_bits: np.ndarray, nthreads: int = 0):
    """bf16 bits [N][K] -> (packed uint8 [N][K/4], S uint16 [N][K/128], ZS uint16 [N][K/128])."""
    lib = load_library()
    w = np.asarray(w_bits)
    if w.dtype != np.uint16 or w.ndim != 2:
        raise ValueError("w_bits must be a 2-D uint16 array of bf16 bit patterns")
    if w.strides[1] != 2:
        w = np.ascontiguousarray(w)
    n, k = w.shape
    ldw = w.strides[0] // 2
    packed = np.empty((n, max(k // 4, 1)), dtype=np.uint8)
    S = np.empty((n, max(k // GROUP, 1)), dtype=np.uint16)
    ZS = np.empty_like(S)
    _check(lib.draft_head_quantize_pack(_ptr(w), n, k, ldw, _ptr(packed), _ptr(S), _ptr(ZS), nthreads))
    return packed, S, ZS


def draft_head_quantize_pack_int4(w_bits: np.ndarray, nthreads: int = 0):
    """bf16 bits [N][K] -> the 4-bit head (packed uint8 [N][K/2], S, ZS uint16 [N][K/128])."""
    lib = load_library()
    w = np.asarray(w_bits)
    if w.dtype != np.uint16 or w.ndim != 2:
        raise ValueError("w_bits must be a 2-D uint16 array of bf16 bit patterns")
    if w.strides[1] != 2:
        w = np.ascontiguousarray(w)
    n, k = w.shape
    packed = np.empty((n, max(k // 2, 1)), dtype=np.uint8)
    S = np.empty((n, max(k // GROUP, 1)), dtype=np.uint16)
    ZS = np.empty_like(S)
    _check(lib.draft_head_quantize_pack_int4(_ptr(w), n, k, w.strides[0] // 2, _ptr(packed), _ptr(S), _ptr(ZS),
                                             nthreads))
    return packed, S, ZS


def draft_head_int4_as_int2(packed4: np.ndarray, S: np.ndarray, ZS: np.ndarray):
    """A 4-bit head as the 2-bit head of length 2K the device path runs:
    (packed uint8 [N][2K/4], S2, ZS2 uint16 [N][2K/128])."""
    lib = load_library()
    packed4 = np.ascontiguousarray(packed4, dtype=np.uint8)
    S = np.ascontiguousarray(S, dtype=np.uint16)
    ZS = np.ascontiguousarray(ZS, dtype=np.uint16)
    n, h = packed4.shape
    k = 2 * h
    packed2 = np.empty((n, h), dtype=np.uint8)
    S2 = np.empty((n, 2 * (k // GROUP)), dtype=np.uint16)
    ZS2 = np.empty_like(S2)
    _check(lib.draft_head_int4_as_int2(_ptr(packed4), _ptr(S), _ptr(ZS), n, k, _ptr(packed2), _ptr(S2), _ptr(ZS2)))
    return packed2, S2, ZS2


def draft_head_tile(packed: np.ndarray, S: np.ndarray, ZS: np.ndarray):
    """Canonical arrays -> (tiled codes uint8 [NBLK*64*K/4], pairs uint32 [NBLK*64*K/128])."""
    lib = load_library()
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    S = np.ascontiguousarray(S, dtype=np.uint16)
    ZS = np.ascontiguousarray(ZS, dtype=np.uint16)
    n, q4 = packed.shape
    k = 4 * q4
    if S.shape != (n, k // GROUP) or ZS.shape != S.shape:
        raise ValueError("S and ZS must be [N][K/128]")
    sizes = draft_head_sizes(n, k)
    tiled = np.empty(sizes["tiled_bytes"], dtype=np.uint8)
    pairs = np.empty(sizes["tiled_pairs"], dtype=np.uint32)
    _check(lib.draft_head_tile(_ptr(packed), _ptr(S), _ptr(ZS), n, k, _ptr(tiled), _ptr(pairs)))
    return tiled, pairs


def draft_head_tile_int4(packed4: np.ndarray, S: np.ndarray, ZS: np.ndarray):
    """A 4-bit head's canonical arrays -> its device form: its own code bytes
    in the tiles of a 2-bit head of length 2K, and its own pairs (tiled uint8
    [NBLK*64*K/2], pairs uint32 [NBLK*64*K/128])."""
    lib = load_library()
    packed4 = np.ascontiguousarray(packed4, dtype=np.uint8)
    S = np.ascontiguousarray(S, dtype=np.uint16)
    ZS = np.ascontiguousarray(ZS, dtype=np.uint16)
    n, h = packed4.shape
    k = 2 * h
    if S.shape != (n, k // GROUP) or ZS.shape != S.shape:
        raise ValueError("S and ZS must be [N][K/128]")
    sizes = draft_head_sizes(n, 2 * k)
    tiled = np.empty(sizes["tiled_bytes"], dtype=np.uint8)
    pairs = np.empty(sizes["tiled_pairs"] // 2, dtype=np.uint32)
    _check(lib.draft_head_tile_int4(_ptr(packed4), _ptr(S), _ptr(ZS), n, k, _ptr(tiled), _ptr(pairs)))
    return tiled, pairs


# ------------------------------------------------------------------ device side
def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _empty(shape, dtype, like):
    import torch
    return torch.empty(shape, dtype=dtype, device=like.device)


def draft_head_workspace_bytes(M: int, K: int) -> int:
    """Device workspace bytes the coarse pass needs for M rows of length K."""
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.draft_head_workspace_bytes(M, K, ctypes.byref(out)))
    return out.value


def workspace_for(M: int, K: int, device):
    """A device workspace for M rows of length K (zero-filled once; the library
    keeps the parts that must start at zero at zero)."""
    import torch
    return torch.zeros(draft_head_workspace_bytes(M, K), dtype=torch.uint8, device=device)


def _ws(workspace):
    return (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())


def draft_head_coarse(x, tiled, pairs, N: int, kcand: int = 8, cand_val=None, cand_id=None,
                      coarse_out=None, workspace=None, stream=None, bits: int = 2):
    """x: CUDA bf16 [M][K]; tiled/pairs: CUDA tensors in the draft_head_tile layout
    (bits = 4: draft_head_tile_int4's form); workspace: CUDA tensor of
    draft_head_workspace_bytes(M, K) bytes (2K for bits = 4; allocated when None).
    Returns (cand_val fp32 [M][NBLK*kcand], cand_id int32 [M][NBLK*kcand])."""
    import torch
    lib = load_library()
    M, K = x.shape
    nblk = (N + BLOCK_N - 1) // BLOCK_N
    if cand_val is None:
        cand_val = _empty((M, nblk * kcand), torch.float32, x)
    if cand_id is None:
        cand_id = _empty((M, nblk * kcand), torch.int32, x)
    if workspace is None:
        workspace = workspace_for(M, K * (2 if bits == 4 else 1), x.device)
    f = lib.draft_head_coarse_int4 if bits == 4 else lib.draft_head_coarse
    _check(f(_ptr(x), M, K, N, _ptr(tiled), _ptr(pairs), kcand, _ptr(cand_val), _ptr(cand_id), _ptr(coarse_out),
             *_ws(workspace), _stream(stream)))
    return cand_val, cand_id


def draft_head_rerank(x, w, cand_val, cand_id, R: int = 32, rr_id=None, rr_val=None, N=None,
                      stream=None):
    """x: CUDA bf16 [M][K]; w: CUDA bf16 [N][ldw]; candidates from draft_head_coarse.
    Returns (rr_id int32 [M][R], rr_val fp32 [M][R])."""
    import torch
    lib = load_library()
    M, K = x.shape
    n = w.shape[0] if N is None else N
    ldw = w.stride(0)
    ncand = cand_val.shape[1]
    if rr_id is None:
        rr_id = _empty((M, R), torch.int32, x)
    if rr_val is None:
        rr_val = _empty((M, R), torch.float32, x)
    _check(lib.draft_head_rerank(_ptr(x), _ptr(w), ldw, M, K, n, _ptr(cand_val), _ptr(cand_id), ncand,
                                 R, _ptr(rr_id), _ptr(rr_val), _stream(stream)))
    return rr_id, rr_val


def draft_head_rerank_e4m3(x, w8, wscale, cand_val, cand_id, R: int = 32, rr_id=None, rr_val=None, N=None,
                           stream=None):
    """draft_head_rerank from e4m3 rows: w8 CUDA uint8 [N][ldw] (e4m3 bytes),
    wscale CUDA fp32 [N].  Returns (rr_id int32 [M][R], rr_val fp32 [M][R])."""
    import torch
    lib = load_library()
    M, K = x.shape
    n = w8.shape[0] if N is None else N
    ncand = cand_val.shape[1]
    if rr_id is None:
        rr_id = _empty((M, R), torch.int32, x)
    if rr_val is None:
        rr_val = _empty((M, R), torch.float32, x)
    _check(lib.draft_head_rerank_e4m3(_ptr(x), _ptr(w8), _ptr(wscale), w8.stride(0), M, K, n, _ptr(cand_val),
                                      _ptr(cand_id), ncand, R, _ptr(rr_id), _ptr(rr_val), _stream(stream)))
    return rr_id, rr_val


def draft_head_rerank_nvfp4(x, w4, bscale, gscale, cand_val, cand_id, R: int = 32, rr_id=None, rr_val=None,
                            N=None, stream=None):
    """draft_head_rerank from NVFP4 rows: w4 CUDA uint8 [N][ldw] (two e2m1
    codes per byte, low nibble first), bscale CUDA uint8 [N][lds] (e4m3 scale
    per 16 elements), gscale CUDA fp32 [1].  Returns (rr_id, rr_val)."""
    import torch
    lib = load_library()
    M, K = x.shape
    n = w4.shape[0] if N is None else N
    ncand = cand_val.shape[1]
    if rr_id is None:
        rr_id = _empty((M, R), torch.int32, x)
    if rr_val is None:
        rr_val = _empty((M, R), torch.float32, x)
    _check(lib.draft_head_rerank_nvfp4(_ptr(x), _ptr(w4), w4.stride(0), _ptr(bscale), bscale.stride(0),
                                       _ptr(gscale), M, K, n, _ptr(cand_val), _ptr(cand_id), ncand, R, _ptr(rr_id),
                                       _ptr(rr_val), _stream(stream)))
    return rr_id, rr_val


def draft_head_logits_row(rr_id, rr_val, N: int, coarse=None, topk_only=False, out=None, stream=None):
    """The bf16 row handed to the caller: bf16(coarse) (or -inf with
    topk_only) with the reranked ids' exact values; returns int16 bits [M][N]."""
    import torch
    lib = load_library()
    M, R = rr_id.shape
    if out is None:
        out = torch.empty((M, N), dtype=torch.int16, device=rr_id.device)
    _check(lib.draft_head_logits_row(_ptr(coarse), _ptr(rr_id), _ptr(rr_val), M, N, R, 1 if topk_only else 0,
                                     _ptr(out), _stream(stream)))
    return out


DH_READ_BLOCKS = 2048


def draft_head_stream_read(buf, out=None, stream=None):
    """Read a CUDA tensor's bytes once (the device read-rate reference);
    returns the uint32 [DH_READ_BLOCKS] XOR folds of the workgroups' spans."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty(DH_READ_BLOCKS, dtype=torch.int32, device=buf.device)
    _check(lib.draft_head_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), _stream(stream)))
    return out


def draft_head_argmax(rr_id, rr_val, out_id=None, out_val=None, stream=None):
    """Returns (out_id int32 [M], out_val fp32 [M])."""
    import torch
    lib = load_library()
    M, R = rr_id.shape
    if out_id is None:
        out_id = _empty((M,), torch.int32, rr_id)
    if out_val is None:
        out_val = _empty((M,), torch.float32, rr_id)
    _check(lib.draft_head_argmax(_ptr(rr_id), _ptr(rr_val), M, R, _ptr(out_id), _ptr(out_val),
                                 _stream(stream)))
    return out_id, out_val


def forward_buffers(M: int, N: int, kcand: int, R: int, device):
    """Output tensors of one full call for M rows (what draft_head_forward fills)."""
    import torch
    ncand = ((N + BLOCK_N - 1) // BLOCK_N) * kcand
    return {"cand_val": torch.empty((M, ncand), dtype=torch.float32, device=device),
            "cand_id": torch.empty((M, ncand), dtype=torch.int32, device=device),
            "rr_id": torch.empty((M, R), dtype=torch.int32, device=device),
            "rr_val": torch.empty((M, R), dtype=torch.float32, device=device),
            "out_id": torch.empty((M,), dtype=torch.int32, device=device),
            "out_val": torch.empty((M,), dtype=torch.float32, device=device)}


def _event(ev):
    if ev is None:
        return None
    if ev.cuda_event == 0:
        raise ValueError("record a timing event once (torch creates it lazily) before passing it")
    return ev.cuda_event


def draft_head_forward(x, tiled, pairs, w, N: int, kcand: int = 8, R: int = 32, out=None,
                       coarse_out=None, workspace=None, stream=None, coarse_events=None, wscale=None,
                       bits: int = 2, bscale=None, gscale=None):
    """One full call (coarse -> rerank -> argmax) in one library call.

    w: the bf16 rows, or with wscale (fp32 [N]) the e4m3 rows (uint8), or
    with bscale and gscale the NVFP4 rows (uint8) of the rerank; out: dict from forward_buffers (allocated when None); workspace:
    as for draft_head_coarse; coarse_events: optional (start, stop)
    torch.cuda.Event pair that takes the coarse kernel's own dispatch
    timestamps.  Returns the dict of output tensors."""
    lib = load_library()
    M, K = x.shape
    if out is None:
        out = forward_buffers(M, N, kcand, R, x.device)
    if workspace is None:
        workspace = workspace_for(M, K * (2 if bits == 4 else 1), x.device)
    e0, e1 = (None, None) if coarse_events is None else (_event(coarse_events[0]), _event(coarse_events[1]))
    outs = (_ptr(out["cand_val"]), _ptr(out["cand_id"]), _ptr(out["rr_id"]), _ptr(out["rr_val"]),
            _ptr(out["out_id"]), _ptr(out["out_val"]), _ptr(coarse_out), *_ws(workspace), _stream(stream), e0, e1)
    if bits == 4:
        if wscale is not None or bscale is not None:
            raise ValueError("the 4-bit head reranks against bf16 rows")
        _check(lib.draft_head_forward_int4(_ptr(x), M, K, N, _ptr(tiled), _ptr(pairs), _ptr(w), w.stride(0),
                                           kcand, R, *outs))
    elif bscale is not None:
        _check(lib.draft_head_forward_nvfp4(_ptr(x), M, K, N, _ptr(tiled), _ptr(pairs), _ptr(w), w.stride(0),
                                            _ptr(bscale), bscale.stride(0), _ptr(gscale), kcand, R, *outs))
    elif wscale is None:
        _check(lib.draft_head_forward(_ptr(x), M, K, N, _ptr(tiled), _ptr(pairs), _ptr(w), w.stride(0), kcand,
                                      R, *outs))
    else:
        _check(lib.draft_head_forward_e4m3(_ptr(x), M, K, N, _ptr(tiled), _ptr(pairs), _ptr(w), _ptr(wscale),
                                           w.stride(0), kcand, R, *outs))
    return out


def draft_head_forward_row(x, tiled, pairs, w, N: int, kcand: int = 8, R: int = 32, topk_only: bool = False,
                           out=None, row=None, workspace=None, stream=None):
    """One call plus the bf16 row for the caller (bf16 rerank rows); returns
    the forward outputs with "row" (int16 [M][N] holding bf16 bits) added."""
    import torch
    lib = load_library()
    M, K = x.shape
    if out is None:
        out = forward_buffers(M, N, kcand, R, x.device)
    if row is None:
        row = torch.empty((M, N), dtype=torch.int16, device=x.device)
    if workspace is None:
        workspace = workspace_for(M, K, x.device)
    _check(lib.draft_head_forward_row(_ptr(x), M, K, N, _ptr(tiled), _ptr(pairs), _ptr(w), w.stride(0), kcand, R,
                                      _ptr(out["cand_val"]), _ptr(out["cand_id"]), _ptr(out["rr_id"]),
                                      _ptr(out["rr_val"]), _ptr(out["out_id"]), _ptr(out["out_val"]), _ptr(row),
                                      1 if topk_only else 0, *_ws(workspace), _stream(stream)))
    out["row"] = row
    return out


def draft_head_forward_noalloc(x, tiled, pairs, w, N: int, kcand: int = 8, R: int = 32, out=None,
                               coarse_out=None, stream=None, coarse_events=None):
    """draft_head_forward with the library's static scratch instead of a
    workspace (bf16 rerank rows); out: dict from forward_buffers (allocated
    here when None, which a caller that cannot allocate passes)."""
    lib = load_library()
    M, K = x.shape
    if out is None:
        out = forward_buffers(M, N, kcand, R, x.device)
    e0, e1 = (None, None) if coarse_events is None else (_event(coarse_events[0]), _event(coarse_events[1]))
    _check(lib.draft_head_forward_noalloc(_ptr(x), M, K, N, _ptr(tiled), _ptr(pairs), _ptr(w), w.stride(0), kcand,
                                          R, _ptr(out["cand_val"]), _ptr(out["cand_id"]), _ptr(out["rr_id"]),
                                          _ptr(out["rr_val"]), _ptr(out["out_id"]), _ptr(out["out_val"]),
                                          _ptr(coarse_out), _stream(stream), e0, e1))
    return out


class DraftHead:
    """Device-resident head: the tiled 2-bit arrays plus the bf16 weight the rerank reads.

    from_weight() quantises on the host with the library, tiles, and uploads.
    __call__(x) runs coarse -> rerank -> argmax on the current stream with one
    library call and returns a dict of the device tensors of every step;
    staged(x) does the same with one library call per step.
    """

    def __init__(self, tiled, pairs, w, N: int, K: int, kcand: int = 8, R: int = 32, wscale=None, bits: int = 2,
                 bscale=None, gscale=None):
        """w: the bf16 rows the rerank reads, or e4m3 rows (uint8) with their
        per-row fp32 scale `wscale` (a per-channel FP8 head), or NVFP4 rows
        (uint8) with their block scales `bscale` and global scale `gscale`.
        bits = 4: tiled and pairs hold a 4-bit head (draft_head_tile_int4)."""
        self.tiled, self.pairs, self.w, self.wscale = tiled, pairs, w, wscale
        self.bscale, self.gscale = bscale, gscale
        self.N, self.K, self.kcand, self.R, self.bits = N, K, kcand, R, bits

    @classmethod
    def from_weight(cls, w_bits: np.ndarray, kcand: int = 8, R: int = 32, device="cuda",
                    packed=None, bits: int = 2):
        """bits = 2: the head of the page's default configuration; bits = 4:
        the 4-bit head (packed: draft_head_quantize_pack_int4's arrays)."""
        import torch
        n, k = w_bits.shape
        if bits == 4:
            packed4 = packed if packed is not None else draft_head_quantize_pack_int4(w_bits)
            tiled, pairs = draft_head_tile_int4(*packed4)
        else:
            if packed is None:
                packed = draft_head_quantize_pack(w_bits)
            tiled, pairs = draft_head_tile(*packed)
        t_tiled = torch.from_numpy(tiled).to(device)
        t_pairs = torch.from_numpy(pairs.view(np.int32)).to(device)
        t_w = torch.from_numpy(np.ascontiguousarray(w_bits).view(np.int16)).to(device)
        return cls(t_tiled, t_pairs, t_w, n, k, kcand, R, bits=bits)

    def __call__(self, x, coarse_out=None, stream=None, out=None, coarse_events=None, workspace=None):
        return draft_head_forward(x, self.tiled, self.pairs, self.w, self.N, self.kcand, self.R, out=out,
                                  coarse_out=coarse_out, workspace=workspace, stream=stream,
                                  coarse_events=coarse_events, wscale=self.wscale, bits=self.bits,
                                  bscale=self.bscale, gscale=self.gscale)

    def logits_row(self, x, topk_only=False, stream=None, out=None, row=None, workspace=None):
        """One call plus the bf16 row the page hands to its caller (full, or
        top-k only), in one library call; returns the forward outputs with
        "row" added."""
        if self.bits != 2 or self.wscale is not None or self.bscale is not None:
            raise ValueError("the row for the caller is built with the 2-bit head and bf16 rerank rows")
        return draft_head_forward_row(x, self.tiled, self.pairs, self.w, self.N, self.kcand, self.R, topk_only,
                                      out=out, row=row, workspace=workspace, stream=stream)

    def logits_row_staged(self, x, topk_only=False, stream=None):
        """The same row from the fp32 coarse row: a forward with coarse_out,
        then draft_head_logits_row."""
        import torch
        coarse = torch.empty((x.shape[0], self.N), dtype=torch.float32, device=x.device)
        out = self(x, coarse_out=coarse, stream=stream)
        out["row"] = draft_head_logits_row(out["rr_id"], out["rr_val"], self.N,
                                           coarse=None if topk_only else coarse, topk_only=topk_only,
                                           stream=stream)
        out["coarse"] = coarse
        return out

    def staged(self, x, coarse_out=None, stream=None):
        """The same call as three library calls (coarse, rerank, argmax)."""
        cv, ci = draft_head_coarse(x, self.tiled, self.pairs, self.N, self.kcand,
                                   coarse_out=coarse_out, stream=stream, bits=self.bits)
        if self.bscale is not None:
            rr_id, rr_val = draft_head_rerank_nvfp4(x, self.w, self.bscale, self.gscale, cv, ci, self.R, N=self.N,
                                                    stream=stream)
        elif self.wscale is None:
            rr_id, rr_val = draft_head_rerank(x, self.w, cv, ci, self.R, N=self.N, stream=stream)
        else:
            rr_id, rr_val = draft_head_rerank_e4m3(x, self.w, self.wscale, cv, ci, self.R, N=self.N, stream=stream)
        out_id, out_val = draft_head_argmax(rr_id, rr_val, stream=stream)
        return {"cand_val": cv, "cand_id": ci, "rr_id": rr_id, "rr_val": rr_val,
                "out_id": out_id, "out_val": out_val}
