"""bf16 conversions for the oracle (own implementation).

bf16 is the upper half of an IEEE float32.  Widening is exact.  Narrowing
follows what the quantiser on the radiance_drafthead.py page does when it
stores the scale pair with `.to(torch.bfloat16)`: round to nearest, ties to
even (reading: the page does not state the mode; this is torch's).
"""
import numpy as np


def to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def to_f64(bits):
    return to_f32(bits).astype(np.float64)


def from_f32(values):
    """float32 -> bf16 bit patterns, round to nearest even; NaN -> canonical NaN."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    isnan = np.isnan(v)
    if np.any(isnan):
        r = np.where(isnan, np.uint16(0x7FC0), r)
    return r
