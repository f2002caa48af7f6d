"""Storage-format decoding and round-to-nearest-even, in float64.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module. It shares no code with the HIP path.

The pages do not state how outputs are rounded (reading: IEEE
round-to-nearest-even, the rounding a dtype cast performs). Rounding here is a
single rounding straight from float64 to the target format.
"""
from __future__ import annotations

import numpy as np


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64 (exact for every format handled here)."""
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be given as uint16 bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        if a.dtype != np.float16:
            raise TypeError("f16 data must be numpy float16")
        return a.astype(np.float64)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 data must be numpy float32")
        return a.astype(np.float64)
    if dtype in ("i8", "i32"):
        return a.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


# (significand bits including the implicit one, smallest normal exponent e such
#  that values in [2**(e-1), 2**e) are normal, largest finite value)
_FORMATS = {
    "bf16": (8, -125, float.fromhex("0x1.fe00000000000p+127")),
    "f16": (11, -13, 65504.0),
}


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest ``dtype`` value, ties to even.

    Values in [2**(e-1), 2**e) are spaced 2**(e - p) apart for a p-bit
    significand; below the smallest normal binade the spacing stays fixed
    (gradual underflow). Scaling by that spacing is exact, and ``numpy.rint``
    rounds half to even. Results beyond the largest finite value become inf.
    ``f32`` returns the input unchanged: the float32 test outputs are compared
    against the unrounded value.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.copy()
    p, emin, fmax = _FORMATS[dtype]
    _, e = np.frexp(x)
    e = np.maximum(e, emin)
    ulp = np.ldexp(1.0, e - p)
    with np.errstate(invalid="ignore", over="ignore"):
        q = np.rint(x / ulp) * ulp
        q = np.where(np.abs(q) > fmax, np.copysign(np.inf, x), q)
    return np.where(np.isfinite(x), q, x)
