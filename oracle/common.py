"""Input widening for the oracle (test infrastructure only).

Logits arrive either as float32 values or as bf16 bit patterns stored in uint16.
Both are widened exactly to float64: a bf16 value is the upper 16 bits of the
float32 with the same sign, exponent and leading mantissa bits.
"""

import numpy as np


def widen_logits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of float32 logits or of bf16 logits given as uint16 bits."""
    if dtype == "bf16":
        bits = np.asarray(values)
        if bits.dtype != np.uint16:
            raise ValueError("bf16 logits must be given as uint16 bit patterns")
        wide = bits.astype(np.uint32) * np.uint32(65536)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "f32":
        vals = np.asarray(values)
        if vals.dtype != np.float32:
            raise ValueError("f32 logits must be float32")
        return vals.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
