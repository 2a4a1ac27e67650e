"""Exact widening of the kernel's input dtypes to float64 (oracle side).

Test infrastructure only (see the package docstring).

bf16 is the upper half of an IEEE fp32, so shifting the 16-bit pattern left by
16 bits gives the fp32 with the same value, which widens to fp64 exactly.
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16/int16 bf16 bit patterns -> float64 values (exact)."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen kernel-side data to float64. ``dtype`` is "bf16" (x holds bit
    patterns) or "f32" (x holds float32 values)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
