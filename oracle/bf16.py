"""Exact bf16 widening and fp64 -> bf16 / fp32 rounding for the oracle.

bf16 is the top half of an IEEE binary32: 1 sign, 8 exponent, 7 fraction bits.
Rounding is round-to-nearest, ties to even, applied once from the fp64 value.
"""

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (float32, or uint16 bf16 bits) -> exact float64 values."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), as fp64.

    For x = m * 2**e with m in [0.5, 1), bf16 keeps 8 significant bits, so the
    spacing is 2**(e - 8); below the normal range the spacing stays 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(np.ones_like(x), e - 8)
    y = np.rint(x / q) * q
    y = np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype; result returned as fp64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


def to_bits(x: np.ndarray) -> np.ndarray:
    """fp64 values that are already bf16-representable -> uint16 bits."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
