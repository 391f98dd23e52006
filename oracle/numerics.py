"""Rounding helpers of the oracle (float64 in, float64 out).

Pinned by tests/test_oracle_pins.py against torch's own float32->bfloat16
cast on values that float32 holds exactly.
"""
import numpy as np


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float64. bfloat16 keeps 8 significant bits; values here are finite
    and far from the bfloat16 overflow and subnormal ranges (zeros pass
    through unchanged)."""
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)              # x = mant * 2**expo, 0.5 <= |mant| < 1
    scaled = np.ldexp(mant, 8)            # 8 significant bits before the point
    return np.ldexp(np.rint(scaled), expo - 8)   # rint = round half to even


def round_to_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
