"""bf16 rounding used by the oracle's outputs (test infrastructure only).

bf16 keeps the top 16 bits of an IEEE binary32 value.  Rounding a float to
bf16 is round-to-nearest, ties-to-even on the 16 dropped bits, taken from the
value's binary32 form.  A float64 result is first rounded to binary32 (the
library's fp32 cast, itself nearest-even); the double rounding this implies is
the documented reading for values produced in float64.
"""
import numpy as np


def round_f32_to_bf16(x32: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest bf16 (ties to even); returns the
    rounded values as float32.  NaN stays NaN; overflow goes to +-inf."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    keep = u >> 16
    low = u & 0xFFFF
    # round up when the dropped half is above the midpoint, or exactly the
    # midpoint and the kept part is odd
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & 1) == 1))
    keep = keep + up.astype(np.uint64)
    out = (keep << 16).astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x32)
    out[nan] = np.float32(np.nan)
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> binary32 -> bf16, returned as float64 holding bf16 values."""
    return round_f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32)).astype(np.float64)


def bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) into float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
