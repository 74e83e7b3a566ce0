"""Shared helpers of the test suite (no method arithmetic here)."""
import sys

import numpy as np


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x: np.ndarray, y: np.ndarray) -> float:
    """max |x - y| / max |y| over one slice (relative to the slice's scale)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    den = np.abs(y).max()
    if den == 0:
        return float(np.abs(x - y).max())
    return float(np.abs(x - y).max() / den)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def cuda_bits(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def host_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)
