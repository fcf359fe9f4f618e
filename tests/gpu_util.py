"""Helpers shared by the GPU tests: host<->device transfer of BF16 bit patterns and
structured test matrices.  No arithmetic of the method lives here."""
import sys

import numpy as np


def say(*a):
    """Print the case about to run and flush, so a failing GPU step names itself."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, torch, dev="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def to_host(t) -> np.ndarray:
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def wide_exponents(shape, g, lo=100, hi=140):
    """Finite BF16 with exponents spread over [lo, hi): many escapes, non-run codebook."""
    n, k = shape
    s = g.integers(0, 2, (n, k)).astype(np.uint32)
    e = g.integers(lo, hi, (n, k)).astype(np.uint32)
    m = g.integers(0, 128, (n, k)).astype(np.uint32)
    return ((s << 15) | (e << 7) | m).astype(np.uint16)


def narrow_exponents(shape, g):
    n, k = shape
    s = g.integers(0, 2, (n, k)).astype(np.uint32)
    e = g.integers(120, 123, (n, k)).astype(np.uint32)
    m = g.integers(0, 128, (n, k)).astype(np.uint32)
    return ((s << 15) | (e << 7) | m).astype(np.uint16)
