"""Helpers shared by the GPU tests: host<->device transfer of BF16 bit patterns,
structured test matrices, and the reference of the RMS GEMM (the oracle's exact product
divided by the row's RMS).  No arithmetic of the method lives here."""
import sys

import numpy as np

from oracle import w12_oracle as o
import w12_inputs as wi


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


def rms_reference(x: np.ndarray, w: np.ndarray):
    """Reference of the RMS GEMM (harness op of the layer chain, not the method):
    (x . W^T) / rms(x) per row, rms(x) = sqrt(mean_k x^2) in FP64 from the BF16 values,
    with the magnitude scale S divided the same way, for oracle.gemm_accept."""
    z, s = o.gemm_reference(x, w)
    xf = wi.bf16_bits_to_f32(x).astype(np.float64)
    r = np.sqrt((xf * xf).mean(axis=1))[:, None]
    return z / r, s / r
