"""Near-tie planting for the LM-head verification workload, driven by the oracle (test
infrastructure: the expected answers always come from the oracle on the final W).

For each planted row (hidden vector x_i):
  * v1 = the oracle's exact argmax of x_i on the current W; v2 != v1 a seeded index not
    used by any other plant;
  * even plants: W[v2] := W[v1], an exact tie whose expected answer is min(v1, v2);
  * odd plants: also move W[v2, k*] by one BF16 step (direction seeded), with k* the
    column minimising |x_ik| * ulp(W[v1, k]) over nonzero finite entries, so that the
    two exact logits differ by far less than one FP32 ulp of the top logit.
Afterwards every planted row is checked: its exact top two are v1 and v2 and their gap
is at most one FP32 ulp of the top logit (exactly zero for even plants)."""
from __future__ import annotations

import math

import numpy as np

from oracle import w12_oracle as o


def _fp32_ulp(v: float) -> float:
    a = abs(np.float32(v))
    return float(np.spacing(a))


def _argmax_among(x_row, w, z64, s64, k):
    """The oracle's exact argmax for one row, given float64 logits of the current W:
    the oracle's rigorous filter picks the candidates, exact logits decide."""
    thr = z64.max() - o.fp64_filter_width(k, s64.max())
    cand = np.nonzero(z64 >= thr)[0]
    sub, _ = o.argmax_exact(x_row[None, :], w[cand])
    return int(cand[int(sub[0])])


def plant_near_ties(x, w, rng_of_row):
    """Plant one near-tie per row of x ([R, K] BF16 bits) into a copy of w ([V, K]).
    rng_of_row(i) -> numpy Generator for plant i.  Returns (w_planted, pairs) with
    pairs[i] = (v1, v2)."""
    w = w.copy()
    r_rows, k = x.shape
    vocab = w.shape[0]
    z64, s64 = o.gemm_reference(x, w)
    used = set()
    pairs = []
    for i in range(r_rows):
        g = rng_of_row(i)
        v1 = _argmax_among(x[i], w, z64[i], s64[i], k)
        used.add(v1)
        while True:
            v2 = int(g.integers(0, vocab))
            if v2 not in used:
                break
        used.add(v2)
        w[v2] = w[v1]
        if i % 2 == 1:
            sg, ex, ma, _ = o.split_fields(w[v1])
            ex = ex.astype(np.int64)
            ok = (ex < 255) & ((ex > 0) | (ma > 0)) & ((x[i] & 0x7FFF) != 0)
            ulp = np.where(ex > 0, 2.0 ** (ex.astype(np.float64) - 134), 2.0 ** -133)
            cost = np.where(ok, np.abs(o.bf16_to_f64(x[i])) * ulp, np.inf)
            kk = int(np.argmin(cost))
            step = 1 if g.integers(0, 2) else -1
            b = int(w[v1, kk])
            if (b & 0x7FFF) == 0x7F7F and step == 1:    # keep the value finite
                step = -1
            w[v2, kk] = np.uint16(b + step)
        zv, sv = o.gemm_reference(x, w[v2:v2 + 1])
        z64[:, v2] = zv[:, 0]
        s64[:, v2] = sv[:, 0]
        pairs.append((v1, v2))
    return w, pairs


def check_plants(x, w, pairs):
    """Assert that each planted row's exact top two are its pair, within one FP32 ulp."""
    am, _ = o.argmax_exact(x, w)
    z64, _ = o.gemm_reference(x, w)
    for i, (v1, v2) in enumerate(pairs):
        z1 = o.exact_logit(x[i], w[v1])
        z2 = o.exact_logit(x[i], w[v2])
        assert int(am[i]) in (v1, v2), (i, int(am[i]), v1, v2)
        ztop = math.ldexp(float(max(z1, z2)), -o.EXACT_SHIFT)
        gap = abs(z1 - z2)
        assert gap <= int(_fp32_ulp(ztop) * 2.0 ** o.EXACT_SHIFT), (i, gap)
        if i % 2 == 0:
            assert gap == 0 and int(am[i]) == min(v1, v2)
        else:
            assert gap > 0
        # the pair is the exact top two: every other index is exactly below both
        lo = math.ldexp(float(min(z1, z2)), -o.EXACT_SHIFT)
        others = np.nonzero(z64[i] >= lo - 1e-6)[0]
        for v in others:
            if v in (v1, v2):
                continue
            assert o.exact_logit(x[i], w[v]) < min(z1, z2), (i, int(v))
    return am
