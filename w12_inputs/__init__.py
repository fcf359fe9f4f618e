"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and rounds them to BF16; it holds none of
the W12 method's arithmetic (no encode, decode, product or argmax).  Both the
CPU oracle tests and the GPU tests/bench take their inputs from here, so the
two sides see identical bits.

Seeding convention: ``numpy.random.default_rng([2026, c, t])`` where ``c`` is
the workload number (1..5, 0 for ad-hoc test cases) and ``t`` a tensor id.
Gaussian tensors are drawn in float32, scaled by ``float32(sigma)`` and
rounded to BF16 with round-to-nearest-even on the float32 bit pattern.

Workload shapes (a dense ~22B decoder: hidden 5120, grouped k/v 1024, MLP
17408, vocabulary 151936, 64 layers):

====  =========================================================================
 1    single linear layer: W [1024, 1024] ~N(0, 0.02^2), x [1, 1024] ~N(0, 1)
 2    attention projection with exponent outliers: W [5120, 5120] ~N(0, 0.02^2)
      with 0.1% of entries (uniform positions, no repeats) scaled by 2^s,
      s ~ U{6..12}; x [1, 5120]
 3    MLP block: gate+up W [34816, 5120], down W [5120, 17408]; x rows ~N(0, 1);
      M in {1, 4, 8, 16, 32}
 4    LM head W [151936, 5120] ~N(0, 0.02^2); M = 16 hidden rows ~N(0, 1)
 5    64 layers x {q, k, v, o, gate, up, down} + LM head, M = 24 (generated
      on the device, see ``device_layer_weight``)
====  =========================================================================
"""
from __future__ import annotations

import numpy as np

SIGMA_W = 0.02

# tensor ids inside one workload
T_W, T_W2, T_X, T_X2, T_OUT_POS, T_OUT_EXP, T_P, T_R, T_TIE = 0, 1, 2, 3, 4, 5, 6, 7, 8

CONFIG_SHAPES = {
    1: {"w": (1024, 1024), "m": (1,)},
    2: {"w": (5120, 5120), "m": (1,)},
    3: {"gate_up": (34816, 5120), "down": (5120, 17408), "m": (1, 4, 8, 16, 32)},
    4: {"w": (151936, 5120), "m": (16,)},
    5: {"hidden": 5120, "kv": 1024, "mlp": 17408, "vocab": 151936, "layers": 64, "m": (24,)},
}

# config 5 layer matrices as (name, n_out, k_in)
LAYER_MATS = (("q", 5120, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 5120),
              ("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408))


def rng(c: int, t: int, extra: int | None = None) -> np.random.Generator:
    key = [2026, int(c), int(t)] if extra is None else [2026, int(c), int(t), int(extra)]
    return np.random.default_rng(key)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (round to nearest, ties to even); returns uint16 bits.
    Inputs here are finite, so no NaN special case is needed."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian_bf16(shape, sigma: float, g: np.random.Generator, chunk_rows: int = 4096) -> np.ndarray:
    """BF16 bits of float32(N(0,1)) * float32(sigma), drawn row-chunk by row-chunk (same
    stream as one big draw) to bound the float32 temporary."""
    n, k = shape
    out = np.empty((n, k), dtype=np.uint16)
    s = np.float32(sigma)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        z = g.standard_normal((r1 - r0, k), dtype=np.float32)
        z *= s
        out[r0:r1] = f32_to_bf16_bits(z)
    return out


def weight(c: int, t: int, shape, sigma: float = SIGMA_W) -> np.ndarray:
    return gaussian_bf16(shape, sigma, rng(c, t))


def activations(c: int, t: int, m: int, k: int) -> np.ndarray:
    """x rows ~N(0,1) in BF16, [m, k]."""
    return gaussian_bf16((m, k), 1.0, rng(c, t, m))


def add_exponent_outliers(w: np.ndarray, frac: float, c: int, lo: int = 6, hi: int = 12) -> np.ndarray:
    """Scale floor(frac*N*K) distinct uniformly placed entries by 2^s, s ~ U{lo..hi}.
    Scaling by a power of two is exact in BF16 (only the exponent field moves), so the
    new bits are formed by adding s to the exponent field; entries whose exponent would
    leave the finite range (or that are zero/subnormal) are left unchanged."""
    w = w.copy()
    flat = w.reshape(-1)
    cnt = int(np.floor(frac * flat.size))
    pos = rng(c, T_OUT_POS).choice(flat.size, size=cnt, replace=False)
    s = rng(c, T_OUT_EXP).integers(lo, hi + 1, size=cnt)
    b = flat[pos].astype(np.int64)
    e = (b >> 7) & 0xFF
    ok = (e > 0) & (e + s < 255)
    e2 = np.where(ok, e + s, e)
    flat[pos] = ((b & 0x807F) | (e2 << 7)).astype(np.uint16)
    return w


def config_weights(c: int):
    """Host BF16 weights for workloads 1..4 (dict name -> uint16 [N, K])."""
    if c == 1:
        return {"w": weight(1, T_W, CONFIG_SHAPES[1]["w"])}
    if c == 2:
        return {"w": add_exponent_outliers(weight(2, T_W, CONFIG_SHAPES[2]["w"]), 0.001, 2)}
    if c == 3:
        return {"gate_up": weight(3, T_W, CONFIG_SHAPES[3]["gate_up"]),
                "down": weight(3, T_W2, CONFIG_SHAPES[3]["down"])}
    if c == 4:
        return {"w": weight(4, T_W, CONFIG_SHAPES[4]["w"])}
    raise ValueError(c)


def random_bits(shape, g: np.random.Generator) -> np.ndarray:
    """Uniformly random 16-bit patterns (every BF16 value including NaN/Inf/subnormals)."""
    return g.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def all_bf16_patterns() -> np.ndarray:
    """A [512, 128] matrix holding each of the 65,536 BF16 bit patterns exactly once."""
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(512, 128)


def device_layer_seed(layer: int, mat: int) -> int:
    """Seed of torch.Generator('cuda') for config-5 matrix `mat` (index into LAYER_MATS,
    7 = LM head) of `layer`."""
    return 2026_0500 + 8 * layer + mat


def device_layer_weight(torch, layer: int, mat: int, n: int, k: int, device="cuda"):
    """Config-5 weights drawn on the device: randn(float32) * 0.02 -> bfloat16 (RNE)."""
    g = torch.Generator(device=device)
    g.manual_seed(device_layer_seed(layer, mat))
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    w.mul_(SIGMA_W)
    return w.to(torch.bfloat16)


# ----------------------------------------------------------------------------- FP8 weights
F8_MAX = 448.0     # largest finite OCP FP8 E4M3 value
F8_BLOCK = 128     # checkpoint block: one scale per 128 x 128 weights


def f8_quantize(torch, w):
    """Checkpoint form of a float32 weight w [n, k] (a torch tensor on any device; k a
    multiple of 128): one FP32 scale per 128 x 128 block, s = (block max |w|) / 448 (1 for
    an all-zero block; the last block row covers the rows past the last multiple of 128),
    and codes q = w / s, clamped to +-448 and cast by torch to float8_e4m3fn (round to
    nearest even), returned as uint8 bytes.  Returns (q uint8 [n, k], s float32
    [ceil(n/128), k/128])."""
    n, k = w.shape
    nbk = (n + F8_BLOCK - 1) // F8_BLOCK
    wp = torch.nn.functional.pad(w, (0, 0, 0, nbk * F8_BLOCK - n))
    amax = wp.abs().reshape(nbk, F8_BLOCK, k // F8_BLOCK, F8_BLOCK).amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / F8_MAX, torch.ones_like(amax)).to(torch.float32)
    srow = s.repeat_interleave(F8_BLOCK, 0)[:n].repeat_interleave(F8_BLOCK, 1)
    v = (w / srow).clamp(-F8_MAX, F8_MAX)
    return v.to(torch.float8_e4m3fn).view(torch.uint8), s


def f8_weight(c: int, t: int, shape, sigma: float = SIGMA_W):
    """Host FP8 checkpoint weight: the BF16 Gaussian weight(c, t, shape) in float32,
    quantized by f8_quantize.  Returns numpy (q uint8 [n, k], s float32)."""
    import torch
    w = torch.from_numpy(bf16_bits_to_f32(weight(c, t, shape, sigma)))
    q, s = f8_quantize(torch, w)
    return q.numpy(), s.numpy()


def device_f8_weight(torch, seed: int, n: int, k: int, device="cuda"):
    """FP8 checkpoint weight drawn on the device: randn(float32) * 0.02 from
    torch.Generator(device) seeded with `seed`, quantized by f8_quantize."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    w.mul_(SIGMA_W)
    return f8_quantize(torch, w)


# ----------------------------------------------------------------------------- workload 4
VERIFY_BATCHES = 3        # batch 0 plain, batches 1-2 carry the 32 near-tie rows


def verify_batch_x(b: int, m: int = 16, k: int = 5120) -> np.ndarray:
    """Hidden rows of LM-head batch b (~N(0,1) BF16)."""
    if b == 0:
        return activations(4, T_X, m, k)
    return gaussian_bf16((m, k), 1.0, rng(4, T_X, 100 + b))


def verify_mismatch(b: int, vocab: int, m: int = 16):
    """(p, r) of batch b: the draft's first mismatch position p in 0..m (m = none) and
    the offset r in [0, vocab - 2] that makes the wrong token."""
    p = int(rng(4, T_P, b).integers(0, m + 1))
    r = int(rng(4, T_R, b).integers(0, vocab - 1))
    return p, r


# Batched verification: 24 requests (the largest of the batched request counts the
# pages report, 16, 20 and 24) of 5 rows each: 4 drafted tokens and the bonus row.
BATCHED_REQUESTS, BATCHED_ROWS = 24, 5


def batched_verify_x(n_req: int = BATCHED_REQUESTS, rows: int = BATCHED_ROWS,
                     k: int = 5120) -> np.ndarray:
    """Hidden rows of the batched verification, request after request (~N(0,1) BF16)."""
    return gaussian_bf16((n_req * rows, k), 1.0, rng(4, T_X, 200))


def batched_verify_table(vocab: int, n_req: int = BATCHED_REQUESTS, rows: int = BATCHED_ROWS):
    """Request table and planted mismatches: row offsets [n_req + 1], draft lengths
    [n_req] (rows - 1 each), and per request the first mismatch position p in
    0..rows-1 (rows - 1 = none) with the offset r in [0, vocab - 2] of the wrong token."""
    off = (np.arange(n_req + 1) * rows).astype(np.int32)
    nd = np.full(n_req, rows - 1, dtype=np.int32)
    p = rng(4, T_P, 200).integers(0, rows, n_req)
    r = rng(4, T_R, 200).integers(0, vocab - 1, n_req)
    return off, nd, p, r


def tie_rng(b: int, row: int) -> np.random.Generator:
    """Random choices of the near-tie plant for row `row` of batch b."""
    return rng(4, T_TIE, 1000 * b + row)


# ----------------------------------------------------------------------------- workload 5
def device_lm_head_seed() -> int:
    return device_layer_seed(64, 7)


def device_lm_head(torch, vocab: int, k: int, device="cuda"):
    """The decode step's LM head, drawn on the device like the layer matrices."""
    return device_layer_weight(torch, 64, 7, vocab, k, device)


def decode_step_x(m: int = 24, k: int = 5120) -> np.ndarray:
    """h0 of the decode-step chain, ~N(0,1) BF16 [m, k]."""
    return activations(5, T_X, m, k)


def decode_step_draft(vocab: int, m: int = 24) -> np.ndarray:
    """Seeded draft tokens for the chain's LM-head verify."""
    return rng(5, T_P).integers(0, vocab, size=m).astype(np.int32)
