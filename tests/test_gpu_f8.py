"""GPU parity of the FP8 GEMM (E4M3 codes with FP32 128 x 128 block scales, BF16
activations) against the CPU oracle, element by element, through the C ABI: the tile
bytes exactly, every output by oracle.gemm_accept (a hand-worked example bit for bit).
Shapes span several tiles, ragged 128-row scale blocks, odd row-block counts, K splits and
the longest K; m covers the 16-, 32-, 64- and 128-column x tiles and their ragged edges.
Also the grouped launches, the RMS forms, the prepared calls and the binding's routing
by weight format."""
import numpy as np
import pytest

from oracle import w12_oracle as o
import w12_inputs as wi
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu

# (n, k): one tile; a partial last scale-block row (144 = 128 + 16); odd row-block counts
# and tile columns; many row-blocks; a long K on few rows (split); 2049 row-blocks (the
# 10-wave workgroups from 17 rows on, a partial last scale block)
SHAPES = [(16, 128), (144, 640), (272, 1280), (2080, 512), (64, 4096), (32784, 256)]
MS = [1, 2, 3, 5, 8, 16, 17, 24, 32, 33, 48, 64, 65, 96, 128]


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import lossless_bit_weight_w12_amd as w12
    w12.lib()
    return torch, w12


def random_codes(shape, g):
    """Uniform E4M3 codes without the NaN pattern: every finite value, subnormals included."""
    q = g.integers(0, 256, shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    return q


def random_scales(n, k, g):
    return (g.uniform(0.5, 2.0, ((n + 127) // 128, k // 128))
            * 2.0 ** g.integers(-14, 2, ((n + 127) // 128, k // 128))).astype(np.float32)


def run(torch, w12, x, q, s):
    n, k = q.shape
    qt = w12.f8_tile(torch.from_numpy(q).to("cuda:0"))
    y = w12.gemm_f8(to_dev(x, torch), qt, torch.from_numpy(s).to("cuda:0"), n, k)
    torch.cuda.synchronize()
    return qt, y


def check(y_dev, x, q, s):
    z, sa = o.gemm_f8_reference(x, q, s)
    ok = o.gemm_accept(to_host(y_dev), z, sa)
    bad = np.argwhere(~ok)
    assert ok.all(), f"{bad.shape[0]} outputs outside tolerance, first {bad[:4].tolist()}"


@pytest.mark.parametrize("n,k", SHAPES)
def test_f8_tile_bytes(env, n, k):
    torch, w12 = env
    g = np.random.default_rng(8100 + n + k)
    q = random_codes((n, k), g)
    say("f8 tile", n, k)
    qt = w12.f8_tile(torch.from_numpy(q).to("cuda:0"))
    torch.cuda.synchronize()
    assert np.array_equal(qt.cpu().numpy(), o.f8_pack(q))


@pytest.mark.parametrize("m", MS)
def test_gemm_f8_checkpoint_weights(env, m):
    """Gaussian weights in checkpoint form (block max mapped to 448), x ~ N(0, 1)."""
    torch, w12 = env
    for i, (n, k) in enumerate(SHAPES):
        say("gemm f8 checkpoint", m, n, k)
        q, s = wi.f8_weight(0, 40 + i, (n, k))
        x = wi.gaussian_bf16((m, k), 1.0, np.random.default_rng(8200 + 16 * m + i))
        _, y = run(torch, w12, x, q, s)
        check(y, x, q, s)


@pytest.mark.parametrize("m", [1, 4, 16, 32, 64, 128])
def test_gemm_f8_random_codes_and_scales(env, m):
    """Every finite code (subnormals included) under block scales spread over 2^-15..2^2."""
    torch, w12 = env
    g = np.random.default_rng(8300 + m)
    for n, k in SHAPES:
        say("gemm f8 random codes", m, n, k)
        q = random_codes((n, k), g)
        s = random_scales(n, k, g)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        _, y = run(torch, w12, x, q, s)
        check(y, x, q, s)


def test_gemm_f8_zero_and_negative_scales(env):
    """A zero block contributes nothing; negative scales are applied with their sign."""
    torch, w12 = env
    g = np.random.default_rng(8400)
    n, k = 272, 1280
    q = random_codes((n, k), g)
    s = random_scales(n, k, g)
    s[0, 3] = 0.0
    s[1, :] *= -1.0
    for m in (3, 32, 100):
        say("gemm f8 zero/negative scales", m)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        _, y = run(torch, w12, x, q, s)
        check(y, x, q, s)


def test_gemm_f8_nan_code_poisons_its_row(env):
    torch, w12 = env
    g = np.random.default_rng(8500)
    n, k = 144, 640
    q = random_codes((n, k), g)
    q[5, 300] = 0x7F
    q[130, 7] = 0xFF
    s = random_scales(n, k, g)
    for m in (2, 40):
        say("gemm f8 NaN code", m)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        _, y = run(torch, w12, x, q, s)
        yf = y.float().cpu().numpy()
        assert np.isnan(yf[:, [5, 130]]).all()
        keep = np.setdiff1d(np.arange(n), [5, 130])
        q2 = q.copy()
        q2[5, 300] = 0
        q2[130, 7] = 0
        z, sa = o.gemm_f8_reference(x, q2, s)
        assert o.gemm_accept(to_host(y)[:, keep], z[:, keep], sa[:, keep]).all()


def test_gemm_f8_deterministic_and_overwrites(env):
    """Repeated calls (K split and whole) give identical bits and overwrite y entirely."""
    torch, w12 = env
    g = np.random.default_rng(8600)
    for m, (n, k) in [(1, (64, 4096)), (24, (272, 1280)), (128, (2080, 512))]:
        say("gemm f8 determinism", m, n, k)
        q = random_codes((n, k), g)
        s = random_scales(n, k, g)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        qt, y0 = run(torch, w12, x, q, s)
        st = torch.from_numpy(s).to("cuda:0")
        xt = to_dev(x, torch)
        out = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        for _ in range(3):
            y = w12.gemm_f8(xt, qt, st, n, k, out=out)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
        check(y0, x, q, s)


@pytest.mark.parametrize("m", [1, 5, 16, 24, 33, 64, 128])
def test_gemm_f8_group(env, m):
    """q, k, v-like and gate, up-like groups in one launch: every output of every weight
    against the oracle (segments with partial last scale blocks and odd row-block counts)."""
    torch, w12 = env
    g = np.random.default_rng(8700 + m)
    for ns, k in (((272, 144, 144), 640), ((2080, 2080), 512), ((64, 48, 16, 32), 4096)):
        say("gemm f8 group", m, ns, k)
        qs = [random_codes((n, k), g) for n in ns]
        ss = [random_scales(n, k, g) for n in ns]
        x = wi.gaussian_bf16((m, k), 1.0, g)
        weights = [(w12.f8_tile(torch.from_numpy(q).to("cuda:0")), torch.from_numpy(s).to("cuda:0"), q.shape[0])
                   for q, s in zip(qs, ss)]
        ys = w12.gemm_f8_group(to_dev(x, torch), weights, k)
        torch.cuda.synchronize()
        for y, q, s in zip(ys, qs, ss):
            check(y, x, q, s)


def test_prepared_f8_calls_match_direct_calls(env):
    """The prepared FP8 calls (marshalled once, re-issued by the layer timing) give the
    direct calls' bits, also when re-issued after the inputs change in place."""
    torch, w12 = env
    g = np.random.default_rng(8800)
    k = 640
    qs = [random_codes((n, k), g) for n in (272, 144)]
    ss = [random_scales(n, k, g) for n in (272, 144)]
    weights = [(w12.f8_tile(torch.from_numpy(q).to("cuda:0")), torch.from_numpy(s).to("cuda:0"), q.shape[0])
               for q, s in zip(qs, ss)]
    x = to_dev(wi.gaussian_bf16((24, k), 1.0, g), torch)
    y1 = torch.empty((24, 272), dtype=torch.bfloat16, device="cuda:0")
    outs = [torch.empty((24, n), dtype=torch.bfloat16, device="cuda:0") for _, _, n in weights]
    p1 = w12.prepare_gemm_f8(x, weights[0][0], weights[0][1], 272, k, y1)
    pg = w12.prepare_gemm_f8_group(x, weights, k, outs)
    for trial in range(2):
        say("prepared f8 calls", trial)
        p1()
        pg()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), w12.gemm_f8(x, weights[0][0], weights[0][1], 272, k).view(torch.int16))
        for o, ref in zip(outs, w12.gemm_f8_group(x, weights, k)):
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
        x.copy_(to_dev(wi.gaussian_bf16((24, k), 1.0, g), torch))


def test_gemm_routes_by_weight_format(env):
    """gemm / gemm_group take an F8Tensor to the FP8 kernels (same bits as the direct
    calls) and a W12Tensor to the W12 ones; a mixed group and an FP8 RMS call are refused."""
    torch, w12 = env
    g = np.random.default_rng(8900)
    k = 512
    q = random_codes((272, k), g)
    s = random_scales(272, k, g)
    t8 = w12.f8_encode(torch.from_numpy(q).to("cuda:0"), torch.from_numpy(s).to("cuda:0"))
    assert (t8.n, t8.k) == (272, k) and t8.nbytes() == 272 * k + 4 * s.size
    w = wi.gaussian_bf16((144, k), 0.02, g)
    t12 = w12.encode(to_dev(w, torch))
    x = wi.gaussian_bf16((5, k), 1.0, g)
    xt = to_dev(x, torch)
    say("gemm routing by weight format")
    y8 = w12.gemm(xt, t8)
    y12 = w12.gemm(xt, t12)
    yg = w12.gemm_group(xt, [t8, t8])
    torch.cuda.synchronize()
    ref8 = w12.gemm_f8(xt, t8.tiles, t8.scale, 272, k)
    assert torch.equal(y8.view(torch.int16), ref8.view(torch.int16))
    check(y8, x, q, s)
    z, sa = o.gemm_reference(x, w)
    assert o.gemm_accept(to_host(y12), z, sa).all()
    for yy in yg:
        check(yy, x, q, s)
    with pytest.raises(ValueError):
        w12.gemm_group(xt, [t8, t12])
    yr = w12.gemm(xt, t8, rms=True)
    torch.cuda.synchronize()
    refr = w12.gemm_f8(xt, t8.tiles, t8.scale, 272, k, rms=True)
    assert torch.equal(yr.view(torch.int16), refr.view(torch.int16))


def test_f8_worked_example_golden(env):
    """The hand-worked FP8 GEMM: tile bytes and output bits exactly (its few products and
    their sums are exact in FP32, so the kernel's result is the rounding of the exact z)."""
    torch, w12 = env
    g, q, s, x = __import__("test_oracle").golden_f8()
    say("f8 worked example")
    qt = w12.f8_tile(torch.from_numpy(q).to("cuda:0"))
    y = w12.gemm_f8(to_dev(x, torch), qt, torch.from_numpy(s).to("cuda:0"), g["n"], g["k"])
    torch.cuda.synchronize()
    tiles = qt.cpu().numpy()
    listed = {off: int(b, 16) for off, b in g["tile_bytes"]}
    assert all(int(tiles[off]) == b for off, b in listed.items())
    assert np.count_nonzero(tiles) == len(listed)
    yb = to_host(y)
    want = np.zeros_like(yb)
    for r, c, b in g["y_bf16"]:
        want[r, c] = int(b, 16)
    assert np.array_equal(yb, want)


@pytest.mark.parametrize("m", [1, 33, 128])
def test_gemm_f8_max_k(env, m):
    """The longest K the shape rules allow (2^20 - 128, 8191 tile and scale columns): the
    largest tile, x and scale offsets, K split over the few row-blocks."""
    torch, w12 = env
    g = np.random.default_rng(8950 + m)
    n, k = 32, (1 << 20) - 128
    q = random_codes((n, k), g)
    s = random_scales(n, k, g)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    say("gemm f8 max k", m, n, k)
    _, y = run(torch, w12, x, q, s)
    check(y, x, q, s)


def rms_f8_reference(x, q, s):
    """Reference of the FP8 RMS GEMM (harness op of a layer chain): the oracle's product
    divided by the row's RMS, sqrt(mean_k x^2) in FP64 from the BF16 values, with the
    magnitude scale divided the same way (for oracle.gemm_accept)."""
    z, sa = o.gemm_f8_reference(x, q, s)
    xf = wi.bf16_bits_to_f32(x).astype(np.float64)
    r = np.sqrt((xf * xf).mean(axis=1))[:, None]
    return z / r, sa / r


@pytest.mark.parametrize("m", [1, 5, 16, 24, 32, 33, 64, 100, 128])
def test_gemm_f8_rms(env, m):
    """The RMS form (single and grouped launches, K whole and split) against the oracle's
    product divided by each x row's RMS."""
    torch, w12 = env
    g = np.random.default_rng(9100 + m)
    for ns, k in (((272,), 1280), ((64,), 4096), ((272, 144, 144), 640), ((2080,), 512)):
        say("gemm f8 rms", m, ns, k)
        qs = [random_codes((n, k), g) for n in ns]
        ss = [random_scales(n, k, g) for n in ns]
        x = wi.gaussian_bf16((m, k), 1.0, g)
        weights = [(w12.f8_tile(torch.from_numpy(q).to("cuda:0")), torch.from_numpy(sc).to("cuda:0"), q.shape[0])
                   for q, sc in zip(qs, ss)]
        xt = to_dev(x, torch)
        ys = (w12.gemm_f8_group(xt, weights, k, rms=True) if len(ns) > 1
              else [w12.gemm_f8(xt, weights[0][0], weights[0][1], ns[0], k, rms=True)])
        torch.cuda.synchronize()
        for y, q, sc in zip(ys, qs, ss):
            z, sa = rms_f8_reference(x, q, sc)
            ok = o.gemm_accept(to_host(y), z, sa)
            assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance"
