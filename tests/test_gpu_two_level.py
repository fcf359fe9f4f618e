"""GPU parity of the two-level verification (screen copy + W12 head) against the CPU
oracle, through the C ABI.

Bars: the screen copy's codes and scales are byte-identical to the oracle's
(screen_encode + screen_pack); its per-row constants are upper bounds of the exact
||r_v||_2 + gamma ||w^_v||_2 (exact integer sums, compared at 60 digits) and within 2^-18
of it; every screen logit is within its reported bound of the exact logit, and within
gamma S8 (+ the underflow allowance) of the float64 screen logit, so a wrong scale or
code would show; argmax and accepted length equal the oracle's exact answer and the
single-level verification's, bit for bit, on planted near-ties, sub-FP64 ties, exact
ties, escape-heavy heads, zero and non-finite rows, every tile width (m up to 128) and
batched requests."""
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import w12_oracle as o
import w12_inputs as wi
from gpu_util import say, to_dev, to_host, wide_exponents
from test_gpu_parity import BIG_HEAD, plant_pairs, sub_fp64_head

pytestmark = pytest.mark.gpu

getcontext().prec = 60


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import lossless_bit_weight_w12_amd as w12
    w12.lib()
    return torch, w12


def screen_parts(sc, n, k):
    """Tiles, C and A of a screen copy (host numpy), per the documented layout."""
    a = lambda v: (v + 255) // 256 * 256
    buf = sc.buf.cpu().numpy()
    nt = (n // 16) * (k // 128) * o.SCREEN_TILE_BYTES
    c0 = a(nt)
    coef = buf[c0:c0 + 4 * n].view(np.float32)
    a0 = c0 + a(4 * n)
    abse = buf[a0:a0 + 4 * n].view(np.float32)
    return buf[:nt], coef, abse


def exact_coef(w_row, q_row, s_row, k):
    r2, q2 = o.screen_row_sums_exact(w_row, q_row, s_row)
    d = Decimal(k // 32 + 64) * Decimal(2) ** -23
    gam = d / (1 - d)
    unit = Decimal(2) ** -133
    return Decimal(r2).sqrt() * unit + gam * Decimal(q2).sqrt() * unit


def screen_mats():
    g = np.random.default_rng(8100)
    yield "gauss_64x512", wi.gaussian_bf16((64, 512), 0.02, g)
    yield "outliers_272x1280", wi.add_exponent_outliers(wi.gaussian_bf16((272, 1280), 0.02, g), 0.01, 9)
    yield "wide_48x640", wide_exponents((48, 640), g, 90, 140)
    bits = wi.random_bits((32, 256), g)
    yield "bits_32x256", bits                                   # non-finite weights included
    sub = wi.random_bits((16, 384), g) & np.uint16(0x807F)      # zeros and subnormals
    yield "subnormal_16x384", sub


SCREEN_MATS = list(screen_mats())


@pytest.mark.parametrize("name,w", SCREEN_MATS, ids=[m[0] for m in SCREEN_MATS])
def test_screen_encode_matches_oracle(env, name, w):
    torch, w12 = env
    n, k = w.shape
    say("screen encode", name, w.shape)
    q, s_bits, fin = o.screen_encode(w)
    sc = w12.screen_encode(to_dev(w, torch))
    torch.cuda.synchronize()
    tiles, coef, abse = screen_parts(sc, n, k)
    assert np.array_equal(tiles, o.screen_pack(q, s_bits))
    s_f = o.bf16_to_f64(s_bits)
    for v in range(n):
        if not fin[v]:
            assert np.isinf(coef[v]) and coef[v] > 0, v
            continue
        c = exact_coef(w[v], q[v], s_bits[v], k)
        got = Decimal(float(coef[v]))
        assert got >= c, (v, got, c)
        assert got <= c * (1 + Decimal(2) ** -18) + Decimal(2) ** -140, (v, got, c)
        a_exact = Decimal(k // 32) * (Decimal(float(s_f[v].max())) * Decimal(2) ** -113 + Decimal(2) ** -125)
        assert Decimal(float(abse[v])) >= a_exact, v


def _gauss_head(g, n, k):
    return wi.gaussian_bf16((n, k), 0.02, g)


@pytest.mark.parametrize("m,n,k", [(1, 2080, 512), (5, 4096, 128), (16, 2064, 1280), (17, 4096, 512),
                                   (32, 1040, 640), (33, 2048, 512), (64, 1024, 256), (128, 528, 512)])
def test_screen_bound_holds(env, m, n, k):
    """Every screen logit of a Gaussian head (plus outlier rows) is within its bound of
    the exact logit; the bound is ||x|| C + A to within 2^-10; the screen logit itself is
    within gamma S8 + A of the float64 screen logit."""
    torch, w12 = env
    g = np.random.default_rng(8200 + m)
    w = _gauss_head(g, n, k)
    w[:16] = wi.add_exponent_outliers(w[:16], 0.05, 9)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    x[0, :8] = 0x0001                                  # a few subnormal x values
    say("screen bound", m, n, k)
    t = w12.encode(to_dev(w, torch))
    sc = w12.screen_encode(to_dev(w, torch))
    z8, bnd = w12.screen_logits_f32(to_dev(x, torch), t, sc)
    torch.cuda.synchronize()
    z8 = z8.cpu().numpy().astype(np.float64)
    bnd = bnd.cpu().numpy().astype(np.float64)
    z, s = o.gemm_reference(x, w)
    q, s_bits, _ = o.screen_encode(w)
    zr, s8 = o.screen_logits_reference(x, q, s_bits)
    _, coef, abse = screen_parts(sc, n, k)
    xn = np.sqrt((o.bf16_to_f64(x) ** 2).sum(axis=1))
    fp64 = (k + 2) * 2.0 ** -52
    assert np.all(np.abs(z8 - z) <= bnd + fp64 * s), np.max(np.abs(z8 - z) - bnd)
    want = xn[:, None] * coef.astype(np.float64)[None, :] + abse.astype(np.float64)[None, :]
    assert np.all(bnd >= want * (1 - 2.0 ** -40)) and np.all(bnd <= want * (1 + 2.0 ** -10) + 1e-30)
    gam = o.screen_gamma(k)
    assert np.all(np.abs(z8 - zr) <= gam * s8 + abse[None, :] + fp64 * s8)
    # the FP32 evaluation is far inside its worst case
    assert np.max(np.abs(z8 - zr) / np.maximum(gam * s8, 1e-30)) < 0.05


def _check_verify2(torch, w12, x, w, am_ref, draft, t=None, sc=None):
    xt = to_dev(x, torch)
    t = t or w12.encode(to_dev(w, torch))
    sc = sc or w12.screen_encode(to_dev(w, torch))
    d = torch.from_numpy(np.ascontiguousarray(draft, dtype=np.int32)).to("cuda:0")
    am2, acc2 = w12.lmhead_verify2(xt, t, sc, d)
    am1, acc1 = w12.lmhead_verify(xt, t, d)
    torch.cuda.synchronize()
    assert am2.cpu().numpy().tolist() == am_ref.tolist()
    assert am1.cpu().numpy().tolist() == am_ref.tolist()
    want = o.accepted_length(am_ref, draft)
    assert int(acc2.item()) == int(acc1.item()) == want
    return t, sc


@pytest.mark.parametrize("m", [1, 2, 7, 15, 16, 24, 32, 33, 64, 128])
def test_verify2_matches_oracle(env, m):
    torch, w12 = env
    g = np.random.default_rng(8300 + m)
    n, k = 4096, 512
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = plant_pairs(x, _gauss_head(g, n, k), list(range(m)), g)
    say("verify2", m, n, k)
    am_ref, _ = o.argmax_exact(x, w)
    t = sc = None
    for p in sorted({0, m // 2, m}):
        draft = am_ref.copy().astype(np.int32)
        if p < m:
            draft[p] = (draft[p] + 1 + int(g.integers(0, n - 1))) % n
        t, sc = _check_verify2(torch, w12, x, w, am_ref, draft, t, sc)
    nc = w12.verify2_candidates(t, m).cpu().numpy()
    # the planted pairs pass the screen together (a later plant may overwrite an earlier
    # pair's rows, so not every row keeps one)
    assert (nc[:, 0] >= 1).all() and (nc[:, 0] >= 2).mean() >= 0.5
    assert (nc[:, 1] >= 1).all() and (nc[:, 1] <= nc[:, 0]).all()


@pytest.mark.parametrize("m", [1, 3, 8, 16])
def test_verify2_large_head(env, m):
    """The 16400-row head (1025 row-blocks: a ragged last group of 8) with near ties."""
    torch, w12 = env
    g = np.random.default_rng(8400 + m)
    n, k = BIG_HEAD
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = plant_pairs(x, _gauss_head(g, n, k), list(range(m)), g)
    say("verify2 large head", m, n, k)
    am_ref, _ = o.argmax_exact(x, w)
    draft = am_ref.astype(np.int32).copy()
    draft[m // 2] = (draft[m // 2] + 7) % n
    t, _ = _check_verify2(torch, w12, x, w, am_ref, draft)
    nc = w12.verify2_candidates(t, m).cpu().numpy()
    say("verify2 large head candidates", nc[:, 0].tolist(), nc[:, 1].tolist())


@pytest.mark.parametrize("m", [2, 5, 16])
def test_verify2_sub_fp64_near_tie(env, m):
    """The sub-FP64 near tie (exact 2^-60 against 2^-61): the screen and the FP64 stage
    cannot separate the pair and the exact sums decide; zero rows answer 0."""
    torch, w12 = env
    g = np.random.default_rng(8500 + m)
    x2, w, want = sub_fp64_head(g)
    k = w.shape[1]
    x = np.concatenate([x2, wi.gaussian_bf16((m - 2, k), 1.0, g)]) if m > 2 else x2
    if m >= 5:
        x[2] = 0
        x[3] = 0x8000
    say("verify2 sub-fp64 near tie", m)
    am_ref, _ = o.argmax_exact(x, w)
    assert am_ref[:2].tolist() == want
    t, _ = _check_verify2(torch, w12, x, w, am_ref, am_ref.astype(np.int32))
    nc = w12.verify2_candidates(t, m).cpu().numpy()
    assert nc[0, 1] >= 2 and nc[1, 1] >= 2


def test_verify2_exact_ties_escapes_and_lut(env):
    """Exact ties (copied rows), an escape-heavy head with a lookup-table codebook and
    widely spread exponents (large screen scales)."""
    torch, w12 = env
    g = np.random.default_rng(8600)
    n, k, m = 1024, 640, 5
    w = wide_exponents((n, k), g, 100, 126)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    z, _ = o.gemm_reference(x, w)
    for mi in range(m):
        v1 = int(np.argmax(z[mi]))
        w[(v1 * 7 + 3) % n] = w[v1]
    am_ref, _ = o.argmax_exact(x, w)
    say("verify2 ties")
    _check_verify2(torch, w12, x, w, am_ref, am_ref.astype(np.int32))


def test_verify2_zero_and_nonfinite_rows(env):
    """Zero rows answer 0 quickly, a row of x with an Inf answers -1, and a head row with
    an Inf weight gives the single-level answer."""
    torch, w12 = env
    g = np.random.default_rng(8700)
    n, k = BIG_HEAD
    w = _gauss_head(g, n, k)
    x = wi.gaussian_bf16((5, k), 1.0, g)
    x[0] = 0
    x[2] = 0x8000
    x[4, 9] = 0x7F80
    say("verify2 zero / non-finite rows")
    t = w12.encode(to_dev(w, torch))
    sc = w12.screen_encode(to_dev(w, torch))
    xt = to_dev(x, torch)
    none = torch.zeros(0, dtype=torch.int32, device="cuda:0")
    am2, _ = w12.lmhead_verify2(xt, t, sc, none)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    am2, acc2 = w12.lmhead_verify2(xt, t, sc, none)
    e1.record()
    am1, _ = w12.lmhead_verify(xt, t, none)
    torch.cuda.synchronize()
    ref, _ = o.argmax_exact(x[[1, 3]], w)
    got = am2.cpu().numpy()
    assert got.tolist() == [0, int(ref[0]), 0, int(ref[1]), -1]
    assert got.tolist() == am1.cpu().numpy().tolist()
    assert int(acc2.item()) == 0
    assert e0.elapsed_time(e1) < 2.0
    # a head row with +Inf weights: the screen cannot bound it (C = +Inf), the FP64 stage
    # sees a non-finite logit; both verifications agree
    w2 = w.copy()
    w2[333, 17] = 0x7F80
    t2 = w12.encode(to_dev(w2, torch))
    sc2 = w12.screen_encode(to_dev(w2, torch))
    xs = to_dev(x[[1, 3]], torch)
    a2, _ = w12.lmhead_verify2(xs, t2, sc2, none)
    a1, _ = w12.lmhead_verify(xs, t2, none)
    torch.cuda.synchronize()
    assert a2.cpu().tolist() == a1.cpu().tolist()


def test_verify2_batched_requests(env):
    """Requests of 1..5 rows in one two-level call: argmax and per-request accepted
    lengths as the oracle's and the single-level batched call's; an invalid entry -1."""
    torch, w12 = env
    g = np.random.default_rng(8800)
    n, k = 4096, 512
    rows = g.integers(1, 6, 24)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    m = int(off[-1])
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = plant_pairs(x, _gauss_head(g, n, k), list(range(0, m, 3)), g)
    say("verify2 batched", m)
    am_ref, _ = o.argmax_exact(x, w)
    nd = np.maximum(rows - 1, 0).astype(np.int32)
    draft = am_ref.astype(np.int32).copy()
    for r in range(len(rows)):
        p = int(g.integers(0, nd[r] + 1))
        if p < nd[r]:
            draft[off[r] + p] = (draft[off[r] + p] + 1) % n
    nd_bad = nd.copy()
    nd_bad[5] = rows[5] + 1
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")
    t = w12.encode(to_dev(w, torch))
    sc = w12.screen_encode(to_dev(w, torch))
    xt = to_dev(x, torch)
    am2, acc2 = w12.lmhead_verify2_batched(xt, t, sc, dev(off), dev(nd_bad), dev(draft))
    am1, acc1 = w12.lmhead_verify_batched(xt, t, dev(off), dev(nd_bad), dev(draft))
    torch.cuda.synchronize()
    assert am2.cpu().tolist() == am1.cpu().tolist() == am_ref.tolist()
    want = o.accepted_lengths_batched(am_ref, draft, off, nd_bad)
    want[5] = -1
    assert acc2.cpu().tolist() == acc1.cpu().tolist() == want.tolist()


def test_verify2_workspace_reuse_and_tickets(env):
    """Calls of different m and heads share one workspace in any order: the row tickets
    are zero after every call, results repeat bit for bit; a prepared call re-reads x."""
    torch, w12 = env
    g = np.random.default_rng(8900)
    heads = [_gauss_head(g, 2048, 512), _gauss_head(g, 4096, 256)]
    tt = [(w12.encode(to_dev(h, torch)), w12.screen_encode(to_dev(h, torch))) for h in heads]
    cases = []
    for m, hi in [(3, 0), (16, 1), (1, 0), (40, 1)]:
        x = wi.gaussian_bf16((m, heads[hi].shape[1]), 1.0, g)
        am_ref, _ = o.argmax_exact(x, heads[hi])
        cases.append((to_dev(x, torch), hi, am_ref))
    none = torch.zeros(0, dtype=torch.int32, device="cuda:0")
    for rep in range(2):
        for i in (2, 0, 3, 1):
            xt, hi, am_ref = cases[i]
            t, sc = tt[hi]
            am, _ = w12.lmhead_verify2(xt, t, sc, none)
            torch.cuda.synchronize()
            assert am.cpu().numpy().tolist() == am_ref.tolist(), (rep, i)
            ws = w12.workspace(w12.workspace_bytes(w12.OP_VERIFY2, xt.shape[0], t.n, t.k), xt.device, "verify2")
            assert int(ws[:4096].count_nonzero().item()) == 0
    # prepared call: new x contents are read on the next call
    xt, hi, _ = cases[1]
    t, sc = tt[hi]
    am = torch.empty(xt.shape[0], dtype=torch.int32, device="cuda:0")
    acc = torch.empty(1, dtype=torch.int32, device="cuda:0")
    call = w12.prepare_verify2(xt, t, sc, none, am, acc)
    x_new = wi.gaussian_bf16(tuple(xt.shape), 1.0, g)
    xt.copy_(to_dev(x_new, torch))
    call()
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == o.argmax_exact(x_new, heads[hi])[0].tolist()


def test_verify2_max_k(env):
    """Two-level verification at the longest K (2^20 - 128: 8191 tile columns, the screen's
    32-bit tile offsets, the FP64 loop over 131056 units of a row) with an exact tie."""
    torch, w12 = env
    g = np.random.default_rng(9100)
    m, n, k = 3, 64, (1 << 20) - 128
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = wi.gaussian_bf16((n, k), 0.02, g)
    w[5] = w[40]
    say("verify2 max k", m, n, k)
    am_ref, _ = o.argmax_exact(x, w)
    draft = am_ref.copy().astype(np.int32)
    draft[1] = (draft[1] + 1) % n
    _check_verify2(torch, w12, x, w, am_ref, draft)
    # the screen copy's codes and scales at this K
    sc = w12.screen_encode(to_dev(w, torch))
    q, s_bits, _ = o.screen_encode(w)
    tiles, _, _ = screen_parts(sc, n, k)
    assert np.array_equal(tiles, o.screen_pack(q, s_bits))
