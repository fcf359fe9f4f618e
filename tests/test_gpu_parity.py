"""GPU parity of libw12.so against the CPU oracle, element by element, through the
C ABI (via the thin binding).  Sizes span several tiles with ragged tails (odd
row-block counts, tile columns not a multiple of the 4-column chunk), split-K shapes,
both codebook paths (run and lookup table), escape-heavy matrices, every M in 1..32,
and greedy verification with planted exact ties and 1-ulp pairs.

Bars: encode bytes, decode bits, argmax and accepted length are bit-exact; a GEMM
output is the BF16 rounding (to nearest even) of a value t with
|t - z| <= 2e-3 * sum|x||w| + 1e-6 (oracle.gemm_accept)."""
import numpy as np
import pytest

from oracle import w12_oracle as o
import w12_inputs as wi
from gpu_util import narrow_exponents, rms_reference, say, to_dev, to_host, wide_exponents

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import lossless_bit_weight_w12_amd as w12
    w12.lib()
    return torch, w12


def matrices():
    g = np.random.default_rng(2026)
    yield "worked_example", __import__("test_oracle").worked_example_matrix()
    yield "all_patterns", wi.all_bf16_patterns()
    yield "gauss_48x384", wi.gaussian_bf16((48, 384), 0.02, g)
    yield "gauss_272x1280", wi.gaussian_bf16((272, 1280), 0.02, g)
    yield "bits_64x256", wi.random_bits((64, 256), g)
    yield "narrow_32x128", narrow_exponents((32, 128), g)
    yield "wide_48x640", wide_exponents((48, 640), g)
    yield "outliers_320x640", wi.add_exponent_outliers(wi.gaussian_bf16((320, 640), 0.02, g), 0.01, 9)


MATS = list(matrices())


@pytest.mark.parametrize("name,w", MATS, ids=[m[0] for m in MATS])
def test_encode_bytes_and_decode(env, name, w):
    torch, w12 = env
    say("encode/decode", name, w.shape)
    ref = o.encode(w)
    t = w12.encode(to_dev(w, torch))
    torch.cuda.synchronize()
    assert t.codebook == tuple(ref.codebook.tolist())
    assert t.e_max == ref.e_max and t.n_esc == ref.n_esc
    assert np.array_equal(t.tiles.cpu().numpy(), ref.tiles)
    assert np.array_equal(t.esc_off.cpu().numpy().view(np.uint32), ref.esc_off)
    assert np.array_equal(t.esc.cpu().numpy().view(np.uint32)[:ref.n_esc], ref.esc)
    dec = w12.decode(t)
    assert np.array_equal(to_host(dec), w)


@pytest.mark.parametrize("delta", [-5, 0, 3])
def test_encode_wrong_escape_count_is_memory_safe(env, delta):
    """w12_encode with a descriptor whose n_esc is off by `delta` from the true count:
    the escape offsets stay within n_esc (no later reader passes the end of `esc`), the
    workspace reports the true count, and with the right count the bytes equal the
    oracle's."""
    import ctypes
    torch, w12 = env
    g = np.random.default_rng(31)
    w = wi.add_exponent_outliers(wi.gaussian_bf16((64, 512), 0.02, g), 0.01, 9)
    ref = o.encode(w)
    assert ref.n_esc > 10
    n, k = w.shape
    cap = ref.n_esc + delta
    say("encode wrong n_esc", delta, ref.n_esc)
    t = w12.W12Tensor(n=n, k=k, n_esc=cap, codebook=tuple(ref.codebook.tolist()), e_max=ref.e_max,
                      tiles=torch.empty(w12.tiles_bytes(n, k), dtype=torch.uint8, device="cuda"),
                      esc_off=torch.empty(n // 16 + 1, dtype=torch.int32, device="cuda"),
                      esc=torch.full((cap + 8,), -1, dtype=torch.int32, device="cuda"))
    ws = torch.zeros(w12.workspace_bytes(w12.OP_ENCODE, 1, n, k), dtype=torch.uint8, device="cuda")
    d = t.desc()
    st = w12.lib().w12_encode(ctypes.c_void_p(to_dev(w, torch).data_ptr()), ctypes.byref(d),
                              ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    off0 = w12.ENCODE_TOTAL_OFFSET
    total = int(ws[off0:off0 + 4].cpu().numpy().view(np.uint32)[0])
    assert total == ref.n_esc
    off = t.esc_off.cpu().numpy().view(np.uint32)
    assert off.max() <= cap and np.all(np.diff(off.astype(np.int64)) >= 0)
    assert np.array_equal(off, np.minimum(ref.esc_off, cap))
    esc = t.esc.cpu().numpy()
    assert np.all(esc[cap:] == -1)   # nothing written past n_esc
    assert np.array_equal(t.tiles.cpu().numpy(), ref.tiles)
    if delta >= 0:
        assert np.array_equal(esc.view(np.uint32)[:ref.n_esc], ref.esc)
        assert np.array_equal(to_host(w12.decode(t)), w)


def _gemm_case(env, w, x, which):
    torch, w12 = env
    xt = to_dev(x, torch)
    if which == "bf16":
        y = w12.gemm_bf16(xt, to_dev(w, torch))
    else:
        t = w12.encode(to_dev(w, torch))
        y = torch.full((x.shape[0], w.shape[0]), -1, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
        w12.gemm(xt, t, out=y)
    torch.cuda.synchronize()
    z, s = o.gemm_reference(x, w)
    yb = to_host(y)
    ok = o.gemm_accept(yb, z, s)
    bad = np.argwhere(~ok)
    assert ok.all(), f"{bad.shape[0]} outside tolerance, first {bad[:4].tolist()} y={wi.bf16_bits_to_f32(yb[tuple(bad[0])])} z={z[tuple(bad[0])]}"
    return yb


# (n, k): ragged row-block counts, partial 4-column chunks, split-K, long K, 1025
# row-blocks over two tile columns (the many-row kernels: an odd row-block count for two
# row-blocks per wave, waves with no column), and 2049 row-blocks (one 10-wave workgroup
# per CU at 17..32 rows, the last one nine of its waves idle)
SHAPES = [(16, 128), (272, 1280), (48, 640), (64, 4096), (2080, 512), (16400, 256), (32784, 128)]


# every decode size, then the batched sizes (64- and 128-column tiles, ragged in both)
@pytest.mark.parametrize("m", list(range(1, 33)) + [33, 48, 64, 65, 100, 128])
def test_gemm_all_m_run_codebook(env, m):
    g = np.random.default_rng(1000 + m)
    for n, k in SHAPES:
        say("gemm run", m, n, k)
        w = wi.gaussian_bf16((n, k), 0.02, g)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        _gemm_case(env, w, x, "w12")


@pytest.mark.parametrize("m", [1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 24, 31, 32, 40, 64, 120, 128])
def test_gemm_lut_codebook_and_escapes(env, m):
    g = np.random.default_rng(2000 + m)
    for n, k in [(48, 640), (320, 1280), (64, 4096)]:
        say("gemm lut", m, n, k)
        w = wide_exponents((n, k), g, 108, 132)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        _gemm_case(env, w, x, "w12")
        w2 = wi.add_exponent_outliers(wi.gaussian_bf16((n, k), 0.02, g), 0.01, 7)
        _gemm_case(env, w2, x, "w12")


# weight groups sharing x: few row-blocks with split K (q/k/v-like), many row-blocks
# (gate/up-like), and ragged groups whose row-block boundaries fall inside workgroups
GROUPS = [[(320, 512), (64, 512), (64, 512)],
          [(1088, 1280), (1088, 1280)],
          [(48, 640), (16, 640), (32, 640), (272, 640)],
          [(16, 4096)],
          [(8192, 256), (8208, 256)],
          [(17408, 256), (17408, 256)]]     # 2176 row-blocks: 10-wave workgroups at 17..32 rows


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 15, 16, 24, 32, 64, 128])
def test_gemm_group(env, m):
    torch, w12 = env
    g = np.random.default_rng(7000 + m)
    for shapes in GROUPS:
        k = shapes[0][1]
        say("gemm group", m, shapes)
        ws = [wi.gaussian_bf16(sh, 0.02, g) for sh in shapes]
        x = wi.gaussian_bf16((m, k), 1.0, g)
        ts = [w12.encode(to_dev(w, torch)) for w in ws]
        outs = [torch.full((m, sh[0]), -1, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
                for sh in shapes]
        w12.gemm_group(to_dev(x, torch), ts, outs)
        torch.cuda.synchronize()
        for w, y in zip(ws, outs):
            z, s = o.gemm_reference(x, w)
            assert o.gemm_accept(to_host(y), z, s).all()


@pytest.mark.parametrize("m", [1, 3, 4, 8, 15, 16, 24, 32, 48, 128])
def test_gemm_rms(env, m):
    """RMS GEMM (harness op of the layer chain): grouped and single launches, split and
    whole K, against the oracle's product divided by the row's RMS."""
    torch, w12 = env
    g = np.random.default_rng(7300 + m)
    for shapes in GROUPS + [[(512, 17408)]]:
        k = shapes[0][1]
        say("gemm rms", m, shapes)
        ws = [wi.gaussian_bf16(sh, 0.02, g) for sh in shapes]
        x = wi.gaussian_bf16((m, k), 3.0, g)
        ts = [w12.encode(to_dev(w, torch)) for w in ws]
        xt = to_dev(x, torch)
        outs = w12.gemm_group(xt, ts, rms=True)
        single = w12.gemm(xt, ts[0], rms=True)
        torch.cuda.synchronize()
        for w, y in zip(ws, outs):
            z, s = rms_reference(x, w)
            assert o.gemm_accept(to_host(y), z, s).all()
        z, s = rms_reference(x, ws[0])
        assert o.gemm_accept(to_host(single), z, s).all()


def test_gemm_group_mixed_codebooks(env):
    """Run and lookup-table codebooks in one call (two launches), escapes in both."""
    torch, w12 = env
    g = np.random.default_rng(7100)
    k = 1280
    ws = [wi.add_exponent_outliers(wi.gaussian_bf16((320, k), 0.02, g), 0.01, 11),
          wide_exponents((64, k), g, 104, 130),
          wi.gaussian_bf16((96, k), 0.02, g),
          wide_exponents((32, k), g, 110, 140)]
    for m in (1, 7, 24):
        say("gemm group mixed", m)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        ts = [w12.encode(to_dev(w, torch)) for w in ws]
        outs = w12.gemm_group(to_dev(x, torch), ts)
        torch.cuda.synchronize()
        for w, y in zip(ws, outs):
            z, s = o.gemm_reference(x, w)
            assert o.gemm_accept(to_host(y), z, s).all()


@pytest.mark.parametrize("m", [1, 2, 4, 5, 8, 12, 15, 16, 20, 32, 64, 128])
def test_gemm_bf16_baseline(env, m):
    g = np.random.default_rng(3000 + m)
    for n, k in SHAPES:
        say("gemm bf16", m, n, k)
        w = wi.gaussian_bf16((n, k), 0.02, g)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        _gemm_case(env, w, x, "bf16")


def tiled_reference(w):
    """The documented 4 KB tile layout built with numpy: tiles in column-major order
    (tile (b, g) at (g * n/16 + b) * 4096), group j, lane l = 16q + r holds row 16b + r,
    columns 128g + 32j + 8q .. +7."""
    n, k = w.shape
    t = w.reshape(n // 16, 16, k // 128, 4, 4, 8)          # b, r, g, j, q, e
    t = t.transpose(2, 0, 3, 4, 1, 5)                      # g, b, j, q, r, e
    return np.ascontiguousarray(t).reshape(-1).view(np.uint8)


@pytest.mark.parametrize("m", [1, 2, 4, 8, 16, 24, 32, 96, 128])
def test_gemm_bf16_tiled_baseline(env, m):
    torch, w12 = env
    g = np.random.default_rng(3500 + m)
    for n, k in SHAPES:
        say("gemm bf16 tiled", m, n, k)
        w = wi.gaussian_bf16((n, k), 0.02, g)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        wt = w12.bf16_tile(to_dev(w, torch))
        torch.cuda.synchronize()
        assert np.array_equal(wt.cpu().numpy(), tiled_reference(w))
        y = w12.gemm_bf16_tiled(to_dev(x, torch), wt, n, k)
        torch.cuda.synchronize()
        z, s = o.gemm_reference(x, w)
        assert o.gemm_accept(to_host(y), z, s).all()


def test_gemm_deterministic_and_overwrites(env):
    torch, w12 = env
    g = np.random.default_rng(4)
    for m, (n, k) in [(1, (64, 4096)), (8, (272, 1280)), (32, (2080, 512))]:
        say("determinism", m, n, k)
        w = wi.gaussian_bf16((n, k), 0.02, g)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        t = w12.encode(to_dev(w, torch))
        xt = to_dev(x, torch)
        y1 = w12.gemm(xt, t)
        y2 = torch.full_like(y1.view(torch.int16), -1).view(torch.bfloat16)
        w12.gemm(xt, t, out=y2)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_gemm_workspace_reuse_across_shapes(env):
    """One workspace serves split-K launches of different shapes in any order: the
    split-K tickets sit at a fixed place and every call leaves them at zero."""
    torch, w12 = env
    g = np.random.default_rng(12)
    cases = []
    for m, (n, k) in [(1, (272, 1280)), (1, (64, 4096)), (8, (64, 4096)), (32, (320, 2048)),
                      (4, (2080, 512))]:
        w = wi.gaussian_bf16((n, k), 0.02, g)
        x = wi.gaussian_bf16((m, k), 1.0, g)
        cases.append((to_dev(x, torch), w12.encode(to_dev(w, torch)), x, w))
    first = []
    for xt, t, x, w in cases:
        say("workspace reuse", x.shape, w.shape)
        y = w12.gemm(xt, t)
        torch.cuda.synchronize()
        z, s = o.gemm_reference(x, w)
        assert o.gemm_accept(to_host(y), z, s).all()
        first.append(y)
    for rep in range(3):
        for i in (4, 0, 3, 1, 2):
            xt, t, _, _ = cases[i]
            y = w12.gemm(xt, t)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), first[i].view(torch.int16)), (rep, i)


@pytest.mark.parametrize("which", ["w12", "bf16", "bf16t"])
def test_split_k_completes_from_fresh_partials(env, which):
    """K-split launches complete inside the GEMM: the split that finishes last in a
    row-block group sums every split's partials in split order.  Between calls the
    workspace past the 4 KB of tickets is filled with NaN bytes; each call must still
    equal the first one bit for bit (and the oracle), leave the tickets at zero, and a
    workspace that held NaN bytes everywhere works once w12_workspace_init has zeroed it.
    Shapes: few row-blocks with long K (split at every m), an RMS launch, and 1..3 rows
    on the BF16 kernels (the wave-column kernel's split path)."""
    import ctypes
    torch, w12 = env
    g = np.random.default_rng(7700)
    n, k = 320, 4096
    w = wi.gaussian_bf16((n, k), 0.02, g)
    wd = to_dev(w, torch)
    t = w12.encode(wd) if which == "w12" else None
    wt = w12.bf16_tile(wd) if which == "bf16t" else None
    for m in (1, 3, 8, 32):
        x = wi.gaussian_bf16((m, k), 1.0, g)
        xt = to_dev(x, torch)
        say("split-k completion", which, m)

        def call(out, rms=False):
            if which == "w12":
                return w12.gemm(xt, t, out=out, rms=rms)
            if which == "bf16":
                return w12.gemm_bf16(xt, wd, out=out)
            return w12.gemm_bf16_tiled(xt, wt, n, k, out=out)
        y0 = call(None)
        torch.cuda.synchronize()
        ws = w12.workspace(256, xt.device)                    # the binding's cached GEMM workspace
        assert int(ws[:4096].count_nonzero()) == 0          # tickets left at zero
        z, s = o.gemm_reference(x, w)
        assert o.gemm_accept(to_host(y0), z, s).all()
        for rep in range(2):
            ws[4096:].fill_(0xFF)                             # partials and row sums: NaN
            y1 = call(None)
            torch.cuda.synchronize()
            assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), (m, rep)
            assert int(ws[:4096].count_nonzero()) == 0
        if which == "w12":                                    # RMS launch, K split
            yr = call(None, rms=True)
            torch.cuda.synchronize()
            zr, sr = rms_reference(x, w)
            assert o.gemm_accept(to_host(yr), zr, sr).all()
    # a workspace of NaN bytes prepared by w12_workspace_init, through the C ABI
    m = 8
    x = wi.gaussian_bf16((m, k), 1.0, g)
    xt = to_dev(x, torch)
    op = w12.OP_GEMM if which == "w12" else w12.OP_GEMM_BF16
    nbytes = w12.workspace_bytes(op, m, n, k)
    assert nbytes > 4096
    fresh = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")
    L = w12.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.w12_workspace_init(ctypes.c_void_p(fresh.data_ptr()), nbytes, stream) == 0
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    if which == "w12":
        d = t.desc()
        st = L.w12_gemm(ctypes.c_void_p(xt.data_ptr()), m, ctypes.byref(d), ctypes.c_void_p(y.data_ptr()),
                        ctypes.c_void_p(fresh.data_ptr()), nbytes, stream)
    elif which == "bf16":
        st = L.w12_gemm_bf16(ctypes.c_void_p(xt.data_ptr()), m, ctypes.c_void_p(wd.data_ptr()), n, k,
                             ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(fresh.data_ptr()), nbytes, stream)
    else:
        st = L.w12_gemm_bf16_tiled(ctypes.c_void_p(xt.data_ptr()), m, ctypes.c_void_p(wt.data_ptr()), n, k,
                                   ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(fresh.data_ptr()), nbytes,
                                   stream)
    assert st == 0
    torch.cuda.synchronize()
    z, s = o.gemm_reference(x, w)
    assert o.gemm_accept(to_host(y), z, s).all()
    assert int(fresh[:4096].count_nonzero()) == 0


def test_gemm_nonfinite_propagates(env):
    torch, w12 = env
    g = np.random.default_rng(5)
    w = wi.gaussian_bf16((32, 256), 0.02, g)
    w[3, 7] = 0x7FC0          # NaN
    w[9, 100] = 0x7F80        # +Inf
    x = wi.gaussian_bf16((2, 256), 1.0, g)
    y = to_host(w12.gemm(to_dev(x, torch), w12.encode(to_dev(w, torch))))
    yf = wi.bf16_bits_to_f32(y)
    assert np.isnan(yf[:, 3]).all() and np.isinf(yf[:, 9]).all()
    finite_cols = [c for c in range(32) if c not in (3, 9)]
    z, s = o.gemm_reference(x, w[finite_cols])
    assert o.gemm_accept(y[:, finite_cols], z, s).all()


# ----------------------------------------------------------------------------- verify
def plant_pairs(x, w, rows, g):
    """Plant near-ties for the given x rows: W[v2] := W[v1] (v1 = float64 argmax of the
    row); for odd plants one weight of both rows is set to a tiny value and W[v2]'s copy
    is moved by one BF16 ulp, so the two logits differ by |x_k| * 2^-27-ish, far below
    one FP32 ulp of the logit.  The expected answers are recomputed by the oracle."""
    w = w.copy()
    n = w.shape[0]
    for idx, m in enumerate(rows):
        z, _ = o.gemm_reference(x[m:m + 1], w)
        v1 = int(np.argmax(z[0]))
        v2 = int(g.integers(0, n - 1))
        v2 = v2 + 1 if v2 >= v1 else v2
        w[v2] = w[v1]
        if idx % 2 == 1:
            kk = int(g.integers(0, w.shape[1]))
            tiny = (int(g.integers(0, 2)) << 15) | (107 << 7) | int(g.integers(1, 127))
            w[v1, kk] = tiny
            w[v2, kk] = tiny + (1 if g.integers(0, 2) else -1)
    return w


@pytest.mark.parametrize("m", [1, 2, 7, 15, 16, 24, 32, 33, 64, 128])
def test_verify_matches_oracle(env, m):
    torch, w12 = env
    g = np.random.default_rng(5000 + m)
    n, k = 4096, 512
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = wi.gaussian_bf16((n, k), 0.02, g)
    w = plant_pairs(x, w, list(range(m)), g)
    say("verify", m, n, k)
    am_ref, ncand = o.argmax_exact(x, w)
    t = w12.encode(to_dev(w, torch))
    xt = to_dev(x, torch)
    for p in sorted({0, m // 2, m}):
        draft = am_ref.copy().astype(np.int32)
        if p < m:
            draft[p] = (draft[p] + 1 + int(g.integers(0, n - 1))) % n
        am, acc = w12.lmhead_verify(xt, t, torch.from_numpy(draft).to("cuda:0"))
        torch.cuda.synchronize()
        assert am.cpu().numpy().tolist() == am_ref.tolist()
        assert int(acc.item()) == o.accepted_length(am_ref, draft) == p
    nc = w12.verify_candidates(t, m).cpu().numpy()
    assert (nc[:, 0] >= 1).all() and (nc[:, 1] >= 1).all() and (nc[:, 1] <= 16 * nc[:, 0]).all()


def test_verify_batched_requests(env):
    """Several requests verified in one call (the batched regime: 24 requests of 1..5
    rows, 16-24 requests in the pages' batched rows): the argmax is the oracle's on every
    row, each valid request's accepted length is the oracle's per-request rule, an entry
    whose draft is longer than its rows gets -1 (the documented rule for invalid
    entries), and a second table over the same rows -- rows in no request, an empty
    draft -- is read from the device on the next call."""
    torch, w12 = env
    g = np.random.default_rng(5600)
    n, k = 4096, 512
    rows = g.integers(1, 6, 24)
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    m = int(off[-1])
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = plant_pairs(x, wi.gaussian_bf16((n, k), 0.02, g), list(range(0, m, 3)), g)
    say("verify batched", m, n, k, "requests", len(rows))
    am_ref, _ = o.argmax_exact(x, w)
    t = w12.encode(to_dev(w, torch))
    xt = to_dev(x, torch)
    nd = np.maximum(rows - 1, 0).astype(np.int32)     # the last row of each is the bonus row
    nd[3] = rows[3]                                     # a request drafting on every row
    nd[7] = 0                                           # a request with no draft
    draft = am_ref.astype(np.int32).copy()
    for r in range(len(rows)):
        p = int(g.integers(0, nd[r] + 1))                # p == nd[r]: no mismatch
        if p < nd[r]:
            i = off[r] + p
            draft[i] = (draft[i] + 1 + int(g.integers(0, n - 1))) % n
    nd_bad = nd.copy()
    nd_bad[11] = rows[11] + 1                           # invalid: more draft than rows
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")
    off_t, nd_t, draft_t = dev(off), dev(nd_bad), dev(draft)
    am, acc = w12.lmhead_verify_batched(xt, t, off_t, nd_t, draft_t)
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    want = o.accepted_lengths_batched(am_ref, draft, off, nd_bad)
    want[11] = -1
    assert acc.cpu().numpy().tolist() == want.tolist()
    assert (want[np.arange(24) != 11] < nd[np.arange(24) != 11]).any()   # mismatches were planted
    # a second table on the same rows through one prepared call: new device contents;
    # rows 0-1 and the padding entries (empty requests at row m) belong to no request
    call = w12.prepare_verify_batched(xt, t, off_t, nd_t, draft_t, am, acc)
    off2 = np.array([2, m // 4, m // 2, m - 3, m], dtype=np.int32)
    nd2 = np.array([m // 4 - 2, 0, 2, 3], dtype=np.int32)
    off_t.copy_(torch.from_numpy(np.concatenate([off2, np.full(len(off) - len(off2), m, np.int32)])))
    nd_t.copy_(torch.from_numpy(np.concatenate([nd2, np.zeros(len(nd) - len(nd2), np.int32)])))
    call()
    torch.cuda.synchronize()
    got = acc.cpu().numpy()
    assert got[:4].tolist() == o.accepted_lengths_batched(am_ref, draft, off2, nd2).tolist()
    assert (got[4:] == 0).all()
    # one request over every row is the single-request entry point
    am1, acc1 = w12.lmhead_verify(xt, t, dev(draft[:m]))
    am2, acc2 = w12.lmhead_verify_batched(xt, t, dev([0, m]), dev([m]), dev(draft))
    torch.cuda.synchronize()
    assert am1.cpu().tolist() == am2.cpu().tolist() == am_ref.tolist()
    assert int(acc1.item()) == int(acc2.item()) == o.accepted_length(am_ref, draft)


def _certified_bound(s_hat, k, e_max, xmax):
    """The bound the verification relies on, as its header states it: K exact products,
    each passing through at most D = K/128 + 192 additions (every tile column summed from
    zero, then added to the running sum) with relative error below 2^-23, plus flushed
    denormals (2K + D events)."""
    d = k // 128 + 192.0
    gam = d * 2.0 ** -23 / (1 - d * 2.0 ** -23)
    a = (2 * k + d) * 2.0 ** -126 * (1 + xmax + 2.0 ** (e_max - 126))
    return gam * (s_hat / (1 - gam) + a) + a, gam, a


@pytest.mark.parametrize("m,kind", [(1, "gauss"), (3, "wide"), (7, "gauss"), (16, "outliers"),
                                    (24, "gauss"), (32, "wide"), (64, "outliers"), (128, "wide")])
def test_verify_pass1_error_within_certified_bound(env, m, kind):
    """The FP32 logits of verification pass 1 (w12_logits_f32: the same kernels and
    summation order) stay within the certified bound of the exact values on every
    output (the assumption the exact-argmax filter rests on), and its error scale
    X_m W_v is a valid scale for it."""
    torch, w12 = env
    g = np.random.default_rng(9000 + m)
    n, k = 2048, 5120
    if kind == "gauss":
        w = wi.gaussian_bf16((n, k), 0.02, g)
    elif kind == "wide":
        w = wide_exponents((n, k), g, 104, 126)
    else:
        w = wi.add_exponent_outliers(wi.gaussian_bf16((n, k), 0.02, g), 0.01, 3)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    t = w12.encode(to_dev(w, torch))
    say("pass-1 bound", m, kind, "codebook", t.codebook)
    z_hat, s_hat = (v.cpu().numpy().astype(np.float64) for v in w12.logits_f32(to_dev(x, torch), t))
    z, s = o.gemm_reference(x, w)
    xmax = np.abs(wi.bf16_bits_to_f32(x).astype(np.float64)).max()
    bound, gam, a = _certified_bound(s_hat, k, t.e_max, xmax)
    err = np.abs(z_hat - z)
    assert (err <= bound).all(), float((err / bound).max())
    assert (s <= s_hat / (1 - gam) + a).all()
    _check_scale_is_cauchy_schwarz(s_hat, x, w, k)
    say("pass-1 bound", m, kind, "max |z^-z| / (g S) =", float((err / (gam * s + 1e-300)).max()))


def _check_scale_is_cauchy_schwarz(s_hat, x, w, k):
    """The first pass's error scale is ||x_m||_2 ||w_v||_2 rounded up (Cauchy-Schwarz
    bounds sum_k |x_k||w_vk| by it): at least that product, and above it by less than
    the slack of the FP32 sums of squares (depth K + 64)."""
    gam = (k + 64.0) * 2.0 ** -23 / (1 - (k + 64.0) * 2.0 ** -23)
    xf = wi.bf16_bits_to_f32(x).astype(np.float64)
    wf = wi.bf16_bits_to_f32(w).astype(np.float64)
    cs = np.sqrt((xf * xf).sum(1))[:, None] * np.sqrt((wf * wf).sum(1))[None, :]
    assert (s_hat >= cs * (1 - 1e-12)).all(), float((s_hat / cs).min())
    assert (s_hat <= cs * (1 + 2 * gam) + 1e-30).all(), float((s_hat / cs).max())


# 1025 row-blocks: from 1024 row-blocks the first pass at 1..3 rows runs the wave-column
# VALU kernel with two row-blocks per wave (the column-synchronous MFMA kernel from 4 rows
# on), here with an odd row-block count so the last wave's second row-block is past the end
BIG_HEAD = (16400, 512)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 15])
def test_verify_small_m_large_head(env, m):
    """Verification below 16 rows on a head with more than 1024 row-blocks, near ties
    planted on every row: argmax and accepted length against the oracle."""
    torch, w12 = env
    g = np.random.default_rng(5300 + m)
    n, k = BIG_HEAD
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = plant_pairs(x, wi.gaussian_bf16((n, k), 0.02, g), list(range(m)), g)
    say("verify large head", m, n, k)
    am_ref, _ = o.argmax_exact(x, w)
    t = w12.encode(to_dev(w, torch))
    xt = to_dev(x, torch)
    for p in sorted({0, m // 2, m}):
        draft = am_ref.copy().astype(np.int32)
        if p < m:
            draft[p] = (draft[p] + 1 + int(g.integers(0, n - 1))) % n
        am, acc = w12.lmhead_verify(xt, t, torch.from_numpy(draft).to("cuda:0"))
        torch.cuda.synchronize()
        assert am.cpu().numpy().tolist() == am_ref.tolist()
        assert int(acc.item()) == o.accepted_length(am_ref, draft) == p


@pytest.mark.parametrize("m,kind", [(1, "gauss"), (2, "wide"), (3, "outliers"), (4, "gauss"),
                                    (8, "wide"), (15, "outliers")])
def test_verify_pass1_bound_small_m_large_head(env, m, kind):
    """The certified bound on the first pass's FP32 logits below 16 rows on a head with
    more than 1024 row-blocks (the wave-column VALU kernel at 1..3 rows, then the
    column-synchronous MFMA kernel)."""
    torch, w12 = env
    g = np.random.default_rng(9300 + m)
    n, k = BIG_HEAD[0], 1280
    if kind == "gauss":
        w = wi.gaussian_bf16((n, k), 0.02, g)
    elif kind == "wide":
        w = wide_exponents((n, k), g, 104, 126)
    else:
        w = wi.add_exponent_outliers(wi.gaussian_bf16((n, k), 0.02, g), 0.01, 3)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    t = w12.encode(to_dev(w, torch))
    say("pass-1 bound large head", m, kind, "codebook", t.codebook)
    z_hat, s_hat = (v.cpu().numpy().astype(np.float64) for v in w12.logits_f32(to_dev(x, torch), t))
    z, s = o.gemm_reference(x, w)
    xmax = np.abs(wi.bf16_bits_to_f32(x).astype(np.float64)).max()
    bound, gam, a = _certified_bound(s_hat, k, t.e_max, xmax)
    err = np.abs(z_hat - z)
    assert (err <= bound).all(), float((err / bound).max())
    assert (s <= s_hat / (1 - gam) + a).all()
    _check_scale_is_cauchy_schwarz(s_hat, x, w, k)


def sub_fp64_head(g):
    """The oracle pin's sub-FP64 near tie (test_oracle.sub_fp64_near_tie) inside a head of
    16400 rows: columns 0..255 of every row take the construction's pattern for an
    uninvolved row (logit -1 for both construction rows of x), its rows 2 and 3 go to
    head rows 9002 and 9003 (one row-block) and its rows 5 and 11 to head rows 700 and
    12011; the rest of the head is Gaussian.  Expected: 9003 for x row 0, 700 for row 1."""
    xs, ws, _ = __import__("test_oracle").sub_fp64_near_tie()
    n, k = BIG_HEAD
    w = wi.gaussian_bf16((n, k), 0.02, g)
    w[:, :256] = ws[0]
    for src, dst in ((2, 9002), (3, 9003), (5, 700), (11, 12011)):
        w[dst, :256] = ws[src]
    x = np.zeros((2, k), dtype=np.uint16)
    x[:, :256] = xs
    return x, w, [9003, 700]


@pytest.mark.parametrize("m", [2, 5, 16])
def test_verify_sub_fp64_near_tie(env, m):
    """Two logits that float64 summation misorders (exact 2^-60 against 2^-61, the
    larger one a cancellation 1 + 2^-60 - 1): the FP32 pass and the FP64 screen cannot
    separate them and the exact integer sums decide.  Rows beyond the first two are
    Gaussian; at m = 5 and 16 one extra row is all +0 and one all -0 (every exact logit
    0, so index 0)."""
    torch, w12 = env
    g = np.random.default_rng(5400 + m)
    x2, w, want = sub_fp64_head(g)
    k = w.shape[1]
    x = np.concatenate([x2, wi.gaussian_bf16((m - 2, k), 1.0, g)]) if m > 2 else x2
    if m >= 5:
        x[2] = 0
        x[3] = 0x8000
    say("verify sub-fp64 near tie", m)
    am_ref, _ = o.argmax_exact(x, w)
    assert am_ref[:2].tolist() == want
    if m >= 5:
        assert am_ref[2] == 0 and am_ref[3] == 0
    t = w12.encode(to_dev(w, torch))
    draft = am_ref.astype(np.int32)
    am, acc = w12.lmhead_verify(to_dev(x, torch), t, torch.from_numpy(draft).to("cuda:0"))
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    assert int(acc.item()) == m
    nc = w12.verify_candidates(t, m).cpu().numpy()
    assert nc[0, 1] >= 2 and nc[1, 1] >= 2          # the pair reached the exact sums


def test_verify_zero_rows_are_fast(env):
    """Rows of x that are all zero (padding rows of a batch) make every exact logit 0:
    the answer is index 0 and must not cost an exact sum per head row.  Four rows (two
    zero, one -0, one Gaussian) on the 16400-row head, timed after a warm-up call."""
    torch, w12 = env
    g = np.random.default_rng(5500)
    n, k = BIG_HEAD
    w = wi.gaussian_bf16((n, k), 0.02, g)
    x = wi.gaussian_bf16((4, k), 1.0, g)
    x[0] = 0
    x[2] = 0x8000
    x[3] = 0
    say("verify zero rows")
    am_ref, _ = o.argmax_exact(x, w)
    assert am_ref[[0, 2, 3]].tolist() == [0, 0, 0]
    t = w12.encode(to_dev(w, torch))
    xt = to_dev(x, torch)
    draft = torch.from_numpy(am_ref.astype(np.int32)).to("cuda:0")
    am, acc = w12.lmhead_verify(xt, t, draft)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    am, acc = w12.lmhead_verify(xt, t, draft)
    e1.record()
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist() and int(acc.item()) == 4
    ms = e0.elapsed_time(e1)
    say("verify zero rows", ms, "ms")
    assert ms < 2.0, ms


def test_verify_exact_tie_lowest_index_and_escapes(env):
    """Rows tie exactly (copies), the head is escape-heavy (lookup-table codebook)."""
    torch, w12 = env
    g = np.random.default_rng(6)
    n, k, m = 1024, 640, 5
    w = wide_exponents((n, k), g, 100, 126)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    z, _ = o.gemm_reference(x, w)
    for mi in range(m):
        v1 = int(np.argmax(z[mi]))
        w[(v1 * 7 + 3) % n] = w[v1]
    am_ref, _ = o.argmax_exact(x, w)
    t = w12.encode(to_dev(w, torch))
    say("verify ties", n, k, m, "codebook", t.codebook)
    draft = am_ref.astype(np.int32)
    am, acc = w12.lmhead_verify(to_dev(x, torch), t, torch.from_numpy(draft).to("cuda:0"))
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    assert int(acc.item()) == m


@pytest.mark.parametrize("m", [2, 5])
def test_verify_group_second_logit(env, m):
    """The group record's second largest logit decides whether pass 2 opens the block
    records of z*'s group.  Each row's winning head row is copied (an exact tie, so the
    lowest index must win) into: row 0 the same 16-row block, row 1 another block of the
    same pass-1 group (eight row-blocks at 5 rows, two at 2), row 2.. another group; a
    second set of rows gets a runner-up one BF16 step below the winner on one weight in
    the same group.  Argmax, accepted length and candidate counts against the oracle."""
    torch, w12 = env
    g = np.random.default_rng(7700 + m)
    n, k = BIG_HEAD
    w = wi.gaussian_bf16((n, k), 0.02, g)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    z, _ = o.gemm_reference(x, w)
    bpg = 8 if m >= 4 else 2
    for mi in range(m):
        v1 = int(np.argmax(z[mi]))
        blk, grp = v1 // 16, v1 // (16 * bpg)
        if mi == 0:
            dst = 16 * blk + (v1 % 16 + 5) % 16                       # same block
        elif mi == 1:
            b2 = grp * bpg + (blk - grp * bpg + 1) % bpg              # same group, other block
            dst = 16 * b2 + 3
        else:
            dst = (v1 + 16 * bpg * 7 + 16 * mi) % n                   # another group
        w[dst] = w[v1]
    am_ref, _ = o.argmax_exact(x, w)
    t = w12.encode(to_dev(w, torch))
    say("verify group second logit", m, n, k)
    draft = am_ref.astype(np.int32)
    am, acc = w12.lmhead_verify(to_dev(x, torch), t, torch.from_numpy(draft).to("cuda:0"))
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    assert int(acc.item()) == m
    nc = w12.verify_candidates(t, m).cpu().numpy()
    assert (nc[:, 0] >= 2).all(), nc[:, 0].tolist()   # both copies reached the FP64 screen
    # a runner-up one BF16 step below on a single weight of the winner's row, same group
    w2 = w.copy()
    for mi in range(m):
        v1 = int(am_ref[mi])
        blk, grp = v1 // 16, v1 // (16 * bpg)
        b2 = grp * bpg + (blk - grp * bpg + 1) % bpg
        dst = 16 * b2 + 7
        if dst // 16 == blk:
            dst = 16 * blk + (v1 % 16 + 1) % 16
        w2[dst] = w2[v1]
        kk = int(np.argmax(np.abs(wi.bf16_bits_to_f32(x[mi]))))
        sgn = 1 if wi.bf16_bits_to_f32(x[mi, kk:kk + 1])[0] > 0 else -1
        bits = int(w2[dst, kk])
        # one BF16 step toward a smaller product x*w
        mag_up = (bits & 0x8000 == 0) == (sgn < 0)
        w2[dst, kk] = np.uint16(bits + 1 if mag_up else bits - 1) if bits & 0x7FFF else bits
    am_ref2, _ = o.argmax_exact(x, w2)
    t2 = w12.encode(to_dev(w2, torch))
    am2, _ = w12.lmhead_verify(to_dev(x, torch), t2, torch.from_numpy(am_ref2.astype(np.int32)).to("cuda:0"))
    torch.cuda.synchronize()
    assert am2.cpu().numpy().tolist() == am_ref2.tolist()


def test_verify_row_norms_beyond_fp32(env):
    """Weights so large that the FP32 sums of their squares overflow (|w| in [2^53, 2^63)
    at k = 640) make every row norm bound infinite: every logit of the head is then a
    candidate, screened in FP64 in chunks of 512, and the answer is still the exact argmax
    (the wave-column VALU kernel at 2 rows, the column-synchronous kernel at 5)."""
    torch, w12 = env
    g = np.random.default_rng(61)
    n, k = 2048, 640
    w = wide_exponents((n, k), g, 180, 190)
    t = w12.encode(to_dev(w, torch))
    for m in (2, 5):
        x = wi.gaussian_bf16((m, k), 1.0, g)
        am_ref, _ = o.argmax_exact(x, w)
        say("verify infinite row norms", n, k, m)
        draft = am_ref.astype(np.int32)
        am, acc = w12.lmhead_verify(to_dev(x, torch), t, torch.from_numpy(draft).to("cuda:0"))
        torch.cuda.synchronize()
        assert am.cpu().numpy().tolist() == am_ref.tolist()
        assert int(acc.item()) == m
        nc = w12.verify_candidates(t, m).cpu().numpy()
        assert (nc[:, 0] == n).all(), nc[:, 0].tolist()


def test_verify_nonfinite_row_reports_minus_one(env):
    torch, w12 = env
    g = np.random.default_rng(7)
    w = wi.gaussian_bf16((256, 256), 0.02, g)
    x = wi.gaussian_bf16((3, 256), 1.0, g)
    x[1, 5] = 0x7F80
    am, acc = w12.lmhead_verify(to_dev(x, torch), w12.encode(to_dev(w, torch)),
                                torch.zeros(0, dtype=torch.int32, device="cuda:0"))
    torch.cuda.synchronize()
    ref, _ = o.argmax_exact(x[[0, 2]], w)
    got = am.cpu().numpy()
    assert got[1] == -1 and got[0] == ref[0] and got[2] == ref[1]
    assert int(acc.item()) == 0


@pytest.mark.parametrize("k", [8, 1024, 5120, 17408])
def test_rms_rescale(env, k):
    torch, w12 = env
    g = np.random.default_rng(8 + k)
    x = wi.gaussian_bf16((24, k), 3.0, g)
    y = to_host(w12.rms_rescale(to_dev(x, torch)))
    yf = wi.bf16_bits_to_f32(y).astype(np.float64)
    xf = wi.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True))
    assert np.all(np.abs(yf - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_stack_small(env, fused):
    """The layer chain on small shapes (hidden 512, MLP 1536, 3 layers, vocab 4096), with
    the RMS rescale folded into the GEMMs and as separate launches: every GEMM of every
    layer against the oracle on its captured input (divided by the input rows' RMS where
    the GEMM applies it), and the final verification against the oracle's exact argmax."""
    torch, w12 = env
    from lossless_bit_weight_w12_amd.decode_step import DecodeStack, MATS
    g = np.random.default_rng(8800 + int(fused))
    hid, mlp, kv, vocab, m, nl = 512, 1536, 128, 4096, 24, 3
    shapes = {"q": (hid, hid), "k": (kv, hid), "v": (kv, hid), "o": (hid, hid),
              "gate": (mlp, hid), "up": (mlp, hid), "down": (hid, mlp)}
    host = [{name: wi.gaussian_bf16(shapes[name], 0.02, g) for name in MATS} for _ in range(nl)]
    layers = [{name: w12.encode(to_dev(L[name], torch)) for name in MATS} for L in host]
    head_w = wi.gaussian_bf16((vocab, hid), 0.02, g)
    stack = DecodeStack(layers, w12.encode(to_dev(head_w, torch)), m, fused_rms=fused)
    x0 = wi.gaussian_bf16((m, hid), 1.0, g)
    draft = g.integers(0, vocab, size=m).astype(np.int32)
    say("decode stack small, fused", fused)
    h, am, acc, caps = stack.step(to_dev(x0, torch), torch.from_numpy(draft).to("cuda:0"),
                                  capture=range(nl))
    torch.cuda.synchronize()
    for li in range(nl):
        for name in MATS:
            x_in, rms = caps[li]["in"][name]
            xh = to_host(x_in)
            z, s = rms_reference(xh, host[li][name]) if rms else o.gemm_reference(xh, host[li][name])
            assert o.gemm_accept(to_host(caps[li][name]), z, s).all(), (li, name)
    am_ref, _ = o.argmax_exact(to_host(h), head_w)
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    assert int(acc.item()) == o.accepted_length(am_ref, draft)


@pytest.mark.parametrize("m", [1, 17, 128])
def test_gemm_max_k(env, m):
    """The longest K the format allows (2^20 - 128, 8191 tile columns): 32-bit tile and x
    offsets at their largest, K split over the few row-blocks, escapes spread over every
    column; W12, tiled and row-major BF16 against the oracle."""
    torch, w12 = env
    g = np.random.default_rng(7000 + m)
    n, k = 32, (1 << 20) - 128
    w = wide_exponents((n, k), g, 110, 130)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    say("gemm max k", m, n, k)
    yb = _gemm_case(env, w, x, "w12")
    z, s = o.gemm_reference(x, w)
    xt, wt = to_dev(x, torch), to_dev(w, torch)
    for y in (w12.gemm_bf16(xt, wt), w12.gemm_bf16_tiled(xt, w12.bf16_tile(wt), n, k)):
        torch.cuda.synchronize()
        assert o.gemm_accept(to_host(y), z, s).all()
    assert yb.shape == (m, n)


def test_verify_max_k(env):
    """Greedy verification at the longest K: exact argmax and accepted length."""
    torch, w12 = env
    g = np.random.default_rng(7100)
    m, n, k = 3, 64, (1 << 20) - 128
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = wi.gaussian_bf16((n, k), 0.02, g)
    w[5] = w[40]        # an exact tie between rows 5 and 40 (lower index wins if it is the max)
    say("verify max k", m, n, k)
    am_ref, _ = o.argmax_exact(x, w)
    draft = am_ref.copy().astype(np.int32)
    draft[1] = (draft[1] + 1) % n
    am, acc = w12.lmhead_verify(to_dev(x, torch), w12.encode(to_dev(w, torch)),
                                torch.from_numpy(draft).to("cuda:0"))
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    assert int(acc.item()) == o.accepted_length(am_ref, draft) == 1


def test_graph_capture_replays_match_eager(env):
    """Prepared calls captured in a HIP graph (split-K GEMM completed in the kernel, grouped RMS
    GEMM, verification with its accept initialisation, two-level verification with its row
    tickets): every replay, with new inputs copied in eagerly between replays, equals the
    eager calls bit for bit."""
    torch, w12 = env
    g = np.random.default_rng(7400)
    dev = "cuda:0"
    w_split = wi.gaussian_bf16((320, 4096), 0.02, g)            # few row-blocks: K split
    ws_grp = [wi.gaussian_bf16(sh, 0.02, g) for sh in [(320, 512), (64, 512), (64, 512)]]
    w_head = wi.gaussian_bf16((4096, 512), 0.02, g)
    t_split = w12.encode(to_dev(w_split, torch))
    t_grp = [w12.encode(to_dev(w, torch)) for w in ws_grp]
    t_head = w12.encode(to_dev(w_head, torch))
    sc_head = w12.screen_encode(to_dev(w_head, torch))
    xs = [(wi.gaussian_bf16((7, 4096), 1.0, g), wi.gaussian_bf16((24, 512), 2.0, g),
           wi.gaussian_bf16((16, 512), 1.0, g)) for _ in range(3)]
    x1, x2, x3 = (to_dev(a, torch) for a in xs[0])
    y1 = torch.empty((7, 320), dtype=torch.bfloat16, device=dev)
    y2 = [torch.empty((24, w.shape[0]), dtype=torch.bfloat16, device=dev) for w in ws_grp]
    am = torch.empty(16, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    am2 = torch.empty(16, dtype=torch.int32, device=dev)
    acc2 = torch.empty(1, dtype=torch.int32, device=dev)
    draft = torch.zeros(16, dtype=torch.int32, device=dev)

    def calls():
        return [w12.prepare_gemm(x1, t_split, y1), w12.prepare_gemm_group(x2, t_grp, y2, rms=True),
                w12.prepare_verify(x3, t_head, draft, am, acc),
                w12.prepare_verify2(x3, t_head, sc_head, draft, am2, acc2)]

    def snapshot():
        return [y1.clone(), *[y.clone() for y in y2], am.clone(), acc.clone(), am2.clone(), acc2.clone()]

    eager = []
    for a, b, c in xs:                       # eager answers for each input set
        x1.copy_(to_dev(a, torch)); x2.copy_(to_dev(b, torch)); x3.copy_(to_dev(c, torch))
        for f in calls():
            f()
        torch.cuda.synchronize()
        eager.append(snapshot())
        assert torch.equal(eager[-1][-2], eager[-1][-4]) and torch.equal(eager[-1][-1], eager[-1][-3])
    say("graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fs = calls()                         # marshalled on the capture stream
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for f in fs:
                f()
    torch.cuda.current_stream().wait_stream(side)
    for r in (1, 0, 2, 1):
        a, b, c = xs[r]
        x1.copy_(to_dev(a, torch)); x2.copy_(to_dev(b, torch)); x3.copy_(to_dev(c, torch))
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(snapshot(), eager[r]):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), r
        torch.zeros(1, device=dev).add_(1)  # eager work between the replays
