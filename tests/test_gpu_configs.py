"""The five workloads at full size on the GPU, through the C ABI, against the oracle.

1  W [1024, 1024], x [1, 1024]: encode bytes, decode, GEMV, every output.
2  W [5120, 5120] with 0.1 % exponent outliers, x [1, 5120]: encode bytes (escape path),
   decode, GEMV, every output.
3  MLP block: gate+up [34816, 5120] and down [5120, 17408], M in {1, 4, 8, 16, 32}:
   encode bytes, decode, every output of every GEMM (W12 and the BF16 kernel).
4  LM head [151936, 5120], three M = 16 batches (batch 0 plain, batches 1-2 the 32 rows
   with planted near-ties): codebook, escape count and decode of the whole head, bytes of
   sampled row-block bands, argmax and accepted length of every row against the oracle.
   The same matrices in FP8 checkpoint form (E4M3, 128 x 128 block scales) at M = 16,
   64 and 128: every output of the FP8 GEMM.
5  Decode step: 64 layers of q, k, v, o, gate, up, down + LM head drawn on the device,
   M = 24, RMS-chained (the rescales folded into the consuming GEMMs); at layers 0, 21,
   42, 63 every GEMM output is checked against the oracle on the captured inputs
   (divided by the input rows' RMS where the GEMM applies it) and every weight's decode
   against its regenerated source; the final verification against the oracle's exact
   argmax.

Bars as in the other GPU tests: bytes, bits, argmax and accepted length exact; GEMM
outputs by oracle.gemm_accept."""
import numpy as np
import pytest

from oracle import w12_oracle as o
import w12_inputs as wi
import plant
from gpu_util import rms_reference, say, to_dev, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import lossless_bit_weight_w12_amd as w12
    w12.lib()
    return torch, w12


def _check_encode(t, w):
    ref = o.encode(w)
    assert t.codebook == tuple(ref.codebook.tolist())
    assert t.e_max == ref.e_max and t.n_esc == ref.n_esc
    assert np.array_equal(t.tiles.cpu().numpy(), ref.tiles)
    assert np.array_equal(t.esc_off.cpu().numpy().view(np.uint32), ref.esc_off)
    assert np.array_equal(t.esc.cpu().numpy().view(np.uint32)[:ref.n_esc], ref.esc)
    assert t.nbytes() == o.blob_bytes(ref)
    return ref


def _check_gemm(y_dev, x, w):
    z, s = o.gemm_reference(x, w)
    y = to_host(y_dev)
    ok = o.gemm_accept(y, z, s)
    bad = np.argwhere(~ok)
    assert ok.all(), f"{bad.shape[0]} outputs outside tolerance, first {bad[:4].tolist()}"


def _check_summary(torch, w12, t, w_host, w_dev, bands):
    """Codebook, e_max and escape count from the oracle's histogram of the whole
    tensor, the whole tensor's decode, and the bytes and escape records of sampled
    row-block bands encoded by the oracle with that codebook."""
    hist = o.exponent_histogram(w_host)
    cb = o.choose_codebook(hist)
    assert t.codebook == tuple(cb.tolist())
    assert t.e_max == o.finite_e_max(hist)
    assert t.n_esc == int(hist.sum() - hist[cb.astype(np.int64)].sum())
    assert torch.equal(w12.decode(t).view(torch.int16), w_dev.view(torch.int16))
    esc_off = t.esc_off.cpu().numpy().view(np.uint32)
    # column-major tiles: the band's tiles of every column, read column by column
    tiles = t.tiles.view(t.k // 128, t.n // 16, 3072)
    for b0, b1 in bands:
        ref = o.encode(w_host[16 * b0:16 * b1], codebook=cb)
        got = tiles[:, b0:b1].contiguous().cpu().numpy().reshape(-1)
        assert np.array_equal(got, ref.tiles), (b0, b1)
        lo, hi = int(esc_off[b0]), int(esc_off[b1])
        assert np.array_equal(esc_off[b0:b1 + 1] - lo, ref.esc_off)
        assert np.array_equal(t.esc[lo:hi].cpu().numpy().view(np.uint32), ref.esc)


def test_config1_layer_1024(env):
    torch, w12 = env
    w = wi.config_weights(1)["w"]
    x = wi.activations(1, wi.T_X, 1, 1024)
    say("config 1", w.shape)
    t = w12.encode(to_dev(w, torch))
    ref = _check_encode(t, w)
    assert np.array_equal(to_host(w12.decode(t)), w)
    _check_gemm(w12.gemm(to_dev(x, torch), t), x, w)
    say("config 1 bits/weight", o.bits_per_weight(ref), "escapes", ref.n_esc)


def test_config2_outliers_escape_path(env):
    torch, w12 = env
    w = wi.config_weights(2)["w"]
    x = wi.activations(2, wi.T_X, 1, 5120)
    say("config 2", w.shape)
    t = w12.encode(to_dev(w, torch))
    ref = _check_encode(t, w)
    assert ref.n_esc >= 0.0005 * w.size
    assert np.array_equal(to_host(w12.decode(t)), w)
    xt = to_dev(x, torch)
    _check_gemm(w12.gemm(xt, t), x, w)
    _check_gemm(w12.gemm_bf16(xt, to_dev(w, torch)), x, w)
    say("config 2 bits/weight", o.bits_per_weight(ref), "escapes", ref.n_esc)


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_config3_mlp_block(env, name):
    torch, w12 = env
    w = wi.weight(3, wi.T_W if name == "gate_up" else wi.T_W2, wi.CONFIG_SHAPES[3][name])
    n, k = w.shape
    say("config 3", name, w.shape)
    wd = to_dev(w, torch)
    t = w12.encode(wd)
    _check_encode(t, w)
    assert torch.equal(w12.decode(t).view(torch.int16), wd.view(torch.int16))
    for m in wi.CONFIG_SHAPES[3]["m"]:
        say("config 3", name, "m", m)
        x = wi.activations(3, wi.T_X if name == "gate_up" else wi.T_X2, m, k)
        xt = to_dev(x, torch)
        y = w12.gemm(xt, t)
        yb = w12.gemm_bf16(xt, wd)
        _check_gemm(y, x, w)
        _check_gemm(yb, x, w)


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_config3_mlp_block_batched(env, name):
    """The MLP matrices at the batched sizes the bench times (M = 64 and 128: several
    requests' draft rows at once), every output against the oracle, W12 and BF16."""
    torch, w12 = env
    w = wi.weight(3, wi.T_W if name == "gate_up" else wi.T_W2, wi.CONFIG_SHAPES[3][name])
    n, k = w.shape
    wd = to_dev(w, torch)
    t = w12.encode(wd)
    wt = w12.bf16_tile(wd)
    for m in (64, 128):
        say("config 3 batched", name, "m", m)
        x = wi.activations(3, wi.T_X if name == "gate_up" else wi.T_X2, m, k)
        xt = to_dev(x, torch)
        _check_gemm(w12.gemm(xt, t), x, w)
        _check_gemm(w12.gemm_bf16_tiled(xt, wt, n, k), x, w)


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_config3_mlp_block_f8(env, name):
    """The MLP matrices in FP8 checkpoint form (the same Gaussian weights quantized to
    E4M3 with 128 x 128 block scales) at the batched sizes the bench times, every output
    against the oracle."""
    torch, w12 = env
    q, s = wi.f8_weight(3, wi.T_W if name == "gate_up" else wi.T_W2, wi.CONFIG_SHAPES[3][name])
    n, k = q.shape
    qt = w12.f8_tile(torch.from_numpy(q).to("cuda:0"))
    st = torch.from_numpy(s).to("cuda:0")
    for m in (16, 64, 128):
        say("config 3 f8", name, "m", m)
        x = wi.activations(3, wi.T_X if name == "gate_up" else wi.T_X2, m, k)
        y = w12.gemm_f8(to_dev(x, torch), qt, st, n, k)
        z, sa = o.gemm_f8_reference(x, q, s)
        ok = o.gemm_accept(to_host(y), z, sa)
        assert ok.all(), f"{int((~ok).sum())} outputs outside tolerance"


@pytest.fixture(scope="module")
def lm_head():
    """Workload 4's head with the 32 near-tie rows of batches 1-2 planted, and the three
    hidden batches."""
    w = wi.config_weights(4)["w"]
    xs = [wi.verify_batch_x(b) for b in range(wi.VERIFY_BATCHES)]
    tie_x = np.concatenate(xs[1:])
    say("config 4 planting", tie_x.shape[0], "near-tie rows")
    w, pairs = plant.plant_near_ties(tie_x, w, lambda i: wi.tie_rng(1 + i // 16, i % 16))
    plant.check_plants(tie_x, w, pairs)
    return w, xs


def test_config4_lm_head_verify(env, lm_head):
    torch, w12 = env
    w, xs = lm_head
    vocab = w.shape[0]
    wd = to_dev(w, torch)
    t = w12.encode(wd)
    nb = vocab // 16
    _check_summary(torch, w12, t, w, wd, [(0, 3), (nb // 2, nb // 2 + 2), (nb - 3, nb)])
    del wd
    x_all = np.concatenate(xs)
    am_ref, ncand_ref = o.argmax_exact(x_all, w)
    say("config 4 oracle candidates per row", ncand_ref.tolist())
    for b, x in enumerate(xs):
        ref = am_ref[16 * b:16 * b + 16]
        p, r = wi.verify_mismatch(b, vocab)
        draft = ref.astype(np.int32).copy()
        if p < 16:
            draft[p] = (draft[p] + 1 + r) % vocab
        say("config 4 batch", b, "p", p)
        am, acc = w12.lmhead_verify(to_dev(x, torch), t, torch.from_numpy(draft).to("cuda:0"))
        torch.cuda.synchronize()
        assert am.cpu().numpy().tolist() == ref.tolist()
        assert int(acc.item()) == o.accepted_length(ref, draft) == p
        nc = w12.verify_candidates(t, 16).cpu().numpy()
        say("config 4 batch", b, "GPU candidates / left after the FP64 screen",
            nc.tolist())
        assert (nc[:, 0] >= 1).all() and (nc[:, 1] >= 1).all()


@pytest.mark.parametrize("m", [1, 8])
def test_config4_lm_head_verify_small_m(env, lm_head, m):
    """Workload 4's head verified at 1 and 8 rows (single-request drafts shorter than 16:
    the first pass takes the wave-column VALU kernel with two row-blocks per wave at 1 row,
    the column-synchronous MFMA kernel at 8): the first m planted near-tie rows of batch 1, argmax and accepted
    length against the oracle; and the certified bound on every FP32 logit of the same
    first pass (w12_logits_f32)."""
    torch, w12 = env
    w, xs = lm_head
    vocab, k = w.shape
    x = xs[1][:m]
    t = w12.encode(to_dev(w, torch))
    say("config 4 small m", m, "oracle argmax")
    am_ref, _ = o.argmax_exact(x, w)
    draft = am_ref.astype(np.int32).copy()
    p = m // 2
    draft[p] = (draft[p] + 1 + 12345) % vocab
    xt = to_dev(x, torch)
    am, acc = w12.lmhead_verify(xt, t, torch.from_numpy(draft).to("cuda:0"))
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    assert int(acc.item()) == o.accepted_length(am_ref, draft) == p
    say("config 4 small m", m, "pass-1 bound")
    z_hat, s_hat = (v.cpu().numpy().astype(np.float64) for v in w12.logits_f32(xt, t))
    z, s = o.gemm_reference(x, w)
    xmax = np.abs(wi.bf16_bits_to_f32(x).astype(np.float64)).max()
    d = k // 128 + 192.0   # the certified depth (tile columns summed from zero)
    gam = d * 2.0 ** -23 / (1 - d * 2.0 ** -23)
    a = (2 * k + d) * 2.0 ** -126 * (1 + xmax + 2.0 ** (t.e_max - 126))
    bound = gam * (s_hat / (1 - gam) + a) + a
    assert (np.abs(z_hat - z) <= bound).all()
    assert (s <= s_hat / (1 - gam) + a).all()


def test_config4_lm_head_verify_batched(env, lm_head):
    """Workload 4's head (near ties planted) verifying 24 requests x 5 rows in one call,
    as the bench times it: every row's argmax is the oracle's exact-logit argmax and every
    request's accepted length the oracle's per-request rule, with the planted first
    mismatches."""
    torch, w12 = env
    w, _ = lm_head
    vocab = w.shape[0]
    t = w12.encode(to_dev(w, torch))
    x = wi.batched_verify_x()
    off, nd, pb, rb = wi.batched_verify_table(vocab)
    say("config 4 batched: oracle argmax of", x.shape[0], "rows")
    am_ref, _ = o.argmax_exact(x, w)
    draft = am_ref.astype(np.int32).copy()
    for r in range(len(nd)):
        if pb[r] < nd[r]:
            i = off[r] + pb[r]
            draft[i] = (draft[i] + 1 + rb[r]) % vocab
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")
    am, acc = w12.lmhead_verify_batched(to_dev(x, torch), t, dev(off), dev(nd), dev(draft))
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    want = o.accepted_lengths_batched(am_ref, draft, off, nd)
    assert acc.cpu().numpy().tolist() == want.tolist() == np.minimum(pb, nd).tolist()


def test_config4_two_level_verify(env, lm_head):
    """Two-level verification on workload 4's head with the planted near ties: the screen
    copy's codes and scales equal the oracle's on sampled row-blocks, every screen logit
    of batch 0 lies within its certified bound of the float64 logit, and every batch's
    argmax and accepted length equal the oracle's (and the single-level call's); then 1
    and 8 rows, and the 24-request batch."""
    torch, w12 = env
    w, xs = lm_head
    vocab, k = w.shape
    wd = to_dev(w, torch)
    t = w12.encode(wd)
    sc = w12.screen_encode(wd)
    torch.cuda.synchronize()
    del wd
    # codes and scales of three sampled row-blocks (tiles of every column)
    nb, gk = vocab // 16, k // 128
    buf = sc.buf.cpu().numpy()
    for b in (0, nb // 2, nb - 1):
        q, s_bits, _ = o.screen_encode(w[16 * b:16 * b + 16])
        want = o.screen_pack(q, s_bits).reshape(gk, o.SCREEN_TILE_BYTES)
        got = np.stack([buf[(g * nb + b) * o.SCREEN_TILE_BYTES:(g * nb + b + 1) * o.SCREEN_TILE_BYTES]
                        for g in range(gk)])
        assert np.array_equal(got, want), b
    say("config 4 two-level: screen bound on batch 0")
    z8, bnd = (v.cpu().numpy().astype(np.float64) for v in w12.screen_logits_f32(to_dev(xs[0], torch), t, sc))
    z, s = o.gemm_reference(xs[0], w)
    assert (np.abs(z8 - z) <= bnd + (k + 2) * 2.0 ** -52 * s).all()
    x_all = np.concatenate(xs)
    am_ref, _ = o.argmax_exact(x_all, w)
    for b, x in enumerate(xs):
        ref = am_ref[16 * b:16 * b + 16]
        p, r = wi.verify_mismatch(b, vocab)
        draft = ref.astype(np.int32).copy()
        if p < 16:
            draft[p] = (draft[p] + 1 + r) % vocab
        say("config 4 two-level batch", b, "p", p)
        am, acc = w12.lmhead_verify2(to_dev(x, torch), t, sc, torch.from_numpy(draft).to("cuda:0"))
        torch.cuda.synchronize()
        assert am.cpu().numpy().tolist() == ref.tolist()
        assert int(acc.item()) == o.accepted_length(ref, draft) == p
        nc = w12.verify2_candidates(t, 16).cpu().numpy()
        say("config 4 two-level batch", b, "candidates / left after FP64", nc.tolist())
        assert (nc[:, 0] >= 1).all() and (nc[:, 1] >= 1).all()
    for m in (1, 8):
        x = xs[1][:m]
        ref = am_ref[16:16 + m]
        draft = ref.astype(np.int32).copy()
        draft[m // 2] = (draft[m // 2] + 1 + 12345) % vocab
        am, acc = w12.lmhead_verify2(to_dev(x, torch), t, sc, torch.from_numpy(draft).to("cuda:0"))
        torch.cuda.synchronize()
        assert am.cpu().numpy().tolist() == ref.tolist()
        assert int(acc.item()) == m // 2
    xb = wi.batched_verify_x()
    off, nd, pb, rb = wi.batched_verify_table(vocab)
    say("config 4 two-level batched: oracle argmax of", xb.shape[0], "rows")
    amb_ref, _ = o.argmax_exact(xb, w)
    draft = amb_ref.astype(np.int32).copy()
    for r in range(len(nd)):
        if pb[r] < nd[r]:
            i = off[r] + pb[r]
            draft[i] = (draft[i] + 1 + rb[r]) % vocab
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")
    am, acc = w12.lmhead_verify2_batched(to_dev(xb, torch), t, sc, dev(off), dev(nd), dev(draft))
    torch.cuda.synchronize()
    assert am.cpu().numpy().tolist() == amb_ref.tolist()
    assert acc.cpu().numpy().tolist() == np.minimum(pb, nd).tolist()


SAMPLED_LAYERS = (0, 21, 42, 63)


def test_config5_decode_step(env):
    torch, w12 = env
    from lossless_bit_weight_w12_amd.decode_step import DecodeStack, MATS
    c5 = wi.CONFIG_SHAPES[5]
    m, hid, vocab = c5["m"][0], c5["hidden"], c5["vocab"]
    shapes = {name: (n, k) for name, n, k in wi.LAYER_MATS}
    layers = []
    for li in range(c5["layers"]):
        if li % 8 == 0:
            say("config 5 encoding layer", li)
        L = {}
        for mi, name in enumerate(MATS):
            n, k = shapes[name]
            L[name] = w12.encode(wi.device_layer_weight(torch, li, mi, n, k))
        layers.append(L)
    head = w12.encode(wi.device_lm_head(torch, vocab, hid))
    stack = DecodeStack(layers, head, m)
    x0 = wi.decode_step_x(m, hid)
    draft = wi.decode_step_draft(vocab, m)
    say("config 5 running the step")
    h, am, acc, caps = stack.step(to_dev(x0, torch), torch.from_numpy(draft).to("cuda:0"),
                                  capture=SAMPLED_LAYERS)
    torch.cuda.synchronize()
    for li in SAMPLED_LAYERS:
        cap = caps[li]
        for mi, name in enumerate(MATS):
            n, k = shapes[name]
            say("config 5 layer", li, name)
            src = wi.device_layer_weight(torch, li, mi, n, k)
            assert torch.equal(w12.decode(layers[li][name]).view(torch.int16), src.view(torch.int16))
            w_host = to_host(src)
            x_in, rms = cap["in"][name]
            x_host = to_host(x_in)
            z, s = rms_reference(x_host, w_host) if rms else o.gemm_reference(x_host, w_host)
            ok = o.gemm_accept(to_host(cap[name]), z, s)
            assert ok.all(), (li, name, int((~ok).sum()))
    # the final h (rescaled on its own) has unit mean square, BF16 rounding aside
    v = h.float()
    assert torch.all(((v * v).mean(dim=1) - 1).abs() < 1e-2)
    # final verification against the oracle on the captured final h
    say("config 5 LM head verify")
    w_head = to_host(wi.device_lm_head(torch, vocab, hid))
    h_host = to_host(h)
    am_ref, _ = o.argmax_exact(h_host, w_head)
    assert am.cpu().numpy().tolist() == am_ref.tolist()
    assert int(acc.item()) == o.accepted_length(am_ref, draft)
