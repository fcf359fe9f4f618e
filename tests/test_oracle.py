"""Pins for the CPU oracle: every check here compares the oracle with something other
than itself -- a hand-derived worked example, closed forms, invariants of the layout,
exact rational brute force, or constructions whose answer is known in advance.
The mutation tests at the end plant plausible mistakes in the oracle (on the CPU) and
show that at least one pin fails for each."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import w12_oracle as o
import w12_inputs as wi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_fraction(b) -> Fraction:
    """Exact value of a BF16 pattern via Python's float (independent of the oracle)."""
    f = np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


# ----------------------------------------------------------------------------- format
def worked_example_matrix():
    w = np.zeros((16, 128), dtype=np.uint16)
    for r in range(16):
        for c in range(128):
            s = 1 if c >= 64 else 0
            w[r, c] = (s << 15) | ((100 + r) << 7) | (c & 0x7F)
    w[5, 77] = (1 << 15) | (30 << 7) | 77
    return w


def test_worked_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "w12_v1_worked_example.json")))
    w = worked_example_matrix()
    b = o.encode(w)
    assert b.codebook.tolist() == g["codebook"]
    assert b.e_max == g["e_max"]
    assert b.esc_off.tolist() == g["esc_off"]
    assert b.esc.tolist() == g["esc"]
    for pos, val in g["tile_bytes"].items():
        assert int(b.tiles[int(pos)]) == val, pos
    for pos, val in g["code_words"].items():
        p = int(pos)
        word = int.from_bytes(bytes(b.tiles[p:p + 4].tolist()), "little")
        assert word == val, pos
    assert o.blob_bytes(b) == g["total_bytes"]
    assert o.bits_per_weight(b) == g["bits_per_weight"]
    assert o.header(b).hex() == g["header_hex"]
    assert np.array_equal(o.decode(b), w)


def test_all_bf16_patterns_roundtrip():
    w = wi.all_bf16_patterns()
    b = o.encode(w)
    # every exponent field occurs 256 times: the tie rule picks 0..15
    assert b.codebook.tolist() == list(range(16))
    assert b.n_esc == 65536 * 240 // 256
    assert b.e_max == 254
    assert np.array_equal(o.decode(b), w)


def test_slot_layout_is_a_bijection():
    r, kap, sm_pos, word_pos, bit = o.slot_layout()
    pairs = set(zip(r.reshape(-1).tolist(), kap.reshape(-1).tolist()))
    assert len(pairs) == 2048 and pairs == {(a, c) for a in range(16) for c in range(128)}
    assert sorted(sm_pos.reshape(-1).tolist()) == list(range(2048))
    nib = set()
    for wp, bt in zip(word_pos.reshape(-1).tolist(), bit.reshape(-1).tolist()):
        nib.add(2 * wp + bt // 4)          # nibble index inside the tile
    assert nib == set(range(2 * 2048, 2 * 3072))


def test_codebook_definition_pairwise():
    """Pairwise form of the rule: each chosen exponent beats each unchosen one by
    (count, then smaller exponent)."""
    g = np.random.default_rng(7)
    for trial in range(200):
        h = g.integers(0, 4, size=256) * g.integers(0, 2, size=256)
        if trial % 3 == 0:
            h[:] = 0
            h[g.choice(256, size=5, replace=False)] = g.integers(1, 9, size=5)
        cb = o.choose_codebook(h).tolist()
        assert cb == sorted(set(cb)) and len(cb) == 16
        chosen = set(cb)
        for c in chosen:
            for d in range(256):
                if d not in chosen:
                    assert (h[c] > h[d]) or (h[c] == h[d] and c < d)


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(a=st.integers(1, 4), bb=st.integers(1, 3), seed=st.integers(0, 2**31 - 1),
       kind=st.sampled_from(["bits", "gauss", "narrow"]))
def test_roundtrip_and_escape_invariants(a, bb, seed, kind):
    n, k = 16 * a, 128 * bb
    g = np.random.default_rng(seed)
    if kind == "bits":
        w = wi.random_bits((n, k), g)
    elif kind == "gauss":
        w = wi.gaussian_bf16((n, k), 0.02, g)
    else:   # few distinct exponents: codebook padded with unused ones
        w = ((g.integers(0, 2, (n, k)) << 15) | (g.integers(120, 123, (n, k)) << 7)
             | g.integers(0, 128, (n, k))).astype(np.uint16)
    b = o.encode(w)
    assert np.array_equal(o.decode(b), w)
    # closed form: n_esc = sum of counts of exponents outside the codebook
    e = (w.astype(np.int64) >> 7) & 0xFF
    assert b.n_esc == int((~np.isin(e, b.codebook.astype(np.int64))).sum())
    assert b.esc_off[0] == 0 and b.esc_off[-1] == b.n_esc
    assert np.all(np.diff(b.esc_off.astype(np.int64)) >= 0)
    for blk in range(n // 16):
        recs = b.esc[b.esc_off[blk]:b.esc_off[blk + 1]].astype(np.int64)
        keys = [((rc >> 8) & 0xFFFFF, rc >> 28) for rc in recs]
        assert keys == sorted(keys)
        for rc in recs:
            r, kk, ee = rc >> 28, (rc >> 8) & 0xFFFFF, rc & 0xFF
            assert e[16 * blk + r, kk] == ee and ee not in b.codebook


@pytest.mark.parametrize("n,k", [(16, 128), (64, 1024), (1024, 1024)])
def test_bits_per_weight_closed_form(n, k):
    w = wi.gaussian_bf16((n, k), 0.02, np.random.default_rng(n + k))
    b = o.encode(w)
    nb, gk = n // 16, k // 128
    expect = 3072 * nb * gk + 4 * b.n_esc + 4 * (nb + 1) + 64
    assert o.blob_bytes(b) == expect
    assert b.tiles.size * 4 == 3 * (2 * n * k)       # tiles are exactly 3/4 of BF16 bytes
    assert o.bits_per_weight(b) == 12 + 8 * (4 * b.n_esc + 4 * (nb + 1) + 64) / (n * k)


def test_gaussian_codebook_and_escape_rate():
    """For N(0, 0.02^2) the 16 most populated binades are e = 108..123 (masses of the
    neighbours: e=107 ~ 3.8e-5, e=124 ~ 4e-10), so escapes are the |w| < 2^-19 tail
    (rate ~ 2*pdf(0)*2^-19 = 7.6e-5)."""
    w = wi.config_weights(1)["w"]
    b = o.encode(w)
    assert b.codebook.tolist() == list(range(108, 124))
    rate = b.n_esc / w.size
    assert 2e-5 < rate < 2e-4


def test_band_encode_with_tensor_codebook_is_a_slice():
    """A band of row-blocks encoded with the whole tensor's codebook gives exactly the
    whole encode's bytes and escape records for those blocks (row-blocks are encoded
    independently once the codebook is fixed); the sampled checks at full size rely
    on this."""
    g = np.random.default_rng(77)
    w = wi.add_exponent_outliers(wi.gaussian_bf16((160, 384), 0.02, g), 0.01, 5)
    w[37, 5] = 0x7F80
    full = o.encode(w)
    for b0, b1 in [(0, 1), (3, 7), (9, 10)]:
        band = o.encode(w[16 * b0:16 * b1], codebook=full.codebook)
        assert np.array_equal(band.tiles, o.band_tiles(full.tiles, 160, 384, b0, b1))
        # column-major tile order: row-block b's tile of column g at (g * 10 + b) * 3072
        for g in range(3):
            for b in range(b0, b1):
                off = (g * 10 + b) * 3072
                assert np.array_equal(full.tiles[off:off + 3072],
                                      band.tiles[(g * (b1 - b0) + b - b0) * 3072:][:3072])
        lo, hi = full.esc_off[b0], full.esc_off[b1]
        assert np.array_equal(band.esc, full.esc[lo:hi])
        assert np.array_equal(band.esc_off, full.esc_off[b0:b1 + 1] - lo)
    with pytest.raises(ValueError):
        o.encode(w, codebook=np.arange(15, dtype=np.uint8))
    with pytest.raises(ValueError):
        o.encode(w, codebook=np.array([5] * 16, dtype=np.uint8))


def test_outlier_workload_escapes():
    w = wi.config_weights(2)["w"]
    b = o.encode(w)
    assert b.n_esc >= 0.0005 * w.size
    assert np.array_equal(o.decode(b), w)


# ----------------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("m", [1, 2, 7, 15, 16, 17, 31, 32])
def test_gemm_reference_vs_exact_rationals(m):
    g = np.random.default_rng(100 + m)
    n, k = 16, 128
    x = wi.gaussian_bf16((m, k), 1.0, g)
    w = wi.gaussian_bf16((n, k), 0.02, g)
    z, s = o.gemm_reference(x, w)
    xf = [[bf16_fraction(v) for v in row] for row in x]
    wf = [[bf16_fraction(v) for v in row] for row in w]
    for mi in range(m):
        for ni in range(n):
            exact = sum(a * c for a, c in zip(xf[mi], wf[ni]))
            sabs = sum(abs(a * c) for a, c in zip(xf[mi], wf[ni]))
            assert abs(Fraction(z[mi, ni]) - exact) <= Fraction(k, 2**52) * sabs
            assert abs(Fraction(s[mi, ni]) - sabs) <= Fraction(k, 2**52) * sabs


def test_gemm_reference_special_case_library():
    """With W in BF16 the reference is the float64 matrix product: torch on the CPU."""
    import torch
    g = np.random.default_rng(5)
    x = wi.gaussian_bf16((4, 256), 1.0, g)
    w = wi.gaussian_bf16((32, 256), 0.02, g)
    z, _ = o.gemm_reference(x, w)
    xt = torch.from_numpy(wi.bf16_bits_to_f32(x).astype(np.float64))
    wt = torch.from_numpy(wi.bf16_bits_to_f32(w).astype(np.float64))
    assert np.allclose(z, (xt @ wt.T).numpy(), rtol=0, atol=1e-12)


def test_tolerance_rule():
    g = np.random.default_rng(3)
    x = wi.gaussian_bf16((2, 512), 1.0, g)
    w = wi.gaussian_bf16((16, 512), 0.02, g)
    z, s = o.gemm_reference(x, w)
    y = wi.f32_to_bf16_bits(z.astype(np.float32))
    assert o.within_tolerance(y, z, s).all()
    bad = y.copy()
    bad[0, 3] ^= 0x0100          # move the exponent: far outside the rule
    assert not o.within_tolerance(bad, z, s)[0, 3]


def test_bf16_round_against_rationals():
    """Direct RNE to BF16, pinned against exact rational rounding (ties included)."""
    g = np.random.default_rng(21)
    vals = list(g.standard_normal(300) * 10.0 ** g.integers(-40, 38, 300))
    vals += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -133 * 1.5,
             2.0 ** -133 * 2.5, 2.0 ** -126 * (1 - 2.0 ** -9), 75.75, 0.0, -0.0]
    got = o.bf16_round(np.array(vals))
    for v, b in zip(vals, got):
        fv = Fraction(v)
        # exact neighbours on the BF16 grid
        if fv == 0:
            assert int(b) & 0x7FFF == 0
            continue
        sign = -1 if fv < 0 else 1
        a = abs(fv)
        e = a.numerator.bit_length() - a.denominator.bit_length()
        while Fraction(2) ** e > a:
            e -= 1
        while Fraction(2) ** (e + 1) <= a:
            e += 1
        step = Fraction(2) ** max(e - 7, -133)
        qf = a / step
        lo_q = qf.numerator // qf.denominator
        rem = qf - lo_q
        q = lo_q + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo_q % 2 == 1) else 0)
        assert bf16_fraction(b) == sign * q * step, v


def test_rounded_rule_accepts_correct_rounding_only():
    g = np.random.default_rng(22)
    x = wi.gaussian_bf16((2, 512), 1.0, g)
    w = wi.add_exponent_outliers(wi.gaussian_bf16((64, 512), 0.02, g), 0.02, 3)
    z, s = o.gemm_reference(x, w)
    y = o.bf16_round(z)
    assert o.within_tolerance_rounded(y, z, s).all()
    assert o.gemm_accept(y, z, s).all()
    # a value two BF16 ulps away from the nearest admissible rounding is rejected
    tau = o.REL_TOL * s + o.ABS_TOL
    far = o.bf16_round(z + tau).astype(np.int32) + np.where(z + tau >= 0, 2, -2)
    assert not o.within_tolerance_rounded(far.astype(np.uint16), z, s).any()


def _golden_vector(spec, k):
    v = np.zeros(k, dtype=np.uint16)
    for key, val in spec.items():
        lo, _, hi = key.partition("..")
        v[int(lo):int(hi or lo) + 1] = int(val, 16)
    return v


def test_acceptance_boundary_golden():
    """Hand-worked boundary of the acceptance rule (tests/golden/gemm_acceptance_boundary.json):
    z and S of each case are exact, the last accepted BF16 value at z + tau and the next one
    beyond are known, and so are the cases where only the rounding-aware rule can accept."""
    g = json.load(open(os.path.join(GOLDEN, "gemm_acceptance_boundary.json")))
    k = g["k"]
    for case in g["cases"]:
        x = _golden_vector(case["x"], k)[None, :]
        w = _golden_vector(case["w"], k)[None, :]
        z, s = o.gemm_reference(x, w)
        assert Fraction(z[0, 0]) == Fraction(case["z"]) and Fraction(s[0, 0]) == Fraction(case["s"])
        tau = o.REL_TOL * s + o.ABS_TOL
        assert Fraction(tau[0, 0]) == Fraction(float(Fraction(case["tau"])))
        for key, rule, want in (("accepted", o.gemm_accept, True), ("rejected", o.gemm_accept, False),
                                ("literal_accepted", o.within_tolerance, True),
                                ("literal_rejected", o.within_tolerance, False)):
            for y in case[key]:
                got = bool(rule(np.array([[int(y, 16)]], dtype=np.uint16), z, s)[0, 0])
                assert got == want, (case["name"], key, y)


def test_rounded_rule_contains_literal_rule():
    """Every BF16 value the literal rule accepts is accepted by the rounding-aware rule
    (it is its own rounding and RNE is monotone), on random rows with and without
    dominating products and on every BF16 value near each z."""
    g = np.random.default_rng(23)
    x = wi.gaussian_bf16((3, 256), 1.0, g)
    w = wi.add_exponent_outliers(wi.gaussian_bf16((48, 256), 0.02, g), 0.02, 4)
    z, s = o.gemm_reference(x, w)
    base = o.bf16_round(z).astype(np.int32)
    for d in range(-40, 41):
        y = np.clip(base + d, 0, 0xFFFF).astype(np.uint16)
        # stay on the side of zero z is on (adding to the bits moves away from zero)
        y = np.where((base >> 15) == (y.astype(np.int32) >> 15), y, base.astype(np.uint16))
        lit = o.within_tolerance(y, z, s)
        assert (o.gemm_accept(y, z, s) | ~lit).all()


# ----------------------------------------------------------------------------- exact argmax
def test_exact_logit_matches_rationals():
    g = np.random.default_rng(11)
    for k in (128, 640):
        x = wi.gaussian_bf16((1, k), 1.0, g)[0]
        w = wi.gaussian_bf16((1, k), 0.02, g)[0]
        w[:5] = [0x0001, 0x8003, 0x0000, 0x7F7F, 0x0080]   # subnormals, zero, max, min normal
        x[:5] = [0x0005, 0x3F80, 0x8000, 0x0001, 0x8081]
        z = o.exact_logit(x, w)
        exact = sum(bf16_fraction(a) * bf16_fraction(c) for a, c in zip(x, w))
        assert Fraction(z, 2**266) == exact


def brute_argmax(x, w):
    out = []
    wf = [[bf16_fraction(v) for v in row] for row in w]
    for row in x:
        xf = [bf16_fraction(v) for v in row]
        vals = [sum(a * c for a, c in zip(xf, wr)) for wr in wf]
        best = max(vals)
        out.append(vals.index(best))     # first (lowest) index attaining the max
    return out


def test_argmax_matches_brute_force():
    g = np.random.default_rng(12)
    x = wi.gaussian_bf16((3, 128), 1.0, g)
    w = wi.gaussian_bf16((48, 128), 0.02, g)
    am, _ = o.argmax_exact(x, w)
    assert am.tolist() == brute_argmax(x, w)


def test_argmax_planted_exact_tie_picks_lowest_index():
    g = np.random.default_rng(13)
    x = wi.gaussian_bf16((1, 256), 1.0, g)
    w = wi.gaussian_bf16((64, 256), 0.02, g)
    v1 = int(o.argmax_exact(x, w)[0][0])
    v2 = 3 if v1 != 3 else 60
    w[v2] = w[v1]
    am, _ = o.argmax_exact(x, w)
    assert am[0] == min(v1, v2)


def test_argmax_planted_one_ulp_pair():
    """Copy the winner's row, then move one weight by one BF16 ulp in the direction that
    raises (or lowers) the logit: the answer is known by construction."""
    g = np.random.default_rng(14)
    x = wi.gaussian_bf16((1, 256), 1.0, g)
    w = wi.gaussian_bf16((64, 256), 0.02, g)
    v1 = int(o.argmax_exact(x, w)[0][0])
    v2 = 10 if v1 > 10 else 63
    for raise_it in (True, False):
        w2 = w.copy()
        w2[v2] = w2[v1]
        kk = next(i for i in range(256) if (w2[v2, i] & 0x7F) not in (0, 0x7F)
                  and (x[0, i] & 0x7FFF) != 0)
        same_sign = ((x[0, kk] >> 15) == (w2[v2, kk] >> 15))
        bump = 1 if same_sign == raise_it else -1       # +1 ulp in magnitude raises x*w if signs agree
        w2[v2, kk] = int(w2[v2, kk]) + bump
        am, _ = o.argmax_exact(x, w2)
        assert am[0] == (v2 if raise_it else v1)


def sub_fp64_near_tie():
    """A head on which float64 summation misorders the top two exact logits.  With x = 1
    at columns 0, 64 and 128 (zero elsewhere), row 3's products are {1, 2^-60, -1} (exact
    logit 2^-60) and row 2's {2^-61} (exact 2^-61); every other row's logit is -1.  A
    float64 sum that adds 2^-60 to 1 before the -1 arrives loses it (1 + 2^-60 rounds to
    1) and gets 0 < 2^-61; the columns are 64 apart so that any blocked summation with up
    to 64 running sums keeps the three terms in one of them, in column order.  Row 11 of
    a second x row repeats the construction with the winner at the lower index (row 5
    {1, 2^-60, -1} at columns 1, 65, 129 against row 11's {2^-61}).  Expected answers by
    construction: 3 and 5."""
    one, m_one, e60, e61 = 0x3F80, 0xBF80, 0x2180, 0x2100      # 1, -1, 2^-60, 2^-61
    k = 256
    x = np.zeros((2, k), dtype=np.uint16)
    x[0, [0, 64, 128]] = one
    x[1, [1, 65, 129]] = one
    w = np.zeros((16, k), dtype=np.uint16)
    w[:, 0] = m_one
    w[:, 1] = m_one
    w[3, [0, 64, 128]] = [one, e60, m_one]
    w[2, 0] = e61
    w[5, [1, 65, 129]] = [one, e60, m_one]
    w[11, 1] = e61
    for v in (3, 2):
        w[v, 1] = 0          # rows 2, 3 take no part in the second construction
    for v in (5, 11):
        w[v, 0] = 0
    return x, w, [3, 5]


def test_argmax_sub_fp64_near_tie():
    """Pins the width of the oracle's float64 filter: the exact winner's float64 logit is
    below the float64 maximum, so a filter that keeps only the float64 maximum answers
    wrongly; the exact answer (by construction, and by rational brute force) is kept."""
    x, w, want = sub_fp64_near_tie()
    z, _ = o.gemm_reference(x, w)
    # the construction does what it is for: float64 misorders both pairs here
    assert z[0, 3] < z[0, 2] and z[1, 5] < z[1, 11], (z[0, [2, 3]], z[1, [5, 11]])
    am, ncand = o.argmax_exact(x, w)
    assert am.tolist() == want == brute_argmax(x, w)
    assert (ncand >= 2).all()


def test_accepted_length_cases():
    am = np.array([5, 6, 7, 8])
    assert o.accepted_length(am, np.array([9, 6, 7, 8])) == 0
    assert o.accepted_length(am, np.array([5, 6, 7, 8])) == 4
    assert o.accepted_length(am, np.array([5, 6, 0, 8])) == 2     # later matches not counted
    assert o.accepted_length(am, np.array([5, 6])) == 2
    assert o.accepted_length(am, np.array([], dtype=np.int64)) == 0


def test_accepted_lengths_batched_cases():
    # four requests over ten rows, worked by hand: request 0 mismatches at its second
    # token, request 1 accepts both, request 2 mismatches at its third of four, request 3
    # drafts nothing (its row is the bonus row only)
    am = np.array([5, 6, 7, 1, 2, 9, 9, 9, 9, 4])
    draft = np.array([5, 0, 7, 1, 2, 9, 9, 3, 9, 8])
    row_off, n_draft = [0, 3, 5, 9, 10], [2, 2, 4, 0]
    assert list(o.accepted_lengths_batched(am, draft, row_off, n_draft)) == [1, 2, 2, 0]
    # tokens past a request's n_draft are not compared (row 2 of request 0, row 9)
    d2 = draft.copy(); d2[2] = 99; d2[9] = 4
    assert list(o.accepted_lengths_batched(am, d2, row_off, n_draft)) == [1, 2, 2, 0]
    # requests are independent: fixing request 0's mismatch moves only its own length
    d3 = draft.copy(); d3[1] = 6
    assert list(o.accepted_lengths_batched(am, d3, row_off, n_draft)) == [2, 2, 2, 0]
    # one request over all rows is the single-request rule
    assert list(o.accepted_lengths_batched(am, draft, [0, 10], [10])) == [o.accepted_length(am, draft)] == [1]


# ----------------------------------------------------------------------------- screen copy
def _golden_screen():
    g = json.load(open(os.path.join(GOLDEN, "screen_copy_worked_example.json")))
    w = np.zeros((g["n"], g["k"]), dtype=np.uint16)
    for r, c, b in g["weights"]:
        w[r, c] = int(b, 16)
    return g, w


def _units(pairs):
    """sum of coef * 2^exp in units of 2^-266."""
    return sum(int(c) << (int(e) + 266) for c, e in pairs)


def test_screen_worked_example_golden():
    g, w = _golden_screen()
    q, s_bits, fin = o.screen_encode(w)
    for r, j, b in g["scales"]:
        assert int(s_bits[r, j]) == int(b, 16), (r, j)
    for r, c, v in g["codes"]:
        assert int(q[r, c]) == v, (r, c)
    for r, f in g["rows_finite"].items():
        assert bool(fin[int(r)]) == f, r
    tiles = o.screen_pack(q, s_bits)
    assert tiles.size == o.SCREEN_TILE_BYTES
    for off, b in g["tile_bytes"]:
        assert int(tiles[off]) == int(b, 16), off
    # every other code byte is zero, every other scale 2^-100
    listed = {off for off, _ in g["tile_bytes"]}
    assert all(tiles[i] == 0 for i in range(2048) if i not in listed)
    for r, sums in g["exact_sums_units_2^-266"].items():
        r2, q2 = o.screen_row_sums_exact(w[int(r)], q[int(r)], s_bits[int(r)])
        assert r2 == _units(sums["R2"]) and q2 == _units(sums["Q2"]), r


def _screen_mats():
    g = np.random.default_rng(77)
    yield wi.gaussian_bf16((32, 512), 0.02, g)
    yield wi.add_exponent_outliers(wi.gaussian_bf16((16, 384), 0.02, g), 0.02, 9)
    yield wi.random_bits((16, 256), g)                       # every pattern, non-finite included
    sub = wi.random_bits((16, 256), g) & np.uint16(0x807F)   # zeros and subnormals only
    yield sub
    tiny = wi.gaussian_bf16((16, 128), 1.0, g)
    tiny = (tiny & np.uint16(0x807F)) | np.uint16(20 << 7)    # exponents far below 2^-100 * 127
    yield tiny


def _prev_bf16(bits):
    return (bits.astype(np.int64) - 1).astype(np.uint16)


def test_screen_invariants():
    for w in _screen_mats():
        n, k = w.shape
        q, s_bits, fin = o.screen_encode(w)
        wf = o.bf16_to_f64(w)
        finite = np.isfinite(wf)
        assert np.array_equal(fin, finite.all(axis=1))
        assert np.all(q[~finite] == 0)
        s = np.repeat(o.bf16_to_f64(s_bits), 32, axis=1)
        assert np.all(np.abs(q.astype(np.int64)) <= 127)
        assert np.all(s >= 2.0 ** -100)
        wz = np.where(finite, wf, 0.0)
        amax = np.abs(wz).reshape(n, k // 32, 32).max(axis=2)
        s_g = o.bf16_to_f64(s_bits)
        assert np.all(amax <= 127 * s_g)                      # exact: 127 * s has 15 bits
        above = s_g > 2.0 ** -100
        prev = o.bf16_to_f64(_prev_bf16(s_bits))
        assert np.all(127 * prev[above] < amax[above])        # s is the smallest such BF16
        r = wz - q * s                                        # exact (at most 8 significant bits)
        assert np.all(np.abs(r) <= s / 2)
        tie = np.abs(r) == s / 2
        assert np.all(q[tie] % 2 == 0)


def test_screen_codes_sit_at_w12_sign_mantissa_positions():
    """The screen copy puts each code where W12 v1 puts the sign/mantissa byte of the same
    element: weights whose sm byte equals the code (one exponent, no escapes) encode to W12
    tiles whose first 2048 bytes equal the screen tiles' code bytes."""
    g = np.random.default_rng(5)
    n, k = 32, 256
    q = g.integers(-127, 128, size=(n, k)).astype(np.int8)
    sm = q.view(np.uint8).astype(np.uint32)
    w = (((sm >> 7) << 15) | (120 << 7) | (sm & 0x7F)).astype(np.uint16)
    blob = o.encode(w)
    assert blob.n_esc == 0
    w12_tiles = blob.tiles.reshape(-1, o.TILE_BYTES)[:, :2048]
    s_bits = np.full((n, k // 32), 0x3C00, dtype=np.uint16)
    scr = o.screen_pack(q, s_bits).reshape(-1, o.SCREEN_TILE_BYTES)[:, :2048]
    assert np.array_equal(w12_tiles, scr)


def test_screen_exact_sums_closed_forms():
    g = np.random.default_rng(9)
    k = 256
    for e in (-20, -7, 3):
        # w = q * 2^e with one |w| = 127 * 2^e per group: s = 2^e, codes = q, r = 0
        q = g.integers(-127, 128, size=(1, k))
        q[0, ::32] = 127
        w = o.bf16_round(np.ldexp(q.astype(np.float64), e))
        qq, s_bits, _ = o.screen_encode(np.vstack([w] * 16))
        assert np.all(s_bits == o.bf16_round(np.array([2.0 ** e]))[0])
        assert np.array_equal(qq[0], q[0].astype(np.int8))
        r2, q2 = o.screen_row_sums_exact(w[0], qq[0], s_bits[0])
        assert r2 == 0
        assert Fraction(q2, 2 ** 266) == sum(bf16_fraction(b) ** 2 for b in w[0])
    # random rows: R2 <= K (s_max / 2)^2
    w = wi.gaussian_bf16((16, k), 0.02, g)
    qq, s_bits, _ = o.screen_encode(w)
    for r in range(16):
        r2, _ = o.screen_row_sums_exact(w[r], qq[r], s_bits[r])
        smax = Fraction(float(o.bf16_to_f64(s_bits[r]).max()))
        assert Fraction(r2, 2 ** 266) <= k * (smax / 2) ** 2


def test_screen_bound_holds_and_is_tight():
    """|z - z8| <= ||x||_2 ||r||_2 for any x, with near equality when x is parallel to r
    (so a bound missing a factor would fail), and the float64 z8 reference is within
    K 2^-53 S8 of the exact screen logit."""
    g = np.random.default_rng(21)
    k = 512
    w = wi.gaussian_bf16((16, k), 0.02, g)
    q, s_bits, _ = o.screen_encode(w)
    what = o.screen_weights(q, s_bits)
    for r in range(4):
        rr = o.bf16_to_f64(w[r]) - what[r]
        xs = [wi.gaussian_bf16((1, k), 1.0, g)[0],
              o.bf16_round(rr / np.abs(rr).max())]            # parallel to r
        for t, x in enumerate(xs):
            xf = [bf16_fraction(b) for b in x]
            d = sum(a * Fraction(float(v)) for a, v in zip(xf, rr))      # z - z8, exact
            x2 = sum(a * a for a in xf)
            r2, _ = o.screen_row_sums_exact(w[r], q[r], s_bits[r])
            bound2 = x2 * Fraction(r2, 2 ** 266)
            assert d * d <= bound2
            if t == 1:
                assert d * d >= Fraction(98, 100) * bound2
            z8, s8 = o.screen_logits_reference(x[None, :], q[r:r + 1], s_bits[r:r + 1])
            z8x = sum(a * Fraction(float(v)) for a, v in zip(xf, what[r]))
            assert abs(Fraction(float(z8[0, 0])) - z8x) <= Fraction(k * 2.0 ** -53 * float(s8[0, 0]))


# ----------------------------------------------------------------------------- FP8 GEMM
# Values of the OCP 8-bit floating point specification's E4M3 format (bias 7, no
# infinities, S.1111.111 NaN): zero, the smallest subnormal 2^-9, the largest subnormal
# 7 * 2^-9, the smallest normal 2^-6, 1, 1.5, 2, 240, and the largest finite 448.
F8_SPEC = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
           0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
# E4M3 codes of small integers (same specification): value -> code
F8_INT = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E, 8: 0x50}


def test_f8_decode_matches_torch_float8():
    """All 256 codes against torch's float8_e4m3fn (a library decoding of the format)."""
    import torch
    b = np.arange(256, dtype=np.uint8)
    mine = o.f8_e4m3_to_f64(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert set(np.flatnonzero(np.isnan(mine)).tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_f8_decode_spec_values():
    for code, v in F8_SPEC.items():
        assert o.f8_e4m3_to_f64(np.array([code], dtype=np.uint8))[0] == v, hex(code)
    for v, code in F8_INT.items():
        assert o.f8_e4m3_to_f64(np.array([code, code | 0x80], dtype=np.uint8)).tolist() == [v, -v]
    assert np.signbit(o.f8_e4m3_to_f64(np.array([0x80], dtype=np.uint8))[0])
    pos = o.f8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()          # codes 0x00..0x7E strictly increasing


def test_f8_values_are_bf16_values():
    """Every finite E4M3 value is a BF16 value (what an exact conversion to BF16 needs)."""
    v = o.f8_e4m3_to_f64(np.arange(256, dtype=np.uint8))
    v = v[~np.isnan(v)]
    assert np.array_equal(o.bf16_to_f64(o.bf16_round(v)), v)


def test_f8_pack_positions():
    """Hand-placed elements of a 32 x 256 weight (2 row-blocks, 2 tile columns): element
    (row 16b + r, column 128g + 32j + 8q' + i) of lane slot l = 16q' + r, t = 8j + i, lands
    at (g*2 + b)*2048 + 1024*(t//16) + 16*l + t%16."""
    q = np.zeros((32, 256), dtype=np.uint8)
    cases = {(17, 200): 7440, (15, 127): 2047, (16, 0): 2048, (0, 128): 4096, (0, 0): 0,
             (1, 8): 16 * 17, (0, 32): 8}
    for i, (rc, _) in enumerate(cases.items()):
        q[rc] = i + 1
    t = o.f8_pack(q)
    assert t.size == 32 * 256 and np.count_nonzero(t) == len(cases)
    for i, (_, pos) in enumerate(cases.items()):
        assert t[pos] == i + 1, pos


def test_f8_pack_is_a_per_tile_permutation():
    g = np.random.default_rng(80)
    q = g.integers(0, 256, (48, 384)).astype(np.uint8)
    t = o.f8_pack(q).reshape(3, 3, 2048)                      # [g, b, bytes]
    for gg in range(3):
        for b in range(3):
            blk = q[16 * b:16 * b + 16, 128 * gg:128 * gg + 128].ravel()
            assert np.array_equal(np.sort(t[gg, b]), np.sort(blk))


def test_gemm_f8_integer_closed_form():
    """Unit scales and small-integer codes: z and S are integer products, exactly."""
    g = np.random.default_rng(81)
    a = g.integers(-8, 9, (144, 256))
    codes = np.vectorize(lambda v: F8_INT[abs(int(v))] | (0x80 if v < 0 else 0))(a).astype(np.uint8)
    xi = g.integers(-20, 21, (3, 256))
    x = wi.f32_to_bf16_bits(xi.astype(np.float32))
    s = np.ones((2, 2), dtype=np.float32)
    z, sa = o.gemm_f8_reference(x, codes, s)
    assert np.array_equal(z, (xi @ a.T).astype(np.float64))
    assert np.array_equal(sa, (np.abs(xi) @ np.abs(a).T).astype(np.float64))


def test_gemm_f8_vs_exact_rationals():
    """Random codes and FP32 scales on a ragged block grid (144 rows: a full and a partial
    128-row block; 3 column blocks): the oracle against exact rational sums of
    x * E4M3(q) * s with the codes decoded by torch and s taken from its FP32 value."""
    import torch
    g = np.random.default_rng(82)
    n, k, m = 144, 384, 2
    q = g.integers(0, 256, (n, k)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3A                                 # no NaN codes
    s = (g.uniform(0.5, 2.0, (2, 3)) * 2.0 ** g.integers(-12, 3, (2, 3))).astype(np.float32)
    x = wi.gaussian_bf16((m, k), 1.0, g)
    qv = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    z, sa = o.gemm_f8_reference(x, q, s)
    for row in range(m):
        xr = [bf16_fraction(v) for v in x[row]]
        for col in range(n):
            acc = Fraction(0)
            mag = Fraction(0)
            for kk in range(k):
                w = Fraction(float(qv[col, kk])) * Fraction(float(s[col // 128, kk // 128]))
                acc += xr[kk] * w
                mag += abs(xr[kk] * w)
            assert abs(Fraction(z[row, col]) - acc) <= k * Fraction(2) ** -53 * mag
            assert abs(Fraction(sa[row, col]) - mag) <= k * Fraction(2) ** -53 * mag


def golden_f8():
    """The hand-worked FP8 GEMM (tests/golden/fp8_gemm_worked_example.json) as arrays."""
    with open(os.path.join(GOLDEN, "fp8_gemm_worked_example.json")) as f:
        g = json.load(f)
    q = np.zeros((g["n"], g["k"]), dtype=np.uint8)
    for r, c, b in g["codes"]:
        q[r, c] = int(b, 16)
    x = np.zeros((2, g["k"]), dtype=np.float32)
    for r, c, v in g["x"]:
        x[r, c] = v
    return g, q, np.array(g["scales"], dtype=np.float32), wi.f32_to_bf16_bits(x)


def test_f8_worked_example_golden():
    g, q, s, x = golden_f8()
    tiles = o.f8_pack(q)
    listed = {off: int(b, 16) for off, b in g["tile_bytes"]}
    assert all(int(tiles[off]) == b for off, b in listed.items())
    assert np.count_nonzero(tiles) == len(listed)
    z, _ = o.gemm_f8_reference(x, q, s)
    want = np.zeros_like(z)
    for r, c, v in g["z"]:
        want[r, c] = v
    assert np.array_equal(z, want)
    y = o.bf16_round(z)
    for r, c, b in g["y_bf16"]:
        assert int(y[r, c]) == int(b, 16), (r, c)


# ----------------------------------------------------------------------------- mutations
def _pins_fail(fn):
    try:
        fn()
    except (AssertionError, ValueError):
        return True
    return False


def test_mutation_tie_rule_is_caught(monkeypatch):
    def bad(hist):
        order = sorted(range(256), key=lambda ex: (-int(hist[ex]), -ex))
        return np.array(sorted(order[:16]), dtype=np.uint8)
    monkeypatch.setattr(o, "choose_codebook", bad)
    assert _pins_fail(test_all_bf16_patterns_roundtrip)


def test_mutation_nibble_order_is_caught(monkeypatch):
    orig = o.slot_layout

    def bad():
        r, kap, sm_pos, word_pos, bit = orig()
        i = np.arange(32)[None, :] % 8
        return r, kap, sm_pos, word_pos, 4 * i * np.ones((64, 1), dtype=np.int64)
    monkeypatch.setattr(o, "slot_layout", bad)
    assert _pins_fail(test_worked_example_golden)


def test_mutation_escape_order_is_caught(monkeypatch):
    orig = o.encode

    def bad(w, rows_per_chunk=4096):
        b = orig(w, rows_per_chunk)
        for blk in range(b.n // 16):
            seg = b.esc[b.esc_off[blk]:b.esc_off[blk + 1]]
            seg[:] = np.array(sorted(seg.tolist()), dtype=np.uint32)   # sorted by r first
        return b
    monkeypatch.setattr(o, "encode", bad)
    assert _pins_fail(lambda: test_roundtrip_and_escape_invariants.hypothesis.inner_test(
        a=2, bb=2, seed=1, kind="bits"))


def test_mutation_sign_in_exact_logit_is_caught(monkeypatch):
    orig = o.exact_parts

    def bad(b):
        s, mant, ex = orig(b)
        return np.ones_like(s), mant, ex
    monkeypatch.setattr(o, "exact_parts", bad)
    assert _pins_fail(test_exact_logit_matches_rationals)


def test_mutation_transposed_gemm_is_caught(monkeypatch):
    orig = o.gemm_reference

    def bad(x, w, rows_per_chunk=8192):
        z, s = orig(x, w, rows_per_chunk)
        return z[:, ::-1].copy(), s
    monkeypatch.setattr(o, "gemm_reference", bad)
    assert _pins_fail(lambda: test_gemm_reference_vs_exact_rationals(1))


def test_mutation_subnormal_exponent_is_caught(monkeypatch):
    orig = o.exact_parts

    def bad(b):
        s, mant, ex = orig(b)
        return s, mant, np.where(mant < 128, ex - 1, ex)
    monkeypatch.setattr(o, "exact_parts", bad)
    assert _pins_fail(test_exact_logit_matches_rationals)


def test_mutation_batched_accept_offsets_are_caught(monkeypatch):
    # a request reading its draft from the batch's first row instead of its own
    def bad(argmax, draft, row_off, n_draft):
        return np.array([o.accepted_length(argmax[int(a):int(a) + int(nd)], draft[:int(nd)])
                         for a, nd in zip(row_off, n_draft)], dtype=np.int64)
    monkeypatch.setattr(o, "accepted_lengths_batched", bad)
    assert _pins_fail(test_accepted_lengths_batched_cases)


def test_mutation_tolerance_tenfold_is_caught(monkeypatch):
    monkeypatch.setattr(o, "REL_TOL", 2e-2)
    assert _pins_fail(test_acceptance_boundary_golden)


def test_mutation_tolerance_doubled_is_caught(monkeypatch):
    monkeypatch.setattr(o, "REL_TOL", 4e-3)
    assert _pins_fail(test_acceptance_boundary_golden)


def test_mutation_rounded_rule_one_ulp_wider_is_caught(monkeypatch):
    def bad(y_bits, z, s):
        tau = o.REL_TOL * s + o.ABS_TOL
        y = o.bf16_to_f64(y_bits)
        lo_b = o.bf16_round(z - tau).astype(np.int32)
        hi_b = o.bf16_round(z + tau).astype(np.int32)
        # one BF16 step further out on each side (away from zero: +1 on the bits)
        lo = o.bf16_to_f64(np.where(lo_b >= 0x8000, lo_b + 1, np.where(lo_b == 0, 0x8001, lo_b - 1)).astype(np.uint16))
        hi = o.bf16_to_f64(np.where(hi_b >= 0x8000, np.where(hi_b == 0x8000, 0x0001, hi_b - 1), hi_b + 1).astype(np.uint16))
        return (lo <= y) & (y <= hi)
    monkeypatch.setattr(o, "within_tolerance_rounded", bad)
    assert _pins_fail(test_acceptance_boundary_golden)


def test_mutation_zero_width_fp64_filter_is_caught(monkeypatch):
    monkeypatch.setattr(o, "fp64_filter_width", lambda k, s_max: 0.0)
    assert _pins_fail(test_argmax_sub_fp64_near_tie)


def test_mutation_screen_scale_rounded_to_nearest_is_caught(monkeypatch):
    monkeypatch.setattr(o, "bf16_round_up", lambda v: o.bf16_round(v))
    assert _pins_fail(test_screen_invariants)


def test_mutation_screen_ties_away_from_zero_is_caught(monkeypatch):
    monkeypatch.setattr(o.np, "rint", lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))
    assert _pins_fail(test_screen_worked_example_golden)


def test_mutation_screen_groups_strided_is_caught(monkeypatch):
    orig = o.screen_encode

    def bad(w):
        n, k = w.shape
        perm = np.arange(k).reshape(k // 32, 32).T.reshape(-1)   # groups of every (k/32)-th column
        q, s, f = orig(w[:, perm])
        inv = np.argsort(perm)
        return q[:, inv], s, f
    monkeypatch.setattr(o, "screen_encode", bad)
    assert _pins_fail(test_screen_worked_example_golden)


def test_mutation_screen_residual_halved_is_caught(monkeypatch):
    orig = o.screen_row_sums_exact
    monkeypatch.setattr(o, "screen_row_sums_exact", lambda w, q, s: (orig(w, q, s)[0] // 4, orig(w, q, s)[1]))
    assert _pins_fail(test_screen_bound_holds_and_is_tight)


def test_mutation_f8_scale_per_16_rows_is_caught(monkeypatch):
    def bad(q, s):
        n, k = q.shape
        srow = np.asarray(s, dtype=np.float64)[np.minimum(np.arange(n) // 16, s.shape[0] - 1)]
        return o.f8_e4m3_to_f64(q) * np.repeat(srow, o.F8_BLOCK, axis=1)[:, :k]
    monkeypatch.setattr(o, "f8_weights", bad)
    assert _pins_fail(test_gemm_f8_vs_exact_rationals)


def test_mutation_f8_subnormal_scale_is_caught(monkeypatch):
    orig = o.f8_e4m3_to_f64

    def bad(b):
        v = orig(b)
        e = (np.asarray(b, dtype=np.uint8) >> 3) & 0xF
        return np.where(e == 0, 2 * v, v)          # subnormals read at 2^-5 instead of 2^-6
    monkeypatch.setattr(o, "f8_e4m3_to_f64", bad)
    assert _pins_fail(test_f8_decode_matches_torch_float8)
    assert _pins_fail(test_f8_decode_spec_values)


def test_mutation_f8_pack_group_halves_swapped_is_caught(monkeypatch):
    orig = o.slot_layout

    def bad():
        r, kap, pos, wp, bit = orig()
        t = np.arange(32)[None, :]
        return r, kap, 1024 * ((t // 8) % 2) + 16 * np.arange(64)[:, None] + (t % 8) + 8 * (t // 16), wp, bit
    monkeypatch.setattr(o, "slot_layout", bad)
    assert _pins_fail(test_f8_pack_positions)
