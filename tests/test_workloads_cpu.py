"""CPU checks of the workload construction used by the full-size GPU tests: the near-tie
planting (on a reduced vocabulary, same code path) and the seeded draws."""
import numpy as np

import w12_inputs as wi
import plant


def test_near_tie_planting_reduced_vocab():
    w = wi.gaussian_bf16((4096, 5120), 0.02, np.random.default_rng(11))
    x = np.concatenate([wi.verify_batch_x(1), wi.verify_batch_x(2)])
    wp, pairs = plant.plant_near_ties(x, w, lambda i: wi.tie_rng(1 + i // 16, i % 16))
    assert len({v for p in pairs for v in p}) >= 33       # v2s are all distinct
    am = plant.check_plants(x, wp, pairs)
    # only the planted rows changed
    changed = np.nonzero((wp != w).any(axis=1))[0]
    assert set(changed.tolist()) <= {v2 for _, v2 in pairs}
    assert am.shape == (32,)


def test_verify_mismatch_draws():
    seen = set()
    for b in range(3):
        p, r = wi.verify_mismatch(b, 151936)
        assert 0 <= p <= 16 and 0 <= r <= 151934
        seen.add(p)
    assert wi.verify_mismatch(1, 151936) == wi.verify_mismatch(1, 151936)
    assert np.array_equal(wi.verify_batch_x(0), wi.activations(4, wi.T_X, 16, 5120))
    assert not np.array_equal(wi.verify_batch_x(1), wi.verify_batch_x(2))
