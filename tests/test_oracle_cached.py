"""The cached-mask oracle against its pins (CPU)."""
import numpy as np

import oracle
import oracle_pins as pins


def test_cached_brute_force():
    pins.check_cached_brute_force(oracle.cached_mask_ref)


def test_cached_properties():
    pins.check_cached_properties(oracle.cached_mask_ref, oracle.row_lse_ref)


def test_cached_layout_and_partial_group():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 10, 4))
    k = rng.standard_normal((1, 1, 7, 4))
    res = oracle.cached_mask_ref(q, k, 4, 0.1, cap=7)
    assert res["idx"].shape == (1, 1, 3, 7) and res["counts"].shape == (1, 1, 3)
    for g in range(3):
        c = res["counts"][0, 0, g]
        assert np.all(res["idx"][0, 0, g, c:] == -1)
    # the partial last group holds rows 8, 9 only
    row = oracle.slice_max_logprob_ref(q, k, 4, 0.5, units=[(0, 0, 2)])[(0, 0, 2)]
    s = q[0, 0, 8:10] @ k[0, 0].T * 0.5
    lse = np.log(np.exp(s).sum(axis=1))
    assert np.allclose(row, (s - lse[:, None]).max(axis=0), atol=1e-12)
