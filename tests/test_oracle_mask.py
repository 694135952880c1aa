"""Pins of the mask oracle (CPU only)."""
import math

import numpy as np

import oracle
import oracle_pins as pins


def test_group_mean():
    pins.check_group_mean(oracle.group_mean_ref)


def test_group_scores():
    pins.check_group_scores(oracle.group_scores_ref)


def test_topk():
    pins.check_topk(oracle.topk_select_ref)


def test_thresh():
    pins.check_thresh(oracle.thresh_select_ref)


def test_mask_ref_layout():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 50, 8)); k = rng.standard_normal((1, 2, 40, 8))
    r = oracle.mask_ref(q, k, 16, "topk", topk=9)
    assert r["idx"].shape == (1, 2, 4, 9) and np.all(r["counts"] == 9)
    assert np.all(np.diff(r["idx"], axis=-1) > 0)
    r = oracle.mask_ref(q, k, 16, "thresh", thresh=1.0 / 40)
    c = r["counts"]
    assert r["idx"].shape == (1, 2, 4, 40) and np.all(c >= 1)
    for h in range(2):
        for g in range(4):
            kept = r["idx"][0, h, g, :c[0, h, g]]
            assert np.all(np.diff(kept) > 0) and np.all(r["idx"][0, h, g, c[0, h, g]:] == -1)
            s = r["s"][0, h, g]
            assert np.all(s[kept] >= r["t"][0, h, g])
    # M = 1 reduces to per-query scoring
    r1 = oracle.mask_ref(q, k, 1, "topk", topk=5, scale=0.25)
    assert np.abs(r1["s"] - 0.25 * np.einsum("bhid,bhjd->bhij", q, k)).max() <= 1e-12
    assert math.isclose(oracle.mask_ref(q, k, 16, "topk", topk=3)["s"][0, 0, 0, 0],
                        float(q[0, 0, :16].mean(axis=0) @ k[0, 0, 0]) / math.sqrt(8), rel_tol=1e-12)
