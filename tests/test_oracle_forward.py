"""Pins of the forward oracle (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins


def test_all_keys_equals_library_sdpa():
    pins.check_all_keys_equals_library(oracle.sparse_attention_ref)


def test_brute_force_tiny():
    pins.check_brute_force_tiny(oracle.sparse_attention_ref)


def test_closed_forms():
    pins.check_closed_forms(oracle.sparse_attention_ref)


def test_invariants():
    pins.check_invariants(oracle.sparse_attention_ref, oracle.sparse_attention_probs_ref)


def test_dense_matches_library():
    import torch
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 19, 8)); k = rng.standard_normal((1, 2, 31, 8)); v = rng.standard_normal((1, 2, 31, 8))
    out, lse = oracle.dense_attention_ref(q, k, v, 0.4)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.4).numpy()
    assert np.abs(out - ref).max() <= 1e-12
    rows = np.array([0, 7, 18])
    out_r, lse_r = oracle.dense_attention_ref(q, k, v, 0.4, rows=rows)
    assert np.array_equal(out_r[:, :, rows], out[:, :, rows]) and np.array_equal(lse_r[:, :, rows], lse[:, :, rows])


def test_restricted_not_masked_full_softmax():
    """The kept-key weights renormalise to 1 (restricted softmax), unlike a masked full softmax."""
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 4, 3)); k = rng.standard_normal((1, 1, 10, 3)); v = np.ones((1, 1, 10, 3))
    idx = np.array([[[[1, 4, 7]]]], dtype=np.int32)
    out, _ = oracle.sparse_attention_ref(q, k, v, idx, np.array([[[3]]], dtype=np.int32), 4, 1.0)
    assert np.abs(out - 1.0).max() <= 1e-14


def test_units_subset_and_validation():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, 10, 4)); k = rng.standard_normal((1, 2, 12, 4)); v = rng.standard_normal((1, 2, 12, 4))
    idx = np.tile(np.arange(12, dtype=np.int32), (1, 2, 3, 1)); cnt = np.full((1, 2, 3), 12, dtype=np.int32)
    full, _ = oracle.sparse_attention_ref(q, k, v, idx, cnt, 4, 0.5)
    part, _ = oracle.sparse_attention_ref(q, k, v, idx, cnt, 4, 0.5, units=[(0, 1, 2)])
    assert np.array_equal(part[0, 1, 8:10], full[0, 1, 8:10]) and np.isnan(part[0, 0]).all()
    bad = idx.copy(); bad[0, 0, 0, 1] = bad[0, 0, 0, 0]
    with pytest.raises(ValueError):
        oracle.sparse_attention_ref(q, k, v, bad, cnt, 4, 0.5)
    bad = idx.copy(); bad[0, 0, 0, 0] = 12
    with pytest.raises(ValueError):
        oracle.sparse_attention_ref(q, k, v, bad, cnt, 4, 0.5)
