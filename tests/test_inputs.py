"""Seeded input generator and workload shapes (CPU only)."""
import math
import os

import numpy as np
import torch

from synth import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            key, val = line.split()
            vals[key] = float(val)
    return vals


def test_chunked_window_matches_longlive_shapes():
    g = _golden("longlive_window_shapes.txt")
    w = inputs.WORKLOADS["chunked_window"]
    assert w.grid_k[1] * w.grid_k[2] == g["tokens_per_latent_frame"]
    assert w.q_frames == g["frames_per_chunk"] and w.n_q == g["tokens_per_chunk"]
    assert w.n_k == g["tokens_per_chunk"] * g["chunks_in_kv_window"]
    assert w.dim == g["head_dim"]
    qt, kp = math.ceil(w.n_q / 128), math.ceil(w.n_k / 128)
    assert (qt, kp) == (g["query_tiles_per_head"], g["key_pages_per_head"])
    assert qt * kp == g["tiles_per_head"] and qt * kp * g["heads"] == g["tiles_per_call"]
    assert round(w.n_q * w.n_k * 2 / 1e6) == g["p_matrix_fp16_mb"]
    # fp32 e^S overflows just above S = 88
    with np.errstate(over="ignore"):
        assert np.isfinite(np.exp(np.float32(g["fp32_exp_overflow_above"])))
        assert np.isinf(np.exp(np.float32(g["fp32_exp_overflow_above"] + 1)))


def test_mask_memory_is_several_gb():
    g = _golden("fgattn_mask_memory.txt")
    n, m = g["seq_len"], g["group"]
    gb = g["min_heads_for_several_gb"] * math.ceil(n / m) * n * g["bytes_per_index"] / 1e9
    assert 3.0 < gb < 6.0


def test_workload_sizes():
    W = inputs.WORKLOADS
    assert (W["tiny"].n_q, W["tiny"].groups, W["tiny"].topk) == (1024, 16, 256)
    assert (W["full_32760"].n_q, W["full_32760"].groups) == (32760, 256)
    assert (W["long_70200"].n_q, W["long_70200"].groups, W["long_70200"].topk) == (70200, 549, 14040)
    assert (W["voxel_70200"].groups, W["voxel_70200"].topk) == (366, 7020)
    assert W["chunked_window"].groups == 55


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 1e-40, 3.0e38], dtype=np.float32)])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_deterministic_and_per_head():
    w = inputs.WORKLOADS["tiny"]
    q, k, v = inputs.generate(w)
    q2, k2, v2 = inputs.generate(w)
    assert q.shape == (1, 2, 1024, 64) and k.shape == (1, 2, 1024, 64)
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    q1, k1, v1 = inputs.generate(w, heads=[1])
    assert np.array_equal(q1[0, 0], q[0, 1]) and np.array_equal(v1[0, 0], v[0, 1])
    qf, kf, vf = (inputs.bf16_bits_to_f32(x) for x in (q, k, v))
    # field variance ~1 plus noise 0.25; V ~ N(0,1)
    assert 0.9 < qf.var() < 1.6 and 0.9 < kf.var() < 1.6 and 0.9 < vf.var() < 1.1
    # spatially local structure: nearby tokens have larger q.k than distant ones
    near = np.mean(np.sum(qf[0, 0, :-1] * kf[0, 0, 1:], axis=-1))
    far = np.mean(np.sum(qf[0, 0, :512] * kf[0, 0, 512:], axis=-1))
    assert near > far + 10


def test_chunked_window_queries_are_last_chunk():
    w = inputs.Workload("cw_small", 1, 1, 8, (4, 3, 5), 3, 1, 4, "thresh", 0.3, 9)
    q, k, v = inputs.generate(w)
    assert q.shape[2] == 15 and k.shape[2] == 60
    # same field at the same positions: the noise-free part is shared, so q and the last-frame k agree in mean
    qf, kf = inputs.bf16_bits_to_f32(q)[0, 0], inputs.bf16_bits_to_f32(k)[0, 0, 45:]
    assert np.corrcoef(qf.ravel(), kf.ravel())[0, 1] > 0.6


def test_voxel_order():
    grid, vox = (5, 6, 9), (2, 3, 4)
    perm = inputs.voxel_order(grid, vox)
    assert sorted(perm.tolist()) == list(range(5 * 6 * 9))
    T, Hg, Wg = grid
    t, y, x = perm // (Hg * Wg), (perm // Wg) % Hg, perm % Wg
    cell = (t // 2) * 100 + (y // 3) * 10 + x // 4
    # every voxel is one contiguous run
    runs = [cell[0]] + [c for a, c in zip(cell[:-1], cell[1:]) if c != a]
    assert len(runs) == len(set(runs))
    # full voxels hold vt*vy*vx tokens
    assert np.sum(cell == 0) == 24


def test_perturb_and_random_lists():
    rng = np.random.default_rng(1)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((2, 100)).astype(np.float32))
    y = inputs.perturb(x, 0.05, 7)
    d = inputs.bf16_bits_to_f32(y) - inputs.bf16_bits_to_f32(x)
    assert 0.03 < d.std() < 0.07
    counts = np.array([[[3, 0, 5]]])
    idx = inputs.random_index_lists(rng, 1, 1, 3, 20, counts, 6)
    assert np.all(np.diff(idx[0, 0, 0, :3]) > 0) and np.all(idx[0, 0, 1] == -1) and np.all(idx[0, 0, 2, 5:] == -1)
