"""GPU check of the voxel reordering (Chipmunk review, "What carries the argument" and Fig. 2 caption: tokens
reordered so that every contiguous chunk is a spatio-temporal cube; voxel (4, 6, 8) in its free parameters):
sattn_permute_tokens forward and inverse against the seeded generator's own permutation, bit for bit, and
the voxel workload's sparse forward un-permuted to raster order against the oracle."""
import dataclasses
import os

import numpy as np
import pytest

import oracle
from gpu_util import f64, scale_of, to_device_bf16, workload
from synth import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


@pytest.fixture(scope="module")
def sattn():
    import sparse_self_attention_amd as s
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(s.library_path()), "libsattn.so is not built"
    return s


def _bits_of(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_permute_tokens_voxel_order(sattn):
    """Raster-order Q/K/V of the 70,200-token grid (heads 0, 5, 23): the device permutation equals
    x[:, :, perm] with perm from the generator and from the library's host call, and the inverse undoes it."""
    w = inputs.WORKLOADS["voxel_70200"]
    raster = dataclasses.replace(w, voxel=None)
    heads = [0, 5, 23]
    qb, kb, vb = inputs.generate(raster, heads=heads)
    perm = inputs.voxel_order(w.grid_k, w.voxel)
    host = sattn.voxel_permutation(w.grid_k, w.voxel).numpy()
    assert np.array_equal(host, perm), "host voxel permutation differs from the generator's"
    p_dev = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    qv, kv, vv = inputs.generate(w, heads=heads)          # the workload's own (voxel-order) tensors
    for name, xb, xv in (("q", qb, qv), ("k", kb, kv), ("v", vb, vv)):
        x = to_device_bf16(xb, DEV)
        y = sattn.permute_tokens(x, p_dev)
        z = sattn.permute_tokens(y, p_dev, inverse=True)
        torch.cuda.synchronize()
        yb = _bits_of(y)
        assert np.array_equal(yb, xb[:, :, perm]), f"{name}: forward permutation differs"
        assert np.array_equal(yb, xv), f"{name}: forward permutation differs from the voxel workload"
        assert np.array_equal(_bits_of(z), xb), f"{name}: inverse does not undo the forward permutation"


def test_permute_tokens_small_shapes(sattn):
    """Several small shapes (D 64 and 128, B and H > 1), a random permutation, forward and inverse."""
    rng = np.random.default_rng(77)
    for (B, H, N, D) in [(2, 3, 37, 64), (1, 2, 1000, 128), (1, 1, 1, 64)]:
        xb = inputs.f32_to_bf16_bits(rng.standard_normal((B, H, N, D)).astype(np.float32))
        perm = rng.permutation(N)
        x = to_device_bf16(xb, DEV)
        p_dev = torch.from_numpy(perm.astype(np.int32)).to(DEV)
        y = sattn.permute_tokens(x, p_dev)
        z = sattn.permute_tokens(x, p_dev, inverse=True)
        torch.cuda.synchronize()
        assert np.array_equal(_bits_of(y), xb[:, :, perm])
        inv = np.empty_like(perm)
        inv[perm] = np.arange(N)
        assert np.array_equal(_bits_of(z), xb[:, :, inv])


def test_voxel_forward_unpermuted_to_raster(sattn):
    """The voxel workload in the benchmark's launch configuration (groups of 192 contiguous voxel-order
    tokens, top 10 %): the bf16 output un-permuted on the device equals the voxel-order output moved back
    to raster order, and sampled groups match the oracle there (within the bar plus bf16 rounding)."""
    w, (qb, kb, vb) = workload("voxel_70200")
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    idx, counts = sattn.mask(q, k, w.group, topk=w.topk)
    out, _ = sattn.forward(q, k, v, idx, counts, w.group, out_dtype=torch.bfloat16)
    perm = inputs.voxel_order(w.grid_k, w.voxel)
    raster = sattn.permute_tokens(out, torch.from_numpy(perm.astype(np.int32)).to(DEV), inverse=True)
    torch.cuda.synchronize()
    ob, rb = _bits_of(out), _bits_of(raster)
    want = np.empty_like(ob)
    want[:, :, perm] = ob
    assert np.array_equal(rb, want), "device un-permutation differs"
    r_f = inputs.bf16_bits_to_f32(rb).astype(np.float64)
    idx_h, cnt_h = idx.cpu().numpy(), counts.cpu().numpy()
    scale = scale_of(w.dim)
    for h in (0, w.heads - 1):
        for g in (0, w.groups // 2, w.groups - 1):
            r0, r1 = g * w.group, min((g + 1) * w.group, w.n_q)
            ro, _ = oracle.sparse_attention_ref(f64(qb[:, h:h + 1]), f64(kb[:, h:h + 1]), f64(vb[:, h:h + 1]),
                                                idx_h[:, h:h + 1], cnt_h[:, h:h + 1], w.group, scale,
                                                units=[(0, 0, g)])
            got = r_f[0, h, perm[r0:r1]]                 # the group's rows, found at their raster positions
            err = np.abs(got - ro[0, 0, r0:r1])
            assert np.all(err <= 1e-2 + 2.0 ** -9 * np.abs(ro[0, 0, r0:r1])), (h, g, err.max())
