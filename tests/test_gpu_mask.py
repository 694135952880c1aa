"""GPU parity of sattn_mask (through the C ABI) against the fp64 mask oracle."""
import os

import numpy as np
import pytest

import oracle
from gpu_util import check_lse, check_mask_sets, check_out, f64, scale_of, to_device_bf16, workload
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


def _bits(rng, shape, std=1.0):
    return inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _all_units(B, H, G):
    return [(b, h, g) for b in range(B) for h in range(H) for g in range(G)]


def _gpu_mask(sattn, qb, kb, group, **kw):
    q, k = to_device_bf16(qb, DEV), to_device_bf16(kb, DEV)
    idx, counts = sattn.mask(q, k, group, **kw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), counts.cpu().numpy()


def test_tiny_workload_topk(sattn):
    w, (qb, kb, _) = workload("tiny")
    ref = oracle.mask_ref(f64(qb), f64(kb), w.group, "topk", topk=w.topk)
    idx, cnt = _gpu_mask(sattn, qb, kb, w.group, topk=w.topk)
    check_mask_sets(idx, cnt, ref, _all_units(1, w.heads, w.groups), "tiny topk", exact_counts=True)


# (D, group, Nq, Nk, mode, param)
CASES = [
    (128, 128, 1000, 3000, "topk", 600), (64, 64, 513, 1025, "topk", 1), (128, 16, 100, 777, "topk", 777),
    (128, 192, 700, 5003, "topk", 501), (64, 48, 300, 4096, "topk", 4095), (128, 256, 260, 70, "topk", 13),
    (128, 128, 1000, 3000, "thresh", 0.0), (128, 128, 1000, 3000, "thresh", 1e-3), (64, 64, 513, 1025, "thresh", 0.5),
    (128, 32, 333, 9000, "thresh", 2e-4), (128, 128, 200, 100, "thresh", 1.0), (64, 16, 40, 33000, "topk", 9999),
]


@pytest.mark.parametrize("D,group,Nq,Nk,mode,param", CASES)
def test_random(sattn, D, group, Nq, Nk, mode, param):
    rng = np.random.default_rng(D + group + Nq + Nk)
    B, H = 1, 3
    qb = _bits(rng, (B, H, Nq, D), 2.0)
    kb = _bits(rng, (B, H, Nk, D))
    kw = {"topk": param} if mode == "topk" else {"thresh": param}
    ref = oracle.mask_ref(f64(qb), f64(kb), group, mode, **({"topk": param} if mode == "topk" else {"thresh": param}))
    idx, cnt = _gpu_mask(sattn, qb, kb, group, **kw)
    G = -(-Nq // group)
    check_mask_sets(idx, cnt, ref, _all_units(B, H, G), f"{mode} D={D} M={group}", exact_counts=(mode == "topk"))
    if mode == "topk" and param == Nk:
        assert np.all(idx[..., :Nk] == np.arange(Nk))
    if mode == "thresh" and param == 0.0:
        assert np.all(cnt == Nk) and np.all(idx == np.arange(Nk))


def test_ties_go_to_lowest_index(sattn):
    """Identical key rows give bitwise-equal scores: top-k must return the lowest indices,
    a threshold above every probability must return index 0 (arg-max, lowest on ties)."""
    rng = np.random.default_rng(7)
    D, group, Nq, Nk = 64, 64, 128, 3000
    qb = _bits(rng, (1, 1, Nq, D))
    row = _bits(rng, (D,))
    kb = np.broadcast_to(row, (1, 1, Nk, D)).copy()
    idx, cnt = _gpu_mask(sattn, qb, kb, group, topk=1234)
    assert np.all(cnt == 1234) and np.all(idx == np.arange(1234))
    idx, cnt = _gpu_mask(sattn, qb, kb, group, thresh=0.9)
    assert np.all(cnt == 1) and np.all(idx[..., 0] == 0)
    # three identical key rows that score highest for group 0: top-2 keeps the two lowest of them
    kb = _bits(rng, (1, 1, Nk, D))
    qm = f64(qb)[0, 0, :group].mean(axis=0)
    kb[0, 0, [10, 2000, 2500]] = inputs.f32_to_bf16_bits((20.0 * qm).astype(np.float32))
    idx, cnt = _gpu_mask(sattn, qb, kb, group, topk=2)
    assert idx[0, 0, 0, :2].tolist() == [10, 2000]
    # top-3: every key at the cut is kept
    idx, cnt = _gpu_mask(sattn, qb, kb, group, topk=3)
    assert cnt[0, 0, 0] == 3 and idx[0, 0, 0, :3].tolist() == [10, 2000, 2500]


def test_chunked_window_threshold_density(sattn):
    """The calibrated tau of the chunked window gives about 30 % density on the GPU as well."""
    w, (qb, kb, _) = workload("chunked_window")
    s = oracle.group_scores_ref(f64(qb[:, :2]), f64(kb[:, :2]), w.group, scale_of(w.dim))
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    tau = float(np.quantile(p, 0.7))
    idx, cnt = _gpu_mask(sattn, qb[:, :2], kb[:, :2], w.group, thresh=tau)
    dens = cnt.sum() / (cnt.size * w.n_k)
    assert abs(dens - 0.3) < 0.01, dens


def test_crowded_cut_bin_uses_global_passes(sattn):
    """More than 8192 keys share the top 12 bits of the cut: the lower digits come from global memory."""
    rng = np.random.default_rng(11)
    D, group, Nq, Nk = 64, 64, 128, 40000
    qb = _bits(rng, (1, 1, Nq, D))
    base = rng.standard_normal(D).astype(np.float32)
    kb = inputs.f32_to_bf16_bits(base[None, None, None, :] + 0.02 * rng.standard_normal((1, 1, Nk, D)).astype(np.float32))
    ref = oracle.mask_ref(f64(qb), f64(kb), group, "topk", topk=9000)
    idx, cnt = _gpu_mask(sattn, qb, kb, group, topk=9000)
    check_mask_sets(idx, cnt, ref, _all_units(1, 1, 2), "crowded topk", exact_counts=True)
    # all-equal scores over more keys than the LDS candidate list holds
    kb = np.broadcast_to(kb[:, :, :1], (1, 1, Nk, D)).copy()
    idx, cnt = _gpu_mask(sattn, qb, kb, group, topk=20000)
    assert np.all(cnt == 20000) and np.all(idx == np.arange(20000))
    # every key ties and every key is kept
    idx, cnt = _gpu_mask(sattn, qb, kb, group, topk=Nk)
    assert np.all(cnt == Nk) and np.all(idx == np.arange(Nk))


def test_maximum_key_count(sattn):
    """Nk at the mask's limit (131072 keys: the longest sample row the select's LDS takes, the largest
    bitmaps): top-k and threshold lists of both groups against the oracle, then the forward on the
    oracle's top-k lists against the oracle."""
    rng = np.random.default_rng(131072)
    D, group, Nq, Nk = 64, 128, 256, 131072
    qb = _bits(rng, (1, 1, Nq, D), 2.0)
    kb = _bits(rng, (1, 1, Nk, D))
    vb = _bits(rng, (1, 1, Nk, D))
    units = _all_units(1, 1, 2)
    kk = Nk // 5
    ref = oracle.mask_ref(f64(qb), f64(kb), group, "topk", topk=kk)
    idx, cnt = _gpu_mask(sattn, qb, kb, group, topk=kk)
    check_mask_sets(idx, cnt, ref, units, "max Nk topk", exact_counts=True)
    ref_t = oracle.mask_ref(f64(qb), f64(kb), group, "thresh", thresh=1e-5)
    idx_t, cnt_t = _gpu_mask(sattn, qb, kb, group, thresh=1e-5)
    check_mask_sets(idx_t, cnt_t, ref_t, units, "max Nk thresh", exact_counts=False)
    # the forward on the oracle's top-k lists (both sides take the same lists; none comes from the GPU)
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    ridx = np.ascontiguousarray(np.maximum(ref["idx"], 0).astype(np.int32))
    rcnt = np.ascontiguousarray(ref["counts"].astype(np.int32))
    ti, tc = torch.from_numpy(ridx).to(DEV), torch.from_numpy(rcnt).to(DEV)
    out, lse = sattn.forward(q, k, v, ti, tc, group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), ridx, rcnt, group, scale_of(D))
    check_out(out.cpu().numpy(), ro, "max Nk forward")
    check_lse(lse.cpu().numpy(), rl, "max Nk forward")
