"""GPU parity of sattn_forward / attn_forward (through the C ABI) against the fp64 oracle."""
import json
import os

import numpy as np
import pytest

import oracle
from gpu_util import (check_lse, check_mask_sets, check_out, f64, scale_of, to_device_bf16, workload)
from synth import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sattn():
    import sparse_self_attention_amd as s
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(s.library_path()), "libsattn.so is not built"
    return s


DEV = "cuda:0"


def _rand_bits(rng, shape, std=1.0):
    return inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _run_sparse(sattn, qb, kb, vb, idx, counts, group, scale=None, out_dtype=None):
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    it = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(DEV)
    ct = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int32)).to(DEV)
    out, lse = sattn.forward(q, k, v, it, ct, group, scale=scale, out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def test_tiny_workload_with_oracle_lists(sattn):
    w, (qb, kb, vb) = workload("tiny")
    ref_mask = oracle.mask_ref(f64(qb), f64(kb), w.group, "topk", topk=w.topk)
    o, l = _run_sparse(sattn, qb, kb, vb, ref_mask["idx"], ref_mask["counts"], w.group)
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), ref_mask["idx"], ref_mask["counts"], w.group,
                                         scale_of(w.dim))
    check_out(o, ro, "tiny")
    check_lse(l, rl, "tiny")


# (D, group, Nq, Nk, q_std): partial last groups, group sizes that are not multiples of 32, ragged counts
RANDOM_CASES = [
    (64, 64, 300, 500, 1.0), (128, 128, 333, 700, 1.0), (128, 48, 200, 300, 2.0), (128, 16, 70, 129, 1.0),
    (128, 192, 500, 900, 1.0), (128, 256, 600, 300, 1.5), (64, 32, 100, 64, 1.0), (128, 80, 250, 1000, 3.0),
    (64, 128, 257, 2000, 1.0), (128, 128, 128, 4100, 8.0),
    # groups wider than 128 rows run as equal slices: 224 -> 2 x 128 (the last group's 2 rows leave the
    # second slice empty), 160 -> 2 x 96 (ragged second slice)
    (128, 224, 450, 800, 1.0), (64, 160, 333, 600, 1.0),
]


@pytest.mark.parametrize("D,group,Nq,Nk,q_std", RANDOM_CASES)
def test_random_lists(sattn, D, group, Nq, Nk, q_std):
    rng = np.random.default_rng(D * 7 + group + Nq + Nk)
    B, H = 2, 2
    qb = _rand_bits(rng, (B, H, Nq, D), q_std)
    kb, vb = _rand_bits(rng, (B, H, Nk, D)), _rand_bits(rng, (B, H, Nk, D))
    G = -(-Nq // group)
    cap = min(Nk, 700)
    special = [min(c, cap) for c in (0, 1, 63, 64, 65, cap, 129)]
    counts = rng.integers(1, cap + 1, size=(B, H, G)).astype(np.int32)
    for i, c in enumerate(special[:counts.size]):
        counts.flat[i] = c
    idx = inputs.random_index_lists(rng, B, H, G, Nk, counts, cap)
    o, l = _run_sparse(sattn, qb, kb, vb, idx, counts, group)
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), idx, counts, group, scale_of(D))
    empty = np.repeat(counts == 0, group, axis=2)[:, :, :Nq]
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(l[empty])), "empty group must give 0 and -inf"
    check_out(o, np.nan_to_num(ro), f"random D={D} M={group}")
    check_lse(l, rl, f"random D={D} M={group}")


def test_huge_logits(sattn):
    """Scores of several hundred: the online softmax must never form exp of an unshifted score."""
    rng = np.random.default_rng(3)
    D, group, Nq, Nk = 128, 64, 128, 777
    qb = _rand_bits(rng, (1, 1, Nq, D), 30.0)
    kb, vb = _rand_bits(rng, (1, 1, Nk, D)), _rand_bits(rng, (1, 1, Nk, D))
    counts = np.full((1, 1, 2), 500, dtype=np.int32)
    idx = inputs.random_index_lists(rng, 1, 1, 2, Nk, counts, 500)
    o, l = _run_sparse(sattn, qb, kb, vb, idx, counts, group)
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), idx, counts, group, scale_of(D))
    assert np.abs(rl).max() > 88
    check_out(o, ro, "huge logits")
    check_lse(l, rl, "huge logits")


@pytest.mark.parametrize("D,Nq,Nk", [(64, 1024, 1024), (128, 300, 1000), (128, 129, 63), (64, 77, 4100)])
def test_dense_matches_oracle(sattn, D, Nq, Nk):
    rng = np.random.default_rng(D + Nq + Nk)
    qb, kb, vb = _rand_bits(rng, (1, 3, Nq, D), 1.5), _rand_bits(rng, (1, 3, Nk, D)), _rand_bits(rng, (1, 3, Nk, D))
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    out, lse = sattn.attn(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_attention_ref(f64(qb), f64(kb), f64(vb), scale_of(D))
    check_out(out.cpu().numpy(), ro, "dense")
    check_lse(lse.cpu().numpy(), rl, "dense")


def test_all_keys_sparse_equals_dense_and_bf16_rounding(sattn):
    rng = np.random.default_rng(9)
    D, group, Nq, Nk = 128, 128, 384, 1000
    qb, kb, vb = _rand_bits(rng, (1, 2, Nq, D)), _rand_bits(rng, (1, 2, Nk, D)), _rand_bits(rng, (1, 2, Nk, D))
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    G = Nq // group
    idx = torch.arange(Nk, dtype=torch.int32, device=DEV).expand(1, 2, G, Nk).contiguous()
    counts = torch.full((1, 2, G), Nk, dtype=torch.int32, device=DEV)
    so, sl = sattn.forward(q, k, v, idx, counts, group, out_dtype=torch.float32)
    do, dl = sattn.attn(q, k, v, out_dtype=torch.float32)
    sb, _ = sattn.forward(q, k, v, idx, counts, group, out_dtype=torch.bfloat16)
    so2, _ = sattn.forward(q, k, v, idx, counts, group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(so, do) and torch.equal(sl, dl), "all-keys sparse path must equal the dense path"
    assert torch.equal(so, so2), "reruns must be bitwise identical"
    assert torch.equal(sb, so.to(torch.bfloat16)), "bf16 output must be the RNE rounding of the fp32 output"
    out_nolse, none = sattn.forward(q, k, v, idx, counts, group, want_lse=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(out_nolse, sb)


def test_validation_mode_rejects_bad_lists(sattn, monkeypatch):
    rng = np.random.default_rng(4)
    D, group, Nq, Nk = 64, 64, 128, 256
    q, k, v = (to_device_bf16(_rand_bits(rng, (1, 1, n, D)), DEV) for n in (Nq, Nk, Nk))
    counts = torch.tensor([[[3, 2]]], dtype=torch.int32, device=DEV)
    good = torch.tensor([[[[1, 5, 9, -1], [0, 255, -1, -1]]]], dtype=torch.int32, device=DEV)
    monkeypatch.setenv("SATTN_VALIDATE", "1")
    sattn.forward(q, k, v, good, counts, group)
    for bad_idx, bad_cnt in [([[1, 5, 5, -1], [0, 255, -1, -1]], [3, 2]),     # duplicate
                             ([[1, 9, 5, -1], [0, 255, -1, -1]], [3, 2]),     # not ascending
                             ([[1, 5, 9, -1], [0, 256, -1, -1]], [3, 2]),     # out of range
                             ([[1, 5, 9, -1], [0, 255, -1, -1]], [5, 2])]:    # count > cap
        it = torch.tensor([[bad_idx]], dtype=torch.int32, device=DEV)
        ct = torch.tensor([[bad_cnt]], dtype=torch.int32, device=DEV)
        with pytest.raises(sattn.SattnError) as e:
            sattn.forward(q, k, v, it, ct, group)
        assert e.value.status == 7


@pytest.mark.parametrize("D,group,Nq,Nk", [(128, 128, 600, 3000), (64, 64, 300, 2000), (128, 192, 500, 4000),
                                           (128, 48, 200, 700)])
def test_pipeline_depth_one_equals_two(sattn, monkeypatch, D, group, Nq, Nk):
    """Race check of the double-buffered gather: with SATTN_SERIAL_GATHER=1 every key block's gather lands
    before the block before it computes (pipeline depth 1); sparse, dense and delta results must equal the
    default order bit for bit, over a shape with several waves per group and ragged lists."""
    rng = np.random.default_rng(D + group + Nq)
    B, H = 1, 2
    G = -(-Nq // group)
    q, k, v = (to_device_bf16(_rand_bits(rng, (B, H, n, D)), DEV) for n in (Nq, Nk, Nk))
    counts = rng.integers(0, Nk + 1, size=(B, H, G)).astype(np.int32)
    counts[0, 0, 0] = Nk
    idx = inputs.random_index_lists(rng, B, H, G, Nk, counts, Nk)
    it, ct = torch.from_numpy(idx).to(DEV), torch.from_numpy(counts).to(DEV)
    lse_in = torch.from_numpy(rng.standard_normal((B, H, Nq)).astype(np.float32) + 6.0).to(DEV)
    prev = torch.from_numpy(rng.standard_normal((B, H, Nq, D)).astype(np.float32)).to(DEV)

    def run():
        o, l = sattn.forward(q, k, v, it, ct, group, out_dtype=torch.float32)
        do, dl = sattn.attn(q, k, v, out_dtype=torch.float32)
        fresh = torch.zeros_like(prev)
        xo = sattn.delta_forward(q, k, v, it, ct, group, lse=lse_in, out_prev=prev, fresh=fresh,
                                 out=torch.empty_like(prev))
        torch.cuda.synchronize()
        return [t.cpu() for t in (o, l, do, dl, xo, fresh)]

    monkeypatch.setenv("SATTN_SERIAL_GATHER", "0")
    two = run()
    monkeypatch.setenv("SATTN_SERIAL_GATHER", "1")
    one = run()
    for name, a, b in zip(("out", "lse", "dense out", "dense lse", "delta out", "delta fresh"), two, one):
        assert torch.equal(a, b), f"{name}: pipeline depth 1 and 2 differ"


def test_log_mode_names_the_kernels(sattn):
    """SATTN_LOG=1 prints the kernel each launch selects (a child process, so the variable is read fresh)."""
    import subprocess
    import sys
    code = ("import torch, sparse_self_attention_amd as s; q = torch.randn(1, 1, 256, 128, device='cuda')"
            ".to(torch.bfloat16); i, c = s.mask(q, q, 128, topk=64); s.forward(q, q, q, i, c, 128); "
            "torch.cuda.synchronize()")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, SATTN_LOG="1", PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "[sattn] mask<D=128> mode top-k" in r.stderr and "[sattn] attn_fwd_lean<D=128, waves=4, sparse" in r.stderr


def _units(rng, H, G, n):
    us = {(0, 0, 0), (0, H - 1, G - 1)}
    while len(us) < n:
        us.add((0, int(rng.integers(H)), int(rng.integers(G))))
    return sorted(us)


def _check_units(sattn, w, qb, kb, vb, idx_h, cnt_h, out, lse, units, what):
    scale = scale_of(w.dim)
    for h in sorted({u[1] for u in units}):
        gs = [(0, 0, g) for (_, hh, g) in units if hh == h]
        ro, rl = oracle.sparse_attention_ref(f64(qb[:, h:h + 1]), f64(kb[:, h:h + 1]), f64(vb[:, h:h + 1]),
                                             idx_h[:, h:h + 1], cnt_h[:, h:h + 1], w.group, scale, units=gs)
        for (_, _, g) in gs:
            r = slice(g * w.group, min((g + 1) * w.group, w.n_q))
            check_out(out[0, h, r], ro[0, 0, r], f"{what} h={h} g={g}")
            check_lse(lse[0, h, r], rl[0, 0, r], f"{what} h={h} g={g}")


@pytest.mark.parametrize("name", ["long_70200", "voxel_70200", "chunked_window"])
def test_full_size_sampled(sattn, name):
    """Full-size workloads in the benchmark's launch configuration, checked on sampled groups:
    the GPU mask against the oracle mask, then the forward on the GPU's lists and on the oracle's."""
    w, (qb, kb, vb) = workload(name)
    rng = np.random.default_rng(len(name))
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    scale = scale_of(w.dim)
    mh = [0, w.heads - 1]
    ref = {h: oracle.mask_ref(f64(qb[:, h:h + 1]), f64(kb[:, h:h + 1]), w.group, "topk", topk=w.topk)
           for h in mh} if w.mode == "topk" else None
    if w.mode == "topk":
        idx, counts = sattn.mask(q, k, w.group, topk=w.topk)
    else:
        # one global tau: the (1 - keep) quantile of the oracle's pooled probabilities over all heads
        s = oracle.group_scores_ref(f64(qb), f64(kb), w.group, scale)
        p = np.exp(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        tau = float(np.quantile(p, 1.0 - w.keep))
        # the value the benchmark reads was written by tests/golden/make_thresholds.py with the same rule
        with open(os.path.join(os.path.dirname(__file__), "golden", "thresholds.json")) as fh:
            stored = json.load(fh)[name]["tau"]
        assert abs(stored - tau) <= 1e-12 * tau, (stored, tau)
        ref = {h: oracle.mask_ref(f64(qb[:, h:h + 1]), f64(kb[:, h:h + 1]), w.group, "thresh", thresh=tau)
               for h in mh}
        idx, counts = sattn.mask(q, k, w.group, thresh=tau)
    out, lse = sattn.forward(q, k, v, idx, counts, w.group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    idx_h, cnt_h, out_h, lse_h = idx.cpu().numpy(), counts.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    if w.mode == "topk":
        assert np.all(cnt_h == w.topk)
    for h in mh:
        units = [(0, 0, g) for g in range(w.groups)]
        check_mask_sets(idx_h[:, h:h + 1], cnt_h[:, h:h + 1], ref[h], units, f"{name} mask h={h}",
                        exact_counts=(w.mode == "topk"))
    units = _units(rng, w.heads, w.groups, 6)
    _check_units(sattn, w, qb, kb, vb, idx_h, cnt_h, out_h, lse_h, units, f"{name} gpu-lists")
    # the oracle's lists for head 0, fed to both sides
    h = 0
    ri, rc = ref[h]["idx"], ref[h]["counts"]
    idx2 = idx.clone()
    cnt2 = counts.clone()
    idx2[:, h, :, :ri.shape[-1]] = torch.from_numpy(ri[:, 0]).to(DEV)
    cnt2[:, h] = torch.from_numpy(rc[:, 0]).to(DEV)
    out2, lse2 = sattn.forward(q, k, v, idx2, cnt2, w.group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_units(sattn, w, qb, kb, vb, idx2.cpu().numpy(), cnt2.cpu().numpy(), out2.cpu().numpy(),
                 lse2.cpu().numpy(), [(0, 0, 0), (0, 0, w.groups - 1), (0, 0, w.groups // 2)],
                 f"{name} oracle-lists")
    if name == "voxel_70200":
        # dense control path on the same permuted inputs, sampled rows
        dout, dlse = sattn.attn(q, k, v, out_dtype=torch.float32)
        torch.cuda.synchronize()
        rows = np.sort(rng.choice(w.n_q, 64, replace=False))
        ro, rl = oracle.dense_attention_ref(f64(qb[:, :1]), f64(kb[:, :1]), f64(vb[:, :1]), scale, rows=rows)
        check_out(dout[0, 0].cpu().numpy()[rows], ro[0, 0, rows], "dense voxel")
        check_lse(dlse[0, 0].cpu().numpy()[rows], rl[0, 0, rows], "dense voxel")


def test_full_32760_density_sweep(sattn):
    w, (qb, kb, vb) = workload("full_32760")
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    scale = scale_of(w.dim)
    rng = np.random.default_rng(5)
    units = _units(rng, w.heads, w.groups, 4)
    dout, dlse = sattn.attn(q, k, v, out_dtype=torch.float32)
    G = w.groups
    idx_all = torch.arange(w.n_k, dtype=torch.int32, device=DEV).expand(1, w.heads, G, w.n_k).contiguous()
    cnt_all = torch.full((1, w.heads, G), w.n_k, dtype=torch.int32, device=DEV)
    sout, slse = sattn.forward(q, k, v, idx_all, cnt_all, w.group, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(sout, dout) and torch.equal(slse, dlse), "100% density: sparse != dense"
    del idx_all
    rows = np.sort(rng.choice(w.n_q, 48, replace=False))
    ro, rl = oracle.dense_attention_ref(f64(qb[:, 3:4]), f64(kb[:, 3:4]), f64(vb[:, 3:4]), scale, rows=rows)
    check_out(dout[0, 3].cpu().numpy()[rows], ro[0, 0, rows], "dense 32760")
    for keep in (0.5, 0.2):
        kk = int(round(keep * w.n_k))
        idx, counts = sattn.mask(q, k, w.group, topk=kk)
        out, lse = sattn.forward(q, k, v, idx, counts, w.group, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check_units(sattn, w, qb, kb, vb, idx.cpu().numpy(), counts.cpu().numpy(), out.cpu().numpy(),
                     lse.cpu().numpy(), units, f"32760 keep={keep}")
