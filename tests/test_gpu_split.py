"""GPU parity of sattn_forward_split (the list of each group in parts, merged) against the fp64 oracle,
through the C ABI: random lists with ragged and empty groups, more parts than key blocks, row slices of
wide groups, bf16 output as the rounding of the fp32 one, and the full-size chunked window on the GPU
mask's threshold lists."""
import json
import os

import numpy as np
import pytest

import oracle
from gpu_util import check_lse, check_out, f64, scale_of, to_device_bf16, workload
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


def _run(sattn, qb, kb, vb, idx, counts, group, splits, out_dtype=torch.float32):
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    it = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(DEV)
    ct = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int32)).to(DEV)
    out, lse = sattn.forward_split(q, k, v, it, ct, group, splits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


# (D, group, Nq, Nk, cap, splits, q_std): partial last groups, row slices (192 -> 2 x 96, 224 -> 2 x 128),
# counts of 0, 1, 31, 32, 33 and cap, parts that get no key block (splits above the block count)
CASES = [
    (128, 128, 300, 2000, 1500, 3, 1.0), (64, 64, 200, 1000, 700, 5, 1.0), (128, 192, 400, 3000, 2000, 4, 2.0),
    (128, 224, 450, 900, 800, 2, 1.0), (64, 32, 100, 500, 300, 8, 1.0), (128, 128, 256, 600, 100, 32, 1.5),
    (128, 16, 70, 129, 129, 2, 1.0), (128, 80, 250, 4100, 4100, 6, 3.0),
]


@pytest.mark.parametrize("D,group,Nq,Nk,cap,splits,q_std", CASES)
def test_split_random_lists(sattn, D, group, Nq, Nk, cap, splits, q_std):
    rng = np.random.default_rng(D + group * 3 + Nq + Nk + splits)
    B, H = 2, 2
    qb = _bits(rng, (B, H, Nq, D), q_std)
    kb, vb = _bits(rng, (B, H, Nk, D)), _bits(rng, (B, H, Nk, D))
    G = -(-Nq // group)
    counts = rng.integers(1, cap + 1, size=(B, H, G)).astype(np.int32)
    for i, c in enumerate([0, 1, 31, 32, 33, cap][:counts.size]):
        counts.flat[i] = min(c, cap)
    idx = inputs.random_index_lists(rng, B, H, G, Nk, counts, cap)
    out, lse = _run(sattn, qb, kb, vb, idx, counts, group, splits)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), idx, counts, group, scale_of(D))
    empty = np.repeat(counts == 0, group, axis=2)[:, :, :Nq]
    assert np.all(o[empty] == 0.0) and np.all(np.isneginf(l[empty])), "empty group must give 0 and -inf"
    check_out(o, np.nan_to_num(ro), f"split D={D} M={group} parts={splits}")
    check_lse(l, rl, f"split D={D} M={group} parts={splits}")
    # the bf16 output is the nearest-even rounding of the fp32 one (the merge rounds once)
    ob, lb = _run(sattn, qb, kb, vb, idx, counts, group, splits, out_dtype=torch.bfloat16)
    want = inputs.f32_to_bf16_bits(o.astype(np.float32))
    got = ob.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), "bf16 output is not the rounding of the fp32 output"
    assert np.array_equal(lb.cpu().numpy(), l)


def test_split_one_part_matches_oracle(sattn):
    """splits = 1: one part per group, the merge only normalises."""
    rng = np.random.default_rng(5)
    D, group, Nq, Nk = 128, 128, 256, 1000
    qb, kb, vb = _bits(rng, (1, 3, Nq, D)), _bits(rng, (1, 3, Nk, D)), _bits(rng, (1, 3, Nk, D))
    counts = np.full((1, 3, 2), 777, dtype=np.int32)
    idx = inputs.random_index_lists(rng, 1, 3, 2, Nk, counts, 777)
    out, lse = _run(sattn, qb, kb, vb, idx, counts, group, 1)
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), idx, counts, group, scale_of(D))
    check_out(out.cpu().numpy(), ro, "split 1")
    check_lse(lse.cpu().numpy(), rl, "split 1")


def test_split_huge_logits(sattn):
    """Scores of several hundred, different in every part: the merge's rescale must stay finite."""
    rng = np.random.default_rng(3)
    D, group, Nq, Nk = 128, 64, 128, 777
    qb = _bits(rng, (1, 1, Nq, D), 30.0)
    kb, vb = _bits(rng, (1, 1, Nk, D)), _bits(rng, (1, 1, Nk, D))
    counts = np.full((1, 1, 2), 500, dtype=np.int32)
    idx = inputs.random_index_lists(rng, 1, 1, 2, Nk, counts, 500)
    out, lse = _run(sattn, qb, kb, vb, idx, counts, group, 7)
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), idx, counts, group, scale_of(D))
    assert np.abs(rl).max() > 88
    check_out(out.cpu().numpy(), ro, "split huge logits")
    check_lse(lse.cpu().numpy(), rl, "split huge logits")


def test_split_full_size_chunked_window(sattn):
    """The chunked window (12 heads, 7,040 queries over 28,160 keys) on the GPU mask's threshold lists
    (tau from tests/golden/thresholds.json), four parts a group as the benchmark runs it; sampled groups
    against the oracle."""
    w, (qb, kb, vb) = workload("chunked_window")
    with open(os.path.join(os.path.dirname(__file__), "golden", "thresholds.json")) as fh:
        tau = json.load(fh)["chunked_window"]["tau"]
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    idx, counts = sattn.mask(q, k, w.group, thresh=tau)
    out, lse = sattn.forward_split(q, k, v, idx, counts, w.group, 4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    idx_h, cnt_h, o, l = idx.cpu().numpy(), counts.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(17)
    scale = scale_of(w.dim)
    for h in (0, w.heads - 1):
        gs = sorted({0, w.groups - 1, int(rng.integers(w.groups))})
        ro, rl = oracle.sparse_attention_ref(f64(qb[:, h:h + 1]), f64(kb[:, h:h + 1]), f64(vb[:, h:h + 1]),
                                             idx_h[:, h:h + 1], cnt_h[:, h:h + 1], w.group, scale,
                                             units=[(0, 0, g) for g in gs])
        for g in gs:
            r = slice(g * w.group, min((g + 1) * w.group, w.n_q))
            check_out(o[0, h, r], ro[0, 0, r], f"chunked split h={h} g={g}")
            check_lse(l[0, h, r], rl[0, 0, r], f"chunked split h={h} g={g}")
