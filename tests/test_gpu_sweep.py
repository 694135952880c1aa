"""A seeded sweep over the shapes the entry points accept: head dim 64 or 128, any group size that is a
multiple of 16 up to 256, query and key counts drawn log-uniformly (single tokens, ragged tails, many
tiles), top-k or threshold masks.  For each shape the GPU mask is checked against the fp64 oracle's sets,
and the GPU sparse forward, fed the oracle's own lists, against the oracle's output and lse."""
import os

import numpy as np
import pytest

import oracle
from gpu_util import check_lse, check_mask_sets, check_out, f64, scale_of, to_device_bf16
from synth import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


def _draw_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        group = 16 * int(rng.integers(1, 17))
        if i < n // 3:       # small and single-token shapes
            Nq = int(np.exp(rng.uniform(0.0, np.log(800.0))))
            Nk = int(np.exp(rng.uniform(0.0, np.log(9000.0))))
        else:                # several groups and key tiles with ragged ends
            Nq, Nk = int(rng.integers(200, 801)), int(rng.integers(300, 9001))
        Nq, Nk = max(Nq, 1), max(Nk, 1)
        if rng.random() < 0.6:
            mode, param = "topk", int(rng.integers(1, Nk + 1))
        else:
            mode, param = "thresh", float(10.0 ** rng.uniform(-5.0, -0.3))
        q_std = float(rng.choice([1.0, 2.0, 4.0]))
        cases.append((i, D, group, Nq, Nk, mode, param, q_std))
    return cases


CASES = _draw_cases(24)


@pytest.fixture(scope="module")
def sattn():
    import sparse_self_attention_amd as s
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(s.library_path()), "libsattn.so is not built"
    return s


def _bits(rng, shape, std=1.0):
    return inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-D{c[1]}-M{c[2]}-{c[3]}x{c[4]}-{c[5]}" for c in CASES])
def test_mask_then_forward(sattn, case):
    i, D, group, Nq, Nk, mode, param, q_std = case
    print(f"sweep case {case}", flush=True)
    rng = np.random.default_rng(1000 + i)
    B, H = 1, 2
    qb = _bits(rng, (B, H, Nq, D), q_std)
    kb, vb = _bits(rng, (B, H, Nk, D)), _bits(rng, (B, H, Nk, D))
    G = -(-Nq // group)
    kw = {"topk": param} if mode == "topk" else {"thresh": param}
    ref = oracle.mask_ref(f64(qb), f64(kb), group, mode, **kw)
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    idx, cnt = sattn.mask(q, k, group, **kw)
    torch.cuda.synchronize()
    units = [(b, h, g) for b in range(B) for h in range(H) for g in range(G)]
    check_mask_sets(idx.cpu().numpy(), cnt.cpu().numpy(), ref, units, f"sweep {i} {mode}", exact_counts=(mode == "topk"))

    ridx = np.ascontiguousarray(np.maximum(ref["idx"], 0).astype(np.int32))
    rcnt = np.ascontiguousarray(ref["counts"].astype(np.int32))
    out, lse = sattn.forward(q, k, v, torch.from_numpy(ridx).to(DEV), torch.from_numpy(rcnt).to(DEV), group,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attention_ref(f64(qb), f64(kb), f64(vb), ridx, rcnt, group, scale_of(D))
    check_out(out.cpu().numpy(), ro, f"sweep {i} forward")
    check_lse(lse.cpu().numpy(), rl, f"sweep {i} forward")
