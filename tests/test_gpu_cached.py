"""GPU parity of sattn_cached_mask (through the C ABI) against the fp64 cached-mask oracle."""
import os

import numpy as np
import pytest

import oracle
from gpu_util import LSE_ABS, MASK_BAND, f64, scale_of, to_device_bf16, workload
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


def check_cached_sets(idx, cnt, rows, log_tau, band, what):
    """Kept sets may differ from the oracle's only on slices whose max log-probability is within
    `band` of ln tau.  rows: {(b, h, g): oracle max log-probability over the group, per key}."""
    for (b, h, g), m in rows.items():
        c = int(cnt[b, h, g])
        got = idx[b, h, g, :c]
        assert np.all(np.diff(got) > 0), f"{what} {b, h, g}: list not strictly ascending"
        want = np.nonzero(m >= log_tau)[0]
        bad = [j for j in set(got.tolist()) ^ set(want.tolist()) if not abs(m[j] - log_tau) <= band]
        assert not bad, f"{what} {b, h, g}: {len(bad)} slices outside the band, e.g. j={bad[0]} " \
                        f"m-ln(tau)={m[bad[0]] - log_tau:.3g}"


# (D, group, Nq, Nk, tau)
CASES = [
    (128, 128, 1000, 3000, 0.5 / 3000), (64, 64, 513, 1025, 0.5 / 1025), (128, 16, 100, 777, 1.0 / 777),
    (128, 192, 700, 5003, 2e-4), (64, 48, 300, 4096, 0.5 / 4096), (128, 256, 260, 70, 0.01),
    (128, 128, 200, 100, 0.0), (128, 128, 200, 100, 1.5), (64, 32, 96, 33000, 0.5 / 33000),
]


@pytest.mark.parametrize("D,group,Nq,Nk,tau", CASES)
def test_random_with_oracle_lse(sattn, D, group, Nq, Nk, tau):
    """The oracle's exact lse is handed to the kernel, so only the score arithmetic differs."""
    rng = np.random.default_rng(D * 7 + group + Nq + Nk)
    B, H = 1, 3
    qb, kb = _bits(rng, (B, H, Nq, D), 2.0), _bits(rng, (B, H, Nk, D))
    q64, k64 = f64(qb), f64(kb)
    scale = scale_of(D)
    lse = oracle.row_lse_ref(q64, k64, scale)
    q, k = to_device_bf16(qb, DEV), to_device_bf16(kb, DEV)
    lse_d = torch.from_numpy(lse.astype(np.float32)).to(DEV)
    idx, cnt = sattn.cached_mask(q, k, lse_d, group, tau=tau)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    ref = oracle.cached_mask_ref(q64, k64, group, tau, scale)
    G = -(-Nq // group)
    rows = {(b, h, g): ref["m"][b, h, g] for b in range(B) for h in range(H) for g in range(G)}
    check_cached_sets(idx, cnt, rows, ref["log_tau"], MASK_BAND + 1e-5, f"D={D} M={group} tau={tau:.3g}")
    if tau <= 0.0:
        assert np.all(cnt == Nk) and np.all(idx == np.arange(Nk))
    if tau > 1.0:
        assert np.all(cnt == 0)


def test_end_to_end_with_dense_lse(sattn):
    """lse from the library's own dense forward; the band widens by the lse tolerance."""
    rng = np.random.default_rng(5)
    B, H, Nq, Nk, D, group = 1, 2, 640, 2500, 128, 128
    qb, kb, vb = _bits(rng, (B, H, Nq, D), 2.0), _bits(rng, (B, H, Nk, D)), _bits(rng, (B, H, Nk, D))
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    _, lse = sattn.attn(q, k, v, out_dtype=torch.float32)
    idx, cnt = sattn.cached_mask(q, k, lse, group)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    tau = 0.5 / Nk
    ref = oracle.cached_mask_ref(f64(qb), f64(kb), group, tau, scale_of(D))
    rows = {(0, h, g): ref["m"][0, h, g] for h in range(H) for g in range(Nq // group)}
    check_cached_sets(idx, cnt, rows, ref["log_tau"], MASK_BAND + LSE_ABS, "dense lse")
    # every query's arg-max key has probability >= 1/Nk > tau, so no group is empty
    assert np.all(cnt >= 1)


def test_cap_truncates_to_first_keys(sattn):
    rng = np.random.default_rng(9)
    B, H, Nq, Nk, D, group = 1, 1, 256, 900, 64, 64
    qb, kb = _bits(rng, (B, H, Nq, D), 2.0), _bits(rng, (B, H, Nk, D))
    q64, k64 = f64(qb), f64(kb)
    lse = oracle.row_lse_ref(q64, k64, scale_of(D))
    q, k = to_device_bf16(qb, DEV), to_device_bf16(kb, DEV)
    lse_d = torch.from_numpy(lse.astype(np.float32)).to(DEV)
    full_idx, full_cnt = sattn.cached_mask(q, k, lse_d, group, tau=1e-4)
    cap = 7
    idx, cnt = sattn.cached_mask(q, k, lse_d, group, tau=1e-4, cap=cap)
    torch.cuda.synchronize()
    full_idx, full_cnt, idx, cnt = (x.cpu().numpy() for x in (full_idx, full_cnt, idx, cnt))
    assert np.all(full_cnt > cap)
    assert np.all(cnt == cap)
    assert np.array_equal(idx, full_idx[..., :cap])


@pytest.mark.parametrize("name", ["long_70200", "chunked_window"])
def test_full_size_sampled(sattn, name):
    """The long-video and chunked-window workloads at full size, lse from the dense forward, checked
    on sampled groups (always including the partial last group) against the fp64 oracle."""
    w, (qb, kb, vb) = workload(name)
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    _, lse = sattn.attn(q, k, v, out_dtype=torch.float32)
    idx, cnt = sattn.cached_mask(q, k, lse, w.group)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    del q, k, v, lse
    rng = np.random.default_rng(17)
    units = [(0, int(rng.integers(w.heads)), int(rng.integers(w.groups))) for _ in range(3)]
    units.append((0, w.heads - 1, w.groups - 1))
    tau = 0.5 / w.n_k
    sel = sorted({h for _, h, _ in units})
    q64, k64 = f64(qb[:, sel]), f64(kb[:, sel])
    rows_local = oracle.slice_max_logprob_ref(q64, k64, w.group, scale_of(w.dim),
                                              units=[(0, sel.index(h), g) for _, h, g in units])
    rows = {(0, sel[h], g): m for (_, h, g), m in rows_local.items()}
    check_cached_sets(idx, cnt, rows, float(np.log(tau)), MASK_BAND + LSE_ABS, name)
    assert np.all(cnt >= 1)
