"""GPU parity of Chipmunk's column-sum selection (sattn_colsum_mask) and sparse-delta step
(sattn_delta_forward) against the fp64 oracle."""
import math
import os

import numpy as np
import pytest

import oracle
from gpu_util import LSE_ABS, check_out, check_out_scaled, f64, scale_of, to_device_bf16, workload
from synth import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"
# column sums are compared on the log scale: sets may differ only where ln c_j is this close to ln t
LOG_BAND = 1e-3


@pytest.fixture(scope="module")
def sattn():
    import sparse_self_attention_amd as s
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(s.library_path()), "libsattn.so is not built"
    return s


def _bits(rng, shape, std=1.0):
    return inputs.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


# fp32's smallest normal number: each probability the kernel adds into a column sum underflows below it (to
# zero or to a few bits), so a sum of a group's M probabilities is lost up to about M times it
FP32_TINY = 2.0 ** -126


def _check_colsum_sets(idx, cnt, rows, topk, band, what, group=1):
    """rows: {(b, h, g): oracle column sums}.  Exact counts; sets differ only near the k-th sum, or, when
    the k-th sum lies where fp32 loses such sums (below 4 M 2^-126, M the group size: very peaked rows),
    among the keys whose sums do too: there they are ties, whatever the oracle's fp64 values."""
    for (b, h, g), c in rows.items():
        n = int(cnt[b, h, g])
        assert n == topk, f"{what} {b, h, g}: count {n} != {topk}"
        got = idx[b, h, g, :n]
        assert np.all(np.diff(got) > 0), f"{what} {b, h, g}: list not strictly ascending"
        order = np.lexsort((np.arange(c.size), -c))
        want = order[:topk]
        t = c[order[topk - 1]]
        lost = 4.0 * group * FP32_TINY
        bad = [j for j in set(got.tolist()) ^ set(want.tolist())
               if not ((t < lost and c[j] < lost) or (c[j] > 0.0 and abs(math.log(c[j]) - math.log(t)) <= band))]
        assert not bad, f"{what} {b, h, g}: {len(bad)} keys outside the band"


# (D, group, Nq, Nk, topk)
COLSUM_CASES = [(128, 192, 700, 3000, 300), (64, 64, 513, 1025, 1), (128, 16, 100, 777, 777), (128, 256, 300, 70, 13),
                (64, 32, 96, 33000, 3300)]


@pytest.mark.parametrize("D,group,Nq,Nk,topk", COLSUM_CASES)
def test_colsum_random(sattn, D, group, Nq, Nk, topk):
    rng = np.random.default_rng(D + 3 * group + Nq + Nk)
    B, H = 1, 2
    qb, kb = _bits(rng, (B, H, Nq, D), 2.0), _bits(rng, (B, H, Nk, D))
    q64, k64 = f64(qb), f64(kb)
    scale = scale_of(D)
    lse = oracle.row_lse_ref(q64, k64, scale)
    q, k = to_device_bf16(qb, DEV), to_device_bf16(kb, DEV)
    idx, cnt = sattn.colsum_mask(q, k, torch.from_numpy(lse.astype(np.float32)).to(DEV), group, topk)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    rows = oracle.colsum_scores_ref(q64, k64, group, scale, lse)
    _check_colsum_sets(idx, cnt, rows, topk, LOG_BAND, f"colsum D={D} M={group}", group)
    if topk == Nk:
        assert np.all(idx == np.arange(Nk))


@pytest.mark.parametrize("D,group,Nq,Nk,cap,out_f32", [(128, 192, 500, 2000, 150, True), (64, 64, 300, 999, 64, False),
                                                      (128, 128, 260, 4100, 700, True), (128, 48, 97, 300, 300, True)])
def test_delta_random(sattn, D, group, Nq, Nk, cap, out_f32):
    rng = np.random.default_rng(D + group + Nq + cap)
    B, H = 1, 2
    G = -(-Nq // group)
    qb, kb, vb = _bits(rng, (B, H, Nq, D), 2.0), _bits(rng, (B, H, Nk, D)), _bits(rng, (B, H, Nk, D))
    q64, k64, v64 = f64(qb), f64(kb), f64(vb)
    scale = scale_of(D)
    lse = oracle.row_lse_ref(q64, k64, scale)
    counts = rng.integers(0, cap + 1, size=(B, H, G)).astype(np.int32)
    counts[0, 0, 0] = 0
    counts[0, -1, -1] = cap
    idx = inputs.random_index_lists(rng, B, H, G, Nk, counts, cap)
    out_prev = rng.standard_normal((B, H, Nq, D)).astype(np.float32)
    fresh_prev = rng.standard_normal((B, H, Nq, D)).astype(np.float32) * 0.1
    ref_out, ref_fresh = oracle.delta_forward_ref(q64, k64, v64, idx, counts, group, scale, lse, out_prev, fresh_prev)
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    fresh = t(fresh_prev)
    out = sattn.delta_forward(q, k, v, t(idx), t(counts), group, lse=t(lse.astype(np.float32)), out_prev=t(out_prev),
                              fresh=fresh, out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    check_out(fresh.cpu().numpy(), ref_fresh, "delta fresh")
    if out_f32:
        check_out(out.cpu().numpy(), ref_out, "delta out")
    else:
        # the bf16 output is the RNE rounding of the fp32 update (whose fresh part is checked above);
        # out is not bounded like a convex combination, so bf16's half-ulp can exceed the fp32 bar
        o32 = out_prev - fresh_prev + fresh.cpu().numpy()
        assert torch.equal(out.cpu(), torch.from_numpy(o32).to(torch.bfloat16))
    # an empty list leaves fresh = 0 for its rows
    assert np.all(fresh[0, 0, :group].cpu().numpy() == 0.0)


def test_delta_unchanged_step_keeps_output(sattn):
    """A step whose inputs equal the cached step's reproduces the cached output (to fp32 rounding)."""
    rng = np.random.default_rng(77)
    B, H, Nq, Nk, D, group = 1, 2, 384, 1500, 128, 192
    qb, kb, vb = _bits(rng, (B, H, Nq, D), 2.0), _bits(rng, (B, H, Nk, D)), _bits(rng, (B, H, Nk, D))
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    dense, lse = sattn.attn(q, k, v, out_dtype=torch.float32)
    idx, cnt = sattn.colsum_mask(q, k, lse, group, 200)
    zeros = torch.zeros_like(dense)
    fresh = torch.zeros_like(dense)
    sattn.delta_forward(q, k, v, idx, cnt, group, lse=lse, out_prev=zeros, fresh=fresh)   # fresh part of the cache
    fresh0 = fresh.clone()
    out = sattn.delta_forward(q, k, v, idx, cnt, group, lse=lse, out_prev=dense, fresh=fresh)
    torch.cuda.synchronize()
    assert torch.equal(fresh, fresh0)          # deterministic: the recomputed part is bit-identical
    # out = (dense - f) + f, equal to dense up to the two fp32 roundings
    bound = 2.0 ** -22 * (dense.abs() + 2.0 * fresh0.abs())
    assert bool(((out - dense).abs() <= bound).all())


@pytest.mark.parametrize("name", ["voxel_70200"])
def test_full_size_sampled(sattn, name):
    """The column-sparse voxel workload (C = 192, 10 % of keys) at full size: dense lse from the
    library, column sums checked on sampled groups against the oracle with its own exact lse;
    then one delta step over seeded random lists with a seeded synthetic lse."""
    w, (qb, kb, vb) = workload(name)
    q, k, v = (to_device_bf16(x, DEV) for x in (qb, kb, vb))
    _, lse = sattn.attn(q, k, v, out_dtype=torch.float32)
    idx, cnt = sattn.colsum_mask(q, k, lse, w.group, w.topk)
    torch.cuda.synchronize()
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    del idx, lse
    rng = np.random.default_rng(19)
    units = [(0, int(rng.integers(w.heads)), int(rng.integers(w.groups))) for _ in range(3)]
    units.append((0, w.heads - 1, w.groups - 1))
    scale = scale_of(w.dim)
    rows = {}
    for (_, h, g) in units:
        r0, r1 = g * w.group, min((g + 1) * w.group, w.n_q)
        qg, kh = f64(qb[:, h:h + 1, r0:r1]), f64(kb[:, h:h + 1])
        lse_rows = oracle.row_lse_ref(qg, kh, scale)
        rows[(0, h, g)] = oracle.colsum_scores_ref(qg, kh, r1 - r0, scale, lse_rows)[(0, 0, 0)]
    # the library's lse is within LSE_ABS of the exact one, which moves a column sum by at most that factor
    _check_colsum_sets(idx_h, cnt_h, rows, w.topk, LOG_BAND + 2 * LSE_ABS, name, w.group)
    # one delta step over seeded random lists (10 % of keys per group) with a synthetic lse
    G = w.groups
    counts = np.full((1, w.heads, G), w.topk, dtype=np.int32)
    srng = np.random.default_rng(23)
    lists = inputs.random_index_lists(srng, 1, w.heads, G, w.n_k, counts, w.topk)
    lse_syn = (12.0 + 0.5 * srng.standard_normal((1, w.heads, w.n_q))).astype(np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out_prev = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    fresh = torch.zeros_like(out_prev)
    out = sattn.delta_forward(q, k, v, t(lists), t(counts), w.group, lse=t(lse_syn), out_prev=out_prev, fresh=fresh)
    torch.cuda.synchronize()
    for (_, h, g) in units:
        r0, r1 = g * w.group, min((g + 1) * w.group, w.n_q)
        ref = oracle.delta_fresh_ref(f64(qb[:, h:h + 1, r0:r1]), f64(kb[:, h:h + 1]), f64(vb[:, h:h + 1]),
                                     lists[:, h:h + 1, g:g + 1], counts[:, h:h + 1, g:g + 1], r1 - r0, scale,
                                     lse_syn[:, h:h + 1, r0:r1])
        check_out_scaled(out[0, h, r0:r1].cpu().numpy(), ref[0, 0], f"{name} delta h={h} g={g}")
