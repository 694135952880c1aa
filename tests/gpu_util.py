"""Helpers shared by the GPU parity tests (device upload, tolerance checks, cached workloads)."""
from __future__ import annotations

import functools
import math

import numpy as np

from synth import inputs

# Parity bar on the fp32 output given identical index lists.
MAX_ABS = 1e-2
REL_L2 = 5e-3
# lse = m ln2 + ln(l), where l sums the bf16-rounded probabilities.  bf16 has 8 significant bits, so its
# unit roundoff is 2^-8: each rounded probability is within 2^-8 of its exact value relative, l within
# 2^-8 of the exact sum, and |ln l - ln l_exact| <= -ln(1 - 2^-8) = 3.914e-3; the fp32 arithmetic of
# m ln2 + ln l adds below 1e-5 for |lse| < 100.
LSE_ABS = 3.93e-3
LSE_ERRORS = []      # (what, max |lse - oracle|) of every check, reported at the end of the session
# mask key sets may differ only on keys whose oracle score is this close (logit scale) to the cut
MASK_BAND = 1e-3


def to_device_bf16(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def f64(bits: np.ndarray) -> np.ndarray:
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def check_out(o_gpu: np.ndarray, o_ref: np.ndarray, what: str, max_abs: float = MAX_ABS):
    o_gpu = o_gpu.astype(np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref).max()
    rel = np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300)
    assert err <= max_abs and rel <= REL_L2, f"{what}: max|err| {err:.3g} (bar {max_abs:.3g}) rel-L2 {rel:.3g}"
    return err, rel


def fp8_tie_rel(D: int) -> float:
    """Error bound of the FP8 and 4-bit-score kernels' scores relative to sum_d |q_d k_d|: each score is an
    fp32 sum of D exact products (bf16 x bf16, or E2M1 x E2M1 with power-of-two scales), then one multiply
    by a constant rounded to fp32 inside the byte's multiply-add: at most (D + 2) 2^-24."""
    return (D + 2) * 2.0 ** -24


def check_fp8_path(o_gpu: np.ndarray, l_gpu: np.ndarray, ref, vmean: np.ndarray, what: str):
    """An FP8 value path (or 4-bit-score) result against its oracle, ref = (out, lse, out_slack, lse_slack,
    loose) from fp8_attention_ref / fp4_attention_ref with tie_rel = fp8_tie_rel(D).

    Output bar per row: the stated one, plus 2^-8 max_b |mean_b| (the block means return through per-block
    sums L_b of the probabilities, which the forward rounds to bf16 for the matrix-core product
    (mean / scale)^T L; bf16's unit roundoff is 2^-8 and the sums are weights of a convex combination),
    plus the row's tie slack: a byte whose pre-rounding value lies within the fp32 error of the kernel's
    scores of a rounding boundary may be taken the other way, one code from the oracle's (both are ExpCast
    bytes of the score; V-Smart/ExpCast summary, third paragraph).  lse bar: the stated one plus the lse
    slack.  Rows whose first reference point is itself such a tie (`loose`: every byte of the row may move
    by one code) are left out here; they must be rare and the caller checks them against the exact
    restricted softmax (check_expcast_bound); the count allowed (2 + 10 % of the rows; the share grows with
    the window, i.e. with |scores|: ~4 % at query spreads of 30) only guards against a window that is far
    too wide.  rel-L2 is taken over the error beyond the mean-restore and tie terms.
    Returns the loose-row mask."""
    out, lse, oslack, lslack, loose = ref
    o_gpu = o_gpu.astype(np.float64)
    l_gpu = l_gpu.astype(np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert loose.sum() <= 2 + 0.1 * loose.size, \
        f"{what}: {int(loose.sum())} of {loose.size} rows have a near-tie reference point"
    keep = ~loose
    allow = 2.0 ** -8 * float(np.abs(vmean).max(initial=0.0)) + oslack     # per row: the analytic terms
    err = np.abs(o_gpu - out)
    row_err = err.max(axis=-1)
    over = keep & (row_err > MAX_ABS + allow)
    assert not over.any(), (f"{what}: max|err| {row_err[over].max():.3g} above the row bar "
                            f"{(MAX_ABS + allow)[over][np.argmax(row_err[over])]:.3g} ({int(over.sum())} rows)")
    # rel-L2 of the error beyond the analytic terms (they are bounded, not random: a row of outputs small
    # next to the block means would otherwise fail on the mean-restore rounding alone)
    excess = np.maximum(err - allow[..., None], 0.0)
    rel = np.linalg.norm(excess[keep]) / max(np.linalg.norm(out[keep]), 1e-300)
    assert rel <= REL_L2, f"{what}: rel-L2 beyond the analytic terms {rel:.3g}"
    ninf = np.isneginf(lse)
    assert np.array_equal(np.isneginf(l_gpu), ninf), f"{what}: -inf pattern of lse differs"
    fin = keep & ~ninf
    if fin.any():
        lerr = np.abs(l_gpu[fin] - lse[fin])
        LSE_ERRORS.append((what, float(lerr.max())))
        assert np.all(lerr <= LSE_ABS + lslack[fin]), f"{what}: lse max|err| {lerr.max():.3g}"
    return loose


def check_out_scaled(o_gpu: np.ndarray, o_ref: np.ndarray, what: str):
    """Like check_out for unnormalised sums (the sparse-delta part with a stale lse): P is rounded to
    bf16 with a relative error, so the absolute bar scales with the magnitude of the reference."""
    o_gpu = o_gpu.astype(np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    mag = max(1.0, float(np.abs(o_ref).max()))
    err = np.abs(o_gpu - o_ref).max()
    rel = np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300)
    assert err <= MAX_ABS * mag and rel <= REL_L2, f"{what}: max|err| {err:.3g} (scale {mag:.3g}) rel-L2 {rel:.3g}"
    return err, rel


def check_lse(l_gpu: np.ndarray, l_ref: np.ndarray, what: str):
    l_gpu = l_gpu.astype(np.float64)
    ninf = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), ninf), f"{what}: -inf pattern of lse differs"
    if (~ninf).any():
        err = np.abs(l_gpu[~ninf] - l_ref[~ninf]).max()
        LSE_ERRORS.append((what, float(err)))
        assert err <= LSE_ABS, f"{what}: lse max|err| {err:.3g}"


def check_mask_sets(idx_gpu, cnt_gpu, ref, units, what, exact_counts):
    """Kept sets may differ from the oracle's only on keys within MASK_BAND of the group's cut.  A threshold
    that no key reaches keeps the arg-max alone (lowest index on ties); scores within MASK_BAND of the
    maximum are ties up to the rounding of either side (the oracle's fp64 matrix product can round
    identical key rows differently), so a single key kept by the GPU is valid if its score is that close
    to the maximum."""
    for (b, h, g) in units:
        c = int(cnt_gpu[b, h, g])
        got = idx_gpu[b, h, g, :c]
        assert c >= 1 and np.all(np.diff(got) > 0), f"{what} {b, h, g}: list not strictly ascending"
        rc = int(ref["counts"][b, h, g])
        if exact_counts:
            assert c == rc, f"{what} {b, h, g}: count {c} != {rc}"
        diff = set(got.tolist()) ^ set(ref["idx"][b, h, g, :rc].tolist())
        s, t = ref["s"][b, h, g], ref["t"][b, h, g]
        argmax_alone = rc == 1 and s[ref["idx"][b, h, g, 0]] < t     # no key reached the cut
        smax = s.max()
        bad = [j for j in diff if not (abs(s[j] - t) <= MASK_BAND
                                       or (argmax_alone and c == 1 and s[j] >= smax - MASK_BAND))]
        assert not bad, f"{what} {b, h, g}: {len(bad)} keys outside the band, e.g. j={bad[0]} s-t={s[bad[0]] - t:.3g}"


@functools.lru_cache(maxsize=2)
def workload(name: str):
    """bf16 bits of a whole workload (all heads), cached per process."""
    w = inputs.WORKLOADS[name]
    return w, inputs.generate(w)


def scale_of(D: int) -> float:
    return 1.0 / math.sqrt(D)


def _stride(nk):
    return 4 * (-(-(-(-nk // 128)) // 4))


def vsmooth_to_device(codes, scale, mean, nk, dev="cuda:0"):
    """The oracle's (codes, scale, mean [B,H,NB,D]) in the library's layout: mean / scale channel-major,
    padded with zeros to the stride (exact: the scale is a power of two)."""
    import torch
    B, H, NB, D = mean.shape
    m = np.zeros((B, H, D, _stride(nk)), dtype=np.float32)
    m[:, :, :, :NB] = np.transpose(mean / scale[:, :, None, :], (0, 1, 3, 2))
    mb = inputs.f32_to_bf16_bits(m)
    assert np.array_equal(inputs.bf16_bits_to_f32(mb), m), "scaled means must be exact in bf16"
    return (torch.from_numpy(np.ascontiguousarray(codes)).to(dev), torch.from_numpy(scale.astype(np.float32)).to(dev),
            to_device_bf16(mb, dev))


def structured_lists(rng, B, H, G, Nk, counts, kind):
    cap = max(1, int(counts.max()))
    if kind == "random":
        return inputs.random_index_lists(rng, B, H, G, Nk, counts, cap)
    idx = np.full((B, H, G, cap), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for g in range(G):
                c = int(counts[b, h, g])
                if kind == "spread":           # one key per 128-token block: 64 blocks in every tile
                    base = rng.integers(0, 128, size=c)
                    keys = np.minimum(np.arange(c) * 128 + base, Nk - 1)
                    keys = np.unique(keys)
                    counts[b, h, g] = keys.size
                elif kind == "jumps":          # runs of 20 keys with gaps of ~40 blocks between runs
                    starts = np.cumsum(rng.integers(4000, 6000, size=-(-c // 20)))
                    keys = np.unique(np.minimum((starts[:, None] + np.arange(20)[None]).ravel()[:c], Nk - 1))
                    counts[b, h, g] = keys.size
                else:                          # one block
                    keys = np.sort(rng.choice(128, size=min(c, 128), replace=False)) + 128 * (g % max(1, Nk // 128))
                    keys = keys[keys < Nk]
                    counts[b, h, g] = keys.size
                idx[b, h, g, :keys.size] = keys
    return idx


# ExpCast (V-Smart/ExpCast summary, third paragraph): each probability byte is at most one code from the
# exactly rounded one, which bounds the per-row total variation of the weights from the exact softmax by
# 3.64 %.  Over the normal E4M3 range the decoded weight lies within [0.9576, 1.1077] of the exact
# probability (scaled), whose worst split gives that 3.64 %; the lse of the ExpCast weights is therefore
# within [ln 0.9576, ln 1.1077] of the exact one.
EXPCAST_TV = 0.0364
EXPCAST_LSE = (math.log(0.9576), math.log(1.1077))


def check_expcast_bound(o_gpu, l_gpu, o_exact, l_exact, vrange, what, slack=2e-3, mean_abs_max=0.0):
    """Output of an ExpCast path against the exact restricted softmax over the same (dequantised) values:
    with weights at total variation TV <= 3.64 % from the exact ones, |out - exact| <= TV * (max - min of
    the listed value rows) per channel; the lse is within the weight ratio's logarithm.  `vrange` has the
    per-row channel ranges; the slack covers fp32 accumulation, and 2^-8 * mean_abs_max the bf16 rounding
    of the per-block probability sums that restore the block means (see check_fp8_path)."""
    o_gpu = o_gpu.astype(np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_exact)
    bound = EXPCAST_TV * vrange + slack + 2.0 ** -8 * mean_abs_max
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{what}: |out - exact| reaches {worst:.3f} of the ExpCast bound (max err {err.max():.3g})"
    fin = np.isfinite(l_exact)
    d = l_gpu.astype(np.float64)[fin] - l_exact[fin]
    if d.size:
        assert EXPCAST_LSE[0] - slack <= d.min() and d.max() <= EXPCAST_LSE[1] + slack, \
            f"{what}: lse - exact in [{d.min():.4f}, {d.max():.4f}]"
    return worst


@functools.lru_cache(maxsize=8)
def oracle_vsmooth_head(name: str, h: int):
    """The oracle's V-Smooth quantisation of one head of a workload's V (codes, scale, mean with a head axis of 1)."""
    import oracle
    _, (_, _, vb) = workload(name)
    return oracle.vsmooth_quantize_ref(f64(vb[:, h:h + 1]))


@functools.lru_cache(maxsize=8)
def oracle_mx4_head(name: str, which: str, h: int):
    """The oracle's MXFP4 codes and exponents of one head of a workload's Q or K."""
    import oracle
    _, (qb, kb, _) = workload(name)
    x = qb if which == "q" else kb
    return oracle.mx4_quantize_ref(f64(x[:, h:h + 1]))


def value_ranges(vhat, idx, counts, group, n_q):
    """[B,H,Nq,D]: per row, the per-channel range (max - min) of the value rows its group lists."""
    B, H, _, D = vhat.shape
    G = idx.shape[2]
    r = np.zeros((B, H, n_q, D))
    for b in range(B):
        for h in range(H):
            for g in range(G):
                c = int(counts[b, h, g])
                if c:
                    rows = vhat[b, h, idx[b, h, g, :c]]
                    r[b, h, g * group:min((g + 1) * group, n_q)] = rows.max(axis=0) - rows.min(axis=0)
    return r


def onehot_case(rng, H, Nq, group, Nk, D=128):
    """Q, K and per head a set U of D keys whose V rows are the unit vectors e_0 .. e_{D-1}; every group
    lists a subset of its head's U.  V-Smooth turns V[U[i]] into exactly (1 + 2^-7) e_i (block mean 2^-7,
    channel scale 2^-8, residual code 256) and every other listed row into 0, so a row's output is its
    weights times 1 + 2^-7, read in U's order."""
    G = -(-Nq // group)
    U = np.stack([np.sort(rng.choice(Nk, size=D, replace=False)) for _ in range(H)])
    v = np.zeros((1, H, Nk, D))
    for h in range(H):
        v[0, h, U[h], np.arange(D)] = 1.0
    sizes = [D, 100, 65, 64, 17, 1, 33, 128]
    counts = np.zeros((1, H, G), dtype=np.int32)
    idx = np.zeros((1, H, G, D), dtype=np.int32)
    for h in range(H):
        for g in range(G):
            c = sizes[(h * G + g) % len(sizes)]
            counts[0, h, g] = c
            idx[0, h, g, :c] = np.sort(rng.choice(U[h], size=c, replace=False))
    return U, inputs.f32_to_bf16_bits(v.astype(np.float32)), idx, counts


def onehot_total_variation(out, U, idx, counts, probs, group, Nq):
    """Per-row total variation between the weights read off the one-hot output and the exact ones."""
    tvs = []
    H, G = counts.shape[1], counts.shape[2]
    for h in range(H):
        pos = {int(u): i for i, u in enumerate(U[h])}
        for g in range(G):
            P = probs(h, g)                                   # exact restricted softmax rows [rows, Nk]
            r0 = g * group
            w_exact = np.zeros((P.shape[0], U.shape[1]))
            for j in idx[0, h, g, :counts[0, h, g]]:
                w_exact[:, pos[int(j)]] = P[:, j]
            w_gpu = out[0, h, r0:r0 + P.shape[0]].astype(np.float64) / (1.0 + 2.0 ** -7)
            tvs.append(0.5 * np.abs(w_gpu - w_exact).sum(axis=1))
    return np.concatenate(tvs)
