"""Helpers shared by the GPU parity tests (device upload, tolerance checks, cached workloads)."""
from __future__ import annotations

import functools
import math

import numpy as np

from synth import inputs

# Parity bar on the fp32 output given identical index lists.
MAX_ABS = 1e-2
REL_L2 = 5e-3
# lse = m ln2 + ln(l), where l sums the bf16-rounded probabilities (each within 2^-9 relative), so its
# error is bounded by about 2^-9; allow two bf16 half-ulps of slack.
LSE_ABS = 4e-3
# mask key sets may differ only on keys whose oracle score is this close (logit scale) to the cut
MASK_BAND = 1e-3


def to_device_bf16(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def f64(bits: np.ndarray) -> np.ndarray:
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def check_out(o_gpu: np.ndarray, o_ref: np.ndarray, what: str):
    o_gpu = o_gpu.astype(np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref).max()
    rel = np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300)
    assert err <= MAX_ABS and rel <= REL_L2, f"{what}: max|err| {err:.3g} rel-L2 {rel:.3g}"
    return err, rel


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
        assert err <= LSE_ABS, f"{what}: lse max|err| {err:.3g}"


def check_mask_sets(idx_gpu, cnt_gpu, ref, units, what, exact_counts):
    """Kept sets may differ from the oracle's only on keys within MASK_BAND of the group's cut."""
    for (b, h, g) in units:
        c = int(cnt_gpu[b, h, g])
        got = idx_gpu[b, h, g, :c]
        assert c >= 1 and np.all(np.diff(got) > 0), f"{what} {b, h, g}: list not strictly ascending"
        rc = int(ref["counts"][b, h, g])
        if exact_counts:
            assert c == rc, f"{what} {b, h, g}: count {c} != {rc}"
        diff = set(got.tolist()) ^ set(ref["idx"][b, h, g, :rc].tolist())
        s, t = ref["s"][b, h, g], ref["t"][b, h, g]
        bad = [j for j in diff if not abs(s[j] - t) <= MASK_BAND]
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
