"""Seeded synthetic Q/K/V for the video-shaped attention workloads.

This module only draws inputs. It contains no attention, masking or softmax
arithmetic, so the CPU oracle and the HIP path can both be fed from it without
sharing any of the method's computation.

Shapes follow the pages:
  * LongLive DiT blog ("The Architecture", "Self Attention"): a chunk is
    8 latent frames x 880 tokens = 7040 tokens, the KV window is 4 chunks
    (one fixed sink chunk plus three rolling), 24 heads of dimension 128.
  * V-Smart/ExpCast summary (first paragraph): a 5 s 720p clip is about 70K
    tokens.
  * Chipmunk review ("Assumptions & free parameters"): chunks of C = 192
    tokens, voxel (4, 6, 8).

Real DiT activations are not available, so Q and K are a smooth, low-frequency
positional field plus noise (which gives spatially local attention), and V is
standard normal.  All tensors are rounded fp32 -> bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# bf16 helpers (storage only: bf16 bits are kept as uint16)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload.

    grid_q / grid_k are (T, H_g, W_g) token grids in raster order
    n = (t * H_g + y) * W_g + x.  For the chunked window the queries are the
    last chunk of the key window (q_t0 is the first query frame).
    """

    name: str
    batch: int
    heads: int
    dim: int
    grid_k: tuple           # (T, H_g, W_g) of the keys
    q_t0: int               # first query frame inside grid_k
    q_frames: int           # number of query frames
    group: int              # M (query tokens per group)
    mode: str               # "topk" | "thresh" | "dense"
    keep: float             # fraction of keys kept per group (top-k) or target density (thresh)
    seed: int
    voxel: Optional[tuple] = None   # voxel edge (vt, vy, vx) for the column-sparse reordering

    @property
    def n_k(self) -> int:
        t, y, x = self.grid_k
        return t * y * x

    @property
    def n_q(self) -> int:
        _, y, x = self.grid_k
        return self.q_frames * y * x

    @property
    def groups(self) -> int:
        return -(-self.n_q // self.group)

    @property
    def topk(self) -> int:
        return max(1, int(round(self.keep * self.n_k)))


WORKLOADS = {
    # tiny: 1x2 heads, D=64, 8x8x16 grid, M=64, top 25 %
    "tiny": Workload("tiny", 1, 2, 64, (8, 8, 16), 0, 8, 64, "topk", 0.25, 0),
    # chunked window: 7040 queries (last chunk) against 28160 keys, M=128, ~30 % by threshold
    "chunked_window": Workload("chunked_window", 1, 12, 128, (32, 22, 40), 24, 8, 128, "thresh", 0.30, 1),
    # full self-attention, N=32760 on a 15x42x52 grid, M=128 (densities swept by the caller)
    "full_32760": Workload("full_32760", 1, 24, 128, (15, 42, 52), 0, 15, 128, "topk", 0.20, 2),
    # long video: N=70200 on a 30x45x52 grid, M=128, 20 % of keys per group
    "long_70200": Workload("long_70200", 1, 24, 128, (30, 45, 52), 0, 30, 128, "topk", 0.20, 3),
    # column-sparse: the long grid in voxel order, C=192 tokens per group, 10 % of keys
    "voxel_70200": Workload("voxel_70200", 1, 24, 128, (30, 45, 52), 0, 30, 192, "topk", 0.10, 4,
                            voxel=(4, 6, 8)),
}


# --------------------------------------------------------------------------
# Field + noise generator
# --------------------------------------------------------------------------

N_WAVES = 4           # plane waves per head channel
NOISE_STD = 0.5       # std of the Q/K noise


def _head_rng(seed: int, b: int, h: int) -> np.random.Generator:
    # one independent stream per (seed, batch, head) so any subset of heads is reproducible
    return np.random.default_rng([seed, b, h])


def _field(rng: np.random.Generator, dim: int, grid: tuple, frames: Sequence[int]) -> tuple:
    """Draw the wave parameters and evaluate the field on all grid frames.

    F[n, d] = sum_s (1/sqrt 2) sin(2 pi (ft t/T + fy y/H + fx x/W) + phi), with
    ft, fy, fx ~ U[0, 2) and phi ~ U[0, 2 pi), drawn per (d, s).
    """
    T, Hg, Wg = grid
    freqs = rng.uniform(0.0, 2.0, size=(dim, N_WAVES, 3))
    phases = rng.uniform(0.0, 2.0 * math.pi, size=(dim, N_WAVES))
    t = np.asarray(frames, dtype=np.float64)[:, None, None, None]
    y = np.arange(Hg, dtype=np.float64)[None, :, None, None]
    x = np.arange(Wg, dtype=np.float64)[None, None, :, None]
    F = np.zeros((len(frames), Hg, Wg, dim), dtype=np.float32)
    amp = 1.0 / math.sqrt(2.0)
    for s in range(N_WAVES):
        at = (2.0 * math.pi * freqs[:, s, 0] / T)[None, None, None, :] * t
        ay = (2.0 * math.pi * freqs[:, s, 1] / Hg)[None, None, None, :] * y
        ax = (2.0 * math.pi * freqs[:, s, 2] / Wg)[None, None, None, :] * x
        F += (amp * np.sin(at + ay + ax + phases[None, None, None, :, s])).astype(np.float32)
    return F.reshape(-1, dim)


def generate_head(w: Workload, b: int, h: int) -> tuple:
    """Return (q, k, v) bf16 bits (uint16) of one (batch, head): [n_q, D], [n_k, D], [n_k, D].

    Draw order per head is fixed: wave frequencies, phases, Q noise, K noise, V.
    """
    rng = _head_rng(w.seed, b, h)
    T = w.grid_k[0]
    Fk = _field(rng, w.dim, w.grid_k, range(T))
    Fq = Fk.reshape(T, -1, w.dim)[w.q_t0:w.q_t0 + w.q_frames].reshape(-1, w.dim)
    qn = rng.standard_normal(size=Fq.shape, dtype=np.float32)
    kn = rng.standard_normal(size=Fk.shape, dtype=np.float32)
    v = rng.standard_normal(size=Fk.shape, dtype=np.float32)
    q = f32_to_bf16_bits(Fq + np.float32(NOISE_STD) * qn)
    k = f32_to_bf16_bits(Fk + np.float32(NOISE_STD) * kn)
    return q, k, f32_to_bf16_bits(v)


def generate(w: Workload, heads: Optional[Sequence[int]] = None) -> tuple:
    """Return (q, k, v) as uint16 bf16 bits of shape [B, H', N, D] for the selected heads."""
    heads = list(range(w.heads)) if heads is None else list(heads)
    q = np.empty((w.batch, len(heads), w.n_q, w.dim), dtype=np.uint16)
    k = np.empty((w.batch, len(heads), w.n_k, w.dim), dtype=np.uint16)
    v = np.empty_like(k)
    for b in range(w.batch):
        for j, h in enumerate(heads):
            q[b, j], k[b, j], v[b, j] = generate_head(w, b, h)
    if w.voxel is not None:
        perm = voxel_order(w.grid_k, w.voxel)
        q, k, v = (np.ascontiguousarray(x[:, :, perm]) for x in (q, k, v))
    return q, k, v


def voxel_order(grid: tuple, voxel: tuple) -> np.ndarray:
    """Token permutation that makes every run of vt*vy*vx tokens one 3D voxel.

    Chipmunk review ("What carries the argument", Fig. 2 caption): tokens are
    reordered so each contiguous chunk is a spatio-temporal cube.  Sorting the
    raster positions by (t//vt, y//vy, x//vx, t%vt, y%vy, x%vx) gives that
    order; a stable sort keeps partial edge voxels in raster order.
    Returns perm with permuted[i] = original[perm[i]].
    """
    T, Hg, Wg = grid
    vt, vy, vx = voxel
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    keys = (x % vx, y % vy, t % vt, x // vx, y // vy, t // vt)   # lexsort: last key is primary
    return np.lexsort(keys).astype(np.int64)


def perturb(x_bits: np.ndarray, rel: float, seed: int, ref_rms: Optional[float] = None) -> np.ndarray:
    """x + rel * rms(x_ref) * N(0,1), rounded to bf16 (the step-to-step drift of the long-video run)."""
    x = bf16_bits_to_f32(x_bits)
    rms = float(np.sqrt(np.mean(np.square(x, dtype=np.float64)))) if ref_rms is None else ref_rms
    rng = np.random.default_rng(seed)
    noise = rng.standard_normal(size=x.shape, dtype=np.float32)
    return f32_to_bf16_bits(x + np.float32(rel * rms) * noise)


def random_index_lists(rng: np.random.Generator, batch: int, heads: int, groups: int, n_k: int,
                       counts: np.ndarray, cap: int) -> np.ndarray:
    """Random unique ascending key lists per group (idx[b,h,g,:counts] defined, rest = -1)."""
    idx = np.full((batch, heads, groups, cap), -1, dtype=np.int32)
    for b in range(batch):
        for h in range(heads):
            for g in range(groups):
                c = int(counts[b, h, g])
                if c:
                    idx[b, h, g, :c] = np.sort(rng.choice(n_k, size=c, replace=False))
    return idx
