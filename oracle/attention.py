"""fp64 oracle of the sparse attention forward and of dense attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
library path.

Definitions followed
--------------------
* FG-Attn review (pith.science/paper/2509.16518), "The pith" and "What carries
  the argument"; Fig. 6 and Fig. 7 captions: the unit of skipping is an Mx1
  slice, M contiguous queries against one key; a group of M queries computes
  scores only for its list of relevant keys.
* Chipmunk review (pith.science/paper/CJ4ETNKV), Referee major comment 1 and
  minor comment 1 (Alg. 3): the deployed sparse attention normalises the
  softmax over the selected keys only.  Masking the unselected scores to -inf
  before an ordinary row softmax is exactly that restricted softmax.
* LongLive DiT blog (woonyee.org/projects/dit), "Self Attention": per-head
  softmax(Q K^T / sqrt d) V with 24 heads of dimension 128.

Everything is computed in float64 over the full dense score matrix, with no
gather, no tiling and no online softmax.  lse is the natural-log
log-sum-exp of the kept, scaled scores of each query row.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _check_index_list(j: np.ndarray, n_k: int) -> None:
    if j.size and (j.min() < 0 or j.max() >= n_k):
        raise ValueError("key index out of range")
    if np.unique(j).size != j.size:
        raise ValueError("duplicate key index in a group's list")


def _softmax_rows(S: np.ndarray) -> tuple:
    """Row softmax of S (entries may be -inf); returns (P, lse).  A row of all -inf gives P = 0, lse = -inf."""
    m = S.max(axis=1, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    E = np.exp(S - m_safe)                    # exp(-inf) = 0 for unselected keys
    l = E.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(finite, E / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(finite[:, 0], m_safe[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)), -np.inf)
    return P, lse


def dense_attention_ref(q, k, v, scale: float, rows=None):
    """softmax(Q K^T * scale) V per (batch, head), every key kept.

    q: [B,H,Nq,D], k, v: [B,H,Nk,D] (any real dtype; widened to fp64).
    rows: optional sorted array of query rows to evaluate (the others are left as NaN).
    Returns (out [B,H,Nq,D] fp64, lse [B,H,Nq] fp64).
    LongLive DiT blog, "Self Attention" (the per-head attention formula).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, D = q.shape
    sel = np.arange(Nq) if rows is None else np.asarray(rows)
    out = np.full((B, H, Nq, D), np.nan)
    lse = np.full((B, H, Nq), np.nan)
    for b in range(B):
        for h in range(H):
            S = (q[b, h, sel] @ k[b, h].T) * scale
            P, l = _softmax_rows(S)
            out[b, h, sel] = P @ v[b, h]
            lse[b, h, sel] = l
    return out, lse


def sparse_attention_probs_ref(q, k, idx, counts, group: int, scale: float, b: int, h: int, g: int):
    """Probability rows P (|g| x Nk, fp64) of one query group; zero off the group's key list.

    FG-Attn review, Fig. 7 caption (Q_tile K_rel over the relevant key set);
    Chipmunk review, Referee major comment 1 (restricted softmax).
    """
    q, k = _as_f64(q), _as_f64(k)
    Nq, Nk = q.shape[2], k.shape[2]
    r0, r1 = g * group, min((g + 1) * group, Nq)
    c = int(counts[b, h, g])
    J = np.asarray(idx[b, h, g, :c], dtype=np.int64)
    _check_index_list(J, Nk)
    S = (q[b, h, r0:r1] @ k[b, h].T) * scale
    keep = np.zeros(Nk, dtype=bool)
    keep[J] = True
    S[:, ~keep] = -np.inf
    P, lse = _softmax_rows(S)
    return P, lse


def sparse_attention_ref(q, k, v, idx, counts, group: int, scale: float, units=None):
    """Fine-grained sparse attention forward: each group of `group` queries attends to its own key list.

    q: [B,H,Nq,D]; k, v: [B,H,Nk,D]; idx: [B,H,G,cap] int with idx[b,h,g,:counts[b,h,g]] the kept keys
    (any order, unique, in [0,Nk)); counts: [B,H,G].  G = ceil(Nq/group); the last group may be partial.
    units: optional iterable of (b,h,g) to evaluate; rows of other groups are left as NaN.
    Returns (out [B,H,Nq,D] fp64, lse [B,H,Nq] fp64); a group with counts = 0 gives out = 0, lse = -inf.

    Definition: for group rows R and kept set J, S = Q[R] K^T * scale, S[:, j not in J] = -inf,
    P = row softmax of S, out[R] = P V, lse[R] = log sum_j exp(S[:, j]).
    FG-Attn review ("What carries the argument"; Fig. 6, Fig. 7 captions) and Chipmunk review
    (Referee major comment 1: softmax over the selected keys only).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, D = q.shape
    G = -(-Nq // group)
    if idx.shape[:3] != (B, H, G) or counts.shape != (B, H, G):
        raise ValueError("idx/counts shape does not match [B,H,ceil(Nq/group)]")
    out = np.full((B, H, Nq, D), np.nan)
    lse = np.full((B, H, Nq), np.nan)
    if units is None:
        units = [(b, h, g) for b in range(B) for h in range(H) for g in range(G)]
    for b, h, g in units:
        r0, r1 = g * group, min((g + 1) * group, Nq)
        P, l = sparse_attention_probs_ref(q, k, idx, counts, group, scale, b, h, g)
        out[b, h, r0:r1] = P @ v[b, h]
        lse[b, h, r0:r1] = l
    return out, lse
