"""fp64 oracle of the mean-query (pooling) mask: group mean, scores, per-group cut, index lists.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
library path.

The mask is a heuristic, so this follows its steps in the pages' order:
  1. FG-Attn review, "The pith" and Referee major comment 2: average the
     queries of a group into q_avg.
  2. Same passage: score every key against q_avg, s_j = k_j . q_avg / sqrt(D).
  3. Keep a key unless its pooled probability exp(s_j) / sum_i exp(s_i) is
     below tau (threshold mode; the garbled "/D" is read as the softmax
     denominator), or keep the k highest-scoring keys (top-k mode, the index
     mask of the Chipmunk review, "What carries the argument").
  4. Emit each group's kept keys as an ascending index list plus a count
     (FG-Attn review, Referee major comment 3: the mask is a [B,H,N/M,N]
     index structure).
"""
from __future__ import annotations

import math

import numpy as np


def group_mean_ref(q, group: int) -> np.ndarray:
    """q_avg[b,h,g] = mean of the group's query rows (the last group divides by its true size).

    FG-Attn review, "The pith": the pooling strategy averages the queries of a group.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, Nq, D = q.shape
    G = -(-Nq // group)
    out = np.empty((B, H, G, D))
    for g in range(G):
        r0, r1 = g * group, min((g + 1) * group, Nq)
        out[:, :, g] = q[:, :, r0:r1].sum(axis=2) / (r1 - r0)
    return out


def group_scores_ref(q, k, group: int, scale: float) -> np.ndarray:
    """s[b,h,g,j] = scale * (q_avg[b,h,g] . k[b,h,j]), fp64.

    FG-Attn review, Referee major comment 2 (the pooled score k . q_avg / sqrt D).
    """
    qm = group_mean_ref(q, group)
    k = np.asarray(k, dtype=np.float64)
    return np.matmul(qm, np.swapaxes(k, -1, -2)) * scale


def topk_select_ref(s_row: np.ndarray, topk: int) -> tuple:
    """Keep the `topk` highest scores of one group; ties go to the lower key index.

    Returns (ascending kept indices, boundary score t = the smallest kept score).
    Keys are ranked by (-s, j); the first topk are kept and emitted in ascending order.
    """
    n = s_row.shape[0]
    order = np.lexsort((np.arange(n), -s_row))     # primary key -s, then index
    kept = order[:topk]
    return np.sort(kept), float(s_row[kept[-1]])


def thresh_select_ref(s_row: np.ndarray, tau: float) -> tuple:
    """Keep key j iff exp(s_j - lse) >= tau, i.e. s_j >= lse + ln(tau); never keep nothing.

    lse = log sum_i exp(s_i) over all keys of the group.  tau = 0 keeps every key.  If no key
    reaches the cut, the arg-max key (lowest index on ties) is kept alone.
    Returns (ascending kept indices, cut t = lse + ln tau).
    """
    m = float(s_row.max())
    lse = m + math.log(float(np.exp(s_row - m).sum()))
    t = -math.inf if tau == 0.0 else lse + math.log(tau)
    kept = np.nonzero(s_row >= t)[0]
    if kept.size == 0:
        kept = np.array([int(np.argmax(s_row))])
    return kept, t


def mask_ref(q, k, group: int, mode: str, topk: int = 0, thresh: float = 0.0, scale: float = None,
             cap: int = None) -> dict:
    """Full mask oracle.  mode "topk" or "thresh".

    Returns a dict with idx [B,H,G,cap] int32 (entries beyond counts = -1), counts [B,H,G] int32,
    t [B,H,G] (the cut per group: the k-th largest score, or lse + ln tau) and the scores s [B,H,G,Nk].
    """
    q = np.asarray(q)
    B, H, Nq, D = q.shape
    Nk = np.asarray(k).shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    s = group_scores_ref(q, k, group, scale)
    G = s.shape[2]
    if cap is None:
        cap = topk if mode == "topk" else Nk
    idx = np.full((B, H, G, cap), -1, dtype=np.int32)
    counts = np.zeros((B, H, G), dtype=np.int32)
    t = np.zeros((B, H, G))
    for b in range(B):
        for h in range(H):
            for g in range(G):
                if mode == "topk":
                    kept, cut = topk_select_ref(s[b, h, g], topk)
                elif mode == "thresh":
                    kept, cut = thresh_select_ref(s[b, h, g], thresh)
                else:
                    raise ValueError(mode)
                if kept.size > cap:
                    raise ValueError("cap too small for the kept key list")
                idx[b, h, g, :kept.size] = kept
                counts[b, h, g] = kept.size
                t[b, h, g] = cut
    return {"idx": idx, "counts": counts, "t": t, "s": s}
