"""Writes tests/golden/thresholds.json: the pooling threshold tau of each threshold-mode workload.

The chunked-window workload keeps about 30 % of its keys by the mean-query threshold, and the pages
give no tau (FG-Attn review, Referee major comment 2 and its list of free parameters).  One global tau
is calibrated on the oracle: the (1 - keep) quantile of the pooled probabilities p_{h,g,j} =
softmax_j(scale * qbar_{h,g} . k_j) over all heads and groups.  Only oracle/ and the seeded input
generator are called.  Run: python tests/golden/make_thresholds.py
"""
import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from synth import inputs  # noqa: E402


def calibrate(name: str) -> float:
    w = inputs.WORKLOADS[name]
    qb, kb, _ = inputs.generate(w)
    f64 = lambda b: inputs.bf16_bits_to_f32(b).astype(np.float64)
    s = oracle.group_scores_ref(f64(qb), f64(kb), w.group, 1.0 / math.sqrt(w.dim))
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    return float(np.quantile(p, 1.0 - w.keep))


def main():
    out = {name: {"tau": calibrate(name), "keep": inputs.WORKLOADS[name].keep,
                  "rule": "(1 - keep) quantile of the oracle's pooled probabilities over all heads and groups"}
           for name, w in inputs.WORKLOADS.items() if w.mode == "thresh"}
    with open(os.path.join(HERE, "thresholds.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
