"""Derive the router bias that makes top-2 expert load follow Zipf(s=1.2).

Reading: the skewed-routing workload wants per-expert shares of the T*k
assignments proportional to (e+1)**-1.2 (expert 0 heaviest).  With router
logits ~ iid N(0,1) (x ~ N(0,1), W_g ~ N(0, 1/d)), a per-expert additive bias
b is fitted by the fixed-point iteration b <- b + 0.5*(ln p - ln share), where
share is measured with the oracle's own top-2 selection on seeded N(0,1)
logits.  The result is written to zipf_bias_e8.json and frozen (rounded to
4 decimals) in the input generator.

Run: python tests/golden/fit_zipf_bias.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
from oracle import topk_gate  # noqa: E402


def shares(logits, b, E=8, k=2):
    ids = topk_gate(logits + b[None, :], k).ids
    return np.bincount(ids.ravel(), minlength=E) / ids.size


def fit(n=400_000, E=8, s=1.2, iters=60, seed=12):
    p = np.array([(e + 1) ** -s for e in range(E)])
    p /= p.sum()
    logits = np.random.Generator(np.random.PCG64(seed)).standard_normal((n, E))
    b = np.zeros(E)
    for _ in range(iters):
        b += 0.5 * (np.log(p) - np.log(shares(logits, b)))
        b -= b.mean()
    return p, b, shares(logits, b)


if __name__ == "__main__":
    p, b, sh = fit()
    out = {"s": 1.2, "target_share": p.round(6).tolist(), "bias": b.round(4).tolist(),
           "achieved_share": sh.round(6).tolist(),
           "note": "iid N(0,1) logits, 400000 tokens, seed 12, 60 half-step fixed-point iterations"}
    path = os.path.join(os.path.dirname(__file__), "zipf_bias_e8.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
