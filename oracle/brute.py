"""Brute-force reference for micro shapes, pure Python loops (test infrastructure).

It evaluates the gate equation literally ("Mixtral and Mixture-of-Experts,
Explained", section "How it works"): every expert's logit, the top-k kept and
all others set to -inf, a softmax over all E entries, and then the output as
a DENSE sum over all E experts ``y = sum_i G(x)_i * Expert_i(x)``, where
non-selected experts are multiplied by an exact zero.  No grouping, no
permutation, no numpy linear algebra: it exists only to cross-check the main
oracle (``oracle/moe_oracle.py``), which groups tokens by expert instead.

Capacity (micro shapes only): a per-expert list of (token, slot, G), sorted by
G descending then token ascending with Python's sort, first ``capacity`` kept.
Overflow fallback ("How Mixtral 8x7B uses mixture of experts", section
"Routing without auxiliary loss": excess tokens go to the next-best expert):
each dropped slot is offered, in slot order, to the token's experts ranked
3rd, 4th, ... by logit; every expert takes such offers, ranked by the slot's
G then token, into the slots it left free, and the output weights the
fallback expert's output by that G.

Shared expert (``n_shared=1``; DeepSeek-V3 remark on the "Mixtral 8x7B"
interview page): expert index E of the weight lists, added to every token's
output with weight 1, outside the softmax and the capacity limit.
"""
from __future__ import annotations

import math
from typing import List, Sequence


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def _expert(x: Sequence[float], w1, w3, w2) -> List[float]:
    F = len(w1)
    h = []
    for j in range(F):
        g = _dot(x, w1[j])
        u = _dot(x, w3[j])
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [_dot(h, w2[i]) for i in range(len(w2))]


def gate(logits: Sequence[float], k: int):
    """Literal Softmax(TopK(logits)) over all E entries; returns (ids, full G list)."""
    E = len(logits)
    order = sorted(range(E), key=lambda e: (-logits[e], e))
    top = order[:k]
    masked = [logits[e] if e in top else -math.inf for e in range(E)]
    m = max(masked)
    ex = [math.exp(v - m) if v != -math.inf else 0.0 for v in masked]
    z = sum(ex)
    return top, [v / z for v in ex]


def layer(x, w_gate, w1, w3, w2, k: int = 2, bias=None, capacity: int = -1,
          overflow: str = "drop", n_shared: int = 0):
    """Dense brute-force layer on nested lists; returns (y, ids, G_full, keep).

    With overflow == "next_best" (and a capacity), ``keep`` holds per slot the
    expert that finally processes it, or None when it is dropped."""
    T, E = len(x), len(w_gate)
    shared = [_expert(x[t], w1[E], w3[E], w2[E]) for t in range(T)] if n_shared else None
    logits = [[_dot(x[t], w_gate[e]) + (bias[e] if bias is not None else 0.0) for e in range(E)]
              for t in range(T)]
    ids, Gf = [], []
    for t in range(T):
        top, g = gate(logits[t], k)
        ids.append(top)
        Gf.append(g)
    keep = [[True] * k for _ in range(T)]
    if capacity >= 0:
        for e in range(E):
            cand = [(Gf[t][e], t, s) for t in range(T) for s in range(k) if ids[t][s] == e]
            cand.sort(key=lambda c: (-c[0], c[1]))
            for _, t, s in cand[capacity:]:
                keep[t][s] = False
    if capacity >= 0 and overflow == "next_best":
        final = [[ids[t][s] if keep[t][s] else None for s in range(k)] for t in range(T)]
        offers = {}                                        # expert -> [(G, t, s)]
        for t in range(T):
            ranked = sorted(range(E), key=lambda e: (-logits[t][e], e))[k:]
            dropped = [s for s in range(k) if not keep[t][s]]
            for j, s in enumerate(dropped):
                if j < len(ranked):
                    offers.setdefault(ranked[j], []).append((Gf[t][ids[t][s]], t, s))
        for e, cand in offers.items():
            used = sum(1 for t in range(T) for s in range(k) if final[t][s] == e)
            cand.sort(key=lambda c: (-c[0], c[1]))
            for _, t, s in cand[:max(0, capacity - used)]:
                final[t][s] = e
        y = []
        for t in range(T):
            acc = [0.0] * len(x[t])
            for e in range(E):                             # dense over ALL experts
                w = sum(Gf[t][ids[t][s]] for s in range(k) if final[t][s] == e)
                out = _expert(x[t], w1[e], w3[e], w2[e])
                for i in range(len(acc)):
                    acc[i] += w * out[i]
            y.append(acc)
        return y, ids, Gf, final
    y = []
    for t in range(T):
        acc = [0.0] * len(x[t])
        for e in range(E):                                 # dense over ALL experts
            w = Gf[t][e]
            if e in ids[t] and not keep[t][ids[t].index(e)]:
                w = 0.0
            out = _expert(x[t], w1[e], w3[e], w2[e])
            for i in range(len(acc)):
                acc[i] += w * out[i]
        if shared is not None:                             # shared expert, weight 1
            for i in range(len(acc)):
                acc[i] += shared[t][i]
        y.append(acc)
    return y, ids, Gf, keep
