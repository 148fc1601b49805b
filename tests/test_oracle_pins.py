"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics (CPU only).

Each test names what it pins.  A plausible slip in the oracle (a dropped term,
a wrong sign, index or slot order, a transposed operand, w1/w3 swapped, the
bias dropped, the wrong gate form) fails at least one of them.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from oracle import brute, fp8
from sparse_mixture_experts_topk_amd import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class _Inp:
    """Minimal stand-in for MoEInputs built from float64 numpy arrays."""

    def __init__(self, cfg, x, wg, w1, w3, w2, bias=None):
        self.cfg, self.x, self.w_gate = cfg, x, wg
        self.w1, self.w3, self.w2 = w1, w3, w2
        self.router_bias = bias
        self.w1_scale = self.w3_scale = self.w2_scale = None


def _micro(T=6, d=8, F=12, E=4, seed=3, capacity=-1, bias=False, overflow="drop", k=2, shared=0):
    g = np.random.default_rng(seed)
    f32 = lambda *s: g.standard_normal(s).astype(np.float32).astype(np.float64)  # noqa: E731
    cfg = synthetic.MoEConfig(name="micro", T=T, d_model=d, d_ff=F, n_experts=E, top_k=k,
                              n_shared=shared, capacity=capacity, act_dtype="f32", w_dtype="f32",
                              overflow=overflow)
    b = f32(E) if bias else None
    EW = E + shared
    return _Inp(cfg, f32(T, d), f32(E, d) / math.sqrt(d), f32(EW, F, d) / math.sqrt(d),
                f32(EW, F, d) / math.sqrt(d), f32(EW, d, F) / math.sqrt(F), b)


def _ffn(x, w1, w3, w2):
    """Dense SwiGLU FFN with torch's own silu and linear (float64)."""
    xt = x if isinstance(x, torch.Tensor) else torch.from_numpy(x)
    return Fn.linear(Fn.silu(Fn.linear(xt, torch.from_numpy(w1))) * Fn.linear(xt, torch.from_numpy(w3)),
                     torch.from_numpy(w2)).numpy()


# ------------------------------------------------------------- routing ---

def test_worked_example_printed_values():
    """Interview article, Step 2: scores -> experts '1' and '3' (ids 0, 2), weights 0.6682 / 0.3318."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    scores = np.array(ex["scores"], dtype=np.float64)
    # Router with W_g = I_8 reproduces the scores exactly as logits.
    logits = oracle.router_logits(scores[None, :], np.eye(8))
    r = oracle.topk_gate(logits, 2)
    assert r.ids[0].tolist() == ex["top2_zero_based"]
    assert [i + 1 for i in r.ids[0]] == ex["top2_one_based_as_printed"]
    assert np.round(r.G[0], ex["printed_decimals"]).tolist() == ex["weights_as_printed"]
    # Closed form of a two-way softmax: the logistic function of the logit gap.
    assert abs(r.G[0, 0] - 1.0 / (1.0 + math.exp(-(2.1 - 1.4)))) < 1e-15


def test_gate_forms_agree():
    """Softmax(TopK(l)) (explainer) == full softmax -> top-2 -> renormalise (n4n listing)."""
    logits = np.random.default_rng(0).standard_normal((2000, 8)) * 2.0
    r = oracle.topk_gate(logits, 2)
    p = torch.softmax(torch.from_numpy(logits), dim=-1)
    w, idx = p.topk(2, dim=-1)
    w = w / w.sum(dim=-1, keepdim=True)
    assert np.array_equal(idx.numpy(), r.ids)
    assert np.max(np.abs(w.numpy() - r.G)) < 1e-12


def test_gate_weights_properties():
    logits = np.random.default_rng(1).standard_normal((5000, 8))
    r = oracle.topk_gate(logits, 2)
    assert np.all(np.abs(r.G.sum(axis=1) - 1.0) <= 1e-15)   # sum of two correctly rounded quotients
    assert np.all(r.G[:, 0] >= r.G[:, 1])
    assert np.all(r.ids[:, 0] != r.ids[:, 1])
    l0 = np.take_along_axis(logits, r.ids[:, :1], 1)[:, 0]
    l1 = np.take_along_axis(logits, r.ids[:, 1:], 1)[:, 0]
    others = logits.copy()
    np.put_along_axis(others, r.ids, -np.inf, axis=1)
    assert np.all(l0 >= l1) and np.all(l1 >= others.max(axis=1))
    assert np.allclose(r.gap12, l0 - l1, rtol=0, atol=0)
    assert np.allclose(r.gap23, l1 - others.max(axis=1), rtol=0, atol=0)


def test_ties_go_to_lower_index():
    logits = np.array([[1.0, 3.0, 3.0, 0.0, 3.0, -1.0, 2.0, 2.0],
                       [0.5] * 8,
                       [0.0, 0.0, 5.0, 0.0, 0.0, 0.0, 0.0, 5.0],
                       [4.0, 1.0, 2.0, 2.0, 2.0, 0.0, 0.0, 0.0]])
    r = oracle.topk_gate(logits, 2)
    assert r.ids.tolist() == [[1, 2], [0, 1], [2, 7], [0, 2]]
    assert r.G[1].tolist() == [0.5, 0.5] and r.G[0].tolist() == [0.5, 0.5]
    # Duplicated router rows give exactly equal logits: the lower index wins.
    x = np.random.default_rng(2).standard_normal((50, 16))
    wg = np.random.default_rng(3).standard_normal((8, 16))
    wg[5] = wg[2] = wg[6] * 3.0
    r2 = oracle.topk_gate(oracle.router_logits(x, wg), 2)
    both = np.isin(r2.ids, [2, 5])
    assert not np.any(r2.ids == 5) or np.all(both.sum(axis=1)[np.any(r2.ids == 5, axis=1)] == 2)
    pos = np.any(r2.ids == 2, axis=1) & np.any(r2.ids == 5, axis=1)
    assert np.all(r2.ids[pos].tolist() == [[2, 5]] * int(pos.sum()))


# ------------------------------------------- full layer vs brute force ---

@pytest.mark.parametrize("capacity,bias", [(-1, False), (-1, True), (1, False), (2, True), (0, False)])
def test_oracle_matches_dense_brute_force(capacity, bias):
    inp = _micro(capacity=capacity, bias=bias)
    res = oracle.forward(inp)
    yb, ids, Gf, keep = brute.layer(inp.x.tolist(), inp.w_gate.tolist(), inp.w1.tolist(),
                                    inp.w3.tolist(), inp.w2.tolist(), 2,
                                    None if inp.router_bias is None else inp.router_bias.tolist(),
                                    capacity)
    assert res.routing.ids.tolist() == ids
    Gb = np.array([[Gf[t][e] for e in ids[t]] for t in range(len(ids))])
    assert np.max(np.abs(Gb - res.routing.G)) < 1e-14
    assert res.keep.tolist() == keep
    assert np.max(np.abs(np.array(yb) - res.y)) < 1e-12
    if capacity == 0:
        assert np.all(res.y == 0.0)


@pytest.mark.parametrize("T,E,capacity,bias,seed", [(6, 4, 1, False, 3), (6, 4, 2, True, 3),
                                                     (6, 4, 0, False, 3), (9, 5, 2, False, 7),
                                                     (8, 3, 2, True, 4), (7, 2, 3, False, 5),
                                                     (12, 6, 3, True, 9)])
def test_fallback_matches_dense_brute_force(T, E, capacity, bias, seed):
    """Overflow fallback: grouped oracle vs the literal per-slot offers of brute.layer."""
    inp = _micro(T=T, E=E, seed=seed, capacity=capacity, bias=bias, overflow="next_best")
    res = oracle.forward(inp)
    yb, ids, Gf, final = brute.layer(inp.x.tolist(), inp.w_gate.tolist(), inp.w1.tolist(),
                                     inp.w3.tolist(), inp.w2.tolist(), 2,
                                     None if inp.router_bias is None else inp.router_bias.tolist(),
                                     capacity, overflow="next_best")
    assert res.routing.ids.tolist() == ids
    for t in range(T):
        for s in range(2):
            if final[t][s] is None:
                assert res.status[t, s] == 1
            else:
                assert res.status[t, s] in (0, 2) and res.final_ids[t, s] == final[t][s]
                assert (res.status[t, s] == 2) == (final[t][s] != ids[t][s])
    assert np.max(np.abs(np.array(yb) - res.y)) < 1e-12
    if capacity == 0:
        assert np.all(res.y == 0.0) and np.all(res.status == 1)


def test_fallback_worked_example():
    """Hand-worked case, E = 4, capacity 1, logits fed through W_g = I.

    t0 logits (4, 3, 2, 1):     top-2 (0, 1), G = (s, 1-s) with s = 1/(1+e^-1); ranks 3, 4 = (2, 3)
    t1 logits (3, 4, 1, 2):     top-2 (1, 0), G = (s, 1-s); ranks 3, 4 = (3, 2)
    t2 logits (3.5, 0, .5, .25): top-2 (0, 2), G = (u, 1-u), u = 1/(1+e^-3); ranks 3, 4 = (3, 1)
    Capacity round: e0 gets t0s0 (s), t1s1 (1-s), t2s0 (u) -> keeps t2s0 (u > s).
    e1 gets t0s1 (1-s), t1s0 (s) -> keeps t1s0.  e2 keeps t2s1.  e3 gets nothing.
    Fallback: t0 lost both slots -> s0 offered to e2, s1 to e3; t1 lost s1 -> offered to e3.
    e2 has no free slot: t0s0 stays dropped.  e3 has one: t0s1 and t1s1 tie on G = 1-s,
    the lower token wins -> t0s1 kept at e3, t1s1 dropped.
    """
    logits = np.array([[4, 3, 2, 1], [3, 4, 1, 2], [3.5, 0, 0.5, 0.25]], dtype=np.float64)
    r = oracle.topk_gate(oracle.router_logits(logits, np.eye(4)), 2)
    assert r.ids.tolist() == [[0, 1], [1, 0], [0, 2]]
    assert r.next_ids.tolist() == [[2, 3], [3, 2], [3, 1]]
    keep, _ = oracle.capacity_select(r.ids, r.G, 4, 1)
    assert keep.tolist() == [[False, False], [True, False], [True, True]]
    final, status, cut2 = oracle.fallback_select(r.ids, r.next_ids, r.G, keep, 4, 1)
    assert status.tolist() == [[1, 2], [0, 1], [0, 0]]
    assert final[0, 1] == 3 and final[1, 0] == 1 and final[2].tolist() == [0, 2]
    assert cut2[2] == np.inf and abs(cut2[3] - (1 - 1 / (1 + math.exp(-1)))) < 1e-15
    p = oracle.permutation(final, status != 1, 4)
    assert p.counts.tolist() == [1, 1, 1, 1]
    assert p.perm_src.tolist() == [4, 2, 5, 1]          # e0: t2s0, e1: t1s0, e2: t2s1, e3: t0s1


def test_fallback_invariants():
    g = np.random.default_rng(21)
    T, E, k = 400, 8, 2
    logits = g.standard_normal((T, E)) + np.array([2.0, 1.0, 0.5, 0, 0, 0, 0, -0.5])
    r = oracle.topk_gate(logits, k)
    for C in (0, 1, 20, 60, 100, 200, 800):
        keep, _ = oracle.capacity_select(r.ids, r.G, E, C)
        final, status, _ = oracle.fallback_select(r.ids, r.next_ids, r.G, keep, E, C)
        assert np.all(status[keep] == 0) and np.all(status[~keep] != 0)
        kept = status != 1
        counts = np.bincount(final[kept], minlength=E)
        assert np.all(counts <= C)
        assert kept.sum() >= keep.sum()
        for t, s in np.argwhere(status == 2):
            e = final[t, s]
            assert e not in r.ids[t] and e in r.next_ids[t]
            assert e == (r.next_ids[t, s] if not keep[t].any() else r.next_ids[t, 0])
        # per expert: the fallback round fills exactly min(free slots, offers)
        target = oracle.fallback_targets(keep, r.next_ids)
        for e in range(E):
            free = C - int(np.count_nonzero((r.ids == e) & keep))
            offers = int(np.count_nonzero(target == e))
            assert int(np.count_nonzero((status == 2) & (final == e))) == min(free, offers)
        if C >= T * k:
            assert np.all(status == 0)
    # next-ranked experts are the 3rd and 4th by (logit desc, index asc), distinct from the top-2
    assert np.all(r.next_ids[:, 0] != r.next_ids[:, 1])
    assert not np.any(np.isin(r.next_ids[:, :1], r.ids) & (r.next_ids[:, :1] == r.ids[:, :1]))
    srt = np.sort(-logits, axis=1)
    assert np.allclose(-srt[:, 2], logits[np.arange(T), r.next_ids[:, 0]])
    assert np.allclose(-srt[:, 3], logits[np.arange(T), r.next_ids[:, 1]])


def test_dense_reduction_all_experts_equal():
    """All experts identical and sum(G) = 1  =>  the layer is one dense SwiGLU FFN."""
    inp = _micro(T=40, d=16, F=24, E=8, seed=5)
    for w in (inp.w1, inp.w3, inp.w2):
        w[:] = w[0]
    res = oracle.forward(inp)
    xt = torch.from_numpy(inp.x)
    dense = Fn.linear(Fn.silu(Fn.linear(xt, torch.from_numpy(inp.w1[0]))) *
                      Fn.linear(xt, torch.from_numpy(inp.w3[0])), torch.from_numpy(inp.w2[0]))
    assert np.max(np.abs(res.y - dense.numpy())) < 1e-12 * max(1.0, np.abs(dense.numpy()).max())


def test_token_output_is_gate_weighted_sum_of_its_two_experts():
    inp = _micro(T=30, d=16, F=20, E=8, seed=7, bias=True)
    res = oracle.forward(inp)
    xt = torch.from_numpy(inp.x)
    for t in range(inp.cfg.T):
        acc = torch.zeros(inp.cfg.d_model, dtype=torch.float64)
        for s in range(2):
            e = int(res.routing.ids[t, s])
            ffn = Fn.linear(Fn.silu(Fn.linear(xt[t], torch.from_numpy(inp.w1[e]))) *
                            Fn.linear(xt[t], torch.from_numpy(inp.w3[e])), torch.from_numpy(inp.w2[e]))
            acc += res.routing.G[t, s] * ffn
        assert np.max(np.abs(acc.numpy() - res.y[t])) < 1e-12


def test_combine_linearity_zeroing_one_expert():
    inp = _micro(T=32, d=8, F=12, E=8, seed=9)
    base = oracle.forward(inp)
    e = int(base.routing.ids[0, 0])
    inp.w2 = inp.w2.copy()
    inp.w2[e] = 0.0
    cut = oracle.forward(inp)
    for t in range(inp.cfg.T):
        expect = base.y[t].copy()
        for s in range(2):
            if base.routing.ids[t, s] == e:
                expect -= base.routing.G[t, s] * base.y_perm[base.perm.slot_to_row[2 * t + s]]
        assert np.max(np.abs(cut.y[t] - expect)) < 1e-12


# ------------------------------------------ general top-k, shared expert ---

@pytest.mark.parametrize("k,E,shared,capacity,bias", [
    (1, 4, 0, -1, False), (3, 6, 0, -1, True), (4, 8, 1, -1, False), (8, 8, 0, -1, False),
    (8, 8, 1, -1, True), (3, 6, 1, 2, False), (1, 4, 1, 1, True), (5, 16, 0, 2, False)])
def test_general_topk_and_shared_match_dense_brute_force(k, E, shared, capacity, bias):
    """Routing, capacity and output for k != 2 and a shared expert vs the literal dense form."""
    inp = _micro(T=9, E=E, k=k, shared=shared, capacity=capacity, bias=bias, seed=10 + k + E)
    res = oracle.forward(inp)
    yb, ids, Gf, keep = brute.layer(inp.x.tolist(), inp.w_gate.tolist(), inp.w1.tolist(),
                                    inp.w3.tolist(), inp.w2.tolist(), k,
                                    None if inp.router_bias is None else inp.router_bias.tolist(),
                                    capacity, n_shared=shared)
    assert res.routing.ids.tolist() == ids
    Gb = np.array([[Gf[t][e] for e in ids[t]] for t in range(len(ids))])
    assert np.max(np.abs(Gb - res.routing.G)) < 1e-14
    assert res.keep.tolist() == keep
    assert np.max(np.abs(np.array(yb) - res.y)) < 1e-12


def test_top1_is_the_single_best_expert_with_weight_one():
    """k = 1: the softmax over one kept logit is exactly 1; y = FFN of the arg-max expert."""
    inp = _micro(T=20, d=8, F=12, E=8, k=1, seed=21)
    res = oracle.forward(inp)
    logits = inp.x @ inp.w_gate.T
    assert res.routing.ids[:, 0].tolist() == np.argmax(logits, axis=1).tolist()
    assert np.all(res.routing.G == 1.0)
    for t in range(inp.cfg.T):
        e = int(res.routing.ids[t, 0])
        assert np.max(np.abs(res.y[t] - _ffn(inp.x[t], inp.w1[e], inp.w3[e], inp.w2[e]))) < 1e-12


def test_topk_equal_to_all_experts_is_the_dense_softmax_mixture():
    """k = E: nothing is masked, so G is the full softmax and y is the dense mixture of experts."""
    E = 6
    inp = _micro(T=12, d=8, F=10, E=E, k=E, seed=22, bias=True)
    res = oracle.forward(inp)
    logits = torch.from_numpy(inp.x @ inp.w_gate.T + inp.router_bias[None, :])
    p = torch.softmax(logits, dim=-1).numpy()
    Gfull = np.zeros((inp.cfg.T, E))
    np.put_along_axis(Gfull, res.routing.ids, res.routing.G, axis=1)
    assert np.max(np.abs(Gfull - p)) < 1e-15
    dense = sum(p[:, e:e + 1] * _ffn(inp.x, inp.w1[e], inp.w3[e], inp.w2[e]) for e in range(E))
    assert np.max(np.abs(res.y - dense)) < 1e-12
    assert np.all(np.isinf(res.routing.gap23))


def test_general_topk_gate_properties_and_ties():
    g = np.random.default_rng(23)
    logits = g.standard_normal((3000, 64)) * 1.5
    for k in (1, 3, 6, 8):
        r = oracle.topk_gate(logits, k)
        srt = -np.sort(-logits, axis=1)
        kept = np.take_along_axis(logits, r.ids, 1)
        assert np.array_equal(kept, srt[:, :k])                     # the k largest, in order
        assert np.all(np.abs(r.G.sum(axis=1) - 1.0) < 1e-14)
        assert np.all(np.diff(r.G, axis=1) <= 0)                    # slot 0 the largest weight
        # softmax invariance: G depends only on differences of the kept logits
        ex = np.exp(kept - kept[:, :1])
        assert np.max(np.abs(r.G - ex / ex.sum(axis=1, keepdims=True))) < 1e-15
        gaps = srt[:, :k - 1] - srt[:, 1:k]
        assert np.array_equal(r.gap12, gaps.min(axis=1) if k > 1 else np.full(len(logits), np.inf))
        assert np.array_equal(r.gap23, srt[:, k - 1] - srt[:, k])
    # equal logits go to the lower index for any k
    tie = np.array([[0.0, 2.0, 1.0, 2.0, 1.0, 2.0, 1.0, 0.0]])
    assert oracle.topk_gate(tie, 5).ids.tolist() == [[1, 3, 5, 2, 4]]
    G = oracle.topk_gate(tie, 3).G
    assert G.tolist() == [[1 / 3, 1 / 3, 1 / 3]] or np.max(np.abs(G - 1 / 3)) < 1e-16


def test_shared_expert_alone_is_a_dense_ffn_and_adds_linearly():
    """Routed experts zeroed => y is the shared expert's dense FFN; otherwise routed + shared."""
    inp = _micro(T=15, d=8, F=12, E=8, k=3, shared=1, seed=24)
    shared_ffn = _ffn(inp.x, inp.w1[8], inp.w3[8], inp.w2[8])
    with_shared = oracle.forward(inp).y
    cfg0 = synthetic.MoEConfig(name="micro", T=15, d_model=8, d_ff=12, n_experts=8, top_k=3,
                               act_dtype="f32", w_dtype="f32")
    routed_only = oracle.forward(_Inp(cfg0, inp.x, inp.w_gate, inp.w1[:8], inp.w3[:8], inp.w2[:8])).y
    assert np.max(np.abs(with_shared - (routed_only + shared_ffn))) < 1e-12
    inp.w2 = inp.w2.copy()
    inp.w2[:8] = 0.0
    assert np.max(np.abs(oracle.forward(inp).y - shared_ffn)) < 1e-12
    # capacity 0 drops every routed slot but never the shared expert
    inp.cfg = dataclasses.replace(inp.cfg, capacity=0)
    res = oracle.forward(inp)
    assert not res.keep.any() and np.max(np.abs(res.y - shared_ffn)) < 1e-12


def test_permutation_with_shared_expert_rows():
    g = np.random.default_rng(25)
    T, E, k = 200, 16, 4
    r = oracle.topk_gate(g.standard_normal((T, E)), k)
    keep = g.random((T, k)) > 0.3
    p = oracle.permutation(r.ids, keep, E, 1)
    assert p.counts[E] == T and p.counts[:E].tolist() == np.bincount(r.ids[keep], minlength=E).tolist()
    assert p.offsets[-1] == keep.sum() + T
    assert p.perm_src[p.offsets[E]:].tolist() == (T * k + np.arange(T)).tolist()
    # slot_to_row inverts perm_src over all T*(k+1) slots, dropped slots -> -1
    assert len(p.slot_to_row) == T * (k + 1)
    assert np.array_equal(p.slot_to_row[p.perm_src], np.arange(len(p.perm_src)))
    assert np.all(p.slot_to_row[:T * k][~keep.ravel()] == -1)
    routed = p.perm_src[:p.offsets[E]]
    assert np.array_equal(p.slot_to_row[routed], np.arange(len(routed)))
    for e in range(E):
        seg = p.perm_src[p.offsets[e]:p.offsets[e + 1]]
        assert np.all(np.diff(seg // k) > 0) and np.all(r.ids.ravel()[seg] == e)


# -------------------------------------------------- capacity + grouping ---

def test_capacity_invariants():
    g = np.random.default_rng(11)
    T, E, k = 300, 8, 2
    logits = g.standard_normal((T, E)) + np.array([2.0, 1.0, 0.5, 0, 0, 0, 0, 0])
    r = oracle.topk_gate(logits, k)
    load = np.bincount(r.ids.ravel(), minlength=E)
    for C in (0, 1, 37, 75, 150, 10_000):
        keep, cut = oracle.capacity_select(r.ids, r.G, E, C)
        p = oracle.permutation(r.ids, keep, E)
        assert p.counts.tolist() == np.minimum(load, C).tolist()
        for e in range(E):
            cand = sorted(((-r.G[t, s], t, s) for t in range(T) for s in range(k) if r.ids[t, s] == e))
            kept = {(t, s) for _, t, s in cand[:C]}
            got = {(t, s) for t in range(T) for s in range(k) if r.ids[t, s] == e and keep[t, s]}
            assert kept == got
        if C >= T:
            assert keep.all()
    # Ties in G at the cutoff go to the lower token index.
    ids = np.zeros((6, 2), dtype=np.int64)
    ids[:, 1] = 1
    G = np.tile([0.6, 0.4], (6, 1))
    keep, _ = oracle.capacity_select(ids, G, 2, 4)
    assert keep[:, 0].tolist() == [True] * 4 + [False] * 2


def test_permutation_invariants():
    g = np.random.default_rng(12)
    T, E, k = 500, 8, 2
    r = oracle.topk_gate(g.standard_normal((T, E)), k)
    keep = g.random((T, k)) > 0.2
    p = oracle.permutation(r.ids, keep, E)
    assert p.counts.tolist() == np.bincount(r.ids[keep], minlength=E).tolist()
    assert p.offsets[0] == 0 and np.array_equal(np.diff(p.offsets), p.counts)
    assert p.offsets[-1] == keep.sum()
    full = oracle.permutation(r.ids, np.ones_like(keep), E)
    assert full.counts.sum() == T * k and np.array_equal(full.counts, np.bincount(r.ids.ravel(), minlength=E))
    for e in range(E):
        seg = p.perm_src[p.offsets[e]:p.offsets[e + 1]]
        assert np.all(np.diff(seg // k) > 0)                        # token-ascending, one slot each
        assert np.all(r.ids.ravel()[seg] == e)
    assert np.array_equal(p.slot_to_row[p.perm_src], np.arange(len(p.perm_src)))
    assert np.all(p.slot_to_row[~keep.ravel()] == -1)


# --------------------------------------------------------------- fp8 ---

def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_decode(codes.numpy())
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok]) and np.nanmax(np.abs(got)) == 448.0


def test_e4m3_encode_matches_torch_rne():
    # every bf16 value in [-448, 448], plus exact midpoints between adjacent codes (ties)
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = bits.to(torch.float64)
    v = v[torch.isfinite(v) & (v.abs() <= 448)]
    pos = np.sort(fp8.e4m3_decode(np.arange(127, dtype=np.uint8)))
    mids = (pos[1:] + pos[:-1]) / 2
    rnd = np.random.default_rng(0).uniform(-448, 448, 200_000)
    allv = np.concatenate([v.numpy(), mids, -mids, rnd])
    ref = torch.from_numpy(allv).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fp8.e4m3_encode(allv.astype(np.float32).astype(np.float64))
    assert np.array_equal(ref, got)


def test_block_quantize_properties():
    g = np.random.default_rng(4)
    a = (g.standard_normal((64, 256)) * np.exp(g.uniform(-8, 8, (64, 1)))).astype(np.float32)
    a[3, 32:64] = 0.0
    codes, e, deq = fp8.block_quantize(a)
    q = fp8.e4m3_decode(codes)
    assert np.all(np.abs(q) <= 448)
    blocks = np.abs(a.astype(np.float64)).reshape(64, 8, 32).max(-1)
    nz = blocks > 0
    scaled_max = blocks * np.exp2(-e.astype(np.float64))
    assert np.all(scaled_max[nz] > 224) and np.all(scaled_max[nz] <= 448)
    assert e[3, 1] == 0 and np.all(deq[3, 32:64] == 0)
    assert np.array_equal(deq, q * np.exp2(np.repeat(e, 32, axis=1)))
    normal = np.abs(a) * np.exp2(-np.repeat(e, 32, axis=1)) >= 2.0 ** -6
    rel = np.abs(deq - a)[normal] / np.abs(a.astype(np.float64))[normal]
    assert np.all(rel <= 2.0 ** -4)
    # values already on the grid (e4m3 code times the block's power of two) are unchanged
    grid = (fp8.e4m3_decode(g.integers(0, 126, (8, 64)).astype(np.uint8)) * 2.0 ** -5)
    grid[:, ::32] = 448 * 2.0 ** -5
    _, _, deq2 = fp8.block_quantize(grid.astype(np.float32))
    assert np.array_equal(deq2, grid)


def test_fp8_weight_dequant_matches_torch():
    w32 = torch.from_numpy(np.random.default_rng(5).standard_normal((3, 16, 64)).astype(np.float32) * 0.02)
    q, s = synthetic.quantize_rows_e4m3(w32)
    ref = (q.to(torch.float32).to(torch.float64) * s.to(torch.float64).unsqueeze(-1)).numpy()
    assert np.array_equal(oracle.dequant_weight(q, s), ref)


def test_act_quant_ffn_reduces_to_plain_ffn_on_grid_inputs():
    """With x and h already representable, the fp8 emulation equals the plain SwiGLU."""
    g = np.random.default_rng(6)
    d, F = 64, 32
    x = fp8.e4m3_decode(g.integers(0, 126, (5, d)).astype(np.uint8))
    x[:, ::32] = 448.0
    w1 = g.standard_normal((F, d)) * 0.0
    w3 = g.standard_normal((F, d)) * 0.0
    w2 = g.standard_normal((d, F))
    y_q, _ = oracle.swiglu_act_quant(x, w1, w3, w2)      # h == 0 exactly, representable
    y_p, _ = oracle.swiglu(x, w1, w3, w2)
    assert np.array_equal(y_q, y_p)


def _h_on_block_grid(h32, block=32):
    """Expected dequantised h: per row and 32-element block along F, the scale 2**e with e the
    smallest integer such that fp32(amax / 448) <= 2**e (0 for an all-zero block), and torch's
    float8_e4m3fn cast (round to nearest even) of the scaled values."""
    R, F = h32.shape
    out = np.empty((R, F))
    for r in range(R):
        for b in range(F // block):
            blk = h32[r, b * block:(b + 1) * block]
            amax = np.float32(np.abs(blk).max())
            e = 0
            if amax > 0:
                ratio = float(np.float32(amax / np.float32(448.0)))
                e = math.ceil(math.log2(ratio))
                while 2.0 ** (e - 1) >= ratio:       # guard the float log2 at powers of two
                    e -= 1
                while 2.0 ** e < ratio:
                    e += 1
            q = torch.from_numpy(blk.astype(np.float64) * 2.0 ** -e).to(torch.float32)
            out[r, b * block:(b + 1) * block] = q.to(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** e
    return out


def test_act_quant_h_step_is_block_quantised_along_F():
    """fp8 emulation, h step: with w2 = I (F = d) the output is the quantised h itself.  It must
    lie on one e4m3 grid scaled by 2**e per (row, 32-block along F), equal torch's e4m3 rounding of
    the fp32 h on that grid, and stay within 2**-4 of h (normal range).  x is put on its grid so
    that its own quantisation is the identity; rows differ in magnitude so that blocking along the
    wrong axis changes the scales."""
    g = np.random.default_rng(61)
    d = F = 128
    R = 6
    x = fp8.e4m3_decode(g.integers(0, 126, (R, d)).astype(np.uint8)) * np.where(g.random((R, d)) < 0.5, -1, 1)
    x[:, ::32] = 448.0
    x *= np.exp2(np.arange(R) * 3 - 15.0)[:, None]           # row scales 2^-15 .. 2^0
    w1 = g.standard_normal((F, d)) * 0.05
    w3 = g.standard_normal((F, d)) * 0.05
    w3[:, :] *= np.exp2(g.integers(-6, 6, F))[:, None]       # channel magnitudes vary along F
    y, hq = oracle.swiglu_act_quant(x, w1, w3, np.eye(d))
    xt = torch.from_numpy(x)
    h = (Fn.silu(Fn.linear(xt, torch.from_numpy(w1))) * Fn.linear(xt, torch.from_numpy(w3))).numpy()
    h32 = h.astype(np.float32)
    ref = _h_on_block_grid(h32)
    assert np.array_equal(y, ref), "h is not the per-(row, 32-block along F) e4m3 quantisation"
    assert np.array_equal(hq, ref)
    big = np.abs(ref) >= 2.0 ** -6 * np.abs(h32).max(axis=1, keepdims=True) / 448 * 2
    assert np.all(np.abs(ref - h32)[big] <= 2.0 ** -4 * np.abs(h32.astype(np.float64))[big])
    assert np.linalg.norm(ref - h) / np.linalg.norm(h) > 1e-3     # the step is not the identity


def test_act_quant_h_step_hand_worked_block():
    """One block worked by hand.  x = e_0 (quantises exactly: 1 * 2^8 = 256 is an e4m3 value),
    w1[:, 0] = 40 so silu(g) = 40 exactly in fp64 (exp(-40) vanishes next to 1), and w3[:, 0]
    sets h = 40 * w3 = (100, -3.3, 0.01, 0.001, 0.0001, 0, ...).  amax 100: e = ceil(log2(100/448))
    = -2, so the codes are e4m3 of 4h:
      400     -> midway between 384 and 416; the even mantissa wins: 384 -> 96
      -13.2   -> -13 (spacing 1 in [8, 16))                          -> -3.25
      0.04    -> 10 * 2^-8 (spacing 2^-8 in [2^-5, 2^-4))            -> 0.009765625
      0.004   -> 2 * 2^-9 (subnormal spacing 2^-9)                   -> 0.0009765625
      0.0004  -> 0 (below half the smallest subnormal)               -> 0"""
    d = F = 32
    x = np.zeros((1, d))
    x[0, 0] = 1.0
    w1 = np.zeros((F, d))
    w1[:, 0] = 40.0
    w3 = np.zeros((F, d))
    w3[:5, 0] = np.array([100.0, -3.3, 0.01, 0.001, 0.0001]) / 40.0
    y, _ = oracle.swiglu_act_quant(x, w1, w3, np.eye(d))
    expect = np.zeros(F)
    expect[:4] = [96.0, -3.25, 0.009765625, 0.0009765625]
    assert y[0].tolist() == expect.tolist()


# ---------------------------------------------------- near-tie overrides ---

def _router_inputs(logits, capacity=-1, overflow="drop", k=2, d=16):
    """Inputs whose fp64 router logits are exactly ``logits`` (W_g = I on the first E inputs)."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    cfg = synthetic.MoEConfig(name="ties", T=T, d_model=d, d_ff=8, n_experts=E, top_k=k,
                              capacity=capacity, overflow=overflow, act_dtype="f32", w_dtype="f32")
    x = np.zeros((T, d))
    x[:, :E] = logits
    wg = np.zeros((E, d))
    wg[:, :E] = np.eye(E)
    g = np.random.default_rng(0)
    return _Inp(cfg, x, wg, g.standard_normal((E, 8, d)), g.standard_normal((E, 8, d)),
                g.standard_normal((E, d, 8)))


def _refuses(inp, **kw):
    with pytest.raises(ValueError):
        oracle.forward(inp, tokens=[], **kw)


def test_override_accepts_only_the_tied_expert():
    """gap23 = 5e-5 on token 0: only expert 2 (tied with the 2nd) may replace expert 1."""
    inp = _router_inputs([[3.0, 1.00005, 1.0, 0.5],      # set near tie (gap23 = 5e-5)
                          [2.0, 1.0, 0.0, -1.0],         # clear gaps everywhere
                          [1.00005, 1.0, -1.0, -2.0]])   # slot order near tie (gap12 = 5e-5)
    base = oracle.forward(inp, tokens=[])
    assert base.routing.ids.tolist() == [[0, 1], [0, 1], [0, 1]]
    res = oracle.forward(inp, tokens=[], override={0: (0, 2), 2: (1, 0)})
    assert res.routing.ids.tolist() == [[0, 2], [0, 1], [1, 0]]
    assert abs(res.routing.G[0, 0] - 1 / (1 + math.exp(-2.0))) < 1e-15
    assert abs(res.routing.G[2, 0] - 1 / (1 + math.exp(0.00005))) < 1e-12
    for bad in ((0, 3), (3, 2), (1, 1), (2, 0), (1, 2), (0,), (0, 1, 2), (0, 4)):
        _refuses(inp, override={0: bad})
    for bad in ((0, 2), (1, 0)):
        _refuses(inp, override={1: bad})
    _refuses(inp, override={2: (1, 2)})          # order may swap, the set may not change
    assert oracle.near_tie_ranking_ok(inp.x[0, :4], (0, 2))
    assert not oracle.near_tie_ranking_ok(inp.x[0, :4], (0, 3))


def test_next_override_accepts_only_near_tie_rankings():
    inp = _router_inputs([[5.0, 4.0, 2.00005, 2.0, 1.0, 0.0],   # ranks 3/4 tied
                          [5.0, 4.0, 3.0, 2.0, 1.0, 0.0],       # clear
                          [5.0, 3.00005, 3.0, 2.0, 1.0, 0.0]],  # ranks 2/3 tied
                         capacity=4, overflow="next_best")
    base = oracle.forward(inp, tokens=[])
    assert base.routing.next_ids.tolist() == [[2, 3], [2, 3], [2, 3]]
    res = oracle.forward(inp, tokens=[], next_override={0: (3, 2)})
    assert res.routing.next_ids[0].tolist() == [3, 2]
    for bad in ((2, 4), (4, 3), (2, 2), (0, 3), (2, -1), (1, 3)):
        _refuses(inp, next_override={0: bad})
    _refuses(inp, next_override={1: (3, 2)})
    # the GPU took expert 2 into the top-2 at the set near tie: expert 1 is then ranked 3rd
    res = oracle.forward(inp, tokens=[], override={2: (0, 2)}, next_override={2: (1, 3)})
    assert res.routing.next_ids[2].tolist() == [1, 3]
    _refuses(inp, override={2: (0, 2)}, next_override={2: (2, 3)})


def test_keep_override_only_at_the_cutoff_and_counts_kept():
    """Capacity 1.  Expert 0 gets tokens 0, 1 (G 5e-5 apart) and 3 (far below): only the swap of
    the two tied tokens is accepted."""
    inp = _router_inputs([[2.0, 1.0, 0.0, -1.0],
                          [2.00025, 1.0, 0.0, -1.0],
                          [-3.0, -3.0, 2.0, 1.0],
                          [0.3, -5.0, 0.0, -5.0]], capacity=1)
    base = oracle.forward(inp, tokens=[])
    G = base.routing.G
    assert 0 < G[1, 0] - G[0, 0] < oracle.NEAR_TIE
    keep = base.keep.copy()
    assert keep[:, 0].tolist() == [False, True, True, False]
    swap = keep.copy()
    swap[0, 0], swap[1, 0] = True, False
    res = oracle.forward(inp, tokens=[], keep_override=swap)
    assert np.array_equal(res.keep, swap)
    both = keep.copy()
    both[0, 0] = True                      # two kept by a capacity-1 expert
    _refuses(inp, keep_override=both)
    far = keep.copy()
    far[3, 0], far[1, 0] = True, False     # token 3 is far below the cutoff
    _refuses(inp, keep_override=far)
    clear = keep.copy()
    clear[2, 0] = False                    # expert 2 was under capacity: no cutoff
    _refuses(inp, keep_override=clear)


def test_status_override_only_at_the_fallback_cutoff():
    """Capacity 1 with the fallback: expert 0 keeps token 2; tokens 0 and 1 (G 5e-5 apart) are
    both offered to expert 3, which has one free slot."""
    inp = _router_inputs([[3.0, 2.0, -5.0, 1.0, -5.0],
                          [3.00025, -5.0, 2.0, 1.0, -5.0],
                          [8.0, -5.0, -5.0, -5.0, 4.0]], capacity=1, overflow="next_best")
    base = oracle.forward(inp, tokens=[])
    assert base.status.tolist() == [[1, 0], [2, 0], [0, 0]]
    st = base.status.copy()
    st[0, 0], st[1, 0] = 2, 1
    res = oracle.forward(inp, tokens=[], status_override=st)
    assert res.status.tolist() == [[2, 0], [1, 0], [0, 0]] and res.final_ids[0, 0] == 3
    both = base.status.copy()
    both[0, 0] = 2                         # expert 3 would take two offers into one slot
    _refuses(inp, status_override=both)
    kept = base.status.copy()
    kept[0, 1] = 1                         # a slot kept by its top-2 expert cannot change
    _refuses(inp, status_override=kept)
    zero = base.status.copy()
    zero[1, 0] = 0
    _refuses(inp, status_override=zero)


def test_check_routing_refuses_a_wrong_expert_at_a_near_tie():
    """The GPU parity check itself: at the set near tie only the tied expert may come in."""
    import parity
    inp = _router_inputs([[3.0, 1.00005, 1.0, 0.5], [2.0, 1.0, 0.0, -1.0]])
    res = oracle.forward(inp, tokens=[])

    def run(ids):
        ids = np.asarray(ids, dtype=np.int32)
        w0 = np.array([1 / (1 + math.exp(res.logits[t, ids[t, 1]] - res.logits[t, ids[t, 0]]))
                       for t in range(2)], dtype=np.float32)
        w = np.stack([w0, np.float32(1) - w0], 1)
        return parity.check_routing(res, ids, w, res.logits.astype(np.float32), 1e-6)

    assert run([[0, 2], [0, 1]]) == {0: (0, 2)}
    for bad in ([[0, 3], [0, 1]], [[3, 2], [0, 1]], [[0, 1], [0, 2]]):
        with pytest.raises(AssertionError):
            run(bad)


# ------------------------------------------------- configs and inputs ---

# --------------------------------------------------------------- MXFP4 ---

def test_e2m1_values_from_the_format_definition():
    """OCP MX FP4 E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign."""
    t = oracle.mxfp4.E2M1_TABLE
    assert t[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert t[8:].tolist() == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(t[8]) and not np.signbit(t[0])
    # largest normal = 2^emax * (1 + 1/2) with emax = 2 (bias 1); smallest subnormal 2^(1-1) * 1/2
    assert t[7] == 2.0 ** 2 * 1.5 and t[1] == 0.5


def test_mxfp4_dequant_packing_and_block_scale():
    # byte 0x72: even element = low nibble 2 (1.0), odd element = high nibble 7 (6.0)
    packed = np.full((1, 16), 0x72, dtype=np.uint8)
    for sbyte, mul in ((127, 1.0), (130, 8.0), (120, 2.0 ** -7)):
        w = oracle.mxfp4.dequant(packed, np.array([[sbyte]], dtype=np.uint8))
        assert w.shape == (1, 32)
        assert w[0, 0::2].tolist() == [1.0 * mul] * 16 and w[0, 1::2].tolist() == [6.0 * mul] * 16
    # two blocks with their own scales; a negative code
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 16] = 0x0B                                # element 32 = code 11 = -1.5
    w = oracle.mxfp4.dequant(packed, np.array([[127, 125]], dtype=np.uint8))
    assert w[0, 32] == -1.5 / 4 and np.count_nonzero(w) == 1


def test_mxfp4_input_quantizer_against_the_oracle_decode():
    """The input generator's MXFP4 encoder, decoded by the oracle: grid values exact,
    ties to the even code, shared exponent floor(log2 amax) - 2, error within half a step."""
    X = -5
    levels = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    # block 0: every level (both signs) exactly; amax = 6 * 2^X -> floor(log2) - 2 = X
    b0 = np.concatenate([levels, -levels, levels, -levels]) * np.float32(2.0 ** X)
    # block 1: midpoints (ties) -> 0, 1, 1, 2, 2, 4, 4 and a value above 6 that saturates;
    # amax 7 * 2^X keeps the same shared exponent
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], dtype=np.float32)
    b1 = np.concatenate([mids, -mids, mids, mids]) * np.float32(2.0 ** X)
    b2 = np.zeros(32, dtype=np.float32)                                  # zero block
    w = np.stack([np.concatenate([b0, b1, b2])])
    packed, sc = synthetic.quantize_blocks_mxfp4(w)
    assert sc.tolist() == [[X + 127, X + 127, 127]]
    back = oracle.mxfp4.dequant(packed, sc)
    assert np.array_equal(back[0, :32], b0.astype(np.float64))
    expect = np.array([0, 1, 1, 2, 2, 4, 4, 6], dtype=np.float64) * 2.0 ** X
    assert np.array_equal(back[0, 32:40], expect) and np.array_equal(back[0, 40:48], -expect)
    assert np.all(back[0, 64:] == 0)
    # random weights: shared exponent and the half-step error bound
    g = np.random.default_rng(7)
    w = (g.standard_normal((6, 512)) * 0.02).astype(np.float32)
    packed, sc = synthetic.quantize_blocks_mxfp4(w)
    back = oracle.mxfp4.dequant(packed, sc)
    blk = w.reshape(6, 16, 32).astype(np.float64)
    Xb = np.floor(np.log2(np.abs(blk).max(-1))) - 2
    assert np.array_equal(sc.astype(np.int64) - 127, Xb.astype(np.int64))
    step = np.exp2(Xb)[..., None]                       # grid spacing is <= 2 * 2^X
    v = np.abs(blk) / step
    gap = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0)) * step
    err = np.abs(back.reshape(6, 16, 32) - blk)
    sat = v > 6
    assert np.all(err[~sat] <= gap[~sat] / 2 + 1e-12)
    assert np.all(err[sat] <= (np.abs(blk) - 6 * step)[sat] + 1e-12)


def test_mxfp4_layer_equals_layer_on_dequantized_weights():
    """The oracle layer on MXFP4 experts is the plain layer on their exact dequantised values."""
    cfg = synthetic.MoEConfig(name="m4", T=24, d_model=64, d_ff=96, n_experts=4, w_dtype="mxfp4",
                              wg_std=0.125, w13_std=0.05, w2_std=0.05, seed=3)
    inp = synthetic.make_inputs(cfg)
    assert tuple(inp.w1.shape) == (4, 96, 32) and tuple(inp.w1_scale.shape) == (4, 96, 2)
    assert tuple(inp.w2.shape) == (4, 64, 48) and tuple(inp.w2_scale.shape) == (4, 64, 3)
    res = oracle.forward(inp)
    deq = lambda w, s: np.stack([oracle.mxfp4.dequant(w[e].numpy(), s[e].numpy()) for e in range(4)])  # noqa: E731
    plain = _Inp(cfg.replace(w_dtype="bf16"), oracle.to_f64(inp.x), oracle.to_f64(inp.w_gate),
                 deq(inp.w1, inp.w1_scale), deq(inp.w3, inp.w3_scale), deq(inp.w2, inp.w2_scale))
    ref = oracle.forward(plain)
    assert np.array_equal(res.routing.ids, ref.routing.ids)
    assert np.max(np.abs(res.y - ref.y)) == 0.0
    # brute force on the same dequantised weights
    yb, _, _, _ = brute.layer(plain.x.tolist(), plain.w_gate.tolist(), plain.w1.tolist(),
                              plain.w3.tolist(), plain.w2.tolist(), 2)
    assert np.max(np.abs(np.array(yb) - res.y)) < 1e-12


def test_configs_shapes_and_capacity():
    c = synthetic.CONFIGS
    assert c["skewed_capacity_bf16"].capacity == 1280
    assert synthetic.capacity_from_factor(1, 2, 8) == 0      # batch-1 edge: 0.3125 -> 0 slots
    dec = c["decode_bf16"]
    assert 3 * dec.d_model * dec.d_ff * 2 == 352_321_536    # bytes of one bf16 expert
    fine = {n for n in c if n.startswith("finegrained")}
    assert all(c[n].n_experts == 8 and c[n].top_k == 2 and c[n].n_shared == 0 for n in c if n not in fine)
    # DeepSeek-V3 remark ("Mixtral 8x7B" interview page): 256 routed, 8 active, 1 shared
    assert fine and all((c[n].n_experts, c[n].top_k, c[n].n_shared) == (256, 8, 1) for n in fine)


def test_zipf_bias_frozen_and_effective():
    fit = json.load(open(os.path.join(GOLDEN, "zipf_bias_e8.json")))
    assert np.max(np.abs(np.array(fit["bias"]) - np.array(synthetic.ZIPF12_BIAS_E8))) < 1e-4
    cfg = synthetic.CONFIGS["skewed_capacity_bf16"]
    inp = synthetic.make_inputs(cfg, with_weights=False)
    r = oracle.topk_gate(oracle.router_logits(oracle.to_f64(inp.x), oracle.to_f64(inp.w_gate),
                                              oracle.to_f64(inp.router_bias)), 2)
    share = np.bincount(r.ids.ravel(), minlength=8) / r.ids.size
    assert np.max(np.abs(share - np.array(fit["target_share"]))) < 0.015


def test_inputs_are_seeded_and_prefix_consistent():
    a = synthetic.make_inputs(synthetic.CONFIGS["tiny_fp32"])
    b = synthetic.make_inputs(synthetic.CONFIGS["tiny_fp32"])
    for u, v in ((a.x, b.x), (a.w1, b.w1), (a.w2, b.w2), (a.w_gate, b.w_gate)):
        assert torch.equal(u, v)
    assert a.x.dtype == torch.float32 and a.w1.shape == (8, 256, 128) and a.w2.shape == (8, 128, 256)
    dec = synthetic.make_inputs(synthetic.CONFIGS["decode_bf16"], with_weights=False)
    pre = synthetic.make_inputs(synthetic.CONFIGS["skewed_capacity_bf16"], with_weights=False)
    assert torch.equal(dec.x, pre.x[:16])


def test_tiny_config_oracle_runs_dropless():
    inp = synthetic.make_inputs(synthetic.CONFIGS["tiny_fp32"])
    res = oracle.forward(inp)
    assert res.perm.counts.sum() == 64 * 2
    assert np.all(res.routing.ids[:, 0] != res.routing.ids[:, 1])
    assert np.isfinite(res.y).all() and res.y.shape == (64, 128)
