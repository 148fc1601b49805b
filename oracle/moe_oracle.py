"""Plain fp64 CPU oracle of the sparse top-k MoE feed-forward layer (top-2 Mixtral form
and the general form of step 8).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code, table or helper with the HIP path and never takes a value from it.

What it computes, step by step, with the passage each step follows:

1. Router logits ``x . W_g^T (+ b)`` -- "Mixtral" study notes, section "MoE
   Layer" (the router is a linear map from d_model to one logit per expert,
   without a bias term); the gate equation on "Mixtral and Mixture-of-Experts,
   Explained", section "How it works".  The additive per-expert bias exists only for the skewed-routing
   workload (added after the dot product).
2. Top-2 by logit, largest first; equal logits go to the lower expert index.
3. Gate weights ``G(x) = Softmax(TopK(x . W_g))`` with every non-selected
   logit set to -inf ("Mixtral and Mixture-of-Experts, Explained", "How it
   works"), so the two kept weights are a softmax over just the two kept
   logits ("Mixtral 8x7B" interview article, "Step 2", worked example).
4. Optional capacity: per expert, its assignments ranked by gate weight
   (descending), ties to the lower token index; the first ``capacity`` are
   kept, the rest dropped and contribute nothing ("How Mixtral 8x7B uses
   mixture of experts", section "Routing without auxiliary loss",
   capacity-limited dispatch).
4b. Optional overflow fallback (same section: tokens over capacity are
   handed to a fallback, most often the token's next-best expert, and the
   dispatch sketch collects them in an overflow buffer).  Reading: an assignment dropped
   in step 4 moves to the best-ranked expert outside the token's top-2 --
   the 3rd-ranked one, or, when both of the token's slots were dropped, the
   3rd-ranked for slot 0 and the 4th-ranked for slot 1 -- keeping its gate
   weight.  Each expert takes such candidates into the slots step 4 left
   free (capacity minus what it kept), ranked by the same key; the rest stay
   dropped.  One round only.
5. Grouping by expert: per-expert counts (the ``bincount`` of the top-2 ids,
   same page, expert activation heatmap listing), exclusive offsets, rows of
   one expert in ascending (token, slot) order.
6. Each kept (token, expert): SwiGLU ``w2(silu(x w1^T) * (x w3^T))`` with
   ``silu(z) = z * sigmoid(z)`` and no biases ("Mixtral" study notes,
   MixtralExpert and section "SwiGLU Experts").
7. ``y = sum_i G(x)_i * Expert_i(x)`` over kept slots; zero when nothing is
   kept ("Mixtral and Mixture-of-Experts, Explained", "How it works"; the
   study notes' MoE layer starts from an all-zero output of x's shape and
   adds each expert's weighted contribution).
8. General top-k and a shared expert (the DeepSeek-V3 remark on "Mixtral 8x7B"
   interview page: many routed experts, several active per token, plus a
   shared one).  Reading: k experts by logit with the same gate (softmax
   over the k kept logits); an optional shared expert, stored after the E
   routed ones, processes every token with weight 1 and no capacity limit.

Every input is converted exactly to float64 from its stored bf16 / fp32 /
fp8-code-times-scale / MXFP4-code-times-block-scale value (``oracle/mxfp4.py``;
MXFP4 experts keep bf16 activations); all arithmetic is float64.  For fp8 expert weights
the computation also includes the declared activation quantisation (see
``oracle/fp8.py``): x and h are block-quantised per row and per 32-element
block before the two contractions (``fp8_act_quant=False`` leaves it out, for
the report-only comparison against plain dequantised weights).  The pages
print no fp8 values; the emulation is pinned by its definition (grid,
exponent rule, nearest rounding, blocking axis) and a hand-worked block.

Near ties.  Where the fp32 arithmetic of a GPU router and the fp64 logits
here may order two experts differently (logit gap below ``NEAR_TIE``),
``forward`` can take the GPU's decision instead, but only a decision that is
a correct top-k ranking up to such near ties (``near_tie_ranking_ok``), and
capacity / fallback marks that differ only at a cutoff near tie and keep
every expert's count.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional

import numpy as np
import torch

from . import fp8 as _fp8
from . import mxfp4 as _mxfp4

# Assignments whose deciding gap is below this are "near ties": the decision is
# not fixed by the arithmetic precision of either side (exemption threshold).
NEAR_TIE = 1e-4


def near_tie_ranking_ok(row_logits: np.ndarray, ranked) -> bool:
    """Is ``ranked`` (distinct expert ids in the order a router ranked them: ranks 1..m)
    the exact top-m ranking of ``row_logits`` up to near ties?

    True when the ids are distinct and in range, no expert left out has a logit
    NEAR_TIE or more above one ranked, and no ranked expert has a logit NEAR_TIE
    or more above one ranked before it.  With gaps of at least NEAR_TIE around
    rank m and between the ranked experts this admits only the exact ranking
    (logit descending, ties to the lower index)."""
    ranked = [int(v) for v in ranked]
    E = len(row_logits)
    if len(set(ranked)) != len(ranked) or any(v < 0 or v >= E for v in ranked):
        return False
    if not ranked:
        return True
    lv = np.asarray(row_logits, dtype=np.float64)
    sel = lv[ranked]
    rest = np.delete(lv, ranked)
    if rest.size and rest.max() - sel.min() >= NEAR_TIE:
        return False
    for i in range(1, len(ranked)):
        if sel[i] - sel[:i].min() >= NEAR_TIE:
            return False
    return True


def to_f64(t) -> np.ndarray:
    """Exact conversion of a stored tensor (fp32 / bf16 / fp64 / numpy) to float64."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    if t.dtype == torch.float8_e4m3fn:
        return _fp8.e4m3_decode(t.view(torch.uint8).numpy())
    return t.detach().to(torch.float64).cpu().numpy()


def dequant_weight(w, scale, w_dtype: str = "") -> np.ndarray:
    """fp8 codes times the per-output-channel fp32 scale; MXFP4 codes times their
    block scales; plain conversion otherwise."""
    if w_dtype == "mxfp4":
        return _mxfp4.dequant(w.numpy() if hasattr(w, "numpy") else w,
                              scale.numpy() if hasattr(scale, "numpy") else scale)
    wf = to_f64(w)
    if scale is None:
        return wf
    return wf * to_f64(scale)[..., :, None]


# ---------------------------------------------------------------- routing ---

def router_logits(x: np.ndarray, w_gate: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * W_g[e, i] (+ b[e]); fp64."""
    logits = x @ w_gate.T
    if bias is not None:
        logits = logits + bias[None, :]
    return logits


@dataclasses.dataclass
class Routing:
    ids: np.ndarray        # [T, k] int64, slot 0 = the larger logit
    G: np.ndarray          # [T, k] float64 gate weights
    gap12: np.ndarray      # [T] smallest gap between consecutive ranks 1..k (slot order)
    gap23: np.ndarray      # [T] logit(k-th) - logit(k+1-th): the selected set (inf when E == k)
    next_ids: np.ndarray   # [T, 2] int64: experts ranked k+1 and k+2 (-1 when E is smaller)
    gap34: np.ndarray      # [T] logit(k+1-th) - logit(k+2-th)  (inf when absent)
    gap45: np.ndarray      # [T] logit(k+2-th) - logit(k+3-th)  (inf when absent)


def topk_gate(logits: np.ndarray, k: int = 2) -> Routing:
    """Top-k by (logit descending, expert index ascending), then softmax over the kept logits."""
    T, E = logits.shape
    # A stable sort of the negated logits keeps equal logits in index order.
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k]
    kept = np.take_along_axis(logits, ids, axis=1)
    # Softmax over the full row with non-selected logits set to -inf.
    masked = np.full_like(logits, -np.inf)
    np.put_along_axis(masked, ids, kept, axis=1)
    m = masked.max(axis=1, keepdims=True)
    ex = np.exp(masked - m)                       # exp(-inf) = 0 exactly
    full = ex / ex.sum(axis=1, keepdims=True)
    G = np.take_along_axis(full, ids, axis=1)
    srt = np.take_along_axis(logits, order, axis=1)
    gap12 = (srt[:, :k - 1] - srt[:, 1:k]).min(axis=1) if k > 1 else np.full(T, np.inf)
    gap23 = srt[:, k - 1] - srt[:, k] if E > k else np.full(T, np.inf)
    nxt = np.full((T, 2), -1, dtype=np.int64)
    for j in range(2):
        if E > k + j:
            nxt[:, j] = order[:, k + j]
    gap34 = srt[:, k] - srt[:, k + 1] if E > k + 1 else np.full(T, np.inf)
    gap45 = srt[:, k + 1] - srt[:, k + 2] if E > k + 2 else np.full(T, np.inf)
    return Routing(ids.astype(np.int64), G, gap12, gap23, nxt, gap34, gap45)


def capacity_select(ids: np.ndarray, G: np.ndarray, n_experts: int, capacity: int):
    """Keep, per expert, the ``capacity`` assignments with the largest G (ties: lower token).

    Returns (keep [T, k] bool, cutoff [E] float64: the smallest kept G of an
    over-capacity expert, NaN when nothing was dropped).
    """
    T, k = ids.shape
    keep = np.ones((T, k), dtype=bool)
    cutoff = np.full(n_experts, np.nan)
    if capacity < 0:
        return keep, cutoff
    tok = np.repeat(np.arange(T), k).reshape(T, k)
    for e in range(n_experts):
        sel = ids == e
        t_e, g_e = tok[sel], G[sel]                    # row-major: ascending t*k+slot
        if len(t_e) <= capacity:
            continue
        rank = np.lexsort((t_e, -g_e))                 # primary -G, secondary token
        flat = np.flatnonzero(sel.ravel())             # positions t*k+slot, token-ascending
        dropped = flat[rank[capacity:]]
        keep.ravel()[dropped] = False
        cutoff[e] = g_e[rank[capacity - 1]] if capacity > 0 else np.inf
    return keep, cutoff


def fallback_targets(keep: np.ndarray, next_ids: np.ndarray) -> np.ndarray:
    """Expert each dropped assignment falls back to (-1: kept, or no such expert).

    One dropped slot goes to the 3rd-ranked expert; when both slots of a token
    are dropped, slot 0 goes to the 3rd-ranked and slot 1 to the 4th-ranked."""
    T, k = keep.shape
    target = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        dropped = [s for s in range(k) if not keep[t, s]]
        for j, s in enumerate(dropped):
            target[t, s] = next_ids[t, j]
    return target


def fallback_select(ids: np.ndarray, next_ids: np.ndarray, G: np.ndarray, keep: np.ndarray,
                    n_experts: int, capacity: int):
    """Second capacity round for the assignments ``capacity_select`` dropped.

    Returns (final_ids [T, k], status [T, k] uint8 -- 0 kept by its top-2
    expert, 1 dropped, 2 kept by its fallback expert -- and cutoff [E]: the
    smallest G an expert took in this round when candidates were left over,
    +inf when it had no free slot for them, NaN otherwise)."""
    T, k = ids.shape
    final = ids.copy()
    status = np.where(keep, 0, 1).astype(np.uint8)
    cutoff = np.full(n_experts, np.nan)
    target = fallback_targets(keep, next_ids)
    tok = np.repeat(np.arange(T), k).reshape(T, k)
    for e in range(n_experts):
        free = capacity - int(np.count_nonzero((ids == e) & keep))
        sel = target == e
        t_e, g_e = tok[sel], G[sel]
        rank = np.lexsort((t_e, -g_e))                 # primary -G, secondary token
        flat = np.flatnonzero(sel.ravel())
        taken = flat[rank[:free]]
        status.ravel()[taken] = 2
        final.ravel()[taken] = e
        if len(t_e) > free:
            cutoff[e] = g_e[rank[free - 1]] if free > 0 else np.inf
    return final, status, cutoff


@dataclasses.dataclass
class Permutation:
    counts: np.ndarray       # [E] int64 kept assignments per expert
    offsets: np.ndarray      # [E+1] exclusive prefix sum
    perm_src: np.ndarray     # [N_kept] t*k + slot of each permuted row
    slot_to_row: np.ndarray  # [T*k] row, or -1 when dropped


def permutation(ids: np.ndarray, keep: np.ndarray, n_experts: int, n_shared: int = 0) -> Permutation:
    """Rows grouped by expert, tokens ascending.  A shared expert (index n_experts) takes
    every token after the routed rows; its rows' source (slot) is T*k + token, and
    slot_to_row covers those T slots after the T*k routed ones."""
    T, k = ids.shape
    flat_ids = ids.ravel()
    flat_keep = keep.ravel()
    counts = np.array([np.count_nonzero((flat_ids == e) & flat_keep) for e in range(n_experts)] +
                      [T] * n_shared, dtype=np.int64)
    offsets = np.zeros(n_experts + n_shared + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm_src = np.empty(int(offsets[-1]), dtype=np.int64)
    slot_to_row = np.full(T * (k + n_shared), -1, dtype=np.int64)
    for e in range(n_experts):
        src = np.flatnonzero((flat_ids == e) & flat_keep)   # ascending t*k+slot
        rows = offsets[e] + np.arange(len(src))
        perm_src[rows] = src
        slot_to_row[src] = rows
    if n_shared:
        perm_src[offsets[n_experts]:] = T * k + np.arange(T)
        slot_to_row[T * k:] = offsets[n_experts] + np.arange(T)
    return Permutation(counts, offsets, perm_src, slot_to_row)


# ------------------------------------------------------------ expert FFN ---

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(xr: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray):
    """w2(silu(x w1^T) * (x w3^T)) for rows xr; nn.Linear [out, in] weights.

    Returns (output rows, intermediate h)."""
    h = silu(xr @ w1.T) * (xr @ w3.T)
    return h @ w2.T, h


def swiglu_act_quant(xr: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray):
    """SwiGLU with the declared fp8 activation quantisation of x and h (fp8 weights).

    x (exact in fp32) and h (rounded to fp32 first: the quantisation decision is
    taken in fp32) are block-quantised per row and 32-element block along the
    contraction.  Returns (output rows, dequantised h)."""
    _, _, xq = _fp8.block_quantize(xr.astype(np.float32))
    h = silu(xq @ w1.T) * (xq @ w3.T)
    _, _, hq = _fp8.block_quantize(h.astype(np.float32))
    return hq @ w2.T, hq


# ----------------------------------------------------------- full layer ---

@dataclasses.dataclass
class OracleResult:
    logits: np.ndarray
    routing: Routing
    keep: np.ndarray                    # [T, k] final: the assignment contributes
    cutoff: np.ndarray
    perm: Permutation
    y: np.ndarray                       # [T, d] (rows not in ``tokens`` are NaN)
    y_perm: Optional[np.ndarray] = None # [N_kept, d] (rows not computed are NaN)
    h: Optional[np.ndarray] = None      # [N_kept, F] when requested
    status: Optional[np.ndarray] = None     # [T, k] 0 kept / 1 dropped / 2 kept by the fallback
    final_ids: Optional[np.ndarray] = None  # [T, k] expert that processes each slot
    cutoff2: Optional[np.ndarray] = None    # [E] cutoff of the fallback round
    keep1: Optional[np.ndarray] = None      # [T, k] kept by the capacity round (before any fallback)


def forward(inputs, tokens: Optional[Iterable[int]] = None,
            override: Optional[Dict[int, Iterable[int]]] = None,
            keep_override: Optional[np.ndarray] = None,
            want_h: bool = False,
            next_override: Optional[Dict[int, Iterable[int]]] = None,
            status_override: Optional[np.ndarray] = None,
            fp8_act_quant: bool = True) -> OracleResult:
    """Run the layer on ``inputs`` (a MoEInputs of host tensors).

    tokens: compute the expert FFN / output only for these tokens (all
        routing, capacity and grouping steps still cover every token).
    override: {token: (e0, .., e_{k-1})} routing decisions to use instead of
        the oracle's own, accepted only when they are a top-k ranking of the
        token's fp64 logits up to near ties (``near_tie_ranking_ok``): only an
        expert tied within NEAR_TIE with the k-th may replace it, and slots may
        swap only where their logits are that close.  G is recomputed from
        the oracle's fp64 logits of the given experts.
    keep_override: a [T, k] keep mask replacing the capacity decision; it must
        agree with the oracle's own except for assignments whose G lies
        within NEAR_TIE of their expert's cutoff, and keep min(load, capacity)
        assignments of every expert.
    next_override: {token: (n0, n1)} experts ranked k+1 and k+2 to use instead
        of the oracle's, accepted only when the token's k experts followed by
        them are a ranking up to near ties (-1 where E is too small, as in the
        oracle's own).
    status_override: a [T, k] fallback-round status (0/1/2) replacing the
        oracle's, accepted only where it differs at a fallback cutoff near
        tie (G within NEAR_TIE of the target expert's cutoff) and every
        expert takes min(offers, free slots) in the round.
    fp8_act_quant: for fp8 expert weights, include the declared activation
        quantisation (the default); False gives the plain SwiGLU on the
        dequantised weights (report-only comparisons).
    """
    cfg = inputs.cfg
    E, k = cfg.n_experts, cfg.top_k
    S = getattr(cfg, "n_shared", 0)
    x = to_f64(inputs.x)
    bias = None if inputs.router_bias is None else to_f64(inputs.router_bias)
    logits = router_logits(x, to_f64(inputs.w_gate), bias)
    r = topk_gate(logits, k)
    if override:
        for t, pair in override.items():
            pair = tuple(int(v) for v in pair)
            if tuple(r.ids[t]) == pair:
                continue
            if len(pair) != k or not near_tie_ranking_ok(logits[t], pair):
                raise ValueError(f"override {pair} of token {t} is not a top-{k} ranking up to "
                                 f"near ties (oracle: {tuple(r.ids[t])})")
            kl = logits[t, list(pair)]
            ex = np.exp(kl - kl.max())
            r.ids[t] = pair
            r.G[t] = ex / ex.sum()
            # ranks k+1 and k+2 follow the experts actually taken
            rest = [e for e in np.argsort(-logits[t], kind="stable") if e not in pair]
            r.next_ids[t] = (rest + [-1, -1])[:2]
    keep, cutoff = capacity_select(r.ids, r.G, E, cfg.capacity)
    if keep_override is not None:
        keep_override = np.asarray(keep_override, dtype=bool)
        if keep_override.shape != keep.shape:
            raise ValueError("keep override has the wrong shape")
        diff = np.argwhere(keep_override != keep)
        for t, s in diff:
            e = r.ids[t, s]
            if not (abs(r.G[t, s] - cutoff[e]) < NEAR_TIE):
                raise ValueError(f"keep override at ({t},{s}) is not at the capacity cutoff")
        for e in np.unique(r.ids[tuple(diff.T)]) if len(diff) else []:
            load = int(np.count_nonzero(r.ids == e))
            if int(np.count_nonzero((r.ids == e) & keep_override)) != min(load, cfg.capacity):
                raise ValueError(f"keep override changes the kept count of expert {e}")
        keep = keep_override
    keep1 = keep
    status = final_ids = cutoff2 = None
    if cfg.capacity >= 0 and getattr(cfg, "overflow", "drop") == "next_best":
        if next_override:
            n_next = min(2, E - k)
            for t, pair in next_override.items():
                pair = tuple(int(v) for v in pair)
                if tuple(r.next_ids[t]) == pair:
                    continue
                ok = len(pair) == 2 and all(v >= 0 for v in pair[:n_next]) and \
                    all(v == -1 for v in pair[n_next:]) and \
                    near_tie_ranking_ok(logits[t], tuple(r.ids[t]) + pair[:n_next])
                if not ok:
                    raise ValueError(f"next-expert override {pair} of token {t} is not a ranking "
                                     f"up to near ties (oracle: {tuple(r.next_ids[t])})")
                r.next_ids[t] = pair
        final_ids, status, cutoff2 = fallback_select(r.ids, r.next_ids, r.G, keep, E, cfg.capacity)
        if status_override is not None:
            status_override = np.asarray(status_override, dtype=np.uint8)
            if status_override.shape != status.shape:
                raise ValueError("status override has the wrong shape")
            target = fallback_targets(keep, r.next_ids)
            diff = np.argwhere(status_override != status)
            for t, s_ in diff:
                e = target[t, s_]
                if status[t, s_] == 0 or status_override[t, s_] not in (1, 2) or e < 0 or \
                        not abs(r.G[t, s_] - cutoff2[e]) < NEAR_TIE:
                    raise ValueError(f"status override at ({t},{s_}) is not at a fallback cutoff")
            for e in np.unique(target[tuple(diff.T)]) if len(diff) else []:
                offers = target == e
                free = cfg.capacity - int(np.count_nonzero((r.ids == e) & keep))
                if int(np.count_nonzero(offers & (status_override == 2))) != \
                        min(int(np.count_nonzero(offers)), free):
                    raise ValueError(f"status override changes what expert {e} takes in the "
                                     "fallback round")
            status = status_override
            final_ids = np.where(status == 2, target, r.ids)
        keep = status != 1
        perm = permutation(final_ids, keep, E, S)
    else:
        perm = permutation(r.ids, keep, E, S)

    T, d = x.shape
    want = np.arange(T) if tokens is None else np.unique(np.asarray(list(tokens), dtype=np.int64))
    want_mask = np.zeros(T, dtype=bool)
    want_mask[want] = True
    n_rows = int(perm.offsets[-1])
    y_perm = np.full((n_rows, d), np.nan)
    h_all = np.full((n_rows, cfg.d_ff), np.nan) if want_h else None
    fp8 = cfg.w_dtype == "fp8_e4m3"
    scaled = cfg.w_dtype in ("fp8_e4m3", "mxfp4")
    T_k = T * k

    def token_of(src):
        return np.where(src < T_k, src // k, src - T_k)

    for e in range(E + S):
        rows = np.arange(perm.offsets[e], perm.offsets[e + 1])
        rows = rows[want_mask[token_of(perm.perm_src[rows])]]
        if len(rows) == 0:
            continue
        xr = x[token_of(perm.perm_src[rows])]
        w1 = dequant_weight(inputs.w1[e], inputs.w1_scale[e] if scaled else None, cfg.w_dtype)
        w3 = dequant_weight(inputs.w3[e], inputs.w3_scale[e] if scaled else None, cfg.w_dtype)
        w2 = dequant_weight(inputs.w2[e], inputs.w2_scale[e] if scaled else None, cfg.w_dtype)
        ffn = swiglu_act_quant if fp8 and fp8_act_quant else swiglu
        y_perm[rows], h = ffn(xr, w1, w3, w2)
        if want_h:
            h_all[rows] = h
        del w1, w3, w2
    y = np.full((T, d), np.nan)
    y[want] = 0.0
    for t in want:
        for s in range(k):
            row = perm.slot_to_row[t * k + s]
            if row >= 0:
                y[t] += r.G[t, s] * y_perm[row]
        if S:
            y[t] += y_perm[perm.offsets[E] + t]      # shared expert, weight 1
    return OracleResult(logits, r, keep, cutoff, perm, y, y_perm, h_all, status, final_ids, cutoff2,
                        keep1)


def near_tie_tokens(res: OracleResult) -> np.ndarray:
    """Tokens whose top-k set (gap23) or slot order (gap12) is a near tie."""
    return np.flatnonzero((res.routing.gap23 < NEAR_TIE) | (res.routing.gap12 < NEAR_TIE))


def near_tie_next_tokens(res: OracleResult) -> np.ndarray:
    """Tokens whose 3rd/4th-ranked experts (the fallback targets) are a near tie."""
    r = res.routing
    return np.flatnonzero(np.minimum(np.minimum(r.gap23, r.gap34), r.gap45) < NEAR_TIE)
