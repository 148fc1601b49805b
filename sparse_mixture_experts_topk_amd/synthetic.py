"""Seeded synthetic inputs for the sparse top-k MoE feed-forward layer.

This module only draws and stores inputs: it holds none of the layer's
arithmetic (no routing, no gating, no expert FFN).  Both the fp64 CPU oracle
(``oracle/``) and the HIP path receive exactly the tensors produced here.

Shapes follow the Mixtral 8x7B MoE layer described on the pages
("How Mixtral 8x7B uses mixture of experts", section "The architecture in one
diagram"; "Mixtral" study notes, section "MoE Layer", classes MixtralMoE and
MixtralExpert): 8 experts, top-2 routing, d_model = 4096 and a SwiGLU expert
of hidden width 14336.  The fine-grained configs follow the DeepSeek-V3 remark
on the "Mixtral 8x7B" interview page (section on how MoE design changed since
Mixtral): 256 routed experts, 8 active per token, plus one shared expert that
every token passes through.  The page gives no expert width; the reading
here keeps d_model = 4096 and takes "smaller experts" as d_ff = 2048 for
routed and shared experts alike.

Reading of the distribution notation: ``N(0, 1/n)`` is a variance (std
n**-0.5), ``N(0, 0.02)`` is a standard deviation.  Every tensor has its own
``numpy.random.SeedSequence`` child stream (order: x, w_gate, w1, w3, w2) and
each expert of w1/w3/w2 its own grandchild stream, so one expert can be drawn
on its own and the draw is independent of thread scheduling.  Values are drawn
in float32 and rounded on the host (round-to-nearest-even) to the storage
dtype before either side sees them.

fp8 expert weights (long-context config): each output channel (row of the
nn.Linear ``[out, in]`` weight) gets an fp32 scale ``s = absmax / 448`` and
codes ``e4m3(w / s)``; the cast is torch's ``float8_e4m3fn`` conversion
(round-to-nearest-even).  An all-zero row gets ``s = 1``.

MXFP4 expert weights (4-bit decode config) follow the conversion of the OCP
Microscaling Formats specification v1.0: per row and block of 32 consecutive
input elements, a shared exponent ``X = floor(log2(amax)) - 2`` (2 is the
largest E2M1 exponent), stored as the byte ``X + 127``, and elements
``w / 2^X`` rounded to the nearest FP4 E2M1 value (ties to the even code),
saturating at +-6.  An all-zero block gets ``X = 0``.  Two codes per byte,
the even element in the low nibble.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

# Router bias that makes top-2 expert load follow Zipf(s=1.2) for iid N(0,1)
# logits (expert 0 heaviest).  Derived by tests/golden/fit_zipf_bias.py, which
# uses only the oracle's top-2 selection; frozen here so that every run and
# both sides see the same constants.
ZIPF12_BIAS_E8 = (1.7688, 0.4414, 0.0618, -0.1817, -0.3475, -0.4783, -0.5894, -0.6750)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                      # tokens (batch * seq_len, flattened)
    d_model: int
    d_ff: int
    n_experts: int = 8          # routed experts
    top_k: int = 2
    n_shared: int = 0           # 0 or 1 shared expert, stored after the routed ones
    capacity: int = -1          # -1: dropless; else slots per expert (0 drops all)
    overflow: str = "drop"      # over-capacity assignments: "drop" | "next_best" (fallback round)
    act_dtype: str = "bf16"     # x, w_gate, y: "f32" | "bf16"
    w_dtype: str = "bf16"       # w1/w3/w2: "f32" | "bf16" | "fp8_e4m3" | "mxfp4"
    x_std: float = 1.0
    wg_std: float = 1.0 / 64.0
    w13_std: float = 0.02
    w2_std: float = 0.02
    router_bias: Optional[str] = None   # None | "zipf1.2"
    seed: int = 0
    description: str = ""

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


def capacity_from_factor(T: int, top_k: int, n_experts: int, factor_num: int = 5,
                         factor_den: int = 4) -> int:
    """floor(cf * T * k / E) with cf = factor_num/factor_den, in exact integers."""
    return (factor_num * T * top_k) // (factor_den * n_experts)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny_fp32": MoEConfig(
        name="tiny_fp32", T=64, d_model=128, d_ff=256, act_dtype="f32", w_dtype="f32",
        x_std=1.0, wg_std=128 ** -0.5, w13_std=128 ** -0.5, w2_std=256 ** -0.5,
        description="tiny MoE layer, fp32, T=64 d=128 F=256 E=8 top-2 dropless"),
    "decode_bf16": MoEConfig(
        name="decode_bf16", T=16, d_model=4096, d_ff=14336,
        description="Mixtral-shape decode, bf16, 16 tokens (batch 16 x seq 1), dropless"),
    "prefill_bf16": MoEConfig(
        name="prefill_bf16", T=8192, d_model=4096, d_ff=14336,
        description="Mixtral-shape prefill, bf16, 8192 tokens (4 x 2048), dropless"),
    "skewed_capacity_bf16": MoEConfig(
        name="skewed_capacity_bf16", T=4096, d_model=4096, d_ff=14336,
        capacity=capacity_from_factor(4096, 2, 8), router_bias="zipf1.2",
        description="Zipf(1.2)-skewed routing, capacity floor(1.25*T*2/E)=1280, bf16"),
    "skewed_fallback_bf16": MoEConfig(
        name="skewed_fallback_bf16", T=4096, d_model=4096, d_ff=14336,
        capacity=capacity_from_factor(4096, 2, 8), router_bias="zipf1.2", overflow="next_best",
        description="as skewed_capacity_bf16, over-capacity assignments re-offered to the "
                    "next-best expert"),
    "decode_mxfp4": MoEConfig(
        name="decode_mxfp4", T=16, d_model=4096, d_ff=14336, w_dtype="mxfp4",
        description="Mixtral-shape decode, 16 tokens, MXFP4 (E2M1 + E8M0 per 32) experts, "
                    "bf16 activations and router, dropless"),
    "finegrained_decode_bf16": MoEConfig(
        name="finegrained_decode_bf16", T=16, d_model=4096, d_ff=2048, n_experts=256, top_k=8,
        n_shared=1,
        description="fine-grained decode, bf16, 16 tokens, 256 routed experts top-8 + 1 shared "
                    "(d_ff 2048), dropless"),
    "finegrained_prefill_bf16": MoEConfig(
        name="finegrained_prefill_bf16", T=8192, d_model=4096, d_ff=2048, n_experts=256, top_k=8,
        n_shared=1,
        description="fine-grained prefill, bf16, 8192 tokens, 256 routed experts top-8 + 1 shared "
                    "(d_ff 2048), dropless"),
    "longctx_fp8": MoEConfig(
        name="longctx_fp8", T=16384, d_model=4096, d_ff=14336, w_dtype="fp8_e4m3",
        description="long-context prefill, 16384 tokens, fp8 e4m3 experts with "
                    "per-output-channel fp32 scales, bf16 activations"),
}


@dataclasses.dataclass
class MoEInputs:
    """Host (CPU) tensors in their storage dtype.

    x [T, d], w_gate [E, d] in the activation dtype; router_bias [E] fp32 or
    None; w1, w3 [E, F, d] and w2 [E, d, F] in the weight dtype (fp8 configs:
    torch.float8_e4m3fn codes) with w*_scale [E, F] / [E, d] fp32 per output
    channel for fp8; MXFP4: uint8 [E, F, d/2] / [E, d, F/2] packed codes with
    uint8 [E, F, d/32] / [E, d, F/32] block scales (None otherwise).
    """
    cfg: MoEConfig
    x: torch.Tensor
    w_gate: torch.Tensor
    router_bias: Optional[torch.Tensor]
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    w1_scale: Optional[torch.Tensor] = None
    w3_scale: Optional[torch.Tensor] = None
    w2_scale: Optional[torch.Tensor] = None


_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(5)   # x, w_gate, w1, w3, w2


def _normal(ss: np.random.SeedSequence, n: int, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _store(a32: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a32)
    return t.to(_TORCH_DTYPE[dtype]) if dtype in _TORCH_DTYPE else t


def quantize_rows_e4m3(w32: torch.Tensor):
    """Per-row (output channel) fp8 e4m3 codes with fp32 scale absmax/448."""
    amax = w32.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (w32 / scale.unsqueeze(-1)).to(torch.float8_e4m3fn)
    return q, scale


# Midpoints between consecutive E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def quantize_blocks_mxfp4(w32: np.ndarray):
    """[rows, cols] fp32 -> (packed E2M1 codes [rows, cols/2] uint8, E8M0 scales [rows, cols/32] uint8)."""
    rows, cols = w32.shape
    blk = w32.reshape(rows, cols // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    X = np.clip(X, -127, 127).astype(np.int32)
    v = np.abs(blk) * np.exp2(-X.astype(np.float32))[..., None]       # exact power-of-two scaling
    idx = np.searchsorted(_E2M1_MIDS, v, side="left")                  # level index 0..7
    tie = (idx < 7) & (v == _E2M1_MIDS[np.minimum(idx, 6)])
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)                 # ties -> even code
    codes = (idx | np.where(blk < 0, 8, 0)).astype(np.uint8).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def _expert_matrix(parent: np.random.SeedSequence, E: int, rows: int, cols: int, std: float,
                   w_dtype: str, threads: int, experts=None):
    children = parent.spawn(E)
    ids = list(range(E)) if experts is None else list(experts)

    def one(e):
        a = _normal(children[e], rows * cols, std).reshape(rows, cols)
        t = torch.from_numpy(a)
        if w_dtype == "fp8_e4m3":
            return quantize_rows_e4m3(t)
        if w_dtype == "mxfp4":
            q, sc = quantize_blocks_mxfp4(a)
            return (torch.from_numpy(q), torch.from_numpy(sc))
        return (t.to(_TORCH_DTYPE[w_dtype]), None)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        parts = list(ex.map(one, ids))
    w = torch.stack([p[0] for p in parts])
    s = torch.stack([p[1] for p in parts]) if w_dtype in ("fp8_e4m3", "mxfp4") else None
    return w, s


def make_inputs(cfg: MoEConfig, threads: int = 8, with_weights: bool = True) -> MoEInputs:
    """Draw the seeded inputs of ``cfg`` on the host."""
    T, d, F, E = cfg.T, cfg.d_model, cfg.d_ff, cfg.n_experts
    s_x, s_g, s_1, s_3, s_2 = _streams(cfg.seed)
    x = _store(_normal(s_x, T * d, cfg.x_std).reshape(T, d), cfg.act_dtype)
    w_gate = _store(_normal(s_g, E * d, cfg.wg_std).reshape(E, d), cfg.act_dtype)
    bias = None
    if cfg.router_bias == "zipf1.2":
        if E != 8:
            raise ValueError("the frozen Zipf(1.2) bias is defined for 8 experts")
        bias = torch.tensor(ZIPF12_BIAS_E8, dtype=torch.float32)
    elif cfg.router_bias is not None:
        raise ValueError(f"unknown router_bias {cfg.router_bias!r}")
    if not with_weights:
        z = torch.empty(0)
        return MoEInputs(cfg, x, w_gate, bias, z, z, z)
    EW = E + cfg.n_shared                                # expert weights incl. the shared one
    w1, s1 = _expert_matrix(s_1, EW, F, d, cfg.w13_std, cfg.w_dtype, threads)
    w3, s3 = _expert_matrix(s_3, EW, F, d, cfg.w13_std, cfg.w_dtype, threads)
    w2, s2 = _expert_matrix(s_2, EW, d, F, cfg.w2_std, cfg.w_dtype, threads)
    return MoEInputs(cfg, x, w_gate, bias, w1, w3, w2, s1, s3, s2)


def unquantized_weights(cfg: MoEConfig, threads: int = 8):
    """The fp32 draws that an fp8 config's weights are quantized from (report-only use)."""
    _, _, s_1, s_3, s_2 = _streams(cfg.seed)
    E, d, F = cfg.n_experts, cfg.d_model, cfg.d_ff
    out = []
    for ss, rows, cols, std in ((s_1, F, d, cfg.w13_std), (s_3, F, d, cfg.w13_std),
                                (s_2, d, F, cfg.w2_std)):
        w, _ = _expert_matrix(ss, E, rows, cols, std, "f32" if cfg.w_dtype in ("fp8_e4m3", "mxfp4") else cfg.w_dtype,
                              threads)
        out.append(w)
    return tuple(out)
