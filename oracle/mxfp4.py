"""OCP Microscaling FP4 (MXFP4) weights for the oracle -- TEST INFRASTRUCTURE ONLY.

Format (OCP "Microscaling Formats (MX)" specification v1.0, FP4 E2M1 element
type with an E8M0 shared scale per block of 32 elements):

* element: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0
  is subnormal (0.5 * m), otherwise 2^(e-1) * (1 + m/2): magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6;
* scale: one unsigned byte per 32 consecutive elements along the
  contraction dimension of a weight row, value 2^(byte - 127);
* packing: two elements per byte, the even-indexed element in the low nibble.

Used for the "4-bit expert weights" of the decode path: the pages keep the
router in bf16 and quantise only the experts to 4 bits ("How Mixtral 8x7B
uses mixture of experts", section "Quantization asymmetry"; the NF4 and AWQ
loaders of the other pages are third-party formats).  Activations stay bf16,
so the layer computes with the exactly dequantised weights.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def e2m1_value(code: int) -> float:
    """Value of one 4-bit code, from the bit fields."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def unpack(packed: np.ndarray) -> np.ndarray:
    """[..., n/2] bytes -> [..., n] codes (even element from the low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Weights in float64: element value times 2^(scale byte - 127) of its 32-element block."""
    codes = unpack(packed)
    vals = E2M1_TABLE[codes]
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return vals * np.repeat(sc, BLOCK, axis=-1)
