"""fp8 e4m3 encoding and block quantisation for the oracle (test infrastructure).

The pages say nothing about fp8 (they discuss 4-bit/8-bit loaders only: "How
Mixtral 8x7B uses mixture of experts", section "Quantization asymmetry").  The
long-context configuration fixes fp8 e4m3 expert weights; the format is the
OCP 8-bit floating point "E4M3" encoding, written here from its definition:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* normal values 2**(E-7) * (1 + M/8) for E in 1..15, except E=15, M=7 which
  is NaN (there is no infinity), so the largest finite magnitude is 448;
* subnormals (E = 0): 2**-6 * M/8, i.e. multiples of 2**-9.

Encoding rounds to nearest, ties to even mantissa.  Inputs here never exceed
448 in magnitude after scaling (checked), so no saturation rule is needed.

Activation block quantisation (the reading used for fp8 MFMA): per row and per
block of 32 consecutive elements along the contraction dimension, the scale is
the power of two ``2**e`` with ``e = ceil(log2(amax / 448))`` (``amax / 448``
taken in fp32, round-to-nearest), clamped to [-127, 127]; an all-zero block
gets ``e = 0``.  Elements are ``e4m3(v * 2**-e)`` -- the product is exact, so
there is a single rounding.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    normal = np.ldexp(1.0 + M / 8.0, (E - 7).astype(np.int64))
    sub = np.ldexp(M / 8.0, -6)
    mag = np.where(E == 0, sub, normal)
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def _finite_table():
    codes = np.arange(128, dtype=np.uint8)            # non-negative codes
    vals = e4m3_decode(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]                    # ascending magnitudes 0 .. 448


_POS_CODES, _POS_VALS = _finite_table()


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float64 values with |v| <= 448 -> uint8 codes, round to nearest, ties to even.

    Implemented as a search over the 127 finite non-negative code values: the
    nearest representable magnitude wins, and on an exact tie the code with
    an even mantissa (even code, since the mantissa is the low bits) wins.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3_encode expects finite |v| <= 448")
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(_POS_VALS[hi] == a, hi, idx)               # exact hits
    code = _POS_CODES[idx].astype(np.uint8)
    neg = (v < 0) | ((v == 0) & np.signbit(v))
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def block_scale_exponent(amax32: np.ndarray) -> np.ndarray:
    """e = ceil(log2(fp32(amax / 448))), clamped to [-127, 127]; 0 for amax == 0."""
    amax32 = np.asarray(amax32, dtype=np.float32)
    r = (amax32 / np.float32(E4M3_MAX)).astype(np.float32)       # one fp32 rounding
    m, ex = np.frexp(r.astype(np.float64))                       # r = m * 2**ex, m in [0.5, 1)
    e = np.where(m == 0.5, ex - 1, ex)                           # exact powers of two
    e = np.where(amax32 == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int32)


def block_quantize(a: np.ndarray, block: int = MX_BLOCK):
    """Quantise rows of ``a`` (values exactly representable in fp32) per block of ``block``.

    Returns (codes uint8 [R, C], exponents int32 [R, C // block], dequantised float64 [R, C]).
    """
    a32 = np.asarray(a, dtype=np.float32)
    R, C = a32.shape
    if C % block:
        raise ValueError("row length must be a multiple of the block size")
    blocks = a32.reshape(R, C // block, block)
    amax = np.abs(blocks).max(axis=-1)
    e = block_scale_exponent(amax)
    scaled = np.ldexp(blocks.astype(np.float64), -e[..., None].astype(np.int64))
    codes = e4m3_encode(scaled)
    deq = np.ldexp(e4m3_decode(codes), e[..., None].astype(np.int64))
    return codes.reshape(R, C), e, deq.reshape(R, C)
