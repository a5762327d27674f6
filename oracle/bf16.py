"""bfloat16 rounding (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

bf16 keeps the fp32 sign and 8-bit exponent and 7 explicit fraction bits
(8 significant bits).  Values are carried as float64 arrays holding exactly
representable bf16 numbers.

Readings (the pages fix no storage precision):
* factors, core and output tensors are stored in bf16 with round-to-nearest,
  ties to even, taken directly from the exact (fp64) value;
* the quantizer's per-group offset is rounded toward -inf and its step toward
  +inf, so the grid always covers the group (the invariant that every rotated
  residual lies within half a step of its code).
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float(np.ldexp(255.0, 120))          # (2 - 2^-7) * 2^127
_QEXP_MIN = -133                                # subnormal quantum 2^-133


def round_nearest(x) -> np.ndarray:
    """Round to the nearest bf16, ties to even, from the exact value (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                          # ax = m * 2^e, 0.5 <= m < 1
    qexp = np.maximum(e - 8, _QEXP_MIN)          # quantum of an 8-bit significand
    r = np.rint(np.ldexp(ax, -qexp))             # np.rint: ties to even
    out = np.ldexp(r, qexp)
    out = np.where(out > BF16_MAX, np.inf, out)
    out = np.where(np.isnan(x), np.nan, out)
    return np.copysign(out, x)


def _f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)


def _bits_to_f64(hi16: np.ndarray) -> np.ndarray:
    return (hi16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_down(x32) -> np.ndarray:
    """Largest bf16 <= x for fp32 input x (round toward -inf)."""
    b = _f32_bits(x32)
    hi = b >> np.uint32(16)
    inexact = (b & np.uint32(0xFFFF)) != 0
    neg = (b >> np.uint32(31)) == 1
    # truncation rounds toward zero; a negative inexact value needs one more
    # unit of magnitude to reach -inf direction.
    hi = np.where(inexact & neg, hi + np.uint32(1), hi)
    return _bits_to_f64(hi)


def round_up(x32) -> np.ndarray:
    """Smallest bf16 >= x for fp32 input x (round toward +inf)."""
    b = _f32_bits(x32)
    hi = b >> np.uint32(16)
    inexact = (b & np.uint32(0xFFFF)) != 0
    pos = (b >> np.uint32(31)) == 0
    hi = np.where(inexact & pos, hi + np.uint32(1), hi)
    return _bits_to_f64(hi)


def to_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16-representable values."""
    b = _f32_bits(np.asarray(x, dtype=np.float64).astype(np.float32))
    return (b >> np.uint32(16)).astype(np.uint16)


def from_bits(bits) -> np.ndarray:
    return _bits_to_f64(np.asarray(bits, dtype=np.uint16))
