"""Low-bit group quantization of the rotated residual (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2), the method sentence (the
residual is rotated by a random orthogonal matrix, then quantized to few
bits); news article paragraph 4 (the rotation makes the quantization error close to independent
and uniform).  Bit-widths b in {1, 2, 3, 4}, groups of 32.

Readings (the pages give no quantizer):
* a group is 32 consecutive rotated features of one (head, token) vector;
* asymmetric min-max uniform grid, per group, in IEEE fp32, in this order:
    mn, mx = min, max of the group (exact)
    m16 = bf16 rounded toward -inf of mn
    L = 2^b - 1
    s32 = (mx - m16) / L           fp32 subtract, then fp32 divide
    s16 = bf16 rounded toward +inf of s32
    code = 0 if s16 == 0, else clamp(rint((y - m16) / s16), 0, L)
  with rint = round half to even and a correctly rounded fp32 divide;
  the group stores (m16, s16) as two bf16;
* dequantization is  y^ = m16 + code * s16;
* packing: a group's 32 codes form a 32*b-bit little-endian bit stream:
  code k occupies stream bits [k*b, (k+1)*b) (its least significant bit
  first) and stream bit j is bit (j mod 8) of byte j // 8, so a group takes
  exactly 4*b bytes.
"""
from __future__ import annotations

import numpy as np

from . import bf16

GROUP = 32


def quantize(Y32: np.ndarray, bits: int):
    """Quantize rows of fp32 values, groups of 32 along the last axis.

    Returns (m16, s16, codes): m16 and s16 have shape [..., D/32] (fp64
    holding bf16 values), codes has shape [..., D/32, 32] (uint8).
    """
    Y32 = np.asarray(Y32, dtype=np.float32)
    if Y32.shape[-1] % GROUP:
        raise ValueError("feature size must be a multiple of 32")
    g = Y32.reshape(Y32.shape[:-1] + (Y32.shape[-1] // GROUP, GROUP))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    m16 = bf16.round_down(mn).astype(np.float32)       # exact: bf16 fits fp32
    L = np.float32(2 ** bits - 1)
    s32 = (mx - m16) / L                                # fp32 ops, RNE
    s16 = bf16.round_up(s32).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - m16[..., None]) / s16[..., None]       # fp32 subtract, divide
    q = np.clip(np.rint(t), np.float32(0), L)           # ties to even
    q = np.where(s16[..., None] == 0, np.float32(0), q)
    return m16.astype(np.float64), s16.astype(np.float64), q.astype(np.uint8)


def dequantize(m16: np.ndarray, s16: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """y^ = m16 + code * s16 in fp64; returns [..., D]."""
    y = m16[..., None] + codes.astype(np.float64) * s16[..., None]
    return y.reshape(y.shape[:-2] + (-1,))


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """[..., 32] codes -> [..., 4*bits] bytes (LSB-first bit stream)."""
    codes = np.asarray(codes, dtype=np.uint8)
    shifts = np.arange(bits, dtype=np.uint8)
    stream = (codes[..., :, None] >> shifts) & np.uint8(1)      # [..., 32, b]
    stream = stream.reshape(codes.shape[:-1] + (GROUP * bits,))
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack(packed: np.ndarray, bits: int) -> np.ndarray:
    """[..., 4*bits] bytes -> [..., 32] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(packed, axis=-1, bitorder="little")
    stream = stream.reshape(packed.shape[:-1] + (GROUP, bits)).astype(np.uint8)
    weights = (np.uint8(1) << np.arange(bits, dtype=np.uint8))
    return (stream * weights).sum(axis=-1).astype(np.uint8)
