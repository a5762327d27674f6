"""Comparison codecs at matched bytes (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2), the sentences naming the two
families the method is set against (per-head or cross-layer low-rank
factorizations, and per-entry quantization); news article on JoLT,
paragraph 3 (at 2x, JoLT's error is about ten times smaller than that of
cross-layer SVD or of 4-bit quantization).  The pages give neither baseline's definition;
these are the readings:

* b-bit quantization: the codec's own residual path with no Tucker part,
  choice (0, 0, b): groups of 32 features, bf16 (offset, step), b-bit codes,
  either after the seeded rotation Q (rotated) or with Q = I (unrotated).
  Bytes: the record size of ``alloc.blob_bytes`` at (0, 0, b).
* cross-layer SVD: one feature basis U (D x r) per unit of the allocation
  (a layer group and a kind), shared by the group's layers: the leading r
  eigenvectors of the feature Grams summed over the group's tensors, i.e. the
  leading left singular vectors of the feature unfoldings of all the group's
  tensors side by side (sign rule of ``tucker.sign_fix``).  Each tensor
  stores its coefficients C_h = bf16(X_h U~) (T x r per head) and the group
  stores U~ = bf16(U) once; the reconstruction is X^_h = C_h U~^T, rounded to
  the input dtype.  Bytes: 2 H T r per tensor + 2 D r per group.
"""
from __future__ import annotations

import numpy as np

from . import bf16, codec, tucker


def unrotated_quant(X, bits: int, dtype: str):
    """Decode of the no-Tucker record with the identity as rotation."""
    D = np.asarray(X).shape[2]
    Q = np.eye(D)
    enc = codec.encode_tensor(X, None, None, (0, 0, bits), Q)
    return codec.decode_tensor(enc, Q, dtype)


def xl_basis(tensors, r: int):
    """Shared feature basis of a group: (eigenvalues of the summed feature
    Gram, descending, clamped >= 0; its leading r eigenvectors, sign-fixed)."""
    G = sum(tucker.gram_D(np.asarray(X, dtype=np.float64)) for X in tensors)
    lam, V = tucker.eig_desc(G)
    return np.maximum(lam, 0.0), V[:, :r]


def xl_encode(X, U):
    """(U~, C): the stored basis and the stored per-head coefficients."""
    Ut = bf16.round_nearest(U)
    C = bf16.round_nearest(np.einsum("htd,dr->htr", np.asarray(X, dtype=np.float64), Ut, optimize=True))
    return Ut, C


def xl_decode(Ut, C, dtype: str):
    return codec.round_to(np.einsum("htr,dr->htd", C, Ut, optimize=True), dtype)


def xl_group_bytes(H: int, T: int, D: int, r: int, layers: int) -> int:
    return layers * 2 * H * T * r + 2 * D * r


def xl_rank_for_budget(H: int, T: int, D: int, layers: int, ratio: float) -> int:
    """Largest r whose group bytes fit the group's share of the budget
    (floor(2 N / ratio) bytes per tensor, N = H T D)."""
    budget = int(np.floor(2.0 * H * T * D / ratio)) * layers
    r = 0
    while r < D and xl_group_bytes(H, T, D, r + 1, layers) <= budget:
        r += 1
    return r
