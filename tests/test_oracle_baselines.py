"""Pins of the oracle's comparison codecs (oracle/baselines.py), CPU only.

* The cross-layer basis is the leading left singular subspace of the group's
  feature unfoldings side by side (numpy SVD, a textbook routine), and its
  eigenvalues are their squared singular values.
* Unrounded, the cross-layer reconstruction error of the group is the tail
  of that spectrum (Eckart-Young), and r = D reconstructs exactly.
* Byte accounting and the rank that fits a budget, hand-worked.
* The unrotated quantizer's error is at most half a step per element in the
  input's own coordinates (the identity rotation), and the seeded rotation
  lowers the error on inputs with outlier channels.
"""
import numpy as np
import pytest

import kvgen
from oracle import baselines, bf16, codec, quant, rotation, tucker


def _group(H=2, T=48, D=16, layers=3, seed=5):
    return [kvgen.tensor(H, T, D, seed=seed, layer=l, kind=0, decay=0.8, rank=6).astype(np.float64)
            for l in range(layers)]


def test_basis_is_leading_singular_subspace_of_side_by_side_unfoldings():
    Xs = _group()
    r = 5
    lam, U = baselines.xl_basis(Xs, r)
    A = np.concatenate([tucker.unfold_D(X) for X in Xs], axis=1)          # D x (layers H T)
    Us, sv, _ = np.linalg.svd(A, full_matrices=False)
    np.testing.assert_allclose(lam[:len(sv)], sv ** 2, rtol=1e-10, atol=1e-10 * sv[0] ** 2)
    # same subspace (sines of the principal angles ~ 0), orthonormal columns
    P = Us[:, :r] @ Us[:, :r].T
    assert np.linalg.norm(U - P @ U, 2) < 1e-10
    np.testing.assert_allclose(U.T @ U, np.eye(r), atol=1e-12)
    # sign rule: largest-magnitude entry of each column positive
    idx = np.argmax(np.abs(U), axis=0)
    assert np.all(U[idx, np.arange(r)] > 0)


@pytest.mark.parametrize("r", [1, 4, 9])
def test_unrounded_error_is_spectrum_tail(r):
    Xs = _group()
    lam, U = baselines.xl_basis(Xs, r)
    err2 = sum(float(np.sum((X - np.einsum("htd,dr,er->hte", X, U, U)) ** 2)) for X in Xs)
    tail = float(np.sum(lam[r:]))
    assert abs(err2 - tail) <= 1e-9 * sum(float(np.sum(X * X)) for X in Xs)


def test_full_rank_is_exact_and_stored_parts_are_bf16():
    Xs = _group(D=16)
    lam, U = baselines.xl_basis(Xs, 16)
    for X in Xs:
        np.testing.assert_allclose(np.einsum("htd,dr,er->hte", X, U, U), X, atol=1e-10 * np.abs(X).max())
    Ut, C = baselines.xl_encode(Xs[0], U[:, :4])
    assert np.array_equal(Ut, bf16.round_nearest(Ut)) and np.array_equal(C, bf16.round_nearest(C))
    Xh = baselines.xl_decode(Ut, C, "bf16")
    assert np.array_equal(Xh, bf16.round_nearest(Xh))


def test_bytes_and_rank_for_budget_hand_worked():
    # 4 layers of [8, 4096, 128]: 4 * 2 * 8 * 4096 * r + 2 * 128 * r bytes
    assert baselines.xl_group_bytes(8, 4096, 128, 63, 4) == 16515072 + 16128
    # budget 4 * floor(2 * 4194304 / 2) = 16777216: r = 64 needs 16777216 + 16384
    assert baselines.xl_rank_for_budget(8, 4096, 128, 4, 2.0) == 63
    # at 3.2x: 4 * floor(2 * 4194304 / 3.2) = 10485760 -> r = 39 (10223616 + 9984), r = 40 too much
    assert baselines.xl_group_bytes(8, 4096, 128, 39, 4) == 10223616 + 9984
    assert baselines.xl_rank_for_budget(8, 4096, 128, 4, 3.2) == 39


@pytest.mark.parametrize("bits", [2, 4])
def test_unrotated_error_within_half_step(bits):
    X = kvgen.tensor(2, 40, 128, seed=3, decay=0.9, dtype="f32").astype(np.float64)
    Xh = baselines.unrotated_quant(X, bits, "f32")
    Y = X.astype(np.float32)                      # the quantizer input with Q = I
    m16, s16, codes = quant.quantize(Y, bits)
    step = np.repeat(s16.reshape(2, 40, 4, 1), 32, axis=3).reshape(2, 40, 128)
    ulp = np.spacing(np.abs(X).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(X - Xh) <= step / 2 + 2 * ulp + 1e-30)


def test_rotation_beats_unrotated_on_outlier_channels():
    X = kvgen.tensor(4, 64, 128, seed=9, decay=0.9, dtype="f32").astype(np.float64)
    Q = rotation.rotation(0, 128)
    rot = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, None, None, (0, 0, 2), Q), Q, "f32"))
    unrot = codec.rel_err(X, baselines.unrotated_quant(X, 2, "f32"))
    assert rot < 0.8 * unrot
