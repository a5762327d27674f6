"""Pins for the oracle's FlashJoLT randomized SVD."""
import numpy as np
import pytest

import kvgen
from oracle import flash, rng, tucker


def _sines(U, V):
    """Largest principal-angle sine between the column spaces of U and V."""
    Qu, _ = np.linalg.qr(U)
    Qv, _ = np.linalg.qr(V)
    # sin of the largest angle = ||(I - Qv Qv^T) Qu||_2 (accurate near zero)
    return float(np.linalg.norm(Qu - Qv @ (Qv.T @ Qu), 2))


def test_omega_indexing():
    Om = flash.omega(3, 77, 5, 4)
    z = rng.normals(3, 77, 20)
    for i in range(5):
        for j in range(4):
            assert Om[i, j] == z[i * 4 + j]


def test_sketch_width():
    assert flash.sketch_width(256, 1024, 1024) == 266
    assert flash.sketch_width(160, 32768, 1024) == 170
    assert flash.sketch_width(60, 64, 1024) == 64


def test_exactly_low_rank_recovered():
    r = np.random.default_rng(0)
    H, T, D, k = 4, 64, 32, 12
    A = np.linalg.qr(r.standard_normal((T, k)))[0]
    B = np.linalg.qr(r.standard_normal((D, k)))[0]
    s = 10.0 * 0.8 ** np.arange(k)
    X = np.stack([(A * (s * r.standard_normal(k))) @ B.T for _ in range(H)])
    mu, _, U, _ = flash.factors_flash(X, 20, seed=1, tag=5)      # l = 30 > k
    lam, _, Ue, _ = tucker.factors_exact(X, k)
    assert _sines(U[:, :k], Ue[:, :k]) < 1e-10
    np.testing.assert_allclose(mu[:k], lam[:k], rtol=1e-10)
    assert np.all(mu[k:] < 1e-18 * mu[0])


def test_full_width_sketch_equals_exact():
    X = kvgen.tensor(2, 48, 32, seed=3, decay=0.8, dtype="f32").astype(np.float64)
    H, T, D = X.shape
    # l = min(R + p, T, HD) = T: the sketch spans everything
    mu, lam_D, U, _ = flash.factors_flash(X, 40, seed=0, tag=9)
    lam, lam_D2, Ue, _ = tucker.factors_exact(X, 40)
    np.testing.assert_allclose(mu, lam[:48], rtol=1e-9, atol=1e-9 * lam[0])
    np.testing.assert_array_equal(lam_D, lam_D2)
    gaps = (lam[:39] - lam[1:40]) / lam[0]
    for kcut in range(1, 40):
        if gaps[kcut - 1] > 1e-6:
            assert _sines(U[:, :kcut], Ue[:, :kcut]) < 1e-7


def test_power_iteration_captures_near_optimal_energy():
    X = kvgen.tensor(8, 256, 128, seed=4, decay=0.9, dtype="f32").astype(np.float64)
    A = tucker.unfold_T(X)
    lam, _, _, _ = tucker.factors_exact(X, 1)
    f2 = float(np.sum(A * A))
    R = 64
    ell = flash.sketch_width(R, A.shape[0], A.shape[1])
    Om = flash.omega(0, 1, A.shape[1], ell)
    tails = []
    for q in (0, 1):
        _, U = flash.rsvd(A, R, Om, q)
        tails.append(f2 - float(np.sum((U.T @ A) ** 2)))
    best = f2 - float(np.sum(lam[:R]))
    assert best <= tails[1] <= tails[0]
    assert tails[1] <= 1.5 * best
