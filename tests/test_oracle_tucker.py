"""Pins for the oracle's partial Tucker (exact path): Grams, spectra, factors,
core, reconstruction, the HOSVD bound and the Eckart-Young special case."""
import itertools

import numpy as np
import pytest

import kvgen
from oracle import tucker


def _x(H, T, D, seed=0):
    return np.random.default_rng(seed).standard_normal((H, T, D)) * \
        np.linspace(0.2, 3.0, D)[None, None, :]


def test_unfoldings_by_definition():
    X = _x(2, 3, 4)
    XT, XD = tucker.unfold_T(X), tucker.unfold_D(X)
    for h, t, d in itertools.product(range(2), range(3), range(4)):
        assert XT[t, h * 4 + d] == X[h, t, d]
        assert XD[d, h * 3 + t] == X[h, t, d]


@pytest.mark.parametrize("shape", [(2, 16, 4), (2, 6, 4), (3, 8, 8)])
def test_gram_traces_symmetry_psd(shape):
    X = _x(*shape)
    f2 = float(np.sum(X * X))
    for G in (tucker.gram_D(X), tucker.gram_T(X)):
        assert np.allclose(G, G.T, atol=1e-12 * f2)
        assert abs(np.trace(G) - f2) <= 1e-12 * f2
        assert np.linalg.eigvalsh(G).min() >= -1e-12 * f2


def test_gram_by_loops():
    X = _x(2, 3, 2, seed=4)
    GD = np.zeros((2, 2))
    for d, e in itertools.product(range(2), range(2)):
        GD[d, e] = sum(X[h, t, d] * X[h, t, e] for h in range(2) for t in range(3))
    np.testing.assert_allclose(tucker.gram_D(X), GD, rtol=1e-14)
    # T=3 <= HD=4: direct token Gram
    GT = np.zeros((3, 3))
    for t, u in itertools.product(range(3), range(3)):
        GT[t, u] = sum(X[h, t, d] * X[h, u, d] for h in range(2) for d in range(2))
    np.testing.assert_allclose(tucker.gram_T(X), GT, rtol=1e-14)


@pytest.mark.parametrize("shape", [(2, 16, 4), (2, 6, 4)])
def test_spectra_are_squared_singular_values(shape):
    X = _x(*shape, seed=7)
    H, T, D = shape
    lam_T, lam_D, U_T, U_D = tucker.factors_exact(X, min(T, H * D))
    sT = np.linalg.svd(tucker.unfold_T(X), compute_uv=False) ** 2
    sD = np.linalg.svd(tucker.unfold_D(X), compute_uv=False) ** 2
    n = min(T, H * D)
    assert len(lam_T) == n and len(lam_D) == D
    np.testing.assert_allclose(lam_T, sT[:n], rtol=1e-12, atol=1e-12 * sT[0])
    np.testing.assert_allclose(lam_D, sD, rtol=1e-12, atol=1e-12 * sD[0])
    assert np.all(np.diff(lam_T) <= 0) and np.all(np.diff(lam_D) <= 0)


def test_dual_and_direct_agree():
    X = _x(2, 16, 4, seed=3)                      # T = 16 > HD = 8: dual
    lam_T, _, U_T, _ = tucker.factors_exact(X, 8)
    XT = tucker.unfold_T(X)
    w, V = np.linalg.eigh(XT @ XT.T)              # the direct 16 x 16 Gram
    w = w[::-1]
    np.testing.assert_allclose(lam_T, w[:8], rtol=1e-12, atol=1e-10)
    # recovered U_T columns are eigenvectors of the direct Gram
    GT = XT @ XT.T
    np.testing.assert_allclose(GT @ U_T, U_T * lam_T[None, :8], atol=1e-9 * w[0])


@pytest.mark.parametrize("shape", [(2, 16, 4), (2, 6, 4), (1, 12, 6)])
def test_factors_orthonormal_and_signed(shape):
    X = _x(*shape, seed=9)
    H, T, D = shape
    r = min(T, H * D)
    _, _, U_T, U_D = tucker.factors_exact(X, r)
    for U in (U_T, U_D):
        np.testing.assert_allclose(U.T @ U, np.eye(U.shape[1]), atol=1e-12)
        idx = np.argmax(np.abs(U), axis=0)
        assert np.all(U[idx, np.arange(U.shape[1])] > 0)


@pytest.mark.parametrize("shape", [(2, 16, 4), (2, 6, 4)])
def test_full_rank_is_exact(shape):
    X = _x(*shape, seed=5)
    H, T, D = shape
    r = min(T, H * D)
    _, _, U_T, U_D = tucker.factors_exact(X, r)
    Xh = tucker.reconstruct(tucker.core(X, U_T, U_D), U_T, U_D)
    assert np.linalg.norm(X - Xh) <= 1e-12 * np.linalg.norm(X)


def test_core_and_reconstruct_by_loops():
    r = np.random.default_rng(1)
    X = r.standard_normal((2, 3, 4))
    Ut = r.standard_normal((3, 2))
    Ud = r.standard_normal((4, 3))
    G = tucker.core(X, Ut, Ud)
    for h, a, b in itertools.product(range(2), range(2), range(3)):
        v = sum(Ut[t, a] * X[h, t, d] * Ud[d, b] for t in range(3) for d in range(4))
        assert abs(G[h, a, b] - v) < 1e-12
    Xr = tucker.reconstruct(G, Ut, Ud)
    for h, t, d in itertools.product(range(2), range(3), range(4)):
        v = sum(Ut[t, a] * G[h, a, b] * Ud[d, b] for a in range(2) for b in range(3))
        assert abs(Xr[h, t, d] - v) < 1e-10


@pytest.mark.parametrize("rT,rD", [(4, 2), (8, 3), (1, 1), (12, 4)])
def test_hosvd_bound_and_energy_identity(rT, rD):
    X = kvgen.tensor(3, 24, 8, seed=2, decay=0.7, dtype="f32").astype(np.float64)
    lam_T, lam_D, U_T, U_D = tucker.factors_exact(X, rT)
    G = tucker.core(X, U_T, U_D[:, :rD])
    Xh = tucker.reconstruct(G, U_T, U_D[:, :rD])
    f2 = float(np.sum(X * X))
    err2 = float(np.sum((X - Xh) ** 2))
    bound = tucker.hosvd_tail(lam_T, f2, rT) + tucker.hosvd_tail(lam_D, f2, rD)
    assert err2 <= bound * (1 + 1e-12)
    assert abs(err2 - (f2 - float(np.sum(G * G)))) <= 1e-10 * f2


def test_single_head_is_eckart_young():
    X = _x(1, 12, 6, seed=8)
    for r in (1, 2, 4):
        _, _, U_T, U_D = tucker.factors_exact(X, r)
        Xh = tucker.reconstruct(tucker.core(X, U_T, U_D[:, :r]), U_T, U_D[:, :r])
        U, s, Vt = np.linalg.svd(X[0])
        best = (U[:, :r] * s[:r]) @ Vt[:r]
        np.testing.assert_allclose(Xh[0], best, atol=1e-12 * s[0])


def test_head_axis_is_not_factored():
    # the head axis stays intact: permuting heads permutes the core's heads
    X = _x(3, 10, 4, seed=6)
    _, _, U_T, U_D = tucker.factors_exact(X, 5)
    G = tucker.core(X, U_T, U_D[:, :3])
    Gp = tucker.core(X[[2, 0, 1]], U_T, U_D[:, :3])
    np.testing.assert_allclose(Gp, G[[2, 0, 1]], atol=1e-12)
    lam_T2, lam_D2, _, _ = tucker.factors_exact(X[[2, 0, 1]], 5)
    lam_T, lam_D, _, _ = tucker.factors_exact(X, 5)
    np.testing.assert_allclose(lam_T2, lam_T, rtol=1e-12)
    np.testing.assert_allclose(lam_D2, lam_D, rtol=1e-12)
