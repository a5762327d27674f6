"""Pins for the seeded Haar rotation Q."""
import numpy as np
import pytest

from oracle import rng, rotation


def _gram_schmidt(A):
    """Classical Gram-Schmidt with one re-orthogonalization pass, column by column."""
    n = A.shape[1]
    Q = np.zeros_like(A)
    for j in range(n):
        v = A[:, j].copy()
        for _ in range(2):
            for i in range(j):
                v -= (Q[:, i] @ v) * Q[:, i]
        Q[:, j] = v / np.linalg.norm(v)
    return Q


@pytest.mark.parametrize("D,seed", [(8, 0), (32, 3), (128, 0)])
def test_rotation_is_gram_schmidt_of_seeded_gaussian(D, seed):
    # the QR factor with positive diag(R) equals Gram-Schmidt on A's columns
    A = rng.normals(seed, rng.TAG_ROTATION, D * D).reshape(D, D)
    Q = rotation.rotation(seed, D)
    np.testing.assert_allclose(Q, _gram_schmidt(A), atol=1e-11)
    # A = Q R with R upper triangular, positive diagonal
    R = Q.T @ A
    assert np.abs(np.tril(R, -1)).max() < 1e-11 * np.abs(R).max()
    assert np.all(np.diag(R) > 0)


def test_orthogonal_and_norm_preserving():
    Q = rotation.rotation(0, 128)
    np.testing.assert_allclose(Q.T @ Q, np.eye(128), atol=1e-13)
    r = np.random.default_rng(0).standard_normal((50, 128))
    np.testing.assert_allclose(np.linalg.norm(r @ Q.T, axis=1), np.linalg.norm(r, axis=1),
                               rtol=1e-13)


def test_haar_statistics():
    # entries of a Haar orthogonal D x D matrix have mean 0 and variance 1/D;
    # over many seeds the first entry's distribution matches that
    D = 16
    v = np.array([rotation.rotation(s, D)[0, 0] for s in range(400)])
    assert abs(v.mean()) < 0.05
    assert abs(v.var() * D - 1.0) < 0.2
    # the determinant is +1 or -1 with both signs occurring (no sign bias)
    dets = [np.linalg.det(rotation.rotation(s, D)) for s in range(40)]
    assert all(abs(abs(d) - 1) < 1e-10 for d in dets)
    assert any(d > 0 for d in dets) and any(d < 0 for d in dets)
