"""FlashJoLT factors: seeded Gaussian-sketch randomized SVD (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2), last sentence: a randomized-SVD
variant, FlashJoLT, makes compression 5-13x faster at 1024-token context with
matched quality; news article paragraph 3.  The pages name no algorithm.

Reading: the randomized range finder with subspace (power) iteration and a
direct SVD of the projected matrix, in the form of Halko, Martinsson & Tropp,
"Finding structure with randomness" (SIAM Review 2011), Algorithms 4.4 and 5.1,
applied to the token-mode unfolding A = X_(T) (T x HD):

1. sketch width l = min(R + p, T, HD), oversampling p = 10, q = 1 power step;
2. Omega (HD x l) from the counter-based normal stream of the tensor, element
   [i, j] at index i*l + j;
3. Y = A Omega, Q = qr(Y); then q times: Z = A^T Q, Q_z = qr(Z), Y = A Q_z,
   Q = qr(Y)  (every product re-orthonormalized);
4. B = Q^T A (l x HD); eigen-decompose B B^T = W Mu W^T (descending);
5. U_T = Q W[:, :R], columns sign-fixed; the Ritz values Mu (l of them) are the
   token-mode spectrum handed to the allocator.

qr is Householder thin QR with diag(R) >= 0.  The feature mode keeps its exact
Gram path: its sketch would need l = min(R_D + p, D) = D columns, whose range
is all of R^D, so the sketched and exact feature factors agree to rounding.
"""
from __future__ import annotations

import numpy as np

from . import rng
from .tucker import eig_desc, gram_D, orthonormalize, sign_fix, unfold_T


def sketch_width(R: int, rows: int, cols: int, p: int = 10) -> int:
    return min(R + p, rows, cols)


def omega(seed: int, tag: int, cols: int, ell: int) -> np.ndarray:
    return rng.normals(seed, tag, cols * ell).reshape(cols, ell)


def rsvd(A: np.ndarray, R: int, Om: np.ndarray, q: int = 1):
    """Randomized SVD of A with a given sketch; returns (Ritz values, U[:, :R])."""
    A = np.asarray(A, dtype=np.float64)
    Q = orthonormalize(A @ Om)
    for _ in range(q):
        Qz = orthonormalize(A.T @ Q)
        Q = orthonormalize(A @ Qz)
    B = Q.T @ A
    mu, W = eig_desc(B @ B.T)
    U = sign_fix(Q @ W[:, :R])
    return np.maximum(mu, 0.0), U


def factors_flash(X: np.ndarray, R_T: int, seed: int, tag: int,
                  p: int = 10, q: int = 1):
    """FlashJoLT factors: (mu_T, lam_D, U_T[:, :R_T], U_D)."""
    X = np.asarray(X, dtype=np.float64)
    H, T, D = X.shape
    A = unfold_T(X)
    ell = sketch_width(R_T, T, H * D, p)
    mu, U_T = rsvd(A, R_T, omega(seed, tag, H * D, ell), q)
    lam_D, U_D = eig_desc(gram_D(X))
    return mu, np.maximum(lam_D, 0.0), U_T, U_D
