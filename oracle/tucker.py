"""Partial Tucker decomposition on the token and feature axes (oracle, exact path).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2), the sentences that view a layer's
cache as a third-order tensor over heads, tokens and features and apply a
partial Tucker decomposition compressing only the token and feature axes, with
the head and layer axes left intact; news article paragraph 4 (no projection
on the heads axis).

Notation.  X in R^{H x T x D}; X_h = X[h] in R^{T x D}.  Unfoldings
X_(T)[t, h*D + d] = X[h, t, d] (T x HD) and X_(D)[d, h*T + t] = X[h, t, d]
(D x HT).  Factors U_T (T x r_T), U_D (D x r_D) are leading left singular
vectors of the unfoldings; the core is G_h = U_T^T X_h U_D and the
reconstruction is X^_h = U_T G_h U_D^T.

Readings (the pages name Tucker but no solver):
* factors are eigenvectors of the Gram of each unfolding;  for the token mode
  the smaller of the two Grams is formed: the direct T x T Gram
  sum_h X_h X_h^T when T <= HD, else the dual HD x HD Gram X_(T)^T X_(T), whose
  nonzero spectrum is the same; from the dual, U_T = X_(T) V_r Lambda_r^{-1/2},
  then re-orthonormalized (Householder QR, diag R >= 0);
* eigenvalues sorted descending, ties by lower index; each factor column is
  signed so that its largest-magnitude entry (lowest index on ties) is
  positive (this changes the core's signs only, never the reconstruction);
* spectra are returned clamped at zero.
"""
from __future__ import annotations

import numpy as np


def unfold_T(X: np.ndarray) -> np.ndarray:
    H, T, D = X.shape
    return np.ascontiguousarray(X.transpose(1, 0, 2)).reshape(T, H * D)


def unfold_D(X: np.ndarray) -> np.ndarray:
    H, T, D = X.shape
    return np.ascontiguousarray(X.transpose(2, 0, 1)).reshape(D, H * T)


def gram_D(X: np.ndarray) -> np.ndarray:
    """Mode-D Gram  sum_h X_h^T X_h  (= X_(D) X_(D)^T), D x D."""
    XD = unfold_D(np.asarray(X, dtype=np.float64))
    return XD @ XD.T


def token_gram_is_dual(H: int, T: int, D: int) -> bool:
    return T > H * D


def gram_T(X: np.ndarray) -> np.ndarray:
    """Mode-T Gram actually formed: direct T x T if T <= HD, else dual HD x HD."""
    H, T, D = X.shape
    XT = unfold_T(np.asarray(X, dtype=np.float64))
    if token_gram_is_dual(H, T, D):
        return XT.T @ XT
    return XT @ XT.T


def sort_desc(w: np.ndarray) -> np.ndarray:
    """Permutation sorting w descending; equal values keep lower index first."""
    return np.argsort(-w, kind="stable")


def sign_fix(U: np.ndarray) -> np.ndarray:
    """Make each column's largest-|.| entry (lowest index on ties) positive."""
    U = np.array(U, dtype=np.float64, copy=True)
    if U.size == 0:
        return U
    idx = np.argmax(np.abs(U), axis=0)            # argmax returns the first maximum
    s = np.sign(U[idx, np.arange(U.shape[1])])
    s[s == 0] = 1.0
    return U * s


def eig_desc(G: np.ndarray):
    """Eigenpairs of a symmetric matrix, descending, sign-fixed vectors."""
    w, V = np.linalg.eigh(np.asarray(G, dtype=np.float64))
    p = sort_desc(w)
    return w[p], sign_fix(V[:, p])


def orthonormalize(U: np.ndarray) -> np.ndarray:
    """Householder thin QR, Q scaled so that diag(R) >= 0."""
    Q, R = np.linalg.qr(np.asarray(U, dtype=np.float64), mode="reduced")
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Q * s


def factors_exact(X: np.ndarray, r_T: int):
    """Exact factors: (lam_T, lam_D, U_T[:, :r_T], U_D) in fp64.

    lam_T has min(T, HD) values, lam_D has D values (both clamped >= 0);
    U_D holds all D columns.
    """
    X = np.asarray(X, dtype=np.float64)
    H, T, D = X.shape
    lam_D, U_D = eig_desc(gram_D(X))
    lam, V = eig_desc(gram_T(X))
    if token_gram_is_dual(H, T, D):
        if r_T > 0:
            if np.any(lam[:r_T] <= 0):
                raise ValueError("dual recovery needs positive eigenvalues up to r_T")
            U_T = unfold_T(X) @ (V[:, :r_T] / np.sqrt(lam[:r_T]))
            U_T = sign_fix(orthonormalize(U_T))
        else:
            U_T = np.zeros((T, 0))
    else:
        U_T = V[:, :r_T]
    return np.maximum(lam, 0.0), np.maximum(lam_D, 0.0), U_T, U_D


def core(X: np.ndarray, U_T: np.ndarray, U_D: np.ndarray) -> np.ndarray:
    """G_h = U_T^T X_h U_D for every head, H x r_T x r_D."""
    X = np.asarray(X, dtype=np.float64)
    return np.einsum("tr,htd,ds->hrs", U_T, X, U_D, optimize=True)


def reconstruct(G: np.ndarray, U_T: np.ndarray, U_D: np.ndarray) -> np.ndarray:
    """X^_h = U_T G_h U_D^T for every head, H x T x D."""
    return np.einsum("tr,hrs,ds->htd", U_T, G, U_D, optimize=True)


def hosvd_tail(lam: np.ndarray, frob2: float, r: int) -> float:
    """Energy a rank-r truncation of one mode discards: ||X||^2 - sum_{i<r} lam_i.

    The prefix sum runs sequentially from the largest value, in fp64.
    """
    s = 0.0
    for i in range(min(r, len(lam))):
        s += float(lam[i])
    return max(0.0, float(frob2) - s)
