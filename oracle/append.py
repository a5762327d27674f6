"""Incremental encode of tokens appended to an encoded tensor (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages are silent on tokens that arrive after a tensor has been encoded
(generation appends one token per step).  Reading ("folding-in" of new rows
into fixed factors, as latent semantic indexing adds documents without
recomputing the SVD: Berry, Dumais & O'Brien, SIAM Review 1995): the base
record's stored feature factor U~_D and core G~ stay fixed; for the new
tokens X_new [H, dT, D] the token-factor rows are the least-squares solution

    U_new = argmin_U || X_new,(T) - U W ||_F,   W = [G~_h U~_D^T]_h  (r_T x H D),

stored as bf16; the residual X_new - U~_new G~_h U~_D^T is rotated and
quantized exactly as in ``codec.encode_tensor``.  The appended tokens form a
record of their own (dT tokens, the base's choice, copies of U~_D and G~),
which decodes like any record.
"""
from __future__ import annotations

import numpy as np

from . import bf16, quant, tucker


def stacked_w(G: np.ndarray, Ud: np.ndarray) -> np.ndarray:
    """W = [G_0 Ud^T | G_1 Ud^T | ...]  (r_T x H D)."""
    H = G.shape[0]
    return np.concatenate([G[h] @ Ud.T for h in range(H)], axis=1)


def fold_in_rows(X_new, G, Ud) -> np.ndarray:
    """The least-squares token-factor rows of the new tokens (fp64, unrounded)."""
    W = stacked_w(np.asarray(G, dtype=np.float64), np.asarray(Ud, dtype=np.float64))
    XT = tucker.unfold_T(np.asarray(X_new, dtype=np.float64))          # dT x H D
    sol, *_ = np.linalg.lstsq(W.T, XT.T, rcond=None)                    # r_T x dT
    return sol.T


def append_encode(X_new, base: dict, Q) -> dict:
    """Encode appended tokens against a base encode (``codec.encode_tensor``
    result with r_T > 0): same fields as an encode of the new tokens."""
    X_new = np.asarray(X_new, dtype=np.float64)
    H, dT, D = X_new.shape
    r_T, r_D, bits = base["choice"]
    G, Ud = base["G"], base["U_D"]
    Ut = bf16.round_nearest(fold_in_rows(X_new, G, Ud))
    R = X_new - tucker.reconstruct(G, Ut, Ud)
    Y = (R.reshape(-1, D) @ Q.T).astype(np.float32).reshape(H, dT, D)
    m16, s16, codes = quant.quantize(Y, bits)
    return dict(shape=(H, dT, D), choice=(r_T, r_D, bits), U_T=Ut, U_D=Ud, G=G,
                Y=Y, m16=m16, s16=s16, codes=codes)
