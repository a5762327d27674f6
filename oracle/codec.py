"""End-to-end JoLT encode / decode of one K or V tensor, and a whole cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2): partial Tucker on the token and
feature axes, then a rotated low-bit residual restoring the energy that
truncation discards; one Lagrangian-dual allocation of ranks and bits per layer
group, K and V separate, under one byte budget; quality reported as relative
Frobenius reconstruction error.

Encode (readings marked R):
  U~_T = bf16(U_T[:, :r_T]), U~_D = bf16(U_D[:, :r_D])        (R: bf16 storage)
  G~_h = bf16(U~_T^T X_h U~_D)                                  (fp64, then RNE)
  R_h  = X_h - U~_T G~_h U~_D^T      (R: residual against the stored factors)
  Y_h  = fp32(R_h Q^T)               (rotation along features, rounded once)
  (m16, s16, codes) = quantize(Y, b)  (``quant``)
  with (r_T, r_D) = (0, 0) meaning no Tucker part (R = X).
Decode:
  X^_h = U~_T G~_h U~_D^T + Y^_h Q,  Y^ = m16 + code * s16  (fp64)
  then rounded to the input dtype (R: output dtype = input dtype).
Error: ||X - X^||_F / ||X||_F in fp64 on the rounded output.
"""
from __future__ import annotations

import numpy as np

from . import alloc, bf16, flash, quant, rng, rotation, tucker


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16.round_nearest(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def encode_tensor(X, U_T, U_D, choice, Q):
    """Encode one tensor with given fp64 factors (at least r_T / r_D columns)."""
    X = np.asarray(X, dtype=np.float64)
    H, T, D = X.shape
    r_T, r_D, bits = choice
    if r_T > 0:
        Ut = bf16.round_nearest(U_T[:, :r_T])
        Ud = bf16.round_nearest(U_D[:, :r_D])
        G = bf16.round_nearest(tucker.core(X, Ut, Ud))
        R = X - tucker.reconstruct(G, Ut, Ud)
    else:
        Ut = np.zeros((T, 0))
        Ud = np.zeros((D, 0))
        G = np.zeros((H, 0, 0))
        R = X
    Y = (R.reshape(-1, D) @ Q.T).astype(np.float32).reshape(H, T, D)
    m16, s16, codes = quant.quantize(Y, bits)
    return dict(shape=(H, T, D), choice=(r_T, r_D, bits), U_T=Ut, U_D=Ud, G=G,
                Y=Y, m16=m16, s16=s16, codes=codes)


def decode_exact(enc, Q) -> np.ndarray:
    """The decoded tensor in fp64, before rounding to an output dtype."""
    H, T, D = enc["shape"]
    r_T = enc["choice"][0]
    Yh = quant.dequantize(enc["m16"], enc["s16"], enc["codes"])        # [H, T, D]
    Xh = (Yh.reshape(-1, D) @ Q).reshape(H, T, D)
    if r_T > 0:
        Xh = Xh + tucker.reconstruct(enc["G"], enc["U_T"], enc["U_D"])
    return Xh


def decode_tensor(enc, Q, dtype: str) -> np.ndarray:
    return round_to(decode_exact(enc, Q), dtype)


def rel_err(X, Xh) -> float:
    X = np.asarray(X, dtype=np.float64)
    Xh = np.asarray(Xh, dtype=np.float64)
    den = float(np.sum(X * X))
    if den == 0.0:
        return 0.0 if float(np.sum(Xh * Xh)) == 0.0 else float("inf")
    return float(np.sqrt(np.sum((X - Xh) ** 2) / den))


def analyze(X, R_T: int, method: str = "exact", seed: int = 0,
            layer: int = 0, kind: int = 0, p: int = 10, q: int = 1):
    """Spectra and max-rank factors of one tensor."""
    if method == "exact":
        lam_T, lam_D, U_T, U_D = tucker.factors_exact(X, R_T)
    elif method == "flash":
        tag = rng.tensor_tag(rng.TAG_SKETCH, layer, kind)
        lam_T, lam_D, U_T, U_D = flash.factors_flash(X, R_T, seed, tag, p, q)
    else:
        raise ValueError(method)
    frob2 = float(np.sum(np.asarray(X, dtype=np.float64) ** 2))
    return dict(lam_T=lam_T, lam_D=lam_D, U_T=U_T, U_D=U_D, frob2=frob2)


def encode_cache(tensors, ratio: float, dtype: str, bits=(1, 2, 3, 4),
                 group_layers: int = 4, method: str = "exact", seed: int = 0,
                 p: int = 10, q: int = 1, step_T: int = 32, step_D: int = 16,
                 r_T_cap: int = 0):
    """Allocate and encode a cache; tensors[layer][kind] = X (fp64 values)."""
    L = len(tensors)
    H, T, D = np.asarray(tensors[0][0]).shape
    cap = r_T_cap if r_T_cap > 0 else alloc.rank_cap_T(H, T, D, ratio, step_T)
    ana = [[analyze(tensors[l][k], cap, method, seed, l, k, p, q) for k in (0, 1)]
           for l in range(L)]
    spectra = [[(a["lam_T"], a["lam_D"], a["frob2"]) for a in ana[l]] for l in range(L)]
    plan = alloc.allocate(spectra, L, H, T, D, ratio, bits, group_layers, cap,
                          step_T, step_D)
    Q = rotation.rotation(seed, D)
    encs, errs = [], []
    for l in range(L):
        row_e, row_r = [], []
        for k in (0, 1):
            ch = plan["choice"][(l // group_layers, k)]
            e = encode_tensor(tensors[l][k], ana[l][k]["U_T"], ana[l][k]["U_D"], ch, Q)
            row_e.append(e)
            row_r.append(rel_err(tensors[l][k], decode_tensor(e, Q, dtype)))
        encs.append(row_e)
        errs.append(row_r)
    return dict(plan=plan, analysis=ana, enc=encs, rel_err=errs, Q=Q)
