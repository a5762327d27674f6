"""Helpers for the GPU parity tests: device transfer, record parsing (the
library's documented record layout), subspace angles."""
from __future__ import annotations

import numpy as np
import torch

D = 128


def a256(n: int) -> int:
    return (n + 255) // 256 * 256


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def parse_blob(blob: torch.Tensor, H: int, T: int, choice):
    """Sections of a record (host copies): U_T, U_D, G as fp64, m16/s16 [H,T,4], packed codes."""
    r_T, r_D, b = choice
    raw = blob.cpu().numpy()
    groups = H * T * D // 32
    ut = 256
    ud = ut + a256(2 * T * r_T)
    g = ud + a256(2 * D * r_D)
    sc = g + a256(2 * H * r_T * r_D)
    cd = sc + a256(4 * groups)

    def bf(off, n, shape):
        return bf16_bits_to_f64(raw[off:off + 2 * n].view(np.uint16)).reshape(shape)

    scales = raw[sc:sc + 4 * groups].view(np.uint16).reshape(H, T, 4, 2)
    return dict(
        header=raw[:64].view(np.uint32),
        U_T=bf(ut, T * r_T, (T, r_T)), U_D=bf(ud, D * r_D, (D, r_D)),
        G=bf(g, H * r_T * r_D, (H, r_T, r_D)),
        m16=bf16_bits_to_f64(scales[..., 0]), s16=bf16_bits_to_f64(scales[..., 1]),
        packed=raw[cd:cd + 4 * b * groups].reshape(H, T, 4, 4 * b),
    )


def max_sine(U: np.ndarray, V: np.ndarray) -> float:
    Qu, _ = np.linalg.qr(U)
    Qv, _ = np.linalg.qr(V)
    return float(np.linalg.norm(Qu - Qv @ (Qv.T @ Qu), 2))


def resolvable_cuts(lam: np.ndarray, rmax: int, n: int):
    """Cuts k <= rmax whose relative gap (lam_k - lam_{k+1}) / lam_1 clears the
    fp32 resolution 1e3 * sqrt(n) * 2^-24 (Davis-Kahan)."""
    thr = 1e3 * np.sqrt(n) * 2.0 ** -24
    out = []
    for k in range(1, min(rmax, len(lam) - 1) + 1):
        if (lam[k - 1] - lam[k]) / lam[0] >= thr:
            out.append(k)
    return out


def check_bf16_rounding(got: np.ndarray, exact: np.ndarray, abs_terms: np.ndarray, gamma: float,
                        max_frac: float = 0.05):
    """bf16 values computed in fp32 arithmetic vs the fp64 exact value rounded.

    Where the two roundings differ, the stored value may be off the exact one
    by at most half a bf16 ulp plus gamma * abs_terms (the fp32 accumulation
    error bound from the sum of |terms|).
    """
    from oracle import bf16
    want = bf16.round_nearest(exact)
    mism = got != want
    assert mism.mean() <= max_frac, mism.mean()
    if mism.any():
        g, e, t = got[mism], exact[mism], abs_terms[mism]
        half_ulp = np.spacing(np.maximum(np.abs(g), np.abs(e)).astype(np.float32)).astype(np.float64) * 2 ** 15
        excess = np.abs(g - e) - half_ulp
        assert np.all(excess <= gamma * t + 1e-30), float(np.max(excess / (t + 1e-30)))
    return float(mism.mean())
