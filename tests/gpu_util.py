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


# ---------------------------------------------------------------------------
# Row-sampled parity at full size: the oracle's arithmetic applied to chosen
# (head, token) rows of a GPU record, so that caches far too large for the
# oracle as a whole are still checked element by element on a sample.

def sample_rows(H: int, T: int, n: int, seed: int = 0):
    """(heads, tokens) of n rows: the four corners plus uniform draws."""
    rng = np.random.default_rng(seed)
    hs = np.concatenate([[0, 0, H - 1, H - 1], rng.integers(0, H, n - 4)])
    ts = np.concatenate([[0, T - 1, 0, T - 1], rng.integers(0, T, n - 4)])
    return hs.astype(np.int64), ts.astype(np.int64)


def residual_bound_factors(r_T: int, r_D: int, D: int):
    """(g_R, g_Y): the kernel's error bounds |d recon| <= g_R |U~_T||G~_h||U~_D|^T
    and |dY| <= |dR||Q|^T + g_Y |R||Q|^T, in units of 2^-24.

    The encoder forms W_h = G~_h U~_D^T with r_D fp32 additions of exact bf16
    products and splits fp32 operands into two bf16 parts, f = hi + lo + r
    (hi = rne(f), lo = rne(f - hi), |lo| <= 2^-9 (1 + 2^-8) |f|, the dropped
    |r| <= 2^-18 |f| = 64 units), accumulating in fp32: recon = U~_T hi (r_T
    terms) + U~_T lo (r_T terms of total size <= 2^-8 of the first) + one
    addition, and W's remainder r -> r_D + r_T + r_T/256 + 64 + 1 (+ slack);
    Y = R_hi Q_hi (D terms) + R_hi Q_lo + R_lo Q_hi (2 D terms of total size
    <= 2^-8) + dropped R_lo Q_lo and the remainders of R and Q (3 x 64) + one
    addition + the fp32 rounding of Q -> D + D/128 + 192 + 1 + 1.  Bounds:
    (1 + 2^-5) r_T + r_D + 68 and D + 200."""
    return (1 + 2.0 ** -5) * r_T + r_D + 68, D + 200


def oracle_rows(X_rows: np.ndarray, parts: dict, choice, Q: np.ndarray, hs, ts):
    """Y = fp32((X - U~_T G~_h U~_D^T) Q^T) on the rows, and the per-element
    bound on the kernel's fp32 error (as in the whole-tensor check)."""
    r_T, r_D, _ = choice
    Xr = np.asarray(X_rows, dtype=np.float64)
    absQ = np.abs(Q)
    gR, gY = residual_bound_factors(r_T, r_D, Q.shape[0])
    if r_T > 0:
        Ut = parts["U_T"][ts]                        # [n, r_T]
        G = parts["G"][hs]                           # [n, r_T, r_D]
        Ud = parts["U_D"]                            # [D, r_D]
        recon = np.einsum("nr,nrs,ds->nd", Ut, G, Ud, optimize=True)
        terms = np.einsum("nr,nrs,ds->nd", np.abs(Ut), np.abs(G), np.abs(Ud), optimize=True)
        R = Xr - recon
        bR = gR * 2.0 ** -24 * terms
    else:
        R, recon, terms = Xr, 0.0 * Xr, 0.0 * Xr
        bR = np.zeros_like(Xr)
    bR = bR + 2.0 ** -24 * np.abs(Xr)
    Y = (R @ Q.T).astype(np.float32)
    bY = bR @ absQ.T + gY * 2.0 ** -24 * (np.abs(R) @ absQ.T)
    return Y, bY


def record_rows(parts: dict, hs, ts, bits: int):
    from oracle import quant
    return (parts["m16"][hs, ts], parts["s16"][hs, ts],
            quant.unpack(parts["packed"][hs, ts], bits))


def check_codes(m16_g, s16_g, codes_g, Y, bY, bits):
    """Scales and codes from the GPU vs the oracle quantizer on the oracle's Y
    (any leading shape, groups of 32 along the last axis of Y).

    They may differ only where the fp32 error bound bY lets a decision flip: a
    group minimum (or step) within the bound of a bf16 rounding boundary, a
    code where (y - m16)/s16 is within bound/s16 of a half-integer."""
    from oracle import bf16, quant
    m16, s16, codes = quant.quantize(Y, bits)
    m16, s16 = m16.reshape(-1, 4), s16.reshape(-1, 4)
    codes = codes.reshape(-1, 4, 32)
    gm, gs = np.asarray(m16_g).reshape(-1, 4), np.asarray(s16_g).reshape(-1, 4)
    got = np.asarray(codes_g).reshape(-1, 4, 32)
    L = 2 ** bits - 1
    g = np.asarray(Y).reshape(-1, 4, 32).astype(np.float64)
    b = np.asarray(bY).reshape(-1, 4, 32)
    bmax = b.max(-1)
    same = (gm == m16) & (gs == s16)
    assert same.mean() > 0.98, same.mean()
    if (~same).any():
        mn = g.min(-1)
        lo = bf16.round_down((mn - bmax).astype(np.float32))
        hi = bf16.round_down((mn + bmax).astype(np.float32))
        assert np.all(((gm >= lo) & (gm <= hi))[~same])
        mx = g.max(-1)
        s_lo = bf16.round_up((((mx - bmax) - hi) / L).astype(np.float32))
        s_hi = bf16.round_up((((mx + bmax) - lo) / L).astype(np.float32) * np.float32(1 + 2 ** -22))
        assert np.all(((gs >= s_lo) & (gs <= s_hi))[~same])
    diff = (got != codes) & same[..., None]
    if diff.any():
        t = (g - m16[..., None]) / np.where(s16 == 0, 1, s16)[..., None]
        frac = np.abs(t - np.floor(t) - 0.5)
        tol = b / np.where(s16 == 0, 1, s16)[..., None] + 1e-6
        assert np.all(frac[diff] <= tol[diff])
        assert np.all(np.abs(got.astype(int) - codes.astype(int))[diff] == 1)
    assert diff.mean() < 1e-2, diff.mean()
    return float((~same).mean()), float(diff.mean())


def check_decode_rows(out_rows, parts: dict, choice, Q: np.ndarray, hs, ts, out_dtype: str):
    """GPU decode rows vs the exact decode of the GPU record, within the
    kernel's error bound: bf16 matrix cores with fp32 accumulation, W = G~ U~_D^T
    as a hi + lo bf16 pair (relative 2^-17 after an fp32 product over r_D), the
    dequantized residual and Q each rounded to bf16 (relative 2^-9 each)."""
    from oracle import quant
    r_T, r_D, bits = choice
    m16, s16, codes = record_rows(parts, hs, ts, bits)
    Yh = quant.dequantize(m16, s16, codes).reshape(-1, D)
    exact = Yh @ Q
    rot_terms = np.abs(Yh) @ np.abs(Q)
    rec_terms = np.zeros_like(exact)
    if r_T > 0:
        Ut, G, Ud = parts["U_T"][ts], parts["G"][hs], parts["U_D"]
        exact = exact + np.einsum("nr,nrs,ds->nd", Ut, G, Ud, optimize=True)
        rec_terms = np.einsum("nr,nrs,ds->nd", np.abs(Ut), np.abs(G), np.abs(Ud), optimize=True)
    terms = rot_terms + rec_terms
    bound = (r_T + r_D + D + 8) * 2.0 ** -24 * terms + 2.0 ** -15 * rec_terms + 2.0 ** -8 * rot_terms
    got = np.asarray(out_rows, dtype=np.float64)
    if out_dtype == "f32":
        ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - exact) <= bound + ulp)
        return 0.0
    return check_bf16_rounding(got, exact, bound, 1.0, max_frac=0.25)


def pack_record(enc: dict, dtype_code: int = 0, seed: int = 0) -> np.ndarray:
    """An oracle encode (``codec.encode_tensor``) as record bytes in the
    library's documented layout (header, then 256-aligned sections U_T, U_D,
    core, scales, codes), so that GPU kernels can be fed inputs made by the
    oracle alone."""
    from oracle import quant
    H, T, Dd = enc["shape"]
    r_T, r_D, b = enc["choice"]
    groups = H * T * Dd // 32
    ut = 256
    ud = ut + a256(2 * T * r_T)
    g = ud + a256(2 * Dd * r_D)
    sc = g + a256(2 * H * r_T * r_D)
    cd = sc + a256(4 * groups)
    total = cd + a256(4 * b * groups)
    out = np.zeros(total, dtype=np.uint8)
    hdr = np.array([0x544C4F4A, 1, H, T, Dd, dtype_code, r_T, r_D, b, 32, seed & 0xffffffff, seed >> 32,
                    0, 0, 0, 0], dtype=np.uint32)
    out[:64] = hdr.view(np.uint8)

    def bf(x):
        u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
        return (u >> 16).astype(np.uint16)          # exact: the stored values are bf16 already

    if r_T > 0:
        out[ut:ut + 2 * T * r_T] = bf(enc["U_T"]).reshape(-1).view(np.uint8)
        out[ud:ud + 2 * Dd * r_D] = bf(enc["U_D"]).reshape(-1).view(np.uint8)
        out[g:g + 2 * H * r_T * r_D] = bf(enc["G"]).reshape(-1).view(np.uint8)
    scales = np.stack([bf(enc["m16"]).reshape(-1), bf(enc["s16"]).reshape(-1)], axis=1)
    out[sc:sc + 4 * groups] = scales.reshape(-1).view(np.uint8)
    out[cd:cd + 4 * b * groups] = quant.pack(enc["codes"], b).reshape(-1)
    return out
