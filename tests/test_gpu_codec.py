"""GPU parity of the HIP path against the fp64 CPU oracle, through the C ABI.

Bars (from the codec's statement and its arithmetic):
* quantization codes and scales bit-exact when the kernel is fed the oracle's
  fp32 rotated residual;
* relative Frobenius reconstruction error within 1e-4 of the oracle's;
* factors: spectra within 2e-5 * lambda_1, orthonormal to 1e-5, principal-angle
  sines <= 1e-3 at every cut the fp32 eigengaps resolve, captured energy within
  1e-4 relative.
"""
import numpy as np
import pytest
import torch

import kvgen
from oracle import alloc, bf16, codec, flash, quant, rng, rotation, tucker

from gpu_util import (D, check_bf16_rounding, check_codes, max_sine, parse_blob, residual_bound_factors,
                      resolvable_cuts, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_compression_mode_amd import jolt
    return jolt


@pytest.fixture(scope="module")
def rot(J):
    return J.rotation(0)


@pytest.fixture(scope="module")
def single():
    cfg = kvgen.CONFIGS["single_k_t1024_f32"]
    X = kvgen.config_tensor(cfg, 0, 0).astype(np.float64)
    return X, codec.analyze(X, 256), rotation.rotation(0, 128)


def _quant_ref(Y, bits):
    m16, s16, c = quant.quantize(Y, bits)
    return m16, s16, quant.pack(c, bits)


def _gpu_quant(J, Y, bits):
    rows = Y.shape[0]
    sc, cd = J.quantize(torch.from_numpy(np.ascontiguousarray(Y, np.float32)).cuda(), bits)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy().view(np.uint16).reshape(rows, 4, 2)
    m16 = (sc[..., 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s16 = (sc[..., 1].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return m16, s16, cd.cpu().numpy().reshape(rows, 4, 4 * bits)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_quantizer_bit_exact_on_oracle_residual(J, single, bits):
    X, a, Q = single
    Y = codec.encode_tensor(X, a["U_T"], a["U_D"], (256, 64, bits), Q)["Y"].reshape(-1, D)
    m, s, p = _quant_ref(Y, bits)
    gm, gs, gp = _gpu_quant(J, Y, bits)
    np.testing.assert_array_equal(gm, m)
    np.testing.assert_array_equal(gs, s)
    np.testing.assert_array_equal(gp, p)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_quantizer_edge_cases(J, bits):
    r = np.random.default_rng(100 + bits)
    rows = 37                                            # ragged: not a multiple of the tile
    Y = (r.standard_normal((rows, D)) * r.uniform(1e-3, 1e3, (rows, 1))).astype(np.float32)
    Y[0] = 3.0                                           # constant row: zero step
    Y[1, :32] = -2.5                                     # one constant group
    Y[2] *= np.float32(1e-40)                            # subnormal values
    Y[3] = -np.abs(Y[3])                                 # all negative
    Y[4, ::2] = Y[4, 1::2]                               # exact ties in a row
    Y[5] = np.arange(D, dtype=np.float32) * 0.5 - 31.75  # grid-aligned, midpoints
    m, s, p = _quant_ref(Y, bits)
    gm, gs, gp = _gpu_quant(J, Y, bits)
    np.testing.assert_array_equal(gm, m)
    np.testing.assert_array_equal(gs, s)
    np.testing.assert_array_equal(gp, p)


def test_quantizer_empty(J):
    sc, cd = J.quantize(torch.empty((0, D), dtype=torch.float32, device="cuda"), 2)
    assert sc.numel() == 0 and cd.numel() == 0


def _oracle_from_blob(X, parts, choice, Q, H, T):
    """The oracle's residual and rotation applied to the GPU's stored parts,
    with a per-element bound on the fp32 error of the kernel's Y:
    |dY| <= (g_R |U~_T||G~_h||U~_D|^T + 2^-24 |X|) |Q|^T + g_Y |R| |Q|^T, the
    factors of the kernel's arithmetic (gpu_util.residual_bound_factors).
    """
    r_T, r_D, _ = choice
    absQ = np.abs(Q)
    gR, gY = residual_bound_factors(r_T, r_D, D)
    if r_T > 0:
        R = X - tucker.reconstruct(parts["G"], parts["U_T"], parts["U_D"])
        bR = gR * 2.0 ** -24 * tucker.reconstruct(np.abs(parts["G"]), np.abs(parts["U_T"]),
                                                  np.abs(parts["U_D"]))
    else:
        R = X
        bR = np.zeros_like(X)
    bR = bR + 2.0 ** -24 * np.abs(X)                       # the subtraction X - recon
    Y = (R.reshape(-1, D) @ Q.T).astype(np.float32).reshape(H, T, D)
    bY = ((bR.reshape(-1, D) @ absQ.T) + gY * 2.0 ** -24 * (np.abs(R).reshape(-1, D) @ absQ.T))
    return Y, bY.reshape(H, T, D)


def _check_codes(parts, Y, bY, bits, H, T):
    return check_codes(parts["m16"], parts["s16"], quant.unpack(parts["packed"], bits), Y, bY, bits)


@pytest.mark.parametrize("choice,xdt", [((256, 64, 2), "f32"), ((256, 64, 3), "bf16"),
                                        ((128, 32, 4), "f32"), ((0, 0, 2), "f32"), ((96, 112, 1), "bf16")])
def test_encode_decode_with_oracle_factors(J, rot, single, choice, xdt):
    X0, a, Q = single
    X = codec.round_to(X0, xdt)
    H, T, _ = X.shape
    r_T, r_D, bits = choice
    # factors rounded to bf16 on the oracle side, so both sides store the same values
    Ut = bf16.round_nearest(a["U_T"][:, :max(r_T, 1)])
    Ud = bf16.round_nearest(a["U_D"][:, :max(r_D, 1)])
    xd = to_dev(X, xdt)
    dev32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    blob = J.encode(xd, choice, dev32(Ut) if r_T else None, dev32(Ud) if r_T else None, rot, seed=0)
    xh = J.decode(blob, H, T, choice, rot, dtype=xd.dtype)
    torch.cuda.synchronize()
    parts = parse_blob(blob, H, T, choice)
    assert list(parts["header"][:10]) == [0x544C4F4A, 1, H, T, D, 1 if xdt == "f32" else 0,
                                          r_T, r_D, bits, 32]
    if r_T:
        np.testing.assert_array_equal(parts["U_T"], Ut[:, :r_T])
        np.testing.assert_array_equal(parts["U_D"], Ud[:, :r_D])
        # the core is formed in fp32 (K = T tokens, then D features): its bf16
        # rounding may differ from the fp64 one only next to a rounding midpoint
        exact = tucker.core(X, Ut[:, :r_T], Ud[:, :r_D])
        terms = tucker.core(np.abs(X), np.abs(Ut[:, :r_T]), np.abs(Ud[:, :r_D]))
        check_bf16_rounding(parts["G"], exact, terms, gamma=(T + D) * 2.0 ** -24)
    Y, bY = _oracle_from_blob(X, parts, choice, Q, H, T)
    _check_codes(parts, Y, bY, bits, H, T)
    # decode parity: the oracle decode of the GPU record, element by element
    enc = dict(shape=(H, T, D), choice=choice, U_T=parts["U_T"], U_D=parts["U_D"], G=parts["G"],
               m16=parts["m16"], s16=parts["s16"], codes=quant.unpack(parts["packed"], bits))
    Xg = xh.float().cpu().numpy().astype(np.float64)
    # exact (unrounded) decode of the GPU record and the fp32 error bound of the kernel
    Yh = quant.dequantize(enc["m16"], enc["s16"], enc["codes"]).reshape(H, T, D)
    exact = (Yh.reshape(-1, D) @ Q).reshape(H, T, D)
    terms = (np.abs(Yh).reshape(-1, D) @ np.abs(Q)).reshape(H, T, D)
    if r_T:
        exact = exact + tucker.reconstruct(enc["G"], enc["U_T"], enc["U_D"])
        terms = terms + tucker.reconstruct(np.abs(enc["G"]), np.abs(enc["U_T"]), np.abs(enc["U_D"]))
    # decode arithmetic: bf16 matrix cores, fp32 accumulation; W = G~ U~_D^T as a
    # hi + lo bf16 pair (relative 2^-17 after an fp32 product over r_D), the
    # dequantized residual and Q each rounded to bf16 (relative 2^-9 each)
    rot_terms = (np.abs(Yh).reshape(-1, D) @ np.abs(Q)).reshape(H, T, D)
    rec_terms = terms - rot_terms
    bound = (r_T + r_D + D + 8) * 2.0 ** -24 * terms + 2.0 ** -15 * rec_terms + 2.0 ** -8 * rot_terms
    if xdt == "f32":
        ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(Xg - exact) <= bound + ulp)
    else:
        # the per-element bound is the check; roundings may flip wherever the
        # bf16-operand error reaches a midpoint, which at 1 bit/element is often
        check_bf16_rounding(Xg, exact, bound, 1.0, max_frac=0.25)
    # end-to-end error against the oracle's own record
    eo = codec.encode_tensor(X, Ut, Ud, choice, Q)
    err_o = codec.rel_err(X, codec.decode_tensor(eo, Q, xdt))
    assert abs(codec.rel_err(X, Xg) - err_o) < 1e-4


def _alloc_single(J, X, xdt, method="exact"):
    xd = to_dev(X, xdt)
    return J.allocate([(xd, xd)], ratio=2.0, method=method), xd


def test_gpu_factors_exact_direct(J, single):
    X, a, Q = single
    res, _ = _alloc_single(J, X, "f32")
    torch.cuda.synchronize()
    R = res.r_T_cap
    assert R == 256
    lam_o, lamD_o = a["lam_T"], a["lam_D"]
    lam_g, lamD_g = res.spectra_T[0], res.spectra_D[0]
    assert np.all(np.abs(lam_g - lam_o[:R]) <= 2e-5 * lam_o[0])
    np.testing.assert_allclose(lam_g[:8], lam_o[:8], rtol=1e-5)
    assert np.all(np.abs(lamD_g - lamD_o) <= 2e-5 * lamD_o[0])
    assert abs(res.frob2[0] - a["frob2"]) <= 1e-12 * a["frob2"]
    Ut, Ud = (t.cpu().numpy().astype(np.float64) for t in res.factors(0))
    assert np.abs(Ut.T @ Ut - np.eye(R)).max() < 1e-5
    assert np.abs(Ud.T @ Ud - np.eye(D)).max() < 1e-5
    for k in resolvable_cuts(lam_o, R, len(lam_o)):
        assert max_sine(Ut[:, :k], a["U_T"][:, :k]) <= 1e-3, k
    for k in resolvable_cuts(lamD_o, D - 1, D):
        assert max_sine(Ud[:, :k], a["U_D"][:, :k]) <= 1e-3, k
    # captured energy: the truncation residual ||X||^2 - ||G||^2 is what the
    # codec quantizes, so compare it (not just ||G||^2) with the oracle's
    f2 = a["frob2"]
    for r_T, r_D in [(256, 64), (96, 32), (32, 16)]:
        eg = np.sum(tucker.core(X, Ut[:, :r_T], Ud[:, :r_D]) ** 2)
        eo = np.sum(tucker.core(X, a["U_T"][:, :r_T], a["U_D"][:, :r_D]) ** 2)
        assert abs(eg - eo) <= 1e-4 * eo
        assert abs((f2 - eg) - (f2 - eo)) <= 5e-3 * (f2 - eo), (r_T, r_D, f2 - eg, f2 - eo)


def _qr_launches(J, X):
    """Allocate on one tensor (keys and values both X) with the QR scopes
    profiled: (CholeskyQR calls, Householder update calls, result)."""
    J.profile_enable("cholqr,qr_update")
    try:
        res, xd = _alloc_single(J, X, "f32")
        torch.cuda.synchronize()
        return J.profile_query("cholqr")["launches"], J.profile_query("qr_update")["launches"], res, xd
    finally:
        J.profile_enable(None)


def test_full_rank_factors_take_cholesky_qr(J):
    """The dual token factor of a full-rank tensor (T > H D) is
    re-orthonormalized by CholeskyQR alone (no Householder update runs), and
    is orthonormal with the oracle's leading subspaces."""
    X = kvgen.tensor(2, 512, D, seed=8, layer=1, kind=0, decay=0.85, dtype="f32").astype(np.float64)
    n_chol, n_hh, res, _ = _qr_launches(J, X)
    assert n_chol > 0 and n_hh == 0, (n_chol, n_hh)
    R = res.r_T_cap
    a = codec.analyze(X, R)
    Ut = res.factors(0)[0].cpu().numpy().astype(np.float64)
    assert np.abs(Ut.T @ Ut - np.eye(R)).max() < 1e-5
    assert np.all(np.abs(res.spectra_T[0] - a["lam_T"][:R]) <= 2e-5 * a["lam_T"][0])
    for k in resolvable_cuts(a["lam_T"], R, 2 * D):
        assert max_sine(Ut[:, :k], a["U_T"][:, :k]) <= 1e-3, k


def test_rank_deficient_input(J, rot):
    """An exactly rank-6 tensor (no noise) in the dual regime with a rank cap
    of 64: the factor is orthonormal, carries the oracle's rank-6 subspace
    and spectrum (the rest of the spectrum within 2e-5 lambda_1 of zero),
    and the end-to-end error matches the oracle's record within 1e-4."""
    X = kvgen.tensor(2, 512, D, seed=9, noise_std=0.0, rank=6, outliers=False, dtype="f32").astype(np.float64)
    _, _, res, xd = _qr_launches(J, X)
    R = res.r_T_cap
    assert R > 6
    a = codec.analyze(X, R)
    lam_o, lam_g = a["lam_T"], res.spectra_T[0]
    assert np.all(np.abs(lam_g - lam_o[:R]) <= 2e-5 * lam_o[0])
    Ut, Ud = res.factors(0)
    Utn = Ut.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(Utn))
    assert np.abs(Utn.T @ Utn - np.eye(R)).max() < 1e-5
    assert max_sine(Utn[:, :6], a["U_T"][:, :6]) <= 1e-3
    choice = (8, 16, 2)
    Q = rotation.rotation(0, D)
    xh = J.decode(J.encode(xd, choice, Ut, Ud, rot), 2, 512, choice, rot, dtype=torch.float32)
    err_g = codec.rel_err(X, xh.cpu().numpy())
    err_o = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, a["U_T"], a["U_D"], choice, Q), Q, "f32"))
    assert abs(err_g - err_o) < 1e-4, (err_g, err_o)


def test_zero_tensor_falls_back_to_householder(J, rot):
    """An all-zero tensor: its token basis X V_R is zero, the first CholeskyQR
    pivot is not above its (zero) diagonal, and the analysis is repeated with
    Householder QR.  Spectra are zero, both factors orthonormal, and the
    record decodes to zeros."""
    X = np.zeros((2, 512, D))
    n_chol, n_hh, res, xd = _qr_launches(J, X)
    assert n_chol > 0 and n_hh > 0, (n_chol, n_hh)
    R = res.r_T_cap
    # the eigensolver's brackets of a zero spectrum are [-DBL_MIN, DBL_MIN]
    assert np.all(np.abs(res.spectra_T[0]) <= 1e-300) and np.all(res.spectra_D[0] == 0.0) and res.frob2[0] == 0.0
    Ut, Ud = res.factors(0)
    Utn, Udn = (t.cpu().numpy().astype(np.float64) for t in (Ut, Ud))
    assert np.abs(Utn.T @ Utn - np.eye(R)).max() < 1e-5
    assert np.abs(Udn.T @ Udn - np.eye(D)).max() < 1e-5
    choice = (16, 16, 2)
    xh = J.decode(J.encode(xd, choice, Ut, Ud, rot), 2, 512, choice, rot, dtype=torch.float32)
    assert torch.count_nonzero(xh).item() == 0


@pytest.mark.parametrize("bits", [2, 4])
def test_end_to_end_single_tensor(J, rot, single, bits):
    X, a, Q = single
    res, xd = _alloc_single(J, X, "f32")
    Ut, Ud = res.factors(0)
    choice = (256, 64, bits)
    blob = J.encode(xd, choice, Ut, Ud, rot)
    xh = J.decode(blob, 8, 1024, choice, rot, dtype=torch.float32)
    err_g = codec.rel_err(X, xh.cpu().numpy())
    err_o = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, a["U_T"], a["U_D"], choice, Q),
                                                 Q, "f32"))
    assert abs(err_g - err_o) < 1e-4


def _cache(L, H, T, seed=0, dtype="bf16"):
    return [[kvgen.tensor(H, T, D, seed=seed, layer=l, kind=k, decay=kvgen.decay_for(seed, l, k),
                          outliers=True, dtype=dtype).astype(np.float64) for k in (0, 1)]
            for l in range(L)]


@pytest.mark.parametrize("method,L,H,T,ratio", [("exact", 4, 2, 512, 2.0),    # dual Gram (T > HD)
                                                ("exact", 2, 4, 200, 2.0),    # direct, ragged T
                                                ("flash", 4, 2, 512, 2.0),
                                                ("flash", 2, 8, 384, 3.0)])
def test_small_cache_end_to_end(J, rot, method, L, H, T, ratio):
    tens = _cache(L, H, T)
    dev = [(to_dev(tens[l][0], "bf16"), to_dev(tens[l][1], "bf16")) for l in range(L)]
    res = J.allocate(dev, ratio=ratio, method=method, group_layers=2)
    torch.cuda.synchronize()
    orc = codec.encode_cache(tens, ratio, "bf16", method=method, group_layers=2)
    R = res.r_T_cap
    Q = orc["Q"]
    # the library's plan equals the oracle dual run on the library's spectra
    sp = [[(res.spectra_T[2 * l + k], res.spectra_D[2 * l + k], res.frob2[2 * l + k]) for k in (0, 1)]
          for l in range(L)]
    want = alloc.allocate(sp, L, H, T, D, ratio, (1, 2, 3, 4), 2)
    assert res.choice == want["choice"] and res.total_bytes == want["total_bytes"]
    assert res.total_bytes <= res.budget_bytes
    for l in range(L):
        for k in (0, 1):
            t = 2 * l + k
            X = tens[l][k]
            an = orc["analysis"][l][k]
            lam_o = an["lam_T"]
            assert np.all(np.abs(res.spectra_T[t] - lam_o[:R]) <= 2e-5 * lam_o[0])
            Ut, Ud = res.factors(t)
            Utn = Ut.cpu().numpy().astype(np.float64)
            assert np.abs(Utn.T @ Utn - np.eye(R)).max() < 1e-5
            for kc in resolvable_cuts(lam_o, R, min(T, H * D)):
                assert max_sine(Utn[:, :kc], an["U_T"][:, :kc]) <= 1e-3
            # encode/decode with the library's own factors under the oracle's plan
            ch = orc["plan"]["choice"][(l // 2, k)]
            blob = J.encode(dev[l][k], ch, Ut, Ud, rot)
            xh = J.decode(blob, H, T, ch, rot, dtype=torch.bfloat16)
            err_g = codec.rel_err(X, xh.float().cpu().numpy())
            assert abs(err_g - orc["rel_err"][l][k]) < 1e-4, (l, k, err_g, orc["rel_err"][l][k])


def test_decode_many_matches_single_records(J, rot, single):
    """One batched call (mixed ranks and bit-widths, a no-Tucker record, more
    records than one launch takes) reproduces the single-record decodes bit
    for bit."""
    X0, a, Q = single
    X = codec.round_to(X0, "bf16")
    H, T, _ = X.shape
    xd = to_dev(X, "bf16")
    Ut32 = torch.from_numpy(np.ascontiguousarray(a["U_T"], dtype=np.float32)).cuda()
    Ud32 = torch.from_numpy(np.ascontiguousarray(a["U_D"], dtype=np.float32)).cuda()
    base = [(256, 64, 2), (96, 112, 3), (0, 0, 4), (32, 16, 1), (224, 128, 4)]
    choices = [base[i % len(base)] for i in range(37)]           # 37 > one launch (32)
    blobs = [J.encode(xd, c, Ut32 if c[0] else None, Ud32 if c[0] else None, rot) for c in choices]
    outs = [torch.empty((H, T, D), dtype=torch.bfloat16, device="cuda") for _ in choices]
    ws = torch.empty(J.decode_many_workspace_bytes(H, T, choices), dtype=torch.uint8, device="cuda")
    J.decode_many(blobs, H, T, choices, rot, outs, ws)
    for b, c, o in zip(blobs, choices, outs):
        single_out = J.decode(b, H, T, c, rot)
        assert torch.equal(single_out, o)
    torch.cuda.synchronize()


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
def test_decode_into_unaligned_output(J, rot, single, odt):
    """An output that starts one element past a 16-byte boundary takes the
    element-wise store path and holds the same values as an aligned one."""
    X0, a, Q = single
    X = codec.round_to(X0, "bf16")
    H, T, _ = X.shape
    xd = to_dev(X, "bf16")
    Ut32 = torch.from_numpy(np.ascontiguousarray(a["U_T"], dtype=np.float32)).cuda()
    Ud32 = torch.from_numpy(np.ascontiguousarray(a["U_D"], dtype=np.float32)).cuda()
    c = (96, 112, 3)
    blob = J.encode(xd, c, Ut32, Ud32, rot)
    ref = J.decode(blob, H, T, c, rot, dtype=odt)
    buf = torch.full((H * T * D + 1,), 7.0, dtype=odt, device="cuda")
    view = buf[1:].view(H, T, D)
    assert view.data_ptr() % 16 != 0
    J.decode(blob, H, T, c, rot, dtype=odt, out=view)
    assert torch.equal(view, ref)
    assert buf[0].item() == 7.0
    torch.cuda.synchronize()
