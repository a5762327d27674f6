"""End-to-end pins for the oracle codec: the error model, JL whitening, the
residual against the stored factors, and a small whole-cache allocation."""
import numpy as np
import pytest
from scipy import stats

import kvgen
from oracle import alloc, bf16, codec, quant, rotation, tucker


@pytest.fixture(scope="module")
def single():
    cfg = kvgen.CONFIGS["single_k_t1024_f32"]
    X = kvgen.config_tensor(cfg, 0, 0).astype(np.float64)
    return X, codec.analyze(X, 256), rotation.rotation(0, 128)


def test_stored_parts_are_bf16(single):
    X, a, Q = single
    e = codec.encode_tensor(X, a["U_T"], a["U_D"], (256, 64, 2), Q)
    for k in ("U_T", "U_D", "G", "m16", "s16"):
        v = e[k]
        np.testing.assert_array_equal(bf16.round_nearest(v), v)
    assert e["U_T"].shape == (1024, 256) and e["U_D"].shape == (128, 64)
    assert e["G"].shape == (8, 256, 64) and e["codes"].shape == (8, 1024, 4, 32)


def test_residual_is_against_stored_factors(single):
    X, a, Q = single
    e = codec.encode_tensor(X, a["U_T"], a["U_D"], (256, 64, 3), Q)
    R = X - tucker.reconstruct(e["G"], e["U_T"], e["U_D"])
    Ydef = (R.reshape(-1, 128) @ Q.T).reshape(R.shape)
    # Y is the fp32 rounding of R Q^T
    np.testing.assert_array_equal(e["Y"], Ydef.astype(np.float32))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_error_model(single, bits):
    # rel_err^2 ~ rho(b) * ||X - recon||^2 / ||X||^2 (uniform error after rotation)
    X, a, Q = single
    e = codec.encode_tensor(X, a["U_T"], a["U_D"], (256, 64, bits), Q)
    Xh = codec.decode_tensor(e, Q, "f32")
    f2 = float(np.sum(X * X))
    R = X - tucker.reconstruct(e["G"], e["U_T"], e["U_D"])
    pred = alloc.rho(bits) * float(np.sum(R * R)) / f2
    err = codec.rel_err(X, Xh) ** 2
    assert 0.75 < err / pred < 1.25


def test_decode_error_within_half_step(single):
    X, a, Q = single
    e = codec.encode_tensor(X, a["U_T"], a["U_D"], (256, 64, 2), Q)
    Yh = quant.dequantize(e["m16"], e["s16"], e["codes"]).reshape(8, 1024, 128)
    dev = np.abs(Yh - e["Y"]).reshape(8, 1024, 4, 32)
    ulp = np.spacing(np.abs(e["Y"])).reshape(8, 1024, 4, 32)
    assert np.all(dev <= e["s16"][..., None] / 2 + 2 * ulp)


def test_jl_rotation_whitens_error(single):
    # errors in the rotated domain, in units of the step, are close to
    # independent U(-1/2, 1/2); without Tucker and with outlier channels the
    # rotation lowers the error (news article, paragraph 4)
    X, a, Q = single
    e = codec.encode_tensor(X, a["U_T"], a["U_D"], (256, 64, 3), Q)
    Yh = quant.dequantize(e["m16"], e["s16"], e["codes"]).reshape(8, 1024, 4, 32)
    Y = e["Y"].reshape(8, 1024, 4, 32).astype(np.float64)
    u = (Y - Yh) / e["s16"][..., None]
    # each group's min and max sit on (or next to) the grid ends by
    # construction; the other 30 elements carry the rounding error
    interior = (Y > Y.min(-1, keepdims=True)) & (Y < Y.max(-1, keepdims=True))
    u = u[interior][:200000]
    assert stats.kstest(u, "uniform", args=(-0.5, 1.0)).statistic < 0.02
    c = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(c) < 0.02
    eye = np.eye(128)
    rot = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, None, None, (0, 0, 2), Q), Q, "f32"))
    plain = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, None, None, (0, 0, 2), eye), eye, "f32"))
    assert rot < 0.8 * plain


def test_more_bits_less_error(single):
    X, a, Q = single
    errs = [codec.rel_err(X, codec.decode_tensor(
        codec.encode_tensor(X, a["U_T"], a["U_D"], (256, 64, b), Q), Q, "f32")) for b in (1, 2, 3, 4)]
    assert errs[0] > errs[1] > errs[2] > errs[3]


def test_bf16_output_metric():
    X = kvgen.tensor(2, 64, 64, seed=1, dtype="bf16").astype(np.float64)
    np.testing.assert_array_equal(codec.round_to(X, "bf16"), X)
    assert codec.rel_err(X, X) == 0.0
    assert codec.rel_err(np.zeros(3), np.zeros(3)) == 0.0


@pytest.mark.parametrize("method", ["exact", "flash"])
def test_small_cache_end_to_end(method):
    L, H, T, D = 4, 2, 256, 64
    tensors = [[kvgen.tensor(H, T, D, seed=0, layer=l, kind=k, decay=0.9, dtype="bf16")
                .astype(np.float64) for k in (0, 1)] for l in range(L)]
    out = {}
    for ratio in (3.0, 2.0):
        res = codec.encode_cache(tensors, ratio, "bf16", method=method, group_layers=2,
                                 step_T=16, step_D=16)
        plan = res["plan"]
        assert plan["total_bytes"] <= plan["budget"]
        errs = np.array(res["rel_err"])
        assert np.all(np.isfinite(errs)) and errs.max() < 0.5
        out[ratio] = errs.mean()
    assert out[2.0] < out[3.0]
