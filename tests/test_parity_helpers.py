"""The row-sampled parity helpers used by the full-size GPU tests, run on
the oracle's own record (no GPU): an exact record must pass every check, and
a planted mistake must fail one."""
import numpy as np
import pytest

import kvgen
from oracle import codec, quant, rotation, tucker

from gpu_util import (check_codes, check_decode_rows, oracle_rows, record_rows, sample_rows)


@pytest.fixture(scope="module")
def rec():
    X = kvgen.tensor(4, 256, 128, seed=3, decay=0.9, dtype="bf16").astype(np.float64)
    lam_T, lam_D, U_T, U_D = tucker.factors_exact(X, 64)
    Q = rotation.rotation(0, 128)
    choice = (64, 48, 3)
    e = codec.encode_tensor(X, U_T, U_D, choice, Q)
    parts = dict(U_T=e["U_T"], U_D=e["U_D"], G=e["G"], m16=e["m16"], s16=e["s16"],
                 packed=quant.pack(e["codes"], 3))
    return X, e, parts, Q, choice


def test_rows_reproduce_the_record(rec):
    X, e, parts, Q, choice = rec
    hs, ts = sample_rows(4, 256, 64, seed=1)
    assert (hs[:4] == [0, 0, 3, 3]).all() and (ts[:4] == [0, 255, 0, 255]).all()
    Y, bY = oracle_rows(X[hs, ts], parts, choice, Q, hs, ts)
    np.testing.assert_array_equal(Y, e["Y"][hs, ts])
    assert np.all(bY > 0)
    m16, s16, codes = record_rows(parts, hs, ts, 3)
    assert check_codes(m16, s16, codes, Y, bY, 3) == (0.0, 0.0)
    out = codec.decode_tensor(e, Q, "bf16")
    check_decode_rows(out[hs, ts], parts, choice, Q, hs, ts, "bf16")


def test_planted_code_error_fails(rec):
    X, e, parts, Q, choice = rec
    hs, ts = sample_rows(4, 256, 64, seed=1)
    Y, bY = oracle_rows(X[hs, ts], parts, choice, Q, hs, ts)
    m16, s16, codes = record_rows(parts, hs, ts, 3)
    bad = codes.copy()
    bad[5, 2, 7] = (bad[5, 2, 7] + 2) % 8
    with pytest.raises(AssertionError):
        check_codes(m16, s16, bad, Y, bY, 3)


def test_planted_decode_error_fails(rec):
    X, e, parts, Q, choice = rec
    hs, ts = sample_rows(4, 256, 64, seed=1)
    out = codec.decode_tensor(e, Q, "f32")[hs, ts].copy()
    out[3, 17] += 1e-2 * max(1.0, abs(out[3, 17]))
    with pytest.raises(AssertionError):
        check_decode_rows(out, parts, choice, Q, hs, ts, "f32")
