"""GPU parity of the decode fused into attention (jolt_attend), through the
C ABI, on records made by the oracle alone (its factors and encode, packed in
the library's documented record layout), against the oracle's attention on
its own exact (fp64, unrounded) decode of those records.

The bar is the kernel's arithmetic, bounded element by element:
* the reconstructions' error as in the decode (bf16 matrix cores, fp32
  accumulation, W as a bf16 hi + lo pair, the dequantized residual and Q in
  bf16): (r_T + r_D + D + 8) 2^-24 (|U~_T||G~||U~_D|^T + |Y^||Q|)
  + 2^-15 |U~_T||G~||U~_D|^T + 2^-8 |Y^||Q|;
* a score moves by at most sum_d |q_d| dK_td / sqrt(D) plus its own fp32
  rounding; the softmax weights by at most 2 (max_t ds_t + e_exp) in l1
  (e_exp = 2^-20: the exponential's error over the range that carries weight);
* an output by at most |dp|_1 max_t |V_t| + sum_t p_t dV_t plus the fp32
  accumulation over the tokens and merged blocks.
Cases: a ragged T with a fully masked wave (GQA group 4, two new tokens), an
MHA shape (40 heads, one query per head), a Tucker and a no-Tucker record, and
the Mistral-shaped layer at T = 4096 and T = 32768.
"""
import numpy as np
import pytest
import torch

import kvgen
from oracle import attention, codec, quant, rotation

from gpu_util import D, pack_record

pytestmark = pytest.mark.gpu

E_EXP = 2.0 ** -20


@pytest.fixture(scope="module")
def J():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_compression_mode_amd import jolt
    return jolt


def _record(X, choice, Q, R):
    if choice[0] > 0:
        a = codec.analyze(X, R)
        enc = codec.encode_tensor(X, a["U_T"], a["U_D"], choice, Q)
    else:
        enc = codec.encode_tensor(X, None, None, choice, Q)
    exact = codec.decode_exact(enc, Q)
    # the decode kernel's error bound per element
    H, T, _ = X.shape
    r_T, r_D, _ = choice
    Yh = quant.dequantize(enc["m16"], enc["s16"], enc["codes"]).reshape(H, T, D)
    rot = np.abs(Yh).reshape(-1, D) @ np.abs(Q)
    rot = rot.reshape(H, T, D)
    rec = np.zeros_like(rot)
    if r_T > 0:
        rec = np.einsum("tr,hrs,ds->htd", np.abs(enc["U_T"]), np.abs(enc["G"]), np.abs(enc["U_D"]), optimize=True)
    bound = (r_T + r_D + D + 8) * 2.0 ** -24 * (rec + rot) + 2.0 ** -15 * rec + 2.0 ** -8 * rot
    return enc, exact, bound


def _queries(K, G, n_new, seed):
    """Half the vectors random (diffuse weights), half aligned with one cached
    key each (one dominant weight)."""
    H, T, _ = K.shape
    r = np.random.default_rng(seed)
    q = 0.3 * r.standard_normal((H * G, n_new, D))
    for hq in range(H * G):
        for s in range(n_new):
            if (hq + s) % 2:
                t = r.integers(0, T)
                k = K[hq // G, t]
                q[hq, s] += 0.05 * k
    return q.astype(np.float32).astype(np.float64)


def _bound(q, Kx, Vx, bK, bV, G, n_blk):
    Hq, n, _ = q.shape
    out = np.empty((Hq, n, D))
    for hq in range(Hq):
        h = hq // G
        s = q[hq] @ Kx[h].T / np.sqrt(D)
        ds = np.abs(q[hq]) @ bK[h].T / np.sqrt(D) + (D + 4) * 2.0 ** -24 * (np.abs(q[hq]) @ np.abs(Kx[h]).T) / np.sqrt(D)
        p = attention.softmax_rows(s)
        dp1 = 2.0 * (ds.max(axis=1) + E_EXP) * 1.01                      # [n]
        vmax = np.abs(Vx[h]).max(axis=0)                                  # [D]
        acc = (40 + n_blk) * 2.0 ** -24 + 3 * E_EXP
        out[hq] = dp1[:, None] * vmax[None, :] + p @ bV[h] + acc * (p @ np.abs(Vx[h]))
    return out


CASES = [
    # H, T, G, n_new, choice K, choice V
    (8, 700, 4, 2, (64, 48, 3), (0, 0, 2)),
    (40, 300, 1, 1, (32, 128, 4), (96, 64, 2)),
    (8, 4096, 4, 1, (192, 128, 4), (128, 128, 4)),
    (8, 32768, 4, 1, (160, 128, 3), (160, 96, 3)),
]


@pytest.mark.parametrize("H,T,G,n_new,ck,cv", CASES)
def test_attend_matches_oracle(J, H, T, G, n_new, ck, cv):
    Q = rotation.rotation(0, D)
    rot = J.rotation(0)
    R = max(ck[0], cv[0], 1)
    Xk = kvgen.tensor(H, T, D, seed=41, layer=0, kind=0, decay=0.9, dtype="bf16").astype(np.float64)
    Xv = kvgen.tensor(H, T, D, seed=41, layer=0, kind=1, decay=0.88, dtype="bf16").astype(np.float64)
    encK, Kx, bK = _record(Xk, ck, Q, R)
    encV, Vx, bV = _record(Xv, cv, Q, R)
    recK, recV = pack_record(encK), pack_record(encV)
    q = _queries(Kx, G, n_new, seed=T)
    ref = attention.attend(q, Kx, Vx, G)
    n_blk = (T + 255) // 256
    bnd = _bound(q, Kx, Vx, bK, bV, G, n_blk)
    bk = torch.from_numpy(recK).cuda()
    bv = torch.from_numpy(recV).cuda()
    qd = torch.from_numpy(q.astype(np.float32)).cuda()
    out = J.attend(bk, ck, bv, cv, H, T, qd, G, rot)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bnd), float(np.max(err / bnd))
