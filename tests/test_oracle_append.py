"""Pins of the oracle's incremental encode (oracle/append.py), CPU only.

* New rows inside the row space of W (X_new,(T) = C W) fold in exactly:
  the solution is C, and the reconstruction reproduces them.
* The normal equations: the unrounded residual X_new,(T) - U_new W is
  orthogonal to every row of W.
* W stacks the heads' G_h U_D^T side by side (hand-built 2-head case).
* No coefficient choice does better: the fold-in residual is at most the
  residual of random perturbations of the solution, and of U = 0.
* End to end on a synthetic tensor: tokens appended from the same
  low-rank-plus-noise source decode to an error close to the base tokens'.
"""
import numpy as np

import kvgen
from oracle import append, codec, rotation, tucker


def _base(H=2, T=96, D=32, rT=12, rD=8, seed=3):
    X = kvgen.tensor(H, T + 24, D, seed=seed, decay=0.8, rank=6, dtype="f32").astype(np.float64)
    a = codec.analyze(X[:, :T], rT)
    Q = rotation.rotation(0, D)
    return X, codec.encode_tensor(X[:, :T], a["U_T"], a["U_D"], (rT, rD, 4), Q), Q


def test_stacked_w_hand_built():
    G = np.arange(2 * 2 * 3, dtype=np.float64).reshape(2, 2, 3)
    Ud = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, 1.0], [1.0, 1.0, 0]])     # D = 4, r_D = 3
    W = append.stacked_w(G, Ud)
    assert W.shape == (2, 8)
    np.testing.assert_array_equal(W[:, :4], G[0] @ Ud.T)
    np.testing.assert_array_equal(W[:, 4:], G[1] @ Ud.T)
    np.testing.assert_array_equal(W[1, 4:], [9.0, 10.0, 11.0, 19.0])


def test_rows_in_row_space_fold_in_exactly():
    X, base, Q = _base()
    W = append.stacked_w(base["G"], base["U_D"])
    C = np.random.default_rng(1).standard_normal((5, W.shape[0]))
    H, D = base["G"].shape[0], base["U_D"].shape[0]
    Xn = (C @ W).reshape(5, H, D).transpose(1, 0, 2)            # X_new,(T) = C W
    U = append.fold_in_rows(Xn, base["G"], base["U_D"])
    np.testing.assert_allclose(U, C, atol=1e-9 * np.abs(C).max())
    np.testing.assert_allclose(tucker.reconstruct(base["G"], U, base["U_D"]), Xn, atol=1e-9 * np.abs(Xn).max())


def test_normal_equations_and_optimality():
    X, base, Q = _base()
    Xn = X[:, 96:]
    U = append.fold_in_rows(Xn, base["G"], base["U_D"])
    W = append.stacked_w(base["G"], base["U_D"])
    R = tucker.unfold_T(Xn) - U @ W
    assert np.abs(R @ W.T).max() <= 1e-9 * np.abs(tucker.unfold_T(Xn)).max() * np.abs(W).max() * W.shape[1]
    best = float(np.sum(R ** 2))
    r = np.random.default_rng(2)
    for _ in range(5):
        Up = U + 1e-3 * r.standard_normal(U.shape)
        assert float(np.sum((tucker.unfold_T(Xn) - Up @ W) ** 2)) >= best
    assert float(np.sum(tucker.unfold_T(Xn) ** 2)) >= best


def test_appended_tokens_decode_close_to_base_tokens():
    cfg = kvgen.CONFIGS["mistral7b_t4096_2x"]
    X = kvgen.tensor(cfg.H, 1024 + 128, cfg.D, seed=5, decay=0.9, dtype="bf16").astype(np.float64)
    Xb, Xn = X[:, :1024], X[:, 1024:]
    a = codec.analyze(Xb, 192)
    Q = rotation.rotation(0, cfg.D)
    base = codec.encode_tensor(Xb, a["U_T"], a["U_D"], (192, 128, 4), Q)
    e_base = codec.rel_err(Xb, codec.decode_tensor(base, Q, "bf16"))
    ext = append.append_encode(Xn, base, Q)
    e_new = codec.rel_err(Xn, codec.decode_tensor(ext, Q, "bf16"))
    # the new tokens' signal lies in the base's factor subspaces: only the
    # noise is left for the residual, as for the base tokens
    assert e_new < 2.0 * e_base, (e_new, e_base)
    # against quantizing the new tokens alone (no Tucker part) at the same bits
    e_q = codec.rel_err(Xn, codec.decode_tensor(codec.encode_tensor(Xn, None, None, (0, 0, 4), Q), Q, "bf16"))
    assert e_new < 0.2 * e_q, (e_new, e_q)
