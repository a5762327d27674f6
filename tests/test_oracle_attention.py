"""Pins of the oracle's attention over a decoded cache (oracle/attention.py):
closed forms and invariants, CPU only.

* One cached token: the output is that token's V row.
* Zero queries (uniform weights): the output is the mean of V over tokens.
* Two tokens: the weight of the first is 1 / (1 + exp(s_2 - s_1)) with the
  scores s = q . k / sqrt(D) written out.
* Permuting the tokens (K and V rows together) leaves the output unchanged.
* GQA grouping: query head hq reads KV head hq // G (with uniform weights,
  each query head's output is the mean of its own KV head's V).
"""
import numpy as np

from oracle import attention


def test_single_token_returns_its_value_row():
    r = np.random.default_rng(1)
    q, K, V = r.standard_normal((2, 3, 16)), r.standard_normal((2, 1, 16)), r.standard_normal((2, 1, 16))
    out = attention.attend(q, K, V, 1)
    np.testing.assert_allclose(out, np.repeat(V, 3, axis=1), rtol=0, atol=1e-15)


def test_zero_queries_give_the_mean():
    r = np.random.default_rng(2)
    K, V = r.standard_normal((3, 7, 8)), r.standard_normal((3, 7, 8))
    out = attention.attend(np.zeros((3, 2, 8)), K, V, 1)
    np.testing.assert_allclose(out, np.repeat(V.mean(axis=1, keepdims=True), 2, axis=1), atol=1e-15)


def test_two_token_closed_form():
    D = 4
    q = np.array([[[1.0, 2.0, 0.0, -1.0]]])
    K = np.array([[[0.5, 0.0, 1.0, 0.0], [0.0, 1.0, 0.0, 3.0]]])
    V = np.array([[[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 1.0]]])
    s1 = (1.0 * 0.5) / 2.0                       # sqrt(4) = 2
    s2 = (2.0 * 1.0 - 1.0 * 3.0) / 2.0
    w1 = 1.0 / (1.0 + np.exp(s2 - s1))
    out = attention.attend(q, K, V, 1)
    np.testing.assert_allclose(out[0, 0], [w1, 0.0, 0.0, 1.0 - w1], atol=1e-15)


def test_token_permutation_invariance():
    r = np.random.default_rng(3)
    q, K, V = r.standard_normal((4, 2, 32)), r.standard_normal((2, 50, 32)), r.standard_normal((2, 50, 32))
    perm = r.permutation(50)
    np.testing.assert_allclose(attention.attend(q, K, V, 2), attention.attend(q, K[:, perm], V[:, perm], 2),
                               atol=1e-12)


def test_gqa_group_mapping():
    r = np.random.default_rng(4)
    H, G, T, D = 3, 4, 9, 8
    V = r.standard_normal((H, T, D))
    out = attention.attend(np.zeros((H * G, 1, D)), r.standard_normal((H, T, D)), V, G)
    for hq in range(H * G):
        np.testing.assert_allclose(out[hq, 0], V[hq // G].mean(axis=0), atol=1e-14)
