"""Pins for the oracle's counter-based generator (SplitMix64 + Box-Muller)."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed1234567.txt")


def _golden():
    with open(GOLDEN) as f:
        return [int(l) for l in f if l.strip() and not l.startswith("#")]


def test_splitmix64_published_vectors():
    # published outputs of the reference SplitMix64 generator, state 1234567
    assert [int(w) for w in rng.sequence(1234567, 0, 5)] == _golden()


def test_sequence_offset_and_scalar_agree():
    full = rng.sequence(987654321, 0, 40)
    part = rng.sequence(987654321, 17, 9)
    assert np.array_equal(full[17:26], part)
    s = 987654321
    for i in range(40):
        s = (s + rng.GAMMA) & rng.MASK64
        assert rng.mix64(s) == int(full[i])


def test_words_use_mixed_key():
    w = rng.words(5, rng.TAG_ROTATION, 0, 4)
    key = rng.mix64(5 ^ rng.TAG_ROTATION)
    assert np.array_equal(w, rng.sequence(key, 0, 4))
    # different streams and seeds differ
    assert not np.array_equal(w, rng.words(5, rng.TAG_SKETCH, 0, 4))
    assert not np.array_equal(w, rng.words(6, rng.TAG_ROTATION, 0, 4))


def test_uniform_is_top53_bits_plus_half():
    w = rng.words(3, 77, 0, 1000)
    u = rng.uniforms(3, 77, 0, 1000)
    for wi, ui in zip(w[:50], u[:50]):
        assert ui == ((int(wi) >> 11) + 0.5) / 2.0 ** 53
    assert u.min() > 0.0 and u.max() < 1.0


def test_box_muller_pairs_identity():
    # z0^2 + z1^2 = -2 ln u1 and atan2(z1, z0) = 2 pi u2 (mod 2 pi) per pair
    n = 2000
    z = rng.normals(11, 99, n)
    u = rng.uniforms(11, 99, 0, n)
    r2 = z[0::2] ** 2 + z[1::2] ** 2
    np.testing.assert_allclose(r2, -2.0 * np.log(u[0::2]), rtol=1e-13, atol=1e-13)
    ang = np.mod(np.arctan2(z[1::2], z[0::2]), 2 * np.pi)
    d = np.abs(ang - 2 * np.pi * u[1::2])
    d = np.minimum(d, 2 * np.pi - d)
    assert d.max() < 1e-9


def test_odd_count_is_prefix():
    a = rng.normals(1, 2, 7)
    b = rng.normals(1, 2, 8)
    assert np.array_equal(a, b[:7])


def test_normals_are_standard_normal():
    z = rng.normals(0, rng.TAG_SKETCH, 200000)
    assert abs(z.mean()) < 0.01
    assert abs(z.var() - 1.0) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # no lag-1 correlation between consecutive elements (pairs or across pairs)
    c = np.corrcoef(z[:-1], z[1:])[0, 1]
    assert abs(c) < 0.01


def test_tensor_tag():
    assert rng.tensor_tag(rng.TAG_SKETCH, 3, 1) == rng.TAG_SKETCH ^ (3 << 8 | 1)
