"""Pins for the oracle's bf16 rounding, group quantizer and bit packing."""
import numpy as np
import pytest

from oracle import bf16, quant


def _all_finite_bf16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    v = v[np.isfinite(v)]
    return np.unique(v)           # sorted, -0 and +0 merged


BF = _all_finite_bf16()


def _random_f32(n, seed):
    r = np.random.default_rng(seed)
    mant = r.uniform(-2.0, 2.0, n)
    ex = r.integers(-140, 120, n).astype(np.float64)
    x = (mant * 2.0 ** ex).astype(np.float32)
    # include exact bf16 values and zeros
    x[:50] = BF[r.integers(0, len(BF), 50)].astype(np.float32)
    x[50] = 0.0
    return x


def test_round_down_up_brute_force():
    x = _random_f32(20000, 1).astype(np.float64)
    down = bf16.round_down(x.astype(np.float32))
    up = bf16.round_up(x.astype(np.float32))
    i = np.searchsorted(BF, x, side="right") - 1       # largest bf16 <= x
    j = np.searchsorted(BF, x, side="left")            # smallest bf16 >= x
    np.testing.assert_array_equal(down, BF[i])
    np.testing.assert_array_equal(up, BF[j])


def test_round_nearest_brute_force():
    r = np.random.default_rng(2)
    x = r.uniform(-3, 3, 20000) * 2.0 ** r.integers(-135, 120, 20000)
    # exact midpoints between neighbours (ties), both signs
    k = r.integers(0, len(BF) - 1, 2000)
    mids = (BF[k] + BF[k + 1]) / 2.0
    x = np.concatenate([x, mids, BF[k]])
    got = bf16.round_nearest(x)
    j = np.clip(np.searchsorted(BF, x), 1, len(BF) - 1)
    lo, hi = BF[j - 1], BF[j]
    dlo, dhi = x - lo, hi - x
    even_hi = (bf16.to_bits(hi) & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(even_hi, hi, lo)))
    want = np.where(x == hi, hi, want)
    np.testing.assert_array_equal(np.abs(got), np.abs(want))
    assert np.all((got == 0) | (np.sign(got) == np.sign(x)))


def test_bits_round_trip():
    v = BF[::97]
    np.testing.assert_array_equal(bf16.from_bits(bf16.to_bits(v)), v)


def _group(vals, fill):
    g = np.full(32, fill, dtype=np.float32)
    g[: len(vals)] = vals
    return g[None, :]


def test_hand_worked_group_two_bits():
    # min -1.5, max 1.5: m16 = -1.5, s32 = 3/3 = 1, s16 = 1; code = rint(y + 1.5)
    # with ties to even: 0.0 -> rint(1.5) = 2, 1.0 -> rint(2.5) = 2, -1.0 -> rint(0.5) = 0
    vals = [-1.5, -0.5, 0.0, 0.5, 1.0, 1.5, -1.0]
    m16, s16, codes = quant.quantize(_group(vals, 0.25), 2)
    assert m16[0, 0] == -1.5 and s16[0, 0] == 1.0
    assert list(codes[0, 0, :7]) == [0, 1, 2, 2, 2, 3, 0]
    assert np.all(codes[0, 0, 7:] == 2)                  # rint(1.75) = 2


def test_constant_group_has_zero_step():
    m16, s16, codes = quant.quantize(np.full((1, 32), 3.0, np.float32), 1)
    assert m16[0, 0] == 3.0 and s16[0, 0] == 0.0 and np.all(codes == 0)
    np.testing.assert_array_equal(quant.dequantize(m16, s16, codes), np.full((1, 32), 3.0))


def test_offset_rounds_toward_minus_inf():
    # -(1 + 2^-8) is not a bf16; the next bf16 below it is -(1 + 2^-7)
    g = _group([-(1 + 2.0 ** -8), 2.0], 0.0)
    m16, s16, codes = quant.quantize(g, 4)
    assert m16[0, 0] == -(1 + 2.0 ** -7)
    s32 = np.float32(np.float32(2.0) - np.float32(m16[0, 0])) / np.float32(15)
    assert s16[0, 0] >= s32 and s16[0, 0] in BF
    assert BF[np.searchsorted(BF, s16[0, 0]) - 1] < s32


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_quantizer_invariants(bits):
    r = np.random.default_rng(bits)
    Y = (r.standard_normal((300, 128)) * r.uniform(0.01, 100, (300, 1))).astype(np.float32)
    Y[:5] *= 1e-38                                       # subnormal-range groups
    m16, s16, codes = quant.quantize(Y, bits)
    L = 2 ** bits - 1
    assert codes.max() <= L
    g = Y.reshape(300, 4, 32).astype(np.float64)
    mn, mx = g.min(-1), g.max(-1)
    # offset: largest bf16 <= min; step: a bf16, grid covers the group
    i = np.searchsorted(BF, mn, side="right") - 1
    np.testing.assert_array_equal(m16, BF[i])
    assert np.all(np.isin(s16, BF))
    assert np.all(m16 + L * s16 >= mx * (1 - 2.0 ** -22) - 1e-45)
    # every element within half a step (+2 ulp of y) of its level
    yh = quant.dequantize(m16, s16, codes).reshape(300, 4, 32)
    ulp = np.spacing(np.abs(g).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(g - yh) <= s16[..., None] / 2 + 2 * ulp)
    # brute force: the chosen level is a nearest level (ties either way)
    levels = m16[..., None, None] + np.arange(L + 1) * s16[..., None, None]   # [300,4,1,L+1]
    dist = np.abs(g[..., None] - levels)
    best = dist.min(-1)
    chosen = np.take_along_axis(dist, codes[..., None].astype(np.int64), -1)[..., 0]
    assert np.all(chosen <= best + 2 * ulp)


def test_pack_hand_worked_bytes():
    c = np.zeros(32, np.uint8)
    c[:6] = [1, 2, 3, 4, 5, 6]
    p3 = quant.pack(c, 3)
    assert p3.shape == (12,)
    # stream bits: 100 010 110 001 101 011 -> byte0 = 0b11010001, byte1 = 0b01011000
    assert p3[0] == 209 and p3[1] == 88
    c4 = np.arange(32, dtype=np.uint8) % 16
    p4 = quant.pack(c4, 4)
    np.testing.assert_array_equal(p4, (c4[0::2] | (c4[1::2] << 4)).astype(np.uint8))
    c1 = (np.arange(32) % 3 == 0).astype(np.uint8)
    p1 = quant.pack(c1, 1)
    want = [sum(int(c1[8 * j + i]) << i for i in range(8)) for j in range(4)]
    assert list(p1) == want
    c2 = (np.arange(32) % 4).astype(np.uint8)
    p2 = quant.pack(c2, 2)
    want = [sum(int(c2[4 * j + i]) << (2 * i) for i in range(4)) for j in range(8)]
    assert list(p2) == want


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_round_trip(bits):
    r = np.random.default_rng(10 + bits)
    c = r.integers(0, 2 ** bits, (7, 4, 32)).astype(np.uint8)
    p = quant.pack(c, bits)
    assert p.shape == (7, 4, 4 * bits)
    np.testing.assert_array_equal(quant.unpack(p, bits), c)
