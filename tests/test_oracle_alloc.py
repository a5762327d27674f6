"""Pins for the oracle's byte model, distortion model and Lagrangian-dual
allocation."""
import itertools

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import alloc, quant


def test_kappa_by_quadrature():
    # kappa = E[(max - min)^2] of 32 iid N(0,1) = integral of 2 r P(range > r)
    n = 32
    phi, Phi = stats.norm.pdf, stats.norm.cdf

    def cdf_range(r):
        f = lambda x: phi(x) * (Phi(x + r) - Phi(x)) ** (n - 1)
        return n * integrate.quad(f, -12, 12, limit=300, epsabs=1e-13)[0]

    k = integrate.quad(lambda r: 2 * r * (1 - cdf_range(r)), 0, 20, limit=300,
                       epsabs=1e-11)[0]
    assert abs(k - alloc.KAPPA_32) < 1e-8


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rho_matches_min_max_quantizer_on_gaussians(bits):
    # rho(b) = kappa / (12 (2^b-1)^2) predicts the MSE of the oracle's
    # quantizer on unit Gaussians (uniform-error model; not valid at b = 1)
    z = np.random.default_rng(bits).standard_normal((20000, 128)).astype(np.float32)
    m16, s16, c = quant.quantize(z, bits)
    mse = np.mean((quant.dequantize(m16, s16, c) - z) ** 2)
    assert abs(mse / alloc.rho(bits) - 1) < 0.08


def test_blob_bytes_hand_worked():
    # H=8 T=1024 D=128, r=(256, 64), b=2: U_T 524288 + U_D 16384 + core 262144
    # + scales 131072 + codes 262144 = 1196032, plus the 256-byte header block
    assert alloc.blob_bytes(8, 1024, 128, 256, 64, 2) == 256 + 1196032
    # no Tucker part: header + scales + codes
    assert alloc.blob_bytes(8, 1024, 128, 0, 0, 4) == 256 + 131072 + 524288
    # sections are padded to 256 bytes
    assert alloc.blob_bytes(1, 32, 32, 1, 1, 1) == 256 + 256 * 5


@pytest.mark.parametrize("H,T,ratio,want", [(8, 4096, 2.0, 256), (8, 1024, 2.0, 256),
                                            (8, 32768, 3.0, 160), (40, 4096, 2.0, 1280)])
def test_rank_cap(H, T, ratio, want):
    assert alloc.rank_cap_T(H, T, 128, ratio) == want


def test_numerical_rank_and_tail():
    lam = [10.0, 1.0, 1e-9, 0.0]
    assert alloc.numerical_rank(lam, 4) == 3            # threshold 8.9e-15 < 1e-9
    assert alloc.numerical_rank(lam, 10 ** 7) == 2      # threshold 2.2e-8 > 1e-9
    assert alloc.tail(lam, 11.0, 0) == 11.0
    assert alloc.tail(lam, 11.0, 1) == 1.0
    assert alloc.tail(lam, 11.0, 4) == 0.0


def test_lower_hull_small():
    pts = [(1, 10.0, 0), (2, 6.0, 1), (3, 5.0, 2), (4, 1.0, 3), (4, 2.0, 4), (5, 1.5, 5)]
    h = alloc.lower_hull(pts)
    # (3, 5) lies above the chord (2,6)-(4,1); (5, 1.5) does not lower distortion
    assert [p[2] for p in h] == [0, 1, 3]


def _spectra(rng, n_layers, T, D, decay_lo=0.7, decay_hi=0.97):
    out = []
    for l in range(n_layers):
        row = []
        for k in (0, 1):
            dt = rng.uniform(decay_lo, decay_hi)
            lamT = 1e4 * dt ** np.arange(T) + rng.uniform(5.0, 15.0)   # above the rank floor
            f2 = float(lamT.sum())
            dd = rng.uniform(decay_lo, decay_hi)
            lamD = dd ** np.arange(D) + 0.01                              # full numerical rank
            lamD = lamD * (f2 / lamD.sum())
            row.append((lamT, lamD, f2))
        out.append(row)
    return out


def _brute(spectra, n_layers, H, T, D, ratio, bits, g, stT, stD):
    cap = alloc.rank_cap_T(H, T, D, ratio, stT)
    units = []
    for grp in range((n_layers + g - 1) // g):
        layers = range(grp * g, min(n_layers, grp * g + g))
        for k in (0, 1):
            m = alloc.menu(cap, D, bits, stT, stD)
            pts = [(len(layers) * alloc.blob_bytes(H, T, D, *c),
                    sum(alloc.layer_distortion(*spectra[l][k], c) for l in layers))
                   for c in m]
            units.append(pts)
    best = {}
    for combo in itertools.product(*units):
        b = sum(p[0] for p in combo)
        d = sum(p[1] for p in combo)
        best[b] = min(best.get(b, np.inf), d)
    return best


@pytest.mark.parametrize("seed,ratio", [(0, 2.0), (1, 2.5), (2, 3.0), (3, 1.6)])
def test_dual_is_optimal_at_its_own_bytes(seed, ratio):
    H, T, D, bits, g, stT, stD = 8, 1024, 128, (2, 4), 2, 128, 64
    sp = _spectra(np.random.default_rng(seed), 4, T, D)
    plan = alloc.allocate(sp, 4, H, T, D, ratio, bits, g, 0, stT, stD)
    assert plan["total_bytes"] <= plan["budget"]
    best = _brute(sp, 4, H, T, D, ratio, bits, g, stT, stD)
    cheaper = [d for b, d in best.items() if b <= plan["total_bytes"]]
    assert min(cheaper) >= plan["objective"] - 1e-12 * max(1.0, plan["objective"])
    # the per-tensor bytes add up and K/V of a group share nothing but the budget
    assert sum(plan["tensor_bytes"].values()) == plan["total_bytes"]


def test_distortion_monotone_in_budget():
    H, T, D = 8, 1024, 128
    sp = _spectra(np.random.default_rng(7), 8, T, D)
    prev = np.inf
    for ratio in (4.0, 3.0, 2.5, 2.0, 1.5):
        plan = alloc.allocate(sp, 8, H, T, D, ratio, (1, 2, 3, 4), 4, 256)
        assert plan["objective"] <= prev + 1e-15
        prev = plan["objective"]


def test_infeasible_budget_raises():
    sp = _spectra(np.random.default_rng(8), 4, 1024, 128)
    with pytest.raises(alloc.BudgetError):
        alloc.allocate(sp, 4, 8, 1024, 128, 40.0, (1, 2), 4)


def test_k_and_v_choose_separately():
    # K with a fast-decaying spectrum, V with a flat one: the plan differs
    H, T, D = 8, 1024, 128
    f2 = 1e6
    kT = 0.9 ** np.arange(T) + 1e-3
    kT *= f2 / kT.sum()
    vT = np.full(T, f2 / T)
    kD = 0.7 ** np.arange(D) + 1e-3
    kD *= f2 / kD.sum()
    vD = np.full(D, f2 / D)
    sp = [[(kT, kD, f2), (vT, vD, f2)] for _ in range(4)]
    plan = alloc.allocate(sp, 4, H, T, D, 2.0, (1, 2, 3, 4), 4)
    ck, cv = plan["choice"][(0, 0)], plan["choice"][(0, 1)]
    assert ck != cv
    assert ck[0] > 0 and cv[0] == 0            # low-rank K uses Tucker, flat V does not
