"""Joint Lagrangian-dual allocation of Tucker ranks and residual bits (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2): one Lagrangian dual allocates the
Tucker ranks and the residual bit-widths together, per layer group and
separately for keys and values, under one byte budget; news article
paragraph 2 (per layer group, K/V budgets separate).  Everything below the
sentence level is a reading:

Units.  A unit is (layer group g, kind in {K, V}); group g holds layers
4g .. 4g+3 (the last group may be shorter).  Every layer keeps its own
factors; a unit shares only its choice (r_T, r_D, b).

Menu.  (0, 0, b) (no Tucker, the residual is X itself) and
(r_T, r_D, b) with r_T in {s_T, 2 s_T, ..., R_T}, r_D in {s_D, ..., R_D},
b in the bit menu; default steps s_T = 32, s_D = 16.  R_T is the smallest of
T, HD, floor(Bbar / (4 T)) rounded down to a multiple of s_T (Bbar = 2N/ratio,
the average per-tensor budget: U_T alone may take at most half of it) and the
numerical rank of every layer's token spectrum; R_D is the smallest of D and
the layers' feature numerical ranks.  Numerical rank counts eigenvalues above
n * 2^-52 * lambda_1 (n = the Gram's dimension, min(T, HD) or D): it only
drops directions that carry no energy at the precision of the fp64 spectra
the dual reads.  (A cap at fp32 resolution, n * 2^-23 * lambda_1, would cut
the whole noise bulk of a cache, whose eigenvalues sit near 1e-6 lambda_1 yet
hold most of the truncation energy, and leave only no-Tucker plans.)  Only the leading R_T token eigenvalues are ever read, so a
spectrum truncated after them gives the same plan.

Bytes.  The compressed record size (see ``blob_bytes``); the budget is
floor(2 * N_total / ratio), i.e. relative to bf16 storage.

Distortion (predicted relative squared error of one layer).
    d = rho(b) * min(1, (E_T(r_T) + E_D(r_D)) / ||X||^2),
    E_m(r) = ||X||^2 - sum_{i<r} lambda_{m,i}   (HOSVD truncation bound),
    rho(b) = kappa / (12 (2^b - 1)^2),
kappa = E[(max - min)^2] of 32 iid N(0, 1): the rotated residual is close to
Gaussian (news article paragraph 4: the rotation whitens it), a min-max grid
of step (max-min)/L leaves a uniform error of variance step^2/12.  A unit's
distortion is the sum over its layers; the objective is the sum over units.

Dual.  Per unit, the lower convex hull of its (bytes, distortion) points with
strictly decreasing distortion.  Start every unit at its cheapest point;
order all hull segments by slope (distortion saved per byte) descending, ties
to the lower unit index, then the lower start bytes; apply segments while the
total stays within budget and stop at the first one that does not fit.  This
is the solution of the Lagrangian relaxation at the multiplier equal to that
slope (Everett, Operations Research 1963).  If the cheapest plan is already
over budget the request is infeasible.
"""
from __future__ import annotations

import math

KAPPA_32 = 17.60642599755      # E[(max-min)^2], 32 iid N(0,1); two quadratures agree to 1e-12
ALIGN = 256
HEADER_BLOCK = 256
GROUP = 32


class BudgetError(ValueError):
    pass


def rho(bits: int) -> float:
    L = (1 << bits) - 1
    return KAPPA_32 / (12.0 * float(L * L))


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


def blob_bytes(H: int, T: int, D: int, r_T: int, r_D: int, bits: int) -> int:
    """Size of one compressed tensor record.

    A 64-byte header padded to 256, then 256-aligned sections: U_T bf16
    [T, r_T], U_D bf16 [D, r_D], core bf16 [H, r_T, r_D], per-group (offset,
    step) bf16 pairs [H, T, D/32, 2], codes [H, T, D/32, 4b] bytes.
    """
    N = H * T * D
    groups = N // GROUP
    return (HEADER_BLOCK + _align(2 * T * r_T) + _align(2 * D * r_D)
            + _align(2 * H * r_T * r_D) + _align(4 * groups)
            + _align(4 * bits * groups))


def rank_cap_T(H: int, T: int, D: int, ratio: float, step: int = 32) -> int:
    N = H * T * D
    bbar = 2.0 * N / ratio
    q = int(math.floor(bbar / (4.0 * T)))
    return min(T, H * D, (q // step) * step)


def numerical_rank(lam, n: int) -> int:
    """Count of eigenvalues above n * 2^-52 * lambda_1 (n = Gram dimension)."""
    lam = [float(v) for v in lam]
    if not lam or lam[0] <= 0.0:
        return 0
    thr = float(n) * (2.0 ** -52) * lam[0]
    return sum(1 for v in lam if v > thr)


def tail(lam, frob2: float, r: int) -> float:
    s = 0.0
    for i in range(min(r, len(lam))):
        s += float(lam[i])
    return max(0.0, float(frob2) - s)


def layer_distortion(lam_T, lam_D, frob2: float, choice) -> float:
    r_T, r_D, b = choice
    if frob2 <= 0.0:
        return 0.0
    e = (tail(lam_T, frob2, r_T) + tail(lam_D, frob2, r_D)) / frob2
    return rho(b) * min(1.0, e)


def menu(R_T: int, R_D: int, bits, step_T: int = 32, step_D: int = 16):
    out = [(0, 0, b) for b in bits]
    for rt in range(step_T, R_T + 1, step_T):
        for rd in range(step_D, R_D + 1, step_D):
            for b in bits:
                out.append((rt, rd, b))
    return out


def lower_hull(points):
    """points: list of (bytes, distortion, menu index); returns hull list."""
    pts = sorted(points, key=lambda p: (p[0], p[1], p[2]))
    hull = []
    for p in pts:
        if hull and p[1] >= hull[-1][1]:
            continue
        while len(hull) >= 2:
            a, b = hull[-2], hull[-1]
            cross = (float(b[0] - a[0]) * (p[1] - a[1])
                     - (b[1] - a[1]) * float(p[0] - a[0]))
            if cross <= 0.0:
                hull.pop()
            else:
                break
        hull.append(p)
    return hull


def allocate(spectra, n_layers: int, H: int, T: int, D: int, ratio: float,
             bits=(1, 2, 3, 4), group_layers: int = 4, r_T_cap: int = 0,
             step_T: int = 32, step_D: int = 16):
    """Lagrangian-dual plan for a whole cache.

    spectra[layer][kind] = (lam_T, lam_D, frob2), kind 0 = K, 1 = V.
    Returns dict(choice={(g, kind): (r_T, r_D, b)}, total_bytes, objective,
    budget, tensor_bytes={(layer, kind): bytes}).
    """
    N = H * T * D
    n_total = N * 2 * n_layers
    budget = int(math.floor(2.0 * n_total / ratio))
    cap = r_T_cap if r_T_cap > 0 else rank_cap_T(H, T, D, ratio, step_T)
    n_T = min(T, H * D)
    n_groups = (n_layers + group_layers - 1) // group_layers
    units = []
    for g in range(n_groups):
        layers = list(range(g * group_layers, min(n_layers, (g + 1) * group_layers)))
        for kind in (0, 1):
            specs = [spectra[l][kind] for l in layers]
            R_T = min([cap] + [numerical_rank(s[0], n_T) for s in specs])
            R_D = min([D] + [numerical_rank(s[1], D) for s in specs])
            m = menu(R_T, R_D, bits, step_T, step_D)
            pts = []
            for i, ch in enumerate(m):
                nbytes = len(layers) * blob_bytes(H, T, D, *ch)
                dist = 0.0
                for s in specs:
                    dist += layer_distortion(s[0], s[1], s[2], ch)
                pts.append((nbytes, dist, i))
            units.append(((g, kind), layers, m, lower_hull(pts)))
    pos = [0] * len(units)
    total = sum(u[3][0][0] for u in units)
    if total > budget:
        raise BudgetError(f"cheapest plan needs {total} bytes > budget {budget}")
    segs = []
    for ui, u in enumerate(units):
        hull = u[3]
        for k in range(len(hull) - 1):
            dB = float(hull[k + 1][0] - hull[k][0])
            dD = hull[k][1] - hull[k + 1][1]
            segs.append((dD / dB, ui, hull[k][0], k))
    segs.sort(key=lambda s: (-s[0], s[1], s[2]))
    for slope, ui, _, k in segs:
        hull = units[ui][3]
        assert pos[ui] == k
        step = hull[k + 1][0] - hull[k][0]
        if total + step > budget:
            break
        total += step
        pos[ui] = k + 1
    choice, tensor_bytes = {}, {}
    objective = 0.0
    for ui, u in enumerate(units):
        key, layers, m, hull = u
        pt = hull[pos[ui]]
        ch = m[pt[2]]
        choice[key] = ch
        objective += pt[1]
        for l in layers:
            tensor_bytes[(l, key[1])] = blob_bytes(H, T, D, *ch)
    return dict(choice=choice, total_bytes=total, objective=objective,
                budget=budget, tensor_bytes=tensor_bytes)
