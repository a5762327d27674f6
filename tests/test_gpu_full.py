"""GPU parity at the full sizes of the cache workloads, in the launch
configuration the benchmark times (one jolt_allocate over the whole cache,
jolt_encode per tensor, one batched jolt_decode_many or a layer-by-layer
stream), checked against the fp64 oracle on what it can compute one by one:

* the plan equals the oracle's dual run on the library's spectra, within the
  byte budget;
* on sampled tensors: spectra within 2e-5 lambda_1 of the oracle's, orthonormal
  factors, principal-angle sines <= 1e-3 at every resolvable cut, truncation
  (residual) energy within 0.5% of the oracle's at the planned ranks;
* on sampled (head, token) rows of those tensors: scales and codes equal to
  the oracle quantizer on the oracle's residual rows (flips only inside the
  fp32 error bound), decoded rows within the decode kernel's error bound;
* relative reconstruction error within 1e-4 of the oracle's encode of the
  whole tensor with the oracle's own fp64 factors (no value from the HIP path
  enters an oracle reference).
"""
import numpy as np
import pytest
import torch

import kvgen
from oracle import alloc, codec, rotation, tucker

from gpu_util import (D, check_codes, check_decode_rows, max_sine, oracle_rows, parse_blob,
                      record_rows, resolvable_cuts, sample_rows)

pytestmark = pytest.mark.gpu

N_ROWS = 384


@pytest.fixture(scope="module")
def J():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_compression_mode_amd import jolt
    return jolt


def _load(cfg):
    xs = [[None, None] for _ in range(cfg.n_layers)]
    items = [(l, k) for l in range(cfg.n_layers) for k in (0, 1)]
    for l, k, x in kvgen.generate(cfg, items, workers=8):
        xs[l][k] = torch.from_numpy(x).to(torch.bfloat16).cuda()
    torch.cuda.synchronize()
    return [tuple(p) for p in xs]


def _plan_matches_oracle(res, cfg):
    L = cfg.n_layers
    sp = [[(res.spectra_T[2 * l + k], res.spectra_D[2 * l + k], res.frob2[2 * l + k]) for k in (0, 1)]
          for l in range(L)]
    want = alloc.allocate(sp, L, cfg.H, cfg.T, cfg.D, cfg.ratio, cfg.bits, 4)
    assert res.choice == want["choice"] and res.total_bytes == want["total_bytes"]
    assert res.total_bytes <= res.budget_bytes


def _check_spectra(res, t, lam_T, lam_D, frob2):
    R = res.r_T_cap
    assert np.all(np.abs(res.spectra_T[t] - lam_T[:R]) <= 2e-5 * lam_T[0])
    assert np.all(np.abs(res.spectra_D[t] - lam_D) <= 2e-5 * lam_D[0])
    assert abs(res.frob2[t] - frob2) <= 1e-9 * frob2


def _check_factors(res, t, X, choice, lam_T, U_T_o=None, U_D_o=None, n_T=None):
    """Orthonormality, sines at resolvable cuts, residual energy at the choice."""
    Ut, Ud = (f.double().cpu().numpy() for f in res.factors(t))
    R = Ut.shape[1]
    assert np.abs(Ut.T @ Ut - np.eye(R)).max() < 1e-5
    assert np.abs(Ud.T @ Ud - np.eye(D)).max() < 1e-5
    if U_T_o is not None:
        for k in resolvable_cuts(lam_T, R, n_T):
            assert max_sine(Ut[:, :k], U_T_o[:, :k]) <= 1e-3, k
    r_T, r_D, _ = choice
    if r_T:
        f2 = float(np.sum(X * X))
        # residual energy of the token factor alone against the oracle's optimum
        XT = tucker.unfold_T(X)
        cap_g = float(np.sum((Ut[:, :r_T].T @ XT) ** 2))
        cap_o = float(np.sum(lam_T[:r_T]))
        assert abs((f2 - cap_g) - (f2 - cap_o)) <= 5e-3 * (f2 - cap_o), (f2 - cap_g, f2 - cap_o)
    return Ut, Ud


def _check_rows(X, blob, H, T, choice, Q, out, seed):
    parts = parse_blob(blob, H, T, choice)
    hs, ts = sample_rows(H, T, N_ROWS, seed)
    Y, bY = oracle_rows(X[hs, ts], parts, choice, Q, hs, ts)
    m16, s16, codes = record_rows(parts, hs, ts, choice[2])
    check_codes(m16, s16, codes, Y, bY, choice[2])
    got = out[torch.from_numpy(hs).cuda(), torch.from_numpy(ts).cuda()].float().cpu().numpy()
    check_decode_rows(got, parts, choice, Q, hs, ts, "bf16")
    return parts


def _err(x_host, xh):
    return codec.rel_err(x_host, xh.float().cpu().numpy())


def _encode_all(J, xs, res, rot, seed):
    blobs, choices = [], []
    for i in range(2 * len(xs)):
        ch = res.choice_of(i // 2, i % 2)
        Ut, Ud = res.factors(i)
        blobs.append(J.encode(xs[i // 2][i % 2], ch, Ut, Ud, rot, seed=seed))
        choices.append(ch)
    return blobs, choices


def test_full_mistral7b_t4096_2x(J):
    """32 layers x {K, V}, 8 KV heads, T = 4096, 2x, exact (dual 1024 x 1024 Gram)."""
    cfg = kvgen.CONFIGS["mistral7b_t4096_2x"]
    H, T = cfg.H, cfg.T
    xs = _load(cfg)
    rot = J.rotation(cfg.seed)
    Q = rotation.rotation(cfg.seed, D)
    res = J.allocate(xs, ratio=cfg.ratio, method=cfg.method, bits=cfg.bits, seed=cfg.seed)
    _plan_matches_oracle(res, cfg)
    blobs, choices = _encode_all(J, xs, res, rot, cfg.seed)
    outs = [torch.empty((H, T, D), dtype=torch.bfloat16, device="cuda") for _ in blobs]
    ws = torch.empty(J.decode_many_workspace_bytes(H, T, choices), dtype=torch.uint8, device="cuda")
    J.decode_many(blobs, H, T, choices, rot, outs, ws)
    torch.cuda.synchronize()
    for l, k in [(0, 0), (17, 1), (31, 0)]:
        t = 2 * l + k
        X = kvgen.config_tensor(cfg, l, k).astype(np.float64)
        a = codec.analyze(X, res.r_T_cap, "exact")
        _check_spectra(res, t, a["lam_T"], a["lam_D"], a["frob2"])
        _check_factors(res, t, X, choices[t], a["lam_T"], a["U_T"], a["U_D"], n_T=min(T, H * D))
        _check_rows(X, blobs[t], H, T, choices[t], Q, outs[t], seed=t)
        e_o = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, a["U_T"], a["U_D"], choices[t], Q),
                                                   Q, "bf16"))
        assert abs(_err(X, outs[t]) - e_o) < 1e-4, (l, k, _err(X, outs[t]), e_o)


def test_full_llama13b_t4096_2x(J):
    """40 layers x {K, V}, 40 heads, T = 4096, 2x, bits {1..4}, exact (direct
    4096 x 4096 token Gram, rank cap 1280)."""
    cfg = kvgen.CONFIGS["llama13b_t4096_2x"]
    H, T = cfg.H, cfg.T
    xs = _load(cfg)
    rot = J.rotation(cfg.seed)
    Q = rotation.rotation(cfg.seed, D)
    res = J.allocate(xs, ratio=cfg.ratio, method=cfg.method, bits=cfg.bits, seed=cfg.seed)
    assert res.r_T_cap == 1280
    _plan_matches_oracle(res, cfg)
    blobs, choices = _encode_all(J, xs, res, rot, cfg.seed)
    sampled = [(0, 0), (39, 1)]
    for l, k in sampled:
        t = 2 * l + k
        X = kvgen.config_tensor(cfg, l, k).astype(np.float64)
        # the oracle's own fp64 factors: eigh of the 4096 x 4096 token Gram
        a = codec.analyze(X, res.r_T_cap, "exact")
        _check_spectra(res, t, a["lam_T"], a["lam_D"], a["frob2"])
        _check_factors(res, t, X, choices[t], a["lam_T"], a["U_T"], a["U_D"], n_T=min(T, H * D))
        out = J.decode(blobs[t], H, T, choices[t], rot)
        torch.cuda.synchronize()
        _check_rows(X, blobs[t], H, T, choices[t], Q, out, seed=t)
        # the oracle's encode and decode with its own factors
        e_o = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, a["U_T"], a["U_D"], choices[t], Q),
                                                   Q, "bf16"))
        assert abs(_err(X, out) - e_o) < 1e-4, (l, k, _err(X, out), e_o)


@pytest.mark.parametrize("method", ["exact", "flash"])
def test_full_mistral7b_t1024(J, method):
    """The FlashJoLT comparison workload: 32 layers x {K, V}, T = 1024, 2x,
    exact (direct 1024 x 1024 Gram) and randomized (p = 10, q = 1)."""
    cfg = kvgen.CONFIGS["mistral7b_t1024_flash"]
    H, T = cfg.H, cfg.T
    xs = _load(cfg)
    rot = J.rotation(cfg.seed)
    Q = rotation.rotation(cfg.seed, D)
    res = J.allocate(xs, ratio=cfg.ratio, method=method, bits=cfg.bits, seed=cfg.seed)
    _plan_matches_oracle(res, cfg)
    blobs, choices = _encode_all(J, xs, res, rot, cfg.seed)
    outs = [torch.empty((H, T, D), dtype=torch.bfloat16, device="cuda") for _ in blobs]
    ws = torch.empty(J.decode_many_workspace_bytes(H, T, choices), dtype=torch.uint8, device="cuda")
    J.decode_many(blobs, H, T, choices, rot, outs, ws)
    torch.cuda.synchronize()
    for l, k in [(0, 1), (22, 0)]:
        t = 2 * l + k
        X = kvgen.config_tensor(cfg, l, k).astype(np.float64)
        a = codec.analyze(X, res.r_T_cap, method, cfg.seed, l, k)
        _check_spectra(res, t, a["lam_T"], a["lam_D"], a["frob2"])
        _check_factors(res, t, X, choices[t], a["lam_T"], a["U_T"], a["U_D"], n_T=min(T, H * D))
        _check_rows(X, blobs[t], H, T, choices[t], Q, outs[t], seed=t)
        e_o = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, a["U_T"], a["U_D"], choices[t], Q),
                                                   Q, "bf16"))
        assert abs(_err(X, outs[t]) - e_o) < 1e-4, (l, k, _err(X, outs[t]), e_o)


def test_full_mistral7b_t32768_3x_streaming(J):
    """Long context: 32 layers x {K, V}, T = 32768, 3x, randomized factors;
    decode streams one layer (K + V) at a time into one reused pair of
    output buffers (128 MiB)."""
    cfg = kvgen.CONFIGS["mistral7b_t32768_3x"]
    H, T = cfg.H, cfg.T
    xs = _load(cfg)
    rot = J.rotation(cfg.seed)
    Q = rotation.rotation(cfg.seed, D)
    res = J.allocate(xs, ratio=cfg.ratio, method=cfg.method, bits=cfg.bits, seed=cfg.seed)
    assert res.r_T_cap == 160
    _plan_matches_oracle(res, cfg)
    blobs, choices = _encode_all(J, xs, res, rot, cfg.seed)
    del xs
    out = [torch.empty((H, T, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ws = torch.empty(max(J.decode_many_workspace_bytes(H, T, choices[2 * l:2 * l + 2])
                         for l in range(cfg.n_layers)), dtype=torch.uint8, device="cuda")
    l_s, k_s = 9, 1
    t = 2 * l_s + k_s
    kept = None
    for l in range(cfg.n_layers):
        J.decode_many(blobs[2 * l:2 * l + 2], H, T, choices[2 * l:2 * l + 2], rot, out, ws)
        if l == l_s:
            kept = out[k_s].clone()
    torch.cuda.synchronize()
    X = kvgen.config_tensor(cfg, l_s, k_s).astype(np.float64)
    a = codec.analyze(X, res.r_T_cap, "flash", cfg.seed, l_s, k_s)
    _check_spectra(res, t, a["lam_T"], a["lam_D"], a["frob2"])
    _check_factors(res, t, X, choices[t], a["lam_T"], a["U_T"], a["U_D"], n_T=min(T, H * D))
    _check_rows(X, blobs[t], H, T, choices[t], Q, kept, seed=t)
    e_o = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, a["U_T"], a["U_D"], choices[t], Q),
                                               Q, "bf16"))
    assert abs(_err(X, kept) - e_o) < 1e-4, (_err(X, kept), e_o)
    # the last layer is what the reused buffers hold at the end
    Xl = kvgen.config_tensor(cfg, cfg.n_layers - 1, 0).astype(np.float64)
    tl = 2 * (cfg.n_layers - 1)
    _check_rows(Xl, blobs[tl], H, T, choices[tl], Q, out[0], seed=tl)
