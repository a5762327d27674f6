"""GPU parity of the compression-ratio sweep (JoLT abstract, the sentences on
the near-lossless 2-3x range and the per-K/V relative Frobenius errors),
through the C ABI, on a GQA-shaped (8 heads, dual token Gram) and an
MHA-shaped (40 heads, direct token Gram) cache of one layer group:

* at every ratio the library's plan equals the oracle's dual run on the
  library's spectra, within its byte budget;
* the predicted objective does not fall as the ratio rises (the budget shrinks);
* on sampled tensors the relative error at the planned choice is within 1e-4
  of the oracle's encode with the oracle's own fp64 factors.
"""
import numpy as np
import pytest
import torch

import kvgen
from oracle import alloc, codec, rotation

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def J():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_compression_mode_amd import jolt
    return jolt


@pytest.mark.parametrize("H,T,outliers", [(8, 2048, "KV"), (40, 1024, "K")])
def test_ratio_sweep_plan_and_errors(J, H, T, outliers):
    L = 4
    xs_h = []
    for l in range(L):
        pair = []
        for k in (0, 1):
            out = (k == 0 and "K" in outliers) or (k == 1 and "V" in outliers)
            pair.append(kvgen.tensor(H, T, D, seed=31, layer=l, kind=k, decay=kvgen.decay_for(31, l, k),
                                     outliers=out, dtype="bf16").astype(np.float64))
        xs_h.append(pair)
    xs = [tuple(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda() for x in p) for p in xs_h]
    rot = J.rotation(0)
    Q = rotation.rotation(0, D)
    prev = None
    for ratio in (2.0, 2.5, 3.0):
        res = J.allocate(xs, ratio=ratio)
        sp = [[(res.spectra_T[2 * l + k], res.spectra_D[2 * l + k], res.frob2[2 * l + k]) for k in (0, 1)]
              for l in range(L)]
        want = alloc.allocate(sp, L, H, T, D, ratio, (1, 2, 3, 4), 4)
        assert res.choice == want["choice"] and res.total_bytes == want["total_bytes"], ratio
        assert res.total_bytes <= res.budget_bytes
        if prev is not None:
            assert res.objective >= prev - 1e-12, (ratio, res.objective, prev)
        prev = res.objective
        for l, k in [(0, 0), (3, 1)]:
            t = 2 * l + k
            ch = res.choice_of(l, k)
            Ut, Ud = res.factors(t)
            out = J.decode(J.encode(xs[l][k], ch, Ut, Ud, rot), H, T, ch, rot)
            torch.cuda.synchronize()
            X = xs_h[l][k]
            a = codec.analyze(X, res.r_T_cap, "exact")
            e_o = codec.rel_err(X, codec.decode_tensor(codec.encode_tensor(X, a["U_T"], a["U_D"], ch, Q), Q, "bf16"))
            e_g = codec.rel_err(X, out.float().cpu().numpy())
            assert abs(e_g - e_o) < 1e-4, (ratio, l, k, e_g, e_o)
