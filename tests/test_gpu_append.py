"""GPU parity of the incremental encode of appended tokens (jolt_append),
through the C ABI, on base records made by the oracle alone (its factors and
encode, packed in the library's record layout), against the oracle's
folding-in (exact least squares against the stored factors) and encode:

* the new record carries the base's stored U~_D and G~ bit for bit;
* the new tokens' Tucker reconstruction U~_new W agrees with the oracle's
  within 2e-3 of the tokens' norm: the fp32 normal equations move the rows
  by ~1e-6 relative, so the stored bf16 rows can differ only where that
  moves a value across a rounding boundary (one bf16 unit, 2^-8 relative);
* the appended tokens' relative error after the library's decode is within
  1e-4 of the oracle's append + decode.
Cases: the Mistral-shaped tensor with 256 new tokens, the MHA shape with fewer
new tokens (64) than r_T (96), and a ragged 37.
"""
import numpy as np
import pytest
import torch

import kvgen
from oracle import append, codec, rotation, tucker

from gpu_util import D, pack_record, parse_blob

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_compression_mode_amd import jolt
    return jolt


@pytest.mark.parametrize("H,T,dT,choice", [(8, 4096, 256, (192, 128, 4)), (40, 1024, 64, (96, 64, 3)),
                                           (8, 1024, 37, (128, 96, 2))])
def test_append_matches_oracle(J, H, T, dT, choice):
    X = kvgen.tensor(H, T + dT, D, seed=51, decay=0.9, dtype="bf16").astype(np.float64)
    Xb, Xn = X[:, :T], X[:, T:]
    Q = rotation.rotation(0, D)
    a = codec.analyze(Xb, choice[0])
    base = codec.encode_tensor(Xb, a["U_T"], a["U_D"], choice, Q)
    rec = torch.from_numpy(pack_record(base)).cuda()
    rot = J.rotation(0)
    xn = torch.from_numpy(np.ascontiguousarray(Xn, dtype=np.float32)).to(torch.bfloat16).cuda()
    blob = J.append(rec, H, T, choice, xn, rot)
    out = J.decode(blob, H, dT, choice, rot)
    torch.cuda.synchronize()
    parts = parse_blob(blob, H, dT, choice)
    np.testing.assert_array_equal(parts["U_D"], base["U_D"])
    np.testing.assert_array_equal(parts["G"], base["G"])
    ext = append.append_encode(Xn, base, Q)
    rec_g = tucker.reconstruct(base["G"], parts["U_T"], base["U_D"])
    rec_o = tucker.reconstruct(base["G"], ext["U_T"], base["U_D"])
    rel = np.linalg.norm(rec_g - rec_o) / np.linalg.norm(Xn)
    assert rel < 2e-3, rel
    e_g = codec.rel_err(Xn, out.float().cpu().numpy())
    e_o = codec.rel_err(Xn, codec.decode_tensor(ext, Q, "bf16"))
    assert abs(e_g - e_o) < 1e-4, (e_g, e_o)
