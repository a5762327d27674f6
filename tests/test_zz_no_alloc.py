"""The allocation-free decode (jolt_decode_many_static) against the decode
with a caller workspace (jolt_decode_many), through the C ABI: identical
outputs on two calls in a row, the second with a smaller input; the first
call's records need more scratch than the static array holds, so it runs in
several launches.  A record whose planes alone exceed the array is refused
with JOLT_ENOSPACE before anything runs."""
import numpy as np
import pytest
import torch

import kvgen

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def J():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_compression_mode_amd import jolt
    return jolt


def _orthonormal(rows, cols, seed):
    q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((rows, cols)))
    return torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()


def _records(J, H, T, choices, rot, seed):
    blobs = []
    for i, ch in enumerate(choices):
        x = kvgen.tensor(H, T, D, seed=seed, layer=i, kind=0, decay=0.9, dtype="bf16")
        xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
        if ch[0] > 0:
            Ut = _orthonormal(T, ch[0], seed + 10 * i)
            Ud = _orthonormal(D, D, seed + 10 * i + 1)
        else:
            Ut = Ud = None
        blobs.append(J.encode(xd, ch, Ut, Ud, rot))
    return blobs


def _both(J, H, T, choices, blobs, rot):
    ref = [torch.empty((H, T, D), dtype=torch.bfloat16, device="cuda") for _ in blobs]
    ws = torch.empty(J.decode_many_workspace_bytes(H, T, choices), dtype=torch.uint8, device="cuda")
    J.decode_many(blobs, H, T, choices, rot, ref, ws)
    got = [torch.full((H, T, D), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in blobs]
    J.decode_many_static(blobs, H, T, choices, rot, got)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    return got


def test_static_decode_matches_workspace_decode(J):
    from kv_cache_compression_mode_amd import _lib
    cap = _lib.lib().jolt_decode_static_scratch_bytes()
    assert cap == 32 << 20
    rot = J.rotation(0)
    # call 1: W planes of 21 + 10.5 + 21 MB, more than the 32 MiB array: two launches
    H1, T1 = 40, 1024
    ch1 = [(1024, 128, 2), (512, 64, 3), (1024, 96, 4)]
    assert sum(2 * 2 * H1 * D * c[0] for c in ch1) > cap
    b1 = _records(J, H1, T1, ch1, rot, seed=21)
    out1 = _both(J, H1, T1, ch1, b1, rot)
    # call 2: a smaller input, reusing the same array
    H2, T2 = 8, 512
    ch2 = [(256, 64, 2), (0, 0, 4)]
    b2 = _records(J, H2, T2, ch2, rot, seed=22)
    out2 = _both(J, H2, T2, ch2, b2, rot)
    assert all(torch.isfinite(o.float()).all() for o in out1 + out2)


def test_static_decode_refuses_oversized_record(J):
    from kv_cache_compression_mode_amd import _lib
    H, T, ch = 64, 2048, (2048, 128, 2)       # planes: 2 * 2 * 64 * 128 * 2048 B = 64 MiB
    nb = J.blob_bytes(H, T, D, ch)
    blob = torch.empty(nb, dtype=torch.uint8, device="cuda")   # never read: refused on the host
    out = torch.empty((H, T, D), dtype=torch.bfloat16, device="cuda")
    rot = J.rotation(0)
    with pytest.raises(_lib.JoltError) as ei:
        J.decode_many_static([blob], H, T, [ch], rot, [out])
    assert ei.value.status == _lib.JOLT_ENOSPACE
