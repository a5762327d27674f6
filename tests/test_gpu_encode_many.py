"""jolt_encode_many against jolt_encode, through the C ABI: the batched path
runs the same kernels with the same arithmetic, so every record must match
byte for byte.  Choices mix Tucker ranks (several (r_T, r_D) groups), bit
widths and the residual-only choice r_T = 0; factors come from a small
allocation of a seeded cache, so the records are those the codec stores."""
import numpy as np
import pytest
import torch

import kvgen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def J():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_compression_mode_amd import jolt
    return jolt


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_encode_many_matches_encode(J, dtype):
    cfg = kvgen.CONFIGS["single_k_t1024_f32"]
    L = 3
    xs = []
    for layer in range(L):
        for kind in (0, 1):
            x = kvgen.config_tensor(cfg, layer, kind).astype(np.float32)
            xs.append(torch.from_numpy(x).to(dtype).cuda().contiguous())
    res = J.allocate([(xs[2 * l], xs[2 * l + 1]) for l in range(L)], ratio=2.0)
    H, T, D = xs[0].shape
    choices = [(64, 32, 2), (128, 64, 3), (0, 0, 4), (64, 32, 1), (96, 64, 2), (128, 64, 4)]
    factors = []
    for i, ch in enumerate(choices):
        Ut, Ud = res.factors(i)
        factors.append((Ut, Ud) if ch[0] > 0 else (None, None))
    rot = J.rotation(7)
    # zeroed records: the padding between 256-aligned sections is written by neither path
    sizes = [J.blob_bytes(H, T, D, ch, dtype) for ch in choices]
    zeros = lambda: [torch.zeros(nb, dtype=torch.uint8, device="cuda") for nb in sizes]
    torch.cuda.synchronize()
    one = [J.encode(x, ch, f[0], f[1], rot, seed=7, out=o)
           for x, ch, f, o in zip(xs, choices, factors, zeros())]
    many = J.encode_many(xs, choices, factors, rot, seed=7, outs=zeros())
    torch.cuda.synchronize()
    assert len(many) == len(one)
    for i, (a, b) in enumerate(zip(one, many)):
        assert a.numel() == b.numel(), i
        assert torch.equal(a, b), f"record {i} ({choices[i]}) differs"
    # and twice in a row (workspace and pointer tables rebuilt per call)
    again = J.encode_many(xs[::-1], choices[::-1], factors[::-1], rot, seed=7, outs=zeros()[::-1])
    torch.cuda.synchronize()
    for a, b in zip(one[::-1], again):
        assert torch.equal(a, b)


def test_encode_many_reads_an_allocation(J):
    """Factors taken from the Allocation in place give the same records as the
    factor views passed one by one (choices with r_T > 0 and r_T = 0)."""
    cfg = kvgen.CONFIGS["single_k_t1024_f32"]
    L = 2
    xs = []
    for layer in range(L):
        for kind in (0, 1):
            x = kvgen.config_tensor(cfg, layer, kind).astype(np.float32)
            xs.append(torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous())
    res = J.allocate([(xs[2 * l], xs[2 * l + 1]) for l in range(L)], ratio=2.0)
    H, T, D = xs[0].shape
    choices = [(64, 32, 2), (0, 0, 3), (128, 64, 4), (96, 64, 1)]
    views = [res.factors(i) if ch[0] > 0 else (None, None) for i, ch in enumerate(choices)]
    rot = J.rotation(3)
    sizes = [J.blob_bytes(H, T, D, ch, torch.bfloat16) for ch in choices]
    zeros = lambda: [torch.zeros(nb, dtype=torch.uint8, device="cuda") for nb in sizes]
    a = J.encode_many(xs, choices, views, rot, seed=3, outs=zeros())
    b = J.encode_many(xs, choices, res, rot, seed=3, outs=zeros())
    torch.cuda.synchronize()
    for i, (u, v) in enumerate(zip(a, b)):
        assert torch.equal(u, v), f"record {i} ({choices[i]}) differs"
    with pytest.raises(ValueError):
        J.encode_many(xs[:2], choices[:2], res, rot, seed=3)
