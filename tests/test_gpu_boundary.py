"""The C ABI's contract under concurrency and on its error paths (GPU).

* Two host threads, each with its own stream and workspaces, run
  jolt_allocate then jolt_encode_many at the same time: plans, spectra and
  records are byte-identical to a serial run of the same calls.  One cache
  has the dual 1024 x 1024 token Gram (the feature factor on an auxiliary
  stream), the other a direct 2048 x 2048 one (two lanes of chunks on two
  streams), so both forking patterns overlap.
* A bounded wait of the eigensolver that gives up (forced from the host with
  a poll limit of zero; every kernel still ends normally) makes
  jolt_allocate return JOLT_EHIP, and the next call with the default limit
  succeeds.
* The binding rejects outputs of the wrong dtype, shape or device, and
  factors too short for the choice, before anything is enqueued.
"""
import threading

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


def _cache(H, T, layers, seed):
    out = []
    for l in range(layers):
        pair = []
        for k in (0, 1):
            x = kvgen.tensor(H, T, D, seed=seed, layer=l, kind=k, decay=kvgen.decay_for(seed, l, k),
                             dtype="bf16")
            pair.append(torch.from_numpy(x).to(torch.bfloat16).cuda())
        out.append(tuple(pair))
    return out


def _run(J, xs, rot):
    """allocate + encode_many on the current stream; host copies of everything."""
    res = J.allocate(xs, ratio=2.0)
    flat = [x for pair in xs for x in pair]
    choices = [res.choice_of(i // 2, i % 2) for i in range(len(flat))]
    blobs = J.encode_many(flat, choices, res, rot)
    torch.cuda.current_stream().synchronize()
    return dict(choice=res.choice, total=res.total_bytes, spT=res.spectra_T.copy(), spD=res.spectra_D.copy(),
                blobs=[b.cpu().numpy().copy() for b in blobs])


def _same(a, b):
    assert a["choice"] == b["choice"] and a["total"] == b["total"]
    np.testing.assert_array_equal(a["spT"], b["spT"])
    np.testing.assert_array_equal(a["spD"], b["spD"])
    assert len(a["blobs"]) == len(b["blobs"])
    for x, y in zip(a["blobs"], b["blobs"]):
        np.testing.assert_array_equal(x, y)


def test_concurrent_calls_match_serial(J):
    caches = [_cache(8, 4096, 4, seed=11), _cache(16, 2048, 4, seed=12)]
    rot = J.rotation(0)
    torch.cuda.synchronize()
    serial = [_run(J, c, rot) for c in caches]
    for _ in range(2):
        results, errors = [None, None], []

        def worker(i):
            try:
                s = torch.cuda.Stream()
                with torch.cuda.stream(s):
                    results[i] = _run(J, caches[i], rot)
            except Exception as e:          # reported by the main thread
                errors.append(e)

        th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        assert not errors, errors
        for i in range(2):
            _same(results[i], serial[i])


def test_chase_wait_give_up_is_an_error(J):
    from kv_cache_compression_mode_amd import _lib
    xs = _cache(8, 4096, 2, seed=13)
    try:
        _lib.lib().jolt_debug_chase_wait_limit(0)
        with pytest.raises(_lib.JoltError) as ei:
            J.allocate(xs, ratio=2.0)
        assert ei.value.status == _lib.JOLT_EHIP
    finally:
        _lib.lib().jolt_debug_chase_wait_limit(-1)
    torch.cuda.synchronize()
    res = J.allocate(xs, ratio=2.0)            # default limit: the same call succeeds
    assert res.total_bytes <= res.budget_bytes


def test_binding_rejects_bad_buffers(J):
    xs = _cache(2, 512, 1, seed=14)
    res = J.allocate(xs, ratio=2.0)
    rot = J.rotation(0)
    ch = res.choice_of(0, 0)
    Ut, Ud = res.factors(0)
    blob = J.encode(xs[0][0], ch, Ut, Ud, rot)
    H, T = 2, 512
    with pytest.raises(ValueError):          # output dtype differs from the requested one
        J.decode(blob, H, T, ch, rot, dtype=torch.float32, out=torch.empty((H, T, D), dtype=torch.bfloat16,
                                                                         device="cuda"))
    with pytest.raises(ValueError):          # undersized output
        J.decode(blob, H, T, ch, rot, out=torch.empty((H, T - 1, D), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):          # output on the host
        J.decode(blob, H, T, ch, rot, out=torch.empty((H, T, D), dtype=torch.bfloat16))
    with pytest.raises(ValueError):          # non-contiguous input
        J.encode(xs[0][0].transpose(0, 1), ch, Ut, Ud, rot)
    if ch[0] > 0:
        with pytest.raises(ValueError):      # token factor shorter than T
            J.encode(xs[0][0], ch, Ut[: T - 1], Ud, rot)
    ws = torch.empty(J.decode_many_workspace_bytes(H, T, [ch]), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        J.decode_many([blob], H, T, [ch], rot, [torch.empty((H, T, D), dtype=torch.float32, device="cuda")], ws)
    out = J.decode(blob, H, T, ch, rot)      # the valid call still works
    torch.cuda.synchronize()
    assert out.shape == (H, T, D)


def test_record_reloaded_from_disk_decodes_identically(J, tmp_path):
    """A record is self-contained bytes: written to a file, read back and
    uploaded again, it decodes to the same output, and every one of its bytes
    (header padding and section tails included) is written by the encoder."""
    from kv_cache_compression_mode_amd import _lib  # noqa: F401
    H, T = 2, 200                                 # ragged T: sections end off 256-byte boundaries
    xs = _cache(H, T, 1, seed=15)
    res = J.allocate(xs, ratio=2.0)
    rot = J.rotation(0)
    outs = []
    for k in (0, 1):
        ch = res.choice_of(0, k)
        Ut, Ud = res.factors(k)
        nb = J.blob_bytes(H, T, D, ch)
        first = torch.full((nb,), 0xAB, dtype=torch.uint8, device="cuda")
        second = torch.full((nb,), 0x5C, dtype=torch.uint8, device="cuda")
        J.encode(xs[0][k], ch, Ut, Ud, rot, out=first)
        J.encode(xs[0][k], ch, Ut, Ud, rot, out=second)
        torch.cuda.synchronize()
        host = first.cpu().numpy()
        np.testing.assert_array_equal(host, second.cpu().numpy())   # no byte left as it was
        path = tmp_path / f"rec{k}.bin"
        host.tofile(path)
        back = torch.from_numpy(np.fromfile(path, dtype=np.uint8)).cuda()
        shape, choice, seed = J.header_parse(back[:64].cpu().numpy().tobytes())
        assert shape == (H, T, D, 0) and choice == tuple(ch) and seed == 0
        a = J.decode(first, H, T, ch, rot)
        b = J.decode(back, H, T, choice, rot)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        outs.append(b)
    assert all(o.shape == (H, T, D) for o in outs)
