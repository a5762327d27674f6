"""The allocation planner (csrc/plan.cpp, host C++) built by the host
compiler with its address and undefined-behaviour sanitizers, run on seeded
spectra: no sanitizer report, and every plan bit-identical to the library's
(jolt_plan_from_spectra) on the same inputs.  CPU only."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from kv_cache_compression_mode_amd import jolt as J
import kv_cache_compression_mode_amd._lib as jl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_compression_mode_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    out = str(tmp_path_factory.mktemp("asan") / "plan_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "plan.cpp"), DRIVER, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _spectra(seed, L, T, H, zero_tensor=False):
    rng = np.random.default_rng(seed)
    nT = min(T, H * 128)
    sT, sD, f2 = [], [], []
    for t in range(2 * L):
        lt = np.sort(1e5 * rng.uniform(0.8, 0.99) ** np.arange(nT) + rng.uniform(1, 40, nT))[::-1]
        ld = np.sort(rng.uniform(0.6, 0.97) ** np.arange(128) + 0.002)[::-1]
        e = float(lt.sum())
        ld *= e / ld.sum()
        if zero_tensor and t == 1:
            lt[:] = 0.0
            ld[:] = 0.0
            e = 0.0
        sT.append(lt)
        sD.append(ld)
        f2.append(e)
    return np.stack(sT), np.stack(sD), np.array(f2)


CASES = [
    # seed, H, T, L, G, ratio, bits, method, r_T_cap, step_T, step_D
    (0, 8, 4096, 32, 4, 2.0, (1, 2, 3, 4), "exact", 0, 0, 0),
    (1, 8, 1024, 6, 4, 3.0, (2, 4), "exact", 0, 0, 0),
    (2, 40, 4096, 4, 4, 2.0, (1, 2, 3, 4), "exact", 0, 0, 0),
    (3, 2, 200, 5, 2, 1.7, (3,), "flash", 0, 0, 0),
    (4, 8, 512, 4, 4, 2.5, (1, 4), "exact", 64, 16, 8),
    (5, 8, 1024, 4, 4, 2.0, (1, 2, 3, 4), "exact", 0, 0, 0),      # a zero tensor
    (6, 8, 1024, 4, 4, 40.0, (1, 2), "exact", 0, 0, 0),           # infeasible budget
]


@pytest.mark.parametrize("case", CASES)
def test_sanitized_planner_matches_library(driver, tmp_path, case):
    seed, H, T, L, G, ratio, bits, method, cap, sT_, sD_ = case
    req = J.make_req(H, T, 128, 0, L, ratio, method=method, bits=bits, group_layers=G, r_T_cap=cap,
                     step_T=sT_, step_D=sD_)
    sT, sD, f2 = _spectra(seed, L, T, H, zero_tensor=(seed == 5))
    lenT = sT.shape[1]                  # the whole spectrum (the planner reads the leading part)
    spec = tmp_path / "spectra.bin"
    with open(spec, "wb") as f:
        for a in (sT, sD, f2):
            f.write(np.ascontiguousarray(a, dtype=np.float64).tobytes())
    b = list(bits) + [0] * (4 - len(bits))
    args = [driver, str(H), str(T), "0", str(L), str(G), repr(float(ratio)), str(len(bits)), *map(str, b),
            str(jl.JOLT_FLASH if method == "flash" else jl.JOLT_EXACT), "10", str(cap), str(sT_), str(sD_),
            str(lenT), str(spec)]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run(args, capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    lines = r.stdout.split("\n")
    status = int(lines[0].split()[1])
    if status != 0:
        assert status == jl.JOLT_EBUDGET
        with pytest.raises(jl.JoltError) as e:
            J.plan_from_spectra(req, sT, sD, f2)
        assert e.value.status == status
        return
    got = J.plan_from_spectra(req, sT, sD, f2)
    head = lines[1].split()
    assert int(head[1]) == got["total_bytes"] and int(head[3]) == got["budget"] and int(head[5]) == got["r_T_cap"]
    assert float.fromhex(head[7]) == got["objective"]
    ch = [tuple(map(int, l.split()[1:])) for l in lines if l.startswith("choice")]
    lib_ch = [tuple(got["choice"][(g, k)]) for g in range(len(ch) // 2) for k in (0, 1)]
    assert ch == lib_ch
    tb = [int(l.split()[1]) for l in lines if l.startswith("bytes")]
    assert tb == list(got["tensor_bytes"])
