"""Host logic of bench.py: the HBM-traffic record built from two rocprofv3
--pmc CSVs (scaled by a plain copy of known size) and its invalidation when
the kernel's source changes.  No GPU."""
import csv
import glob
import json
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, kernel_values, copy_values):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        i = 0
        for v in kernel_values:
            w.writerow(dict(Correlation_Id=i, Dispatch_Id=i, Counter_Name=counter, Counter_Value=v,
                            Kernel_Name="void jolt::(anonymous namespace)::k_chase<8>(float*, ...)"))
            i += 1
        for v in copy_values:
            w.writerow(dict(Correlation_Id=i, Dispatch_Id=i, Counter_Name=counter, Counter_Value=v,
                            Kernel_Name="void at::native::vectorized_elementwise_kernel<4, ...>"))
            i += 1


def test_record_and_invalidate(tmp_path):
    copy = 1 << 30
    kib = copy / 1024
    # the fetch counter reads half the bytes of a plain copy, the write counter all of them
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [100.0, 300.0], [20.0, kib / 2, kib / 2])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [50.0, 150.0], [kib, kib, kib])
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    rec_path = str(tmp_path / "traffic.json")
    bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), copy, "chase",
                         "test_workload", rec_path, (str(src),))
    rec = json.load(open(rec_path))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["traffic_bytes_per_launch"] == (200.0 * 2 + 100.0) * 1024
    assert bench.measured_traffic((str(src),), rec_path) == rec["traffic_bytes_per_launch"]
    src.write_text("kernel v2")
    assert bench.measured_traffic((str(src),), rec_path) is None
    assert bench.measured_traffic((str(src),), str(tmp_path / "missing.json")) is None


def test_gemm_records_keep_their_kernels(tmp_path):
    """The fp32 GEMM record counts k_gemm<...> and k_gemm_bf16, the bf16
    matrix-core record only k_gemm_x<...> (one name is a prefix of the other)."""
    copy = 1 << 30
    kib = copy / 1024
    names = {"jolt::(anonymous namespace)::k_gemm<float, float>(jolt::GemmArgs)": 10.0,
             "jolt::(anonymous namespace)::k_gemm_bf16(jolt::GemmArgs)": 30.0,
             "void jolt::(anonymous namespace)::k_gemm_x<2, 1>(jolt::GemmArgs)": 1000.0}
    for counter, fname, cval in (("FETCH_SIZE", "f.csv", kib / 2), ("WRITE_SIZE", "w.csv", kib)):
        with open(tmp_path / fname, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Correlation_Id", "Dispatch_Id", "Counter_Name", "Counter_Value",
                                              "Kernel_Name"])
            w.writeheader()
            rows = list(names.items()) + [("void at::native::vectorized_elementwise_k", cval)] * 2
            for i, (kn, v) in enumerate(rows):
                w.writerow(dict(Correlation_Id=i, Dispatch_Id=i, Counter_Name=counter, Counter_Value=v,
                                Kernel_Name=kn))
    src = tmp_path / "k.hip"
    src.write_text("kernel")
    for name, want in (("gemm", 20.0), ("gemm_bf16", 1000.0)):
        rec_path = str(tmp_path / f"{name}.json")
        bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), copy, name, "w", rec_path,
                             (str(src),))
        rec = json.load(open(rec_path))
        assert rec["fetch_kib_per_dispatch"] == want and rec["write_kib_per_dispatch"] == want


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "traffic_*.json"))))
def test_committed_record_matches_layout(path):
    rec = json.load(open(path))
    for k in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "fetch_scale", "write_scale",
              "traffic_bytes_per_launch", "source_sha256"):
        assert k in rec
    want = (rec["fetch_kib_per_dispatch"] * rec["fetch_scale"]
            + rec["write_kib_per_dispatch"] * rec["write_scale"]) * 1024
    assert abs(rec["traffic_bytes_per_launch"] - want) <= 1e-5 * want


def test_roofline_bound_choice():
    st = dict(launches=2, total_ms=2.0, bytes=2e9, flops=2e9 * 30)   # intensity 30 > fp32 ridge
    r = bench.roofline_for("gemm", st, "no_such_workload")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    # per launch: 1 ms, 1 GB, 30 GFLOP -> 30 TFLOP/s
    assert abs(r["achieved"] - 30.0) < 1e-9 and r["frac"] == round(30.0 / 157.3, 4)
    st = dict(launches=2, total_ms=2.0, bytes=2e9, flops=2e9)
    r = bench.roofline_for("gemm", st, "no_such_workload")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and abs(r["achieved"] - 1000.0) < 1e-9
    # the bf16 matrix-core GEMM: ridge 2500 / 8 = 312.5 flop/B
    st = dict(launches=2, total_ms=2.0, bytes=2e9, flops=2e9 * 30)
    r = bench.roofline_for("gemm_bf16", st, "no_such_workload")
    assert r["bound"] == "hbm" and abs(r["ridge"] - 312.5) < 1e-9
    st = dict(launches=2, total_ms=2.0, bytes=2e9, flops=2e9 * 400)
    r = bench.roofline_for("gemm_bf16", st, "no_such_workload")
    assert r["bound"] == "mfma" and r["peak"] == 2500.0 and r["frac"] == round(400.0 / 2500.0, 4)


def test_multi_gpu_refused():
    import subprocess
    import sys
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stdout
