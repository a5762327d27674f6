"""Throughput of the JoLT codec hot path on one MI355X.

One step = the whole path over one synthetic cache: spectra, factors and the
Lagrangian-dual allocation of all layers x {K, V} (jolt_allocate), encode of
every tensor (jolt_encode_many), decode of every tensor (jolt_decode_many).  The
default workload is the Mistral-7B-v0.3-shaped GQA cache: 32 layers x {K, V},
8 KV heads, T = 4096, D = 128, bf16, 2x byte budget, exact Gram factors.
``--config`` selects another cache workload: the LLaMA-2-13B-shaped MHA cache
(40 heads), the T = 1024 FlashJoLT comparison (the exact path is timed too;
the encode-time ratio and the error delta are reported) or the T = 32768 3x
long context (randomized factors; decode streams one layer at a time into
two reused output buffers).

Prints one JSON line.  ``value`` is cache tokens per second of the full step
(T tokens of the whole cache through allocate + encode + decode); the encode
throughput (tokens/s) and decode HBM throughput (GB/s) are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_FP32_PEAK_TFLOPS = 157.3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--config", default="mistral7b_t4096_2x")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tensors", type=int, default=0,
                   help="tensors the oracle runs on (0: a per-workload default of about 10-30 s)")
    p.add_argument("--profile-step", action="store_true",
                   help="run warmup + one step, then a plain copy of a known size (rocprofv3 runs)")
    p.add_argument("--copy-mib", type=int, default=1024,
                   help="size of the calibration copy in --profile-step mode")
    p.add_argument("--traffic-kernel", default="gemm", help="kernel of the --record-traffic record")
    p.add_argument("--compare", action="store_true",
                   help="instead of timing: relative errors of JoLT over a 2x..3x budget sweep (K and V "
                        "separately) and of the comparison codecs at matched bytes, one JSON line")
    p.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn the counter_collection.csv files of two rocprofv3 --pmc runs of "
                        "--profile-step (FETCH_SIZE, then WRITE_SIZE) into the traffic record "
                        "the roofline reads, and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic, args.copy_mib << 20, args.traffic_kernel, args.config)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this codec benchmark runs on one GPU only: the path has no "
                                   "cross-GPU step (tensors shard by layer with no collective); "
                                   "run with --gpus 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import kvgen
    from kv_cache_compression_mode_amd import jolt

    cfg = kvgen.CONFIGS[args.config]
    if cfg.ratio <= 0:
        print(json.dumps({"error": f"{cfg.name} has a fixed choice and no byte budget: it is a parity "
                                   "case, not a benchmark workload"}))
        sys.exit(2)
    L, H, T, D = cfg.n_layers, cfg.H, cfg.T, cfg.D
    streaming = cfg.name in STREAMING       # decode one layer at a time into reused buffers
    compare = cfg.name in COMPARE_EXACT     # also time the exact path on the same inputs
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {L}x2 tensors [{H},{T},{D}] {cfg.dtype}", file=sys.stderr, flush=True)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    xs = [[None, None] for _ in range(L)]
    for l, k, x in kvgen.generate(cfg, [(l, k) for l in range(L) for k in (0, 1)], workers=8):
        xs[l][k] = torch.from_numpy(x).to(tdt).to(dev)
    xs = [tuple(p) for p in xs]
    flat = [xs[l][k] for l in range(L) for k in (0, 1)]
    rot = jolt.rotation(cfg.seed)
    n_out = 2 if streaming else 2 * L
    outs = [torch.empty((H, T, D), dtype=tdt, device=dev) for _ in range(n_out)]
    stream = torch.cuda.current_stream(dev)
    print("[bench] inputs resident", file=sys.stderr, flush=True)

    def decode_all(blobs, choices, dws, validate=True):
        if streaming:
            for l in range(L):
                jolt.decode_many(blobs[2 * l:2 * l + 2], H, T, choices[2 * l:2 * l + 2], rot, outs, dws,
                                 dtype=tdt, validate=validate)
        else:
            jolt.decode_many(blobs, H, T, choices, rot, outs, dws, dtype=tdt, validate=validate)

    def decode_ws_bytes(choices):
        if streaming:
            return max(jolt.decode_many_workspace_bytes(H, T, choices[2 * l:2 * l + 2], tdt) for l in range(L))
        return jolt.decode_many_workspace_bytes(H, T, choices, tdt)

    state = {}

    def step(method, record=None):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        res = jolt.allocate(xs, ratio=cfg.ratio, method=method, bits=cfg.bits, seed=cfg.seed)
        ev[1].record(stream)
        choices = [res.choice_of(i // 2, i % 2) for i in range(len(flat))]
        blobs = jolt.encode_many(flat, choices, res, rot, seed=cfg.seed)
        ev[2].record(stream)
        dws = torch.empty(decode_ws_bytes(choices), dtype=torch.uint8, device=dev)
        decode_all(blobs, choices, dws)
        ev[3].record(stream)
        state.update(res=res, blobs=blobs, choices=choices)
        if record is not None:
            record.append(ev)

    def run(method, K, profile):
        """Warmup, then K timed steps.  `profile`: kernel names whose launches
        are bracketed by HIP events on their launch stream, with their
        algorithmic work, over the timed region (a few launches per step)."""
        for _ in range(args.warmup):
            step(method)
        torch.cuda.synchronize()
        evs = []
        if profile:
            jolt.profile_enable(",".join(profile))
        t0 = time.perf_counter()
        for _ in range(K):
            step(method, evs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        stats = {}
        if profile:
            stats = {name: jolt.profile_query(name) for name in profile}
            jolt.profile_enable(None)
        ph = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(3)]
        return wall * 1e3 / K, ph, stats

    def errors():
        """Relative Frobenius error of every tensor (outside the timed region)."""
        blobs, choices = state["blobs"], state["choices"]
        dws = torch.empty(decode_ws_bytes(choices), dtype=torch.uint8, device=dev)
        errs = []
        for l in range(L):
            if streaming:
                jolt.decode_many(blobs[2 * l:2 * l + 2], H, T, choices[2 * l:2 * l + 2], rot, outs, dws,
                                 dtype=tdt)
                pair = outs
            else:
                pair = outs[2 * l:2 * l + 2]
            if not streaming and l == 0:
                decode_all(blobs, choices, dws)
            for k in (0, 1):
                xd = xs[l][k].double()
                errs.append(float(torch.linalg.vector_norm(xd - pair[k].double()) / torch.linalg.vector_norm(xd)))
        return np.array(errs).reshape(L, 2)

    if args.compare:
        print(json.dumps(compare_codecs(jolt, cfg, xs, flat, rot, outs, tdt, dev)), flush=True)
        return

    K = 1 if args.profile_step else args.steps
    kstats = {}
    dominant = None
    if not args.profile_step:
        # per-kernel breakdown from one step with every kernel bracketed by
        # events (outside the timed region: the extra events cost time); the
        # dominant kernel among those that account their algorithmic work is
        # then timed inside the timed region
        step(cfg.method)
        jolt.profile_enable("*")
        step(cfg.method)
        torch.cuda.synchronize()
        kstats = {name: jolt.profile_query(name) for name in KERNELS}
        jolt.profile_enable(None)
        cands = [k for k in ROOF if kstats[k]["launches"] and kstats[k]["bytes"] > 0]
        dominant = max(cands, key=lambda k: kstats[k]["total_ms"]) if cands else None
    timed = [k for k in TIMED_ROOF if k != dominant] + ([dominant] if dominant else [])
    ms_step, (ms_alloc, ms_enc, ms_dec), tstats = run(cfg.method, K, None if args.profile_step else timed)
    # the standalone group quantizer (not on the step's path: the encoder
    # fuses it) on a synthetic rotated residual of the whole cache's rows
    q_rows = 2 * L * H * T
    q_bits = 2
    qy = torch.randn((q_rows, D), dtype=torch.float32, device=dev)
    jolt.quantize(qy, q_bits)                   # warmup
    torch.cuda.synchronize()
    if not args.profile_step:
        jolt.profile_enable("quantize")
    for _ in range(3):
        jolt.quantize(qy, q_bits)
    torch.cuda.synchronize()
    qstats = None
    if not args.profile_step:
        qstats = jolt.profile_query("quantize")
        jolt.profile_enable(None)
    del qy
    attn = attend_leg(jolt, cfg, state, rot, dev, tdt, args.profile_step)
    appended = append_leg(jolt, cfg, state, xs, rot, dev, tdt) if not args.profile_step else None
    if args.profile_step:
        # a plain copy of known size (read n bytes, write n bytes), against
        # which the FETCH_SIZE / WRITE_SIZE counters are scaled
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"profile_step_ms": ms_step, "copy_bytes": n}), flush=True)
        return

    res, blobs, choices = state["res"], state["blobs"], state["choices"]
    blob_total = sum(b.numel() for b in blobs)
    in_bytes = sum(x.numel() * x.element_size() for x in flat)

    # decode roofline: algorithmic bytes = every record read once + every output
    # written once, over the decode of the whole cache (one batched call, or the
    # layer-by-layer stream), timed live with HIP events on the launch stream
    dws = torch.empty(decode_ws_bytes(choices), dtype=torch.uint8, device=dev)
    reps = 5
    de0, de1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    decode_all(blobs, choices, dws)                    # the binding checks the buffers once
    de0.record(stream)
    for _ in range(reps):
        decode_all(blobs, choices, dws, validate=False)
    de1.record(stream)
    torch.cuda.synchronize()
    dec_ms = de0.elapsed_time(de1) / reps
    dec_bytes = (blob_total - 256 * len(flat)) + in_bytes
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    errs = errors()

    dec_kernel = ("jolt_decode_many per layer (K + V) into two reused buffers, all layers" if streaming
                  else "jolt_decode_many (k_make_w + k_decode, whole cache)")
    line = {
        "metric": "JoLT encode tokens/s + decode GB/s, Mistral-7B KV shape, 2x budget, 1 GPU",
        "value": round(T / (ms_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 storage, fp32 accumulate",
        "data": "synthetic (seeded low-rank + noise + outlier channels, model cache shapes)",
        "config": {"workload": cfg.name, "layers": L, "kv_heads": H, "tokens": T, "head_dim": D,
                   "input_dtype": cfg.dtype, "budget_ratio": cfg.ratio, "method": cfg.method,
                   "tensors": 2 * L, "decode": "streamed per layer" if streaming else "one batched call"},
        "phases_ms": {"allocate": round(ms_alloc, 3), "encode": round(ms_enc, 3),
                      "decode": round(ms_dec, 3)},
        "encode_tokens_per_s": round(T / ((ms_alloc + ms_enc) * 1e-3), 2),
        "decode_GBps": round(dec_gbps, 1),
        "decode_ms": round(dec_ms, 4),
        "decode_output_GBps": round(in_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "compression_ratio_vs_bf16": round(in_bytes * (2 / flat[0].element_size()) / blob_total, 4),
        "plan_bytes": int(res.total_bytes), "budget_bytes": int(res.budget_bytes),
        "rel_err_K_mean": round(float(errs[:, 0].mean()), 6),
        "rel_err_V_mean": round(float(errs[:, 1].mean()), 6),
        "roofline": (roofline_for(dominant, tstats[dominant], cfg.name)
                     if dominant and tstats.get(dominant, {}).get("launches") else None),
        # the kernels with roofline targets, timed the same way inside the
        # timed steps (the quantizer in its own leg on the cache's rows)
        "roofline_encode": (roofline_for("encode_residual", tstats["encode_residual"], cfg.name)
                            if tstats.get("encode_residual", {}).get("launches") else None),
        "roofline_decode_kernel": (roofline_for("decode", tstats["decode"], cfg.name)
                                   if tstats.get("decode", {}).get("launches") else None),
        "roofline_quantize": (dict(roofline_for("quantize", qstats, cfg.name),
                                   workload=f"{q_rows} rows x {D} fp32 (the cache's rows), b = {q_bits}")
                              if qstats and qstats["launches"] else None),
        "roofline_gram": (roofline_for("gram", tstats["gram"], cfg.name)
                          if tstats.get("gram", {}).get("launches") else None),
        "attend": attn,
        "append": appended,
        "roofline_decode": {"kernel": dec_kernel,
                            "bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                            "algorithmic_bytes_per_call": int(dec_bytes),
                            "avg_call_ms": round(dec_ms, 5)},
        # the other kernels that account their work, from the per-kernel
        # breakdown step (events around every launch, outside the timed steps)
        "roofline_more": {k: roofline_for(k, kstats[k], cfg.name) for k in ROOF
                          if k != dominant and k not in TIMED_ROOF and k in kstats and kstats[k]["launches"]
                          and kstats[k]["bytes"] > 0},
        "kernel_ms_per_step": {k: round(v["total_ms"], 3) for k, v in kstats.items()},
        "kernel_launches_per_step": {k: v["launches"] for k, v in kstats.items()},
    }
    if compare:
        # the exact Gram path on the same inputs, same budget, its own plan
        ex_step, (ex_alloc, ex_enc, _), _ = run("exact", K, False)
        ex_errs = errors()
        line["exact_path"] = {
            "ms_per_step": round(ex_step, 3),
            "encode_ms": round(ex_alloc + ex_enc, 3),
            "rel_err_K_mean": round(float(ex_errs[:, 0].mean()), 6),
            "rel_err_V_mean": round(float(ex_errs[:, 1].mean()), 6)}
        line["encode_time_ratio_exact_over_flash"] = round((ex_alloc + ex_enc) / (ms_alloc + ms_enc), 3)
        line["rel_err_delta_flash_minus_exact"] = {
            "K": round(float(errs[:, 0].mean() - ex_errs[:, 0].mean()), 7),
            "V": round(float(errs[:, 1].mean() - ex_errs[:, 1].mean()), 7)}

    if not args.no_cpu_baseline:
        n_cpu = args.cpu_sample_tensors if args.cpu_sample_tensors > 0 else CPU_SAMPLE.get(cfg.name, 2)
        line["cpu_baseline"] = cpu_baseline(cfg, n_cpu)
    print(json.dumps(line), flush=True)


# workloads whose decode streams one layer (K + V) at a time into two reused
# output buffers, and workloads that also time the exact path (FlashJoLT
# comparison); oracle sample sizes that take about 10-30 s on the host
STREAMING = {"mistral7b_t32768_3x"}
COMPARE_EXACT = {"mistral7b_t1024_flash"}
CPU_SAMPLE = {"mistral7b_t4096_2x": 24, "mistral7b_t1024_flash": 64, "llama13b_t4096_2x": 2,
              "mistral7b_t32768_3x": 4}

KERNELS = ("qr_panel", "qr_update", "cholqr", "cholqr_gemm", "gemm", "gemm_bf16", "gram", "band", "chase", "tri_eig", "chase_back",
           "band_back", "encode_w", "encode_residual", "quantize", "decode_w", "decode", "attend")
# kernels with roofline targets, timed inside the timed steps
TIMED_ROOF = ("gram", "encode_residual", "decode")
CSRC = os.path.join(ROOT, "kv_cache_compression_mode_amd", "csrc")
MFMA_BF16_PEAK_TFLOPS = 2500.0
# fp32 vector arithmetic without packed instructions (which the build turns
# off): 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz
VALU_FP32_PEAK_TFLOPS = 78.6
# kernels whose launches account their algorithmic work (bytes, flops):
# name -> (description, symbol, pattern of its kernel names in profiler
#          traces, sources of the kernel, peak of the matrix cores it runs on
#          in TFLOP/s)
ROOF = {
    "chase": ("k_chase: bulge chasing, band to tridiagonal, one workgroup per matrix, sweeps pipelined over its "
              "waves (fp32 vector arithmetic)",
              "k_chase", r"k_chase<", ("tridiag.hip", "device.hpp"), VALU_FP32_PEAK_TFLOPS, "alu"),
    "chase_back": ("k_cb_tfac + k_cb_apply: the chase reflectors applied to the eigenvectors in compact-WY "
                   "blocks of 32 sweeps (fp32 matrix cores)",
                   "k_cb_apply", r"k_cb_(apply|tfac)\b", ("tridiag.hip", "device.hpp"), MFMA_FP32_PEAK_TFLOPS,
                   "mfma"),
    "band": ("k_qr_reg + k_symm_v + k_w_form + k_syr2k: dense to band, per panel a register QR, the symmetric "
             "product, W, and the lower-triangle rank-64 update (fp32 matrix cores)",
             "k_syr2k", r"k_(qr_reg|symm_v|w_form|syr2k)\b", ("tridiag.hip", "qr.hip", "device.hpp"),
             MFMA_FP32_PEAK_TFLOPS, "mfma"),
    "band_back": ("k_apply_wy: the panel reflectors applied to the eigenvectors (fp32 matrix cores)",
                  "k_apply_wy", r"k_apply_wy\b", ("tridiag.hip", "device.hpp"), MFMA_FP32_PEAK_TFLOPS, "mfma"),
    "qr_update": ("k_wy_part + k_wy_mid + k_wy_upd: block reflectors applied to tall blocks in the Householder "
                  "QR of the token factor (fp32 matrix cores)",
                  "k_wy_upd", r"k_wy_(part|mid|upd)\b", ("qr.hip", "device.hpp"), MFMA_FP32_PEAK_TFLOPS, "mfma"),
    "gemm": ("k_gemm: strided batched 64x64-tile GEMM on fp32 matrix cores (small products)",
             "k_gemm", r"k_gemm(<|_bf16\b)", ("gemm.hip", "device.hpp"), MFMA_FP32_PEAK_TFLOPS, "mfma"),
    "gram": ("k_gemm_x on the token and feature Grams of the tensors (bf16 matrix cores; a triangle-only "
             "output counts the symmetric half, M (M + 1) K flops)",
             "k_gemm_x_gram", None, ("gemm.hip", "device.hpp"), MFMA_BF16_PEAK_TFLOPS, "mfma"),
    "encode_residual": ("k_encode_residual_many: reconstruction U~_T (G~ U~_D^T), residual, JL rotation R Q^T, "
                        "group quantization and packing in one pass over X (bf16 matrix cores over two-part "
                        "splits)",
                        "k_encode_residual_many", r"k_encode_residual(_many)?<", ("codec.hip", "device.hpp"),
                        MFMA_BF16_PEAK_TFLOPS, "mfma"),
    "decode": ("k_decode: X^ = U~_T W + Y^ Q with dequantization fused, all records of a launch (bf16 matrix "
               "cores, W = G~ U~_D^T as bf16 hi + lo)",
               "k_decode", r"k_decode<", ("codec.hip", "device.hpp"), MFMA_BF16_PEAK_TFLOPS, "mfma"),
    "quantize": ("k_quantize: group quantizer alone, one group of 32 per thread (fp32 in, b-bit codes and bf16 "
                 "offset/step out)",
                 "k_quantize", r"k_quantize\b", ("codec.hip", "device.hpp"), None, "hbm"),
    "attend": ("k_attn_decode: attention of new query vectors over a layer's K and V records, the records "
               "decoded tile by tile in registers (bf16 matrix cores), block softmax partials",
               "k_attn_decode", r"k_attn_decode\b", ("attn.hip", "device.hpp"), MFMA_BF16_PEAK_TFLOPS, "mfma"),
    "gemm_bf16": ("k_gemm_x: 128x128-tile GEMM on bf16 matrix cores (token and feature Grams, factor recovery, "
                  "Rayleigh and core products; fp32 operands enter as bf16 hi + lo)",
                  "k_gemm_x", r"k_gemm_x<", ("gemm.hip", "device.hpp"), MFMA_BF16_PEAK_TFLOPS, "mfma"),
}


def traffic_file(symbol, workload):
    return os.path.join(ROOT, "profiles", f"traffic_{symbol}_{workload}.json")


def kernel_sources(name):
    return tuple(os.path.join(CSRC, f) for f in ROOF[name][3])


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(source_paths, record_path):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE runs,
    or None when the kernel's source has changed since they were taken."""
    if not os.path.exists(record_path):
        return None
    with open(record_path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != sources_sha256(source_paths):
        return None
    return rec["traffic_bytes_per_launch"]


def _pmc_means(path, counter, symbol, pattern):
    """Mean counter value (KiB per dispatch) of one kernel (trace names
    matching `pattern`) and of the calibration copy (the last elementwise
    dispatch: the copies follow the fill that allocates their source)."""
    import csv
    import re
    ker, copy = [], []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            if re.search(pattern, r["Kernel_Name"]):
                ker.append(float(r["Counter_Value"]))
            elif "elementwise" in r["Kernel_Name"]:
                copy.append(float(r["Counter_Value"]))
    if not ker or len(copy) < 2:
        raise SystemExit(f"{path}: no {symbol} or calibration-copy dispatches of {counter}")
    return sum(ker) / len(ker), copy[-1], len(ker)


def record_traffic(fetch_csv, write_csv, copy_bytes, name="gemm", workload="mistral7b_t4096_2x",
                   record_path=None, source_paths=None):
    symbol, pattern = ROOF[name][1], ROOF[name][2]
    if pattern is None:
        raise SystemExit(f"{name}: its launches share a kernel with other products; no traffic record")
    source_paths = source_paths or kernel_sources(name)
    jf, cf, n = _pmc_means(fetch_csv, "FETCH_SIZE", symbol, pattern)
    jw, cw, _ = _pmc_means(write_csv, "WRITE_SIZE", symbol, pattern)
    kib = copy_bytes / 1024.0
    f_scale, w_scale = kib / cf, kib / cw      # known bytes / counted KiB of a plain copy
    rec = {"kernel": symbol, "workload": f"{workload} (one step)", "dispatches": n,
           "fetch_kib_per_dispatch": round(jf, 3), "write_kib_per_dispatch": round(jw, 3),
           "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": round(f_scale, 6), "write_scale": round(w_scale, 6),
           "traffic_bytes_per_launch": round((jf * f_scale + jw * w_scale) * 1024.0),
           "sources": [os.path.relpath(p, ROOT) for p in source_paths],
           "source_sha256": sources_sha256(source_paths)}
    record_path = record_path or traffic_file(symbol, workload)
    os.makedirs(os.path.dirname(record_path), exist_ok=True)
    with open(record_path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def roofline_for(name, st, workload):
    """Roofline of a kernel from its launches in the timed steps: time from HIP
    events around every launch on its stream, algorithmic bytes and flops as
    the launches account them (the GEMM: operands read once and the output
    written once, 2 M N K flops)."""
    launches = max(st["launches"], 1)
    avg_ms = st["total_ms"] / launches
    bytes_l = st["bytes"] / launches
    flops_l = st["flops"] / launches
    ai = flops_l / max(bytes_l, 1.0)
    gbps = bytes_l / (avg_ms * 1e-3) / 1e9
    tflops = flops_l / (avg_ms * 1e-3) / 1e12
    peak_tf, kind = ROOF[name][4], ROOF[name][5]
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBPS * 1e9) if peak_tf else float("inf")
    if ai < ridge:
        bound, achieved, peak, unit = "hbm", gbps, HBM_PEAK_GBPS, "GB/s"
    else:
        bound, achieved, peak, unit = kind, tflops, peak_tf, "TFLOP/s"
    desc, symbol, pattern = ROOF[name][0], ROOF[name][1], ROOF[name][2]
    traffic = (measured_traffic(kernel_sources(name), traffic_file(symbol, workload)) if pattern else None)
    extra = {"frac_hbm": round(gbps / HBM_PEAK_GBPS, 4)}
    if peak_tf:
        extra["frac_mfma"] = round(tflops / peak_tf, 4)
    if traffic:
        extra["traffic_over_algorithmic"] = round(traffic / max(bytes_l, 1.0), 3)
    return {"kernel": desc, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic, **extra,
            "algorithmic_bytes_per_launch": round(bytes_l),
            "algorithmic_flops_per_launch": round(flops_l),
            "arithmetic_intensity": round(ai, 2), "ridge": round(ridge, 2),
            "GBps": round(gbps, 1), "TFLOPs": round(tflops, 2),
            "avg_launch_ms": round(avg_ms, 5), "launches": st["launches"]}


def attend_leg(jolt, cfg, state, rot, dev, tdt, quiet):
    """The decode fused into attention on the encoded cache: one new token's
    query vectors per layer (GQA group 4 for the 8-KV-head shape, 1 for MHA),
    every layer's K and V records attended in one call each, against decoding
    the layer to memory and attending over the decoded K and V with torch's
    batched products and softmax."""
    import torch
    L, H, T, D = cfg.n_layers, cfg.H, cfg.T, cfg.D
    G = 4 if H == 8 else 1
    blobs, choices = state["blobs"], state["choices"]
    q = torch.randn((H * G, 1, D), dtype=torch.float32, device=dev) * 0.3
    ws = torch.empty(max(jolt.attend_workspace_bytes(H, T, choices[2 * l], choices[2 * l + 1], G, 1, tdt)
                         for l in range(L)), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    def fused():
        for l in range(L):
            jolt.attend(blobs[2 * l], choices[2 * l], blobs[2 * l + 1], choices[2 * l + 1], H, T, q, G, rot,
                        dtype=tdt, out=out, workspace=ws)

    kv = [torch.empty((H, T, D), dtype=tdt, device=dev) for _ in range(2)]
    dws = torch.empty(max(jolt.decode_many_workspace_bytes(H, T, choices[2 * l:2 * l + 2], tdt) for l in range(L)),
                      dtype=torch.uint8, device=dev)
    # query columns per KV head, [H, D, G] contiguous: every batched product
    # below takes a contiguous right operand
    qcol = q.view(H, G, D).transpose(1, 2).contiguous().to(tdt)
    scale = 1.0 / D ** 0.5

    def unfused():
        for l in range(L):
            jolt.decode_many(blobs[2 * l:2 * l + 2], H, T, choices[2 * l:2 * l + 2], rot, kv, dws, dtype=tdt)
            sc = torch.matmul(kv[0], qcol)                                  # [H, T, G]
            p = torch.softmax(sc.float() * scale, dim=1).to(tdt)
            torch.matmul(p.transpose(1, 2).contiguous(), kv[1])             # [H, G, D]

    def timed(fn, reps=3, prof=None):
        fn()
        torch.cuda.synchronize()
        if prof:
            jolt.profile_enable(prof)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        st = jolt.profile_query(prof) if prof else None
        if prof:
            jolt.profile_enable(None)
        return e0.elapsed_time(e1) / reps, st

    if quiet:
        fused()
        torch.cuda.synchronize()
        return None
    ms_f, st = timed(fused, prof="attend")
    ms_u, _ = timed(unfused)
    rec_bytes = sum(b.numel() - 256 for b in blobs)
    kv_bytes = 2 * L * H * T * D * (2 if tdt == torch.bfloat16 else 4)
    line = {"workload": f"{L} layers, one new token, {H * G} query heads over {H} KV heads",
            "fused_ms_per_cache": round(ms_f, 4), "decode_then_sdpa_ms_per_cache": round(ms_u, 4),
            "speedup_over_decode_then_sdpa": round(ms_u / ms_f, 3),
            "records_GBps": round(rec_bytes / (ms_f * 1e-3) / 1e9, 1),
            "uncompressed_kv_equivalent_GBps": round(kv_bytes / (ms_f * 1e-3) / 1e9, 1)}
    if st and st["launches"]:
        line["roofline"] = roofline_for("attend", st, cfg.name)
    return line


def append_leg(jolt, cfg, state, xs, rot, dev, tdt, n_new=256):
    """Incremental encode: n_new tokens appended to every tensor of the
    encoded cache (folding-in against the record's stored factors; a tensor
    with no Tucker part gets the new tokens quantized alone).  The appended
    tokens are synthetic rows of the same source: the first n_new tokens of
    each tensor, rolled by one row, stand in for tokens that arrive later."""
    import torch
    L, H, T, D = cfg.n_layers, cfg.H, cfg.T, cfg.D
    blobs, choices = state["blobs"], state["choices"]
    news = [torch.roll(xs[i // 2][i % 2][:, :n_new + 1], 1, dims=1)[:, 1:].contiguous() for i in range(2 * L)]
    outs = [torch.empty(jolt.blob_bytes(H, n_new, D, choices[i], tdt), dtype=torch.uint8, device=dev)
            for i in range(2 * L)]
    need = [jolt.append_workspace_bytes(H, T, choices[i], n_new, tdt) for i in range(2 * L) if choices[i][0] > 0]
    ws = torch.empty(max(need + [1]), dtype=torch.uint8, device=dev)

    def run():
        for i in range(2 * L):
            if choices[i][0] > 0:
                jolt.append(blobs[i], H, T, choices[i], news[i], rot, out=outs[i], workspace=ws)
            else:
                jolt.encode(news[i], choices[i], None, None, rot, out=outs[i])

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3
    errs = {0: [], 1: []}
    for i in range(2 * L):
        o = jolt.decode(outs[i], H, n_new, choices[i], rot, dtype=tdt)
        x = news[i].double()
        errs[i % 2].append(float(torch.linalg.vector_norm(x - o.double()) / torch.linalg.vector_norm(x)))
    return {"workload": f"{n_new} tokens appended to each of the cache's {2 * L} tensors",
            "ms_per_cache": round(ms, 3), "tokens_per_s": round(n_new / (ms * 1e-3), 1),
            "rel_err_K_mean": round(sum(errs[0]) / len(errs[0]), 6),
            "rel_err_V_mean": round(sum(errs[1]) / len(errs[1]), 6)}


SWEEP_RATIOS = (2.0, 2.25, 2.5, 2.75, 3.0)


def xl_rank(H, T, D, layers, ratio):
    """Largest cross-layer SVD rank whose group bytes (2 H T r per tensor +
    2 D r per group) fit the group's share of the budget."""
    budget = int(2.0 * H * T * D / ratio) * layers
    r = 0
    while r < D and layers * 2 * H * T * (r + 1) + 2 * D * (r + 1) <= budget:
        r += 1
    return r


def compare_codecs(jolt, cfg, xs, flat, rot, outs, tdt, dev):
    """Relative Frobenius errors (mean over the cache's K and V tensors) of
    JoLT across a 2x..3x budget sweep, and of the comparison codecs at
    matched bytes: rotated and unrotated b-bit quantization (the largest
    b <= 4 that fits), cross-layer SVD (one feature basis per layer group
    and kind), and JoLT at the 4-bit quantizer's byte total."""
    import numpy as np
    import torch
    L, H, T, D = cfg.n_layers, cfg.H, cfg.T, cfg.D
    G = 4
    n_in = H * T * D

    def decode_into(blobs, choices, q):
        ws = torch.empty(jolt.decode_many_workspace_bytes(H, T, choices, tdt), dtype=torch.uint8, device=dev)
        res = {}
        for l in range(L):                     # two output buffers per layer when streaming
            jolt.decode_many(blobs[2 * l:2 * l + 2], H, T, choices[2 * l:2 * l + 2], q, outs[:2] if len(outs) == 2
                             else outs[2 * l:2 * l + 2], ws, dtype=tdt)
            for k in (0, 1):
                o = outs[k] if len(outs) == 2 else outs[2 * l + k]
                xd = xs[l][k].double()
                res[(l, k)] = float(torch.linalg.vector_norm(xd - o.double()) / torch.linalg.vector_norm(xd))
        e = np.array([[res[(l, k)] for k in (0, 1)] for l in range(L)])
        return {"K": round(float(e[:, 0].mean()), 6), "V": round(float(e[:, 1].mean()), 6)}

    def jolt_at(ratio):
        res = jolt.allocate(xs, ratio=ratio, method=cfg.method, bits=cfg.bits, seed=cfg.seed)
        choices = [res.choice_of(i // 2, i % 2) for i in range(2 * L)]
        blobs = jolt.encode_many(flat, choices, res, rot, seed=cfg.seed)
        e = decode_into(blobs, choices, rot)
        plan = {}
        for (g, k), c in sorted(res.choice.items()):
            plan.setdefault("KV"[k], []).append(list(c))
        return {"ratio": ratio, "bytes": int(res.total_bytes), "budget": int(res.budget_bytes),
                "rel_err": e, "plan": plan}

    def quant_at(b, q):
        choices = [(0, 0, b)] * (2 * L)
        blobs = jolt.encode_many(flat, choices, [(None, None)] * (2 * L), q, seed=cfg.seed)
        return {"bits": b, "bytes": int(sum(x.numel() for x in blobs)), "rel_err": decode_into(blobs, choices, q)}

    def xl_at(ratio):
        r = xl_rank(H, T, D, G, ratio)
        err = np.zeros((L, 2))
        nbytes = 0
        for g0 in range(0, L, G):
            layers = list(range(g0, min(L, g0 + G)))
            for k in (0, 1):
                basis, coeffs, _ = jolt.xl_encode([xs[l][k] for l in layers], r)
                dec = jolt.xl_decode(basis, coeffs, dtype=tdt)
                nbytes += 2 * D * r + sum(c.numel() * 2 for c in coeffs)
                for l, o in zip(layers, dec):
                    xd = xs[l][k].double()
                    err[l, k] = float(torch.linalg.vector_norm(xd - o.double()) / torch.linalg.vector_norm(xd))
                del dec, coeffs
        return {"rank": r, "bytes": int(nbytes),
                "rel_err": {"K": round(float(err[:, 0].mean()), 6), "V": round(float(err[:, 1].mean()), 6)}}

    ident = jolt.rotation_from(np.eye(D), device=dev)
    sweep = [jolt_at(r) for r in SWEEP_RATIOS]
    b4 = jolt.blob_bytes(H, T, D, (0, 0, 4))
    r4 = 2.0 * n_in / b4                          # the 4-bit quantizer's compression ratio
    at2 = {"budget_ratio": 2.0, "jolt": sweep[0],
           "rotated_quant": quant_at(4, rot), "unrotated_quant": quant_at(4, ident), "cross_layer_svd": xl_at(2.0)}
    at4 = {"budget_ratio": round(r4, 4), "jolt": jolt_at(r4),
           "rotated_quant": quant_at(4, rot), "unrotated_quant": quant_at(4, ident), "cross_layer_svd": xl_at(r4)}
    for m in (at2, at4):
        j = m["jolt"]["rel_err"]
        m["error_over_jolt"] = {name: {kv: round(m[name]["rel_err"][kv] / j[kv], 2) for kv in "KV"}
                                for name in ("rotated_quant", "unrotated_quant", "cross_layer_svd")}
    return {"metric": "relative Frobenius error (mean over the cache's tensors), JoLT vs comparison codecs",
            "config": {"workload": cfg.name, "layers": L, "kv_heads": H, "tokens": T, "head_dim": D,
                       "input_dtype": cfg.dtype, "method": cfg.method},
            "data": "synthetic (seeded low-rank + noise + outlier channels, model cache shapes)",
            "sweep": sweep, "matched_bytes_2x": at2, "matched_bytes_4bit": at4}


def cpu_baseline(cfg, n_tensors):
    """The fp64 oracle on a bounded sample of the same workload (host cores):
    BLAS threads set to the cores this process may run on; analyze + encode +
    decode per sampled tensor at a fixed choice, scaled to the whole cache."""
    import numpy as np

    import kvgen
    from oracle import alloc, codec, rotation
    cores = len(os.sched_getaffinity(0))
    blas, limits = [], None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = sorted({f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads before)"
                       for i in threadpool_info() if i.get("user_api") == "blas"})
        limits = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        pass
    cap = alloc.rank_cap_T(cfg.H, cfg.T, cfg.D, cfg.ratio)
    choice = (cap, 64, 2)
    Q = rotation.rotation(cfg.seed, cfg.D)
    t_enc = t_dec = 0.0
    errs = {0: [], 1: []}
    done = 0
    try:
        for i in range(n_tensors):
            l, k = i // 2, i % 2
            X = kvgen.config_tensor(cfg, l, k).astype(np.float64)   # input generation is not timed
            t0 = time.perf_counter()
            a = codec.analyze(X, cap, cfg.method, cfg.seed, l, k)
            e = codec.encode_tensor(X, a["U_T"], a["U_D"], choice, Q)
            t1 = time.perf_counter()
            xh = codec.decode_tensor(e, Q, cfg.dtype)
            t2 = time.perf_counter()
            t_enc += t1 - t0
            t_dec += t2 - t1
            errs[k].append(codec.rel_err(X, xh))
            done += 1
    finally:
        if limits is not None:
            limits.restore_original_limits()
    frac = done / (2 * cfg.n_layers)
    out_bytes = done * cfg.H * cfg.T * cfg.D * (2 if cfg.dtype == "bf16" else 4)
    dt = t_enc + t_dec
    return {"value": round(cfg.T * frac / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {2 * cfg.n_layers} tensors (layers 0..{(done - 1) // 2}): analyze "
                      f"({cfg.method} fp64 factors) + encode at (r_T={cap}, r_D=64, b=2) + decode; "
                      f"the dual allocation over the whole cache (milliseconds) is not included; "
                      f"tokens/s scaled by the sampled fraction of the cache, {dt:.1f} s",
            "blas": blas, "blas_threads": int(cores),
            "encode_tokens_per_s": round(cfg.T * frac / t_enc, 2),
            "decode_output_GBps": round(out_bytes / t_dec / 1e9, 4),
            "rel_err_K_mean": round(float(np.mean(errs[0])), 6) if errs[0] else None,
            "rel_err_V_mean": round(float(np.mean(errs[1])), 6) if errs[1] else None}


if __name__ == "__main__":
    main()
