"""Throughput of the JoLT codec hot path on one MI355X.

One step = the whole path over one synthetic cache: spectra, factors and the
Lagrangian-dual allocation of all layers x {K, V} (jolt_allocate), encode of
every tensor (jolt_encode), decode of every tensor (jolt_decode).  The default
workload is the Mistral-7B-v0.3-shaped GQA cache: 32 layers x {K, V},
8 KV heads, T = 4096, D = 128, bf16, 2x byte budget, exact Gram factors.

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
    p.add_argument("--cpu-sample-tensors", type=int, default=2)
    p.add_argument("--profile-step", action="store_true",
                   help="run warmup + one step only (for rocprofv3 runs)")
    return p.parse_args()


def main():
    args = parse()
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
    L, H, T, D = cfg.n_layers, cfg.H, cfg.T, cfg.D
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {L}x2 tensors [{H},{T},{D}] {cfg.dtype}", file=sys.stderr, flush=True)
    host = [[kvgen.config_tensor(cfg, l, k) for k in (0, 1)] for l in range(L)]
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    xs = [tuple(torch.from_numpy(host[l][k]).to(tdt).to(dev) for k in (0, 1)) for l in range(L)]
    flat = [xs[l][k] for l in range(L) for k in (0, 1)]
    rot = jolt.rotation(cfg.seed)
    out = torch.empty((H, T, D), dtype=tdt, device=dev)
    outs = [torch.empty((H, T, D), dtype=tdt, device=dev) for _ in range(2 * L)]
    stream = torch.cuda.current_stream(dev)

    state = {}

    def step(record=None):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e2 = torch.cuda.Event(enable_timing=True)
        e3 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        res = jolt.allocate(xs, ratio=cfg.ratio, method=cfg.method, bits=cfg.bits, seed=cfg.seed)
        e1.record(stream)
        blobs, choices = [], []
        for i, x in enumerate(flat):
            ch = res.choice_of(i // 2, i % 2)
            Ut, Ud = res.factors(i)
            blobs.append(jolt.encode(x, ch, Ut, Ud, rot, seed=cfg.seed))
            choices.append(ch)
        e2.record(stream)
        dws = torch.empty(jolt.decode_many_workspace_bytes(H, T, choices, tdt), dtype=torch.uint8,
                          device=dev)
        jolt.decode_many(blobs, H, T, choices, rot, outs, dws, dtype=tdt)
        e3.record(stream)
        state.update(res=res, blobs=blobs, choices=choices, ev=(e0, e1, e2, e3))
        if record is not None:
            record.append(state["ev"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = 1 if args.profile_step else args.steps
    evs = []
    t0 = time.perf_counter()
    for _ in range(K):
        step(evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_alloc = np.mean([a.elapsed_time(b) for a, b, c, d in evs])
    ms_enc = np.mean([b.elapsed_time(c) for a, b, c, d in evs])
    ms_dec = np.mean([c.elapsed_time(d) for a, b, c, d in evs])
    ms_step = wall * 1e3 / K
    if args.profile_step:
        print(json.dumps({"profile_step_ms": ms_step}), flush=True)
        return

    res, blobs, choices = state["res"], state["blobs"], state["choices"]
    blob_total = sum(b.numel() for b in blobs)
    in_bytes = sum(x.numel() * x.element_size() for x in flat)

    # decode roofline: algorithmic bytes = every record read once + every output
    # written once, over the batched decode of the whole cache, timed live with
    # HIP events on the launch stream
    dws = torch.empty(jolt.decode_many_workspace_bytes(H, T, choices, tdt), dtype=torch.uint8, device=dev)
    reps = 5
    de0, de1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    de0.record(stream)
    for _ in range(reps):
        jolt.decode_many(blobs, H, T, choices, rot, outs, dws, dtype=tdt)
    de1.record(stream)
    torch.cuda.synchronize()
    dec_ms = de0.elapsed_time(de1) / reps
    dec_bytes = (blob_total - 256 * len(flat)) + in_bytes
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9

    # quality on every tensor (outside the timed region)
    errs = []
    for i, x in enumerate(flat):
        xh = outs[i]
        xd = x.double()
        errs.append(float(torch.linalg.vector_norm(xd - xh.double()) / torch.linalg.vector_norm(xd)))
    errs = np.array(errs).reshape(L, 2)

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
                   "tensors": 2 * L},
        "phases_ms": {"allocate": round(ms_alloc, 3), "encode": round(ms_enc, 3),
                      "decode": round(ms_dec, 3)},
        "encode_tokens_per_s": round(T / ((ms_alloc + ms_enc) * 1e-3), 2),
        "decode_GBps": round(dec_gbps, 1),
        "decode_ms": round(dec_ms, 4),
        "decode_output_GBps": round(in_bytes / (ms_dec * 1e-3) / 1e9, 1),
        "compression_ratio_vs_bf16": round(in_bytes * (2 / flat[0].element_size()) / blob_total, 4),
        "plan_bytes": int(res.total_bytes), "budget_bytes": int(res.budget_bytes),
        "rel_err_K_mean": round(float(errs[:, 0].mean()), 6),
        "rel_err_V_mean": round(float(errs[:, 1].mean()), 6),
        "roofline": {"kernel": "jolt_decode_many (k_make_w + k_decode, whole cache)", "bound": "hbm",
                     "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_call": int(dec_bytes),
                     "avg_call_ms": round(dec_ms, 5)},
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, host, args.cpu_sample_tensors)
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, host, n_tensors):
    """The fp64 oracle on a bounded sample of the same workload (host cores)."""
    import numpy as np

    from oracle import alloc, codec, rotation
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    cap = alloc.rank_cap_T(cfg.H, cfg.T, cfg.D, cfg.ratio)
    Q = rotation.rotation(cfg.seed, cfg.D)
    t0 = time.perf_counter()
    done = 0
    for i in range(n_tensors):
        l, k = i // 2, i % 2
        X = host[l][k].astype(np.float64)
        a = codec.analyze(X, cap, cfg.method, cfg.seed, l, k)
        e = codec.encode_tensor(X, a["U_T"], a["U_D"], (cap, 64, 2), Q)
        codec.decode_tensor(e, Q, cfg.dtype)
        done += 1
    dt = time.perf_counter() - t0
    frac = done / (2 * cfg.n_layers)
    return {"value": round(cfg.T * frac / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {2 * cfg.n_layers} tensors (layers 0..{(done - 1) // 2}): analyze "
                      f"(exact fp64 factors) + encode at (r_T={cap}, r_D=64, b=2) + decode; "
                      f"the dual allocation over the whole cache (milliseconds) is not included; "
                      f"tokens/s scaled by the sampled fraction of the cache, {dt:.1f} s"}


if __name__ == "__main__":
    main()
