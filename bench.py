#!/usr/bin/env python3
"""Benchmark one Muon step (momentum + quintic Newton-Schulz + update) of the
GPT-2-124M body (12 layers, d = 768: 48 [768,768] + 12 [768,3072] + 12
[3072,768] matrices) on one MI355X through libmuon's C ABI.

Prints one JSON line. `value` is the Newton-Schulz algorithmic TFLOP/s of the
whole step (all kernels, inputs resident in HBM); `ms_per_step` is the step
latency. `roofline` covers the dominant kernel, timed with HIP events around
each of its launches inside the timed region; `cpu_baseline` times the
float64 CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon step ms + NS TFLOP/s (% bf16 MFMA peak), GPT-2-124M body, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
GRAD_POOL = 4               # distinct gradient sets cycled through the timed steps


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("kernels_ns.hip", "kernels_ns_mfma.hip", "kernels_elementwise.hip", "kernel_common.hpp"):
        with open(os.path.join(ROOT, "muon_newton_schulz_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str, launches_bytes: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            t = json.load(f)
        if t.get("source_hash") != _kernel_source_hash():
            return None
        return float(t["hbm_bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(seconds: float) -> dict:
    """The oracle (float64 NumPy, bf16 rounding contract) on layer 0 of the body."""
    import numpy as np

    import oracle as O
    from workloads import custom_workload, gen_grads, gen_params
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    d = 768
    layer = custom_workload(1, [(d, d, 4, "spike"), (d, 4 * d, 1, "spike"), (4 * d, d, 1, "spike")])
    orc = O.OracleMuon(layer.entries, layer.total, mode="bf16")
    p = gen_params(layer).astype(np.float64)
    flops_per_step = 0.0
    for _gi, _ei, _k, _off, r, c in layer.submatrices():
        m, n = min(r, c), max(r, c)
        flops_per_step += 5 * (m * (m + 1) * n + m * (m + 1) * m + 2 * m * m * n)
    steps = 0
    el = 0.0  # oracle time only; drawing the gradients is not timed
    while el < seconds:
        g = gen_grads(layer, steps)
        t1 = time.perf_counter()
        p = orc.step(p, g, lr=0.02)
        el += time.perf_counter() - t1
        steps += 1
    return {
        "value": flops_per_step * steps / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"layer 0 of the 124M body (4x[768,768] + [768,3072] + [3072,768]), bf16-contract "
                  f"float64 oracle, {steps} full step(s) incl. momentum and update, {el:.1f} s; "
                  f"rate = NS algorithmic FLOP / wall time",
        "ms_per_layer_step": el / steps * 1e3,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, help="workload id (1 = GPT-2-124M body)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true", help="do not time kernels with events")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the sharded "
              "multi-GPU step is not part of it.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from muon_newton_schulz_04_amd import binding as B
    from workloads import gen_grads, gen_params, get_workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    w = get_workload(args.config)
    hp = B.make_hparams(momentum=w.momentum, nesterov=w.nesterov, ns_steps=w.ns_steps, precision=w.ns_precision,
                        normuon=w.normuon, normuon_beta2=w.normuon_beta2, normuon_eps=w.normuon_eps,
                        weight_decay=w.weight_decay)
    H = B.MuonHandle(w.entries, hp)
    work = B.muon_work_stats(H.h)
    dev = torch.device("cuda:0")
    params = torch.from_numpy(gen_params(w)).to(dev)
    mom = torch.zeros(w.total, dtype=torch.float32, device=dev)
    pool = [torch.from_numpy(gen_grads(w, t)).to(dev) for t in range(GRAD_POOL)]
    stream = torch.cuda.current_stream(dev)
    print(f"# workload {w.name}: {w.num_matrices} matrices, {w.total} elements, "
          f"workspace {H.ws_bytes / 2**20:.0f} MiB", file=sys.stderr, flush=True)

    for t in range(args.warmup):
        H.step(params, pool[t % GRAD_POOL], mom, w.lr)
    H.reset(mom)  # warm-up dirtied the optimizer state
    torch.cuda.synchronize()

    if not args.no_events:
        B.muon_profile_enable(H.h, 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for t in range(args.steps):
        H.step(params, pool[t % GRAD_POOL], mom, w.lr)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    B.muon_profile_enable(H.h, 0)
    ms = start.elapsed_time(stop) / args.steps
    assert np.isfinite(params[:1000].cpu().numpy()).all()

    ns_flops = work.flops[B.MUON_KERNEL_GRAM] + work.flops[B.MUON_KERNEL_POLY] + work.flops[B.MUON_KERNEL_UPDATE]
    value = ns_flops / (ms * 1e-3) / 1e12
    fp32 = w.ns_precision == "fp32"
    peak = PEAK_FP32_TFLOPS if fp32 else PEAK_BF16_TFLOPS

    kernels = {}
    if not args.no_events:
        for k, name in enumerate(B.KERNEL_NAMES):
            s, n, tot = B.muon_profile_read(H.h, k, 0)
            if n == 0:
                continue
            per_launch_ms = tot / n
            entry = {"launches": n, "avg_ms": per_launch_ms, "ms_per_step": tot / args.steps}
            lps = work.launches[k]
            if work.flops[k] > 0:
                entry["tflops"] = work.flops[k] / lps / (per_launch_ms * 1e-3) / 1e12
            if work.bytes[k] > 0:
                entry["gbs"] = work.bytes[k] / lps / (per_launch_ms * 1e-3) / 1e9
            kernels[name] = entry
        B.muon_profile_read(H.h, 0, 1)
    ns_ms = sum(kernels.get(k, {}).get("ms_per_step", 0.0) for k in ("gram", "poly", "update"))
    roofline = None
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
        kidx = B.KERNEL_NAMES.index(dom)
        e = kernels[dom]
        if work.flops[kidx] > 0:
            achieved = e["tflops"]
            roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                        "frac": achieved / peak, "kernel": dom,
                        "alg_per_launch": work.flops[kidx] / work.launches[kidx]}
        else:
            achieved = e["gbs"]
            roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": achieved / PEAK_HBM_GBS, "kernel": dom,
                        "alg_per_launch": work.bytes[kidx] / work.launches[kidx]}
        roofline["avg_launch_ms"] = e["avg_ms"]
        roofline["traffic"] = _traffic(dom, w.name, roofline["alg_per_launch"])

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if fp32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": len(w.entries) // 3 if args.config in (1, 2, 3) else None,
                   "matrices": w.num_matrices, "elements": w.total, "ns_steps": w.ns_steps,
                   "ns_precision": w.ns_precision, "normuon": w.normuon, "parallelism": "single GPU"},
        "ns_alg_gflop_per_step": ns_flops / 1e9,
        "ns_tflops_kernels": (ns_flops / (ns_ms * 1e-3) / 1e12) if ns_ms > 0 else None,
        "pct_bf16_peak_step": value / PEAK_BF16_TFLOPS * 100.0,
        "roofline": roofline,
        "kernels": kernels,
        "wall_s": wall,
        "device": torch.cuda.get_device_name(0),
        "source_hash": _kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
