#!/usr/bin/env python3
"""Benchmark one Muon step (momentum + quintic Newton-Schulz + update) of the
GPT-2-124M body (12 layers, d = 768: 48 [768,768] + 12 [768,3072] + 12
[3072,768] matrices) on one MI355X through libmuon's C ABI.

Prints one JSON line. `value` is the Newton-Schulz algorithmic TFLOP/s of the
whole step (all kernels, inputs resident in HBM); `ms_per_step` is the step
latency, `step_ms` its per-step mean, std, median and min. `roofline` covers
the dominant kernel, timed with HIP events around each of its launches on its
own stream; `cpu_baseline` times the float64 CPU oracle on a bounded sample of
the same workload (bf16-contract and exact modes, plus one 1.5B-body layer
extrapolated to 48). `per_config` repeats the measurement for the other four
workloads (the tiny fp32 block, the 124M body with NorMuon, the stress batch
and the 1.5B body, the last with one gradient set); `env` records the
software and hardware.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-other-configs]
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
    """Hash of the kernel and planner sources with comments and blank space
    removed, so that a committed counter summary stays matched to the code it
    was taken on across comment-only edits."""
    import re
    h = hashlib.sha256()
    for f in ("kernels_ns.hip", "kernels_ns_mfma.hip", "kernels_ns_small.hip", "kernels_ns_panel.hip",
              "kernels_elementwise.hip", "kernel_common.hpp", "ns_mfma_common.hpp",
              "device_types.hpp", "plan.cpp", "api.cpp"):
        with open(os.path.join(ROOT, "muon_newton_schulz_04_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)   # block comments
        src = re.sub(r"//[^\n]*", "", src)                  # line comments
        src = "\n".join(ln.strip() for ln in src.splitlines() if ln.strip())
        h.update(src.encode("utf-8"))
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            t = json.load(f)
        if t.get("source_hash") != _kernel_source_hash():
            return None
        return float(t["kernels"][kernel]["hbm_bytes_per_launch"])
    except Exception:
        return None


COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written


def copy_calibration() -> None:
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) measured on the same box."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    # torch's elementwise negation: one streaming read and one streaming write
    # of 1 GiB each (a same-dtype copy_ would go to the DMA engines instead).
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _pmc_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        yield from csv.DictReader(f)


def _pmc_args(workload_id: int):
    """Directory suffix, bench.py arguments and time limit (s) of the counter
    runs for a workload (the 1.5B body's inputs take minutes to generate)."""
    if workload_id == 1:
        return "", " --no-other-configs", 120
    return f"_c{workload_id}", f" --config {workload_id}", 300


def pmc_summary(fetch_dir: str, write_dir: str, workload: str, workload_id: int = 1) -> dict:
    """Per-launch HBM traffic of each NS kernel class from two rocprofv3
    --pmc runs (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), each scaled by
    what the same counter reads for the 1 GiB calibration copy."""
    import statistics
    per = {}
    unmatched = set()
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = {}
        for r in _pmc_rows(d):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = _kernel_class(name)
            if not key:
                unmatched.add(name[:80])
                continue
            grid = int(r["Grid_Size"])
            vals.setdefault(key, {}).setdefault(grid, []).append(float(r["Counter_Value"]) * 1024.0)
        # per kernel class, the launches with the largest grid: the kernel
        # pass's one-stream launches, which the roofline is measured on
        per[counter] = {k: statistics.median(v[max(v)]) for k, v in vals.items()}
    fscale = COPY_BYTES / per["FETCH_SIZE"]["copy"]
    wscale = COPY_BYTES / per["WRITE_SIZE"]["copy"]
    sfx, cfg, lim = _pmc_args(workload_id)
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL " + str(lim) + " rocprofv3 --pmc {c} -f csv -d $REPO/gpurun_out/{d} "
           "-o run -- python3 $REPO/bench.py" + cfg + " --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration")
    out = {"workload": workload, "source_hash": _kernel_source_hash(),
           "commands": [cmd.format(c="FETCH_SIZE", d="pmc_fetch" + sfx), cmd.format(c="WRITE_SIZE", d="pmc_write" + sfx),
                        f"python3 bench.py{cfg} --pmc-summary gpurun_out/pmc_fetch{sfx} gpurun_out/pmc_write{sfx}"],
           "note": "FETCH_SIZE/WRITE_SIZE are KiB per dispatch; each is scaled so that the 1 GiB calibration "
                   "read/write (torch.neg over 2^28 floats) counts 2^30 bytes; medians over the dispatches with "
                   "the largest grid of each kernel class (the one-stream kernel pass the roofline is timed on)",
           "copy_fetch_bytes": per["FETCH_SIZE"]["copy"], "copy_write_bytes": per["WRITE_SIZE"]["copy"],
           "fetch_scale": fscale, "write_scale": wscale, "kernels": {}}
    for k in per["FETCH_SIZE"]:
        if k == "copy" or k not in per["WRITE_SIZE"]:
            continue
        out["kernels"][k] = {"fetch_bytes": per["FETCH_SIZE"][k] * fscale,
                             "write_bytes": per["WRITE_SIZE"][k] * wscale,
                             "hbm_bytes_per_launch": per["FETCH_SIZE"][k] * fscale + per["WRITE_SIZE"][k] * wscale}
    if unmatched:
        print("unmatched kernels:", sorted(unmatched), file=sys.stderr)
    return out


LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS")


def lds_summary(pmc_dir: str, workload_id: int) -> dict:
    """LDS behaviour of each kernel class from one rocprofv3 --pmc run of
    SQ_LDS_BANK_CONFLICT, SQ_LDS_ADDR_CONFLICT, SQ_LDS_IDX_ACTIVE and
    SQ_INSTS_LDS: the cycles LDS is stalled by bank (and address) conflicts
    as a share of the cycles it spends on indexed (ds_*) operations, and the
    LDS instructions issued; medians over the largest-grid dispatches of each
    class (the one-stream kernel pass). The direct-to-LDS loads of the NS
    kernels are not indexed operations and are not counted here."""
    import statistics
    from workloads import get_workload
    w = get_workload(workload_id)
    per = {}
    for r in _pmc_rows(pmc_dir):
        key = _kernel_class(r["Kernel_Name"])
        if not key or key == "copy":
            continue
        d = per.setdefault(key, {}).setdefault(int(r["Grid_Size"]), {})
        d.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    sfx, cfg, lim = _pmc_args(workload_id)
    out = {"workload": w.name, "source_hash": _kernel_source_hash(),
           "commands": [f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL {lim} rocprofv3 --pmc "
                        + " ".join(LDS_COUNTERS) + f" -f csv -d $REPO/gpurun_out/pmc_lds{sfx} -o run -- python3 "
                        f"$REPO/bench.py{cfg} --steps 3 --warmup 1 --no-cpu-baseline",
                        f"python3 bench.py{cfg} --pmc-lds-summary gpurun_out/pmc_lds{sfx}"],
           "note": "bank_conflict_pct = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE x 100 (both summed over the "
                   "GPU); addr_conflict_pct likewise for SQ_LDS_ADDR_CONFLICT; lds_insts = SQ_INSTS_LDS",
           "kernels": {}}
    for key, grids in sorted(per.items()):
        launches = [d for d in grids[max(grids)].values() if all(c in d for c in LDS_COUNTERS)]
        if not launches:
            continue
        act = statistics.median(d["SQ_LDS_IDX_ACTIVE"] for d in launches)
        bank = statistics.median(d["SQ_LDS_BANK_CONFLICT"] for d in launches)
        addr = statistics.median(d["SQ_LDS_ADDR_CONFLICT"] for d in launches)
        out["kernels"][key] = {"dispatches": len(launches), "lds_idx_active_cycles": act,
                               "bank_conflict_cycles": bank, "bank_conflict_pct": 100.0 * bank / act if act else None,
                               "addr_conflict_cycles": addr, "addr_conflict_pct": 100.0 * addr / act if act else None,
                               "lds_insts": statistics.median(d["SQ_INSTS_LDS"] for d in launches)}
    return out


def _ns_alg_flops(workload) -> dict:
    """Algorithmic FLOP of one GRAM / POLY / UPDATE launch over every active
    bf16 matrix of a workload (symmetric Gram and A A count m(m+1) k)."""
    out = {"gram": 0.0, "poly": 0.0, "update": 0.0}
    for e in workload.entries:
        if e.frozen:
            continue
        m, n = min(e.rows, e.cols), max(e.rows, e.cols)
        out["gram"] += e.count * m * (m + 1) * n
        out["poly"] += e.count * m * (m + 1) * m
        out["update"] += e.count * 2 * m * m * n
    return out


def mfma_summary(pmc_dir: str, workload_id: int) -> dict:
    """MFMA utilisation of each NS kernel class from one rocprofv3 --pmc run
    (MfmaUtil, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE,
    SQ_INSTS_VALU_MFMA_MOPS_BF16): rocprofiler's derived MfmaUtil (MFMA busy
    cycles summed over all SIMDs / (the largest per-XCD GUI-active count x
    SIMDs)) and the bf16 MFMA work executed against the algorithmic work,
    medians over the largest-grid dispatches (the one-stream kernel pass)."""
    import statistics
    from workloads import get_workload
    w = get_workload(workload_id)
    alg = _ns_alg_flops(w)
    per = {}
    for r in _pmc_rows(pmc_dir):
        key = _kernel_class(r["Kernel_Name"])
        if key not in ("gram", "poly", "update"):
            continue
        d = per.setdefault(key, {}).setdefault(int(r["Grid_Size"]), {})
        d.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
    sfx, cfg, lim = _pmc_args(workload_id)
    out = {"workload": w.name, "source_hash": _kernel_source_hash(),
           "commands": [f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL {lim} rocprofv3 --pmc MfmaUtil "
                        "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 -f csv -d "
                        f"$REPO/gpurun_out/pmc_mfma{sfx} -o run -- python3 $REPO/bench.py{cfg} --steps 3 --warmup 1 "
                        "--no-cpu-baseline",
                        f"python3 bench.py{cfg} --pmc-mfma-summary gpurun_out/pmc_mfma{sfx}"],
           "note": "mfma_util_pct is rocprofiler's MfmaUtil (sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (max over "
                   "the XCDs of GRBM_GUI_ACTIVE x SIMDs) x 100); executed_flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; "
                   "alg_flop counts the symmetric Gram and A A as m(m+1)k, so executed / alg > 1 is the diagonal "
                   "tiles' lower halves and the padding",
           "kernels": {}}
    for key, grids in per.items():
        launches = list(grids[max(grids)].values())
        util = statistics.median(d["MfmaUtil"] for d in launches)
        ex = statistics.median(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0 for d in launches)
        out["kernels"][key] = {"dispatches": len(launches), "mfma_util_pct": util, "executed_flop": ex,
                               "alg_flop": alg[key], "executed_over_alg": ex / alg[key] if alg[key] else None,
                               "mfma_busy_cycles": statistics.median(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in launches)}
    return out


def _kernel_class(name: str) -> str:
    """gram / poly / update / ns_small / ns_panel / momentum / apply / copy for a kernel name, or '' otherwise."""
    if "neg_kernel" in name:
        return "copy"
    if "k_ns_big<" in name or "k_ns<" in name:
        mode = name.split("<", 1)[1].split(">", 1)[0].split(",")
        return {"0": "gram", "1": "poly", "2": "update"}[mode[2].strip()]
    for k in ("ns_small", "ns_panel", "momentum", "apply"):
        if "k_" + k in name:
            return k
    return ""


def _short_kernel(name: str) -> str:
    """A readable label for a libmuon kernel from its demangled name."""
    import re
    mode = {"0": "GRAM", "1": "POLY", "2": "UPDATE"}
    m = re.search(r"k_ns_big<(\d+), (\d+), (\d), (\w+)(?:, (\w+))?>", name)
    if m:
        return (f"k_ns_big {mode[m.group(3)]} T={m.group(1)} waves={2 * int(m.group(2))}"
                + (" +rowstats" if m.group(4) == "true" else "") + (" +nt" if m.group(5) == "true" else ""))
    m = re.search(r"k_ns<([^,]+), (\d+), (\d)>", name)
    if m:
        return f"k_ns<{'bf16' if 'bf' in m.group(1) else 'f32'}> {mode[m.group(3)]} T={m.group(2)}"
    for k in ("k_ns_small", "k_ns_panel", "k_momentum", "k_apply", "k_normuon", "k_zero_momentum", "k_fill_zero"):
        if k in name:
            return k
    return name[:60]


def trace_summary(trace_dir: str, workload: str, command: str) -> str:
    """Markdown table of a rocprofv3 --kernel-trace run: per kernel and grid
    size (the stream-group launches of a stage have smaller grids than the
    one-stream launches of the kernel pass), calls and durations."""
    import csv
    import glob
    import statistics
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = {}
    total = 0.0
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(wg, 1)
            rows.setdefault((_short_kernel(r["Kernel_Name"]), grid), []).append(dur)
            total += dur
    out = [f"# rocprofv3 kernel trace — Muon step, {workload}", "",
           "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
           f"Kernel sources hash (bench.py `source_hash`): `{_kernel_source_hash()}`. The bench runs the timed steps "
           "with the shipped stream-group schedule (a stage's launches split over up to three streams, smaller "
           "grids), then "
           "the kernel pass with every launch on one stream (full grids); the roofline uses the full-grid rows.", "",
           "| kernel | workgroups | calls | avg µs | median µs | min µs | max µs | share |",
           "|---|---|---|---|---|---|---|---|"]
    for (k, grid), d in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {grid} | {len(d)} | {statistics.mean(d):.1f} | {statistics.median(d):.1f} | "
                   f"{min(d):.1f} | {max(d):.1f} | {100 * sum(d) / total:.1f}% |")
    return "\n".join(out) + "\n"


def _oracle_layer(d: int, seed: int):
    from workloads import custom_workload
    return custom_workload(seed, [(d, d, 4, "spike"), (d, 4 * d, 1, "spike"), (4 * d, d, 1, "spike")])


def _ns_alg_flops_step(layer, ns_steps: int = 5) -> float:
    f = 0.0
    for _gi, _ei, _k, _off, r, c in layer.submatrices():
        m, n = min(r, c), max(r, c)
        f += ns_steps * (m * (m + 1) * n + m * (m + 1) * m + 2 * m * m * n)
    return f


def _time_oracle(layer, mode: str, seconds: float, min_steps: int = 1):
    """Full oracle steps (momentum, NS, update) on one layer until `seconds`
    of oracle time have passed (at least min_steps); gradient generation is
    not timed. Returns (steps, seconds)."""
    import numpy as np

    import oracle as O
    from workloads import gen_grads, gen_params
    orc = O.OracleMuon(layer.entries, layer.total, mode=mode)
    p = gen_params(layer).astype(np.float64)
    steps, el = 0, 0.0
    while el < seconds or steps < min_steps:
        g = gen_grads(layer, steps)
        t1 = time.perf_counter()
        p = orc.step(p, g, lr=0.02)
        el += time.perf_counter() - t1
        steps += 1
    return steps, el


def cpu_baseline(seconds: float) -> dict:
    """The oracle (float64 NumPy) timed on the host: full steps of layer 0 of
    the 124M body in the bf16-contract mode (the reported value) and in the
    exact mode, and one step of one layer of the 1.5B body (exact mode),
    extrapolated to its 48 layers."""
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    layer = _oracle_layer(768, 1)
    f_layer = _ns_alg_flops_step(layer)
    sc, ec = _time_oracle(layer, "bf16", seconds)
    se, ee = _time_oracle(layer, "exact", seconds * 0.5)
    big = _oracle_layer(1600, 3)
    sb, eb = _time_oracle(big, "exact", 0.0, min_steps=1)
    out = {
        "value": f_layer * sc / ec / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"layer 0 of the 124M body (4x[768,768] + [768,3072] + [3072,768]), bf16-contract "
                  f"float64 oracle, {sc} full step(s) incl. momentum and update, {ec:.1f} s; "
                  f"rate = NS algorithmic FLOP / wall time",
        "ms_per_layer_step": ec / sc * 1e3,
        "modes": {
            "bf16_contract": {"steps": sc, "seconds": ec, "ms_per_layer_step": ec / sc * 1e3,
                              "tflops": f_layer * sc / ec / 1e12,
                              "ms_per_step_12_layers_extrapolated": 12 * ec / sc * 1e3},
            "exact": {"steps": se, "seconds": ee, "ms_per_layer_step": ee / se * 1e3,
                      "tflops": f_layer * se / ee / 1e12,
                      "ms_per_step_12_layers_extrapolated": 12 * ee / se * 1e3},
        },
        "body_1p5b": {"sample": "one layer of the 1.5B body (4x[1600,1600] + [1600,6400] + [6400,1600]), exact "
                                "float64 oracle, one full step",
                      "ms_per_layer_step": eb / sb * 1e3,
                      "tflops": _ns_alg_flops_step(big) * sb / eb / 1e12,
                      "ms_per_step_48_layers_extrapolated": 48 * eb / sb * 1e3,
                      "note": "extrapolation: one measured layer x 48 layers"},
    }
    return out


def env_snapshot() -> dict:
    """Versions and hardware of the run (GPU, ROCm, hipcc, torch, host CPU)."""
    import platform

    import numpy as np
    import torch
    env = {"gpu": torch.cuda.get_device_name(0) if torch.cuda.is_available() else None,
           "torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
           "python": platform.python_version(), "numpy": np.__version__, "host_cores": os.cpu_count()}
    try:
        props = torch.cuda.get_device_properties(0)
        env["gpu_arch"] = getattr(props, "gcnArchName", None)
        env["gpu_cus"] = props.multi_processor_count
        env["gpu_mem_gib"] = round(props.total_memory / 2 ** 30, 1)
    except Exception:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    # the compiler that built libmuon, as the build recorded it (no child
    # process is started here: under a profiler it would inherit a GPU context)
    try:
        with open(os.path.join(ROOT, "muon_newton_schulz_04_amd", "libmuon.build.txt")) as f:
            env["hipcc"] = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("hipcc:")), None)
    except OSError:
        env["hipcc"] = None
    try:
        with open("/proc/cpuinfo") as f:
            env["cpu"] = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        env["cpu"] = None
    return env


def _stats(xs):
    import statistics
    return {"mean": statistics.mean(xs), "std": statistics.stdev(xs) if len(xs) > 1 else 0.0,
            "median": statistics.median(xs), "min": min(xs), "max": max(xs), "n": len(xs)}


def measure(w, steps: int, warmup: int, kernel_steps: int, pool: int, stream_groups: int, events: bool = True):
    """Time workload w on cuda:0 through the C ABI.

    Timed pass: the shipped stream-group schedule, a HIP event on the
    caller's stream before the first step and after every step (each step
    joins the caller's stream at its end, and the next starts after it), so
    per-step times and the mean come from the same run. Kernel pass: the same
    steps with every launch on one stream, each launch bracketed by the
    library's own HIP events on that stream (per-kernel averages, roofline).
    Inputs are resident in HBM before timing; `pool` gradient sets are
    cycled."""
    import numpy as np
    import torch

    from muon_newton_schulz_04_amd import binding as B
    from workloads import gen_grads, gen_params

    hpkw = dict(momentum=w.momentum, nesterov=w.nesterov, ns_steps=w.ns_steps, precision=w.ns_precision,
                normuon=w.normuon, normuon_beta2=w.normuon_beta2, normuon_eps=w.normuon_eps,
                weight_decay=w.weight_decay)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    params = torch.from_numpy(gen_params(w)).to(dev)
    grads = [torch.from_numpy(gen_grads(w, t)).to(dev) for t in range(pool)]
    t_gen = time.perf_counter() - t_gen
    mom = torch.zeros(w.total, dtype=torch.float32, device=dev)
    H = B.MuonHandle(w.entries, B.make_hparams(**hpkw, stream_groups=stream_groups))
    work = B.muon_work_stats(H.h)
    stream = torch.cuda.current_stream(dev)
    print(f"# workload {w.name}: {w.num_matrices} matrices, {w.total} elements, workspace "
          f"{H.ws_bytes / 2**20:.0f} MiB, inputs drawn in {t_gen:.1f} s", file=sys.stderr, flush=True)
    for t in range(warmup):
        H.step(params, grads[t % pool], mom, w.lr)
    H.reset(mom)  # warm-up dirtied the optimizer state
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for t in range(steps):
        H.step(params, grads[t % pool], mom, w.lr)
        ev[t + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [ev[t].elapsed_time(ev[t + 1]) for t in range(steps)]
    ms = ev[0].elapsed_time(ev[steps]) / steps
    ns_flops = sum(work.flops[k] for k in (B.MUON_KERNEL_GRAM, B.MUON_KERNEL_POLY, B.MUON_KERNEL_UPDATE,
                                            B.MUON_KERNEL_NS_SMALL, B.MUON_KERNEL_NS_PANEL))
    fp32 = w.ns_precision == "fp32"
    peak = PEAK_FP32_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    res = {"workload": w.name, "steps": steps, "warmup": warmup, "grad_sets": pool, "ms_per_step": ms,
           "stream_groups": int(work.launches[B.MUON_KERNEL_MOMENTUM]),
           "step_ms": _stats(per_step), "wall_s": wall, "ns_alg_gflop_per_step": ns_flops / 1e9,
           "ns_tflops_step": ns_flops / (ms * 1e-3) / 1e12, "pct_peak_step": ns_flops / (ms * 1e-3) / 1e12 / peak * 100,
           "peak_tflops": peak, "dtype": "fp32" if fp32 else "bf16", "elements": w.total,
           "matrices": w.num_matrices}
    del H
    kernels = {}
    if events and kernel_steps > 0:
        H1 = B.MuonHandle(w.entries, B.make_hparams(**hpkw, stream_groups=1))
        for t in range(min(warmup, 3)):
            H1.step(params, grads[t % pool], mom, w.lr)
        torch.cuda.synchronize()
        B.muon_profile_enable(H1.h, 1)
        for t in range(kernel_steps):
            H1.step(params, grads[t % pool], mom, w.lr)
        torch.cuda.synchronize()
        B.muon_profile_enable(H1.h, 0)
        work1 = B.muon_work_stats(H1.h)
        for k, name in enumerate(B.KERNEL_NAMES):
            s, n, tot = B.muon_profile_read(H1.h, k, 0)
            if n == 0:
                continue
            per_launch_ms = tot / n
            entry = {"launches": n, "avg_ms": per_launch_ms, "ms_per_step": tot / kernel_steps}
            lps = work1.launches[k]
            if work1.flops[k] > 0:
                entry["tflops"] = work1.flops[k] / lps / (per_launch_ms * 1e-3) / 1e12
                entry["pct_peak"] = entry["tflops"] / peak * 100
            if work1.bytes[k] > 0:
                entry["gbs"] = work1.bytes[k] / lps / (per_launch_ms * 1e-3) / 1e9
                entry["pct_hbm_peak"] = entry["gbs"] / PEAK_HBM_GBS * 100
            kernels[name] = entry
        B.muon_profile_read(H1.h, 0, 1)
        ns_ms = sum(kernels.get(k, {}).get("ms_per_step", 0.0)
                    for k in ("gram", "poly", "update", "ns_small", "ns_panel"))
        res["ns_tflops_kernels"] = ns_flops / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None
        res["kernel_pass_steps"] = kernel_steps
        if kernels:
            dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
            kidx = B.KERNEL_NAMES.index(dom)
            e = kernels[dom]
            if work1.flops[kidx] > 0:
                rf = {"bound": "mfma", "achieved": e["tflops"], "peak": peak, "unit": "TFLOP/s",
                      "frac": e["tflops"] / peak, "alg_per_launch": work1.flops[kidx] / work1.launches[kidx]}
            else:
                rf = {"bound": "hbm", "achieved": e["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": e["gbs"] / PEAK_HBM_GBS, "alg_per_launch": work1.bytes[kidx] / work1.launches[kidx]}
            rf["kernel"] = dom
            rf["avg_launch_ms"] = e["avg_ms"]
            rf["traffic"] = _traffic(dom, w.name)
            res["roofline"] = rf
        del H1
    res["kernels"] = kernels
    assert np.isfinite(params[:1000].cpu().numpy()).all()
    del params, grads, mom
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# the other workloads: (config id, timed steps, kernel-pass steps, gradient sets)
OTHER_CONFIGS = ((0, 50, 20, 4), (2, 50, 20, 4), (4, 50, 20, 4), (3, 10, 3, 1))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, help="workload id (1 = GPT-2-124M body)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true", help="do not time kernels with events")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="measure only the headline workload (no per-config section)")
    ap.add_argument("--stream-groups", type=int, default=0,
                    help="stream groups of the timed pass (0: the library's choice, 1 .. 4)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 1 GiB once per pass (HBM counter calibration)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "COMMAND"),
                    help="summarise a rocprofv3 --kernel-trace run into profiles/kernel_stats_<workload>.md and exit")
    ap.add_argument("--pmc-mfma-summary", metavar="PMC_DIR",
                    help="summarise a rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16 into profiles/mfma_<workload>.json and exit")
    ap.add_argument("--pmc-lds-summary", metavar="PMC_DIR",
                    help="summarise a rocprofv3 --pmc run of " + ", ".join(LDS_COUNTERS)
                         + " into profiles/lds_<workload>.json and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into "
                         "profiles/traffic_<workload>.json and exit")
    args = ap.parse_args()

    if args.trace_summary:
        from workloads import get_workload as _gw
        wname = _gw(args.config).name
        md = trace_summary(args.trace_summary[0], wname, args.trace_summary[1])
        with open(os.path.join(ROOT, "profiles", f"kernel_stats_{wname}.md"), "w") as f:
            f.write(md)
        print(md)
        return 0

    if args.pmc_mfma_summary:
        t = mfma_summary(args.pmc_mfma_summary, args.config)
        path = os.path.join(ROOT, "profiles", f"mfma_{t['workload']}.json")
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
        return 0

    if args.pmc_lds_summary:
        t = lds_summary(args.pmc_lds_summary, args.config)
        path = os.path.join(ROOT, "profiles", f"lds_{t['workload']}.json")
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
        return 0

    if args.pmc_summary:
        from workloads import get_workload as _gw
        wname = _gw(args.config).name
        t = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], wname, args.config)
        path = os.path.join(ROOT, "profiles", f"traffic_{wname}.json")
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py: libmuon's step runs on one GPU only (asked for --gpus {args.gpus}); a sharded "
              "multi-GPU step is not implemented.", file=sys.stderr)
        return 2

    import torch

    from workloads import get_workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    w = get_workload(args.config)
    head = measure(w, args.steps, args.warmup, 0 if args.no_events else args.steps, GRAD_POOL, args.stream_groups,
                   events=not args.no_events)
    others = {}
    if not args.no_other_configs and args.config == 1:
        for cid, st, kst, pool in OTHER_CONFIGS:
            wo = get_workload(cid)
            others[wo.name] = measure(wo, st, min(args.warmup, 10), 0 if args.no_events else kst, pool,
                                      args.stream_groups, events=not args.no_events)
    fp32 = w.ns_precision == "fp32"
    out = {
        "metric": METRIC,
        "value": head["ns_tflops_step"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if fp32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": len(w.entries) // 3 if args.config in (1, 2, 3) else None,
                   "matrices": w.num_matrices, "elements": w.total, "ns_steps": w.ns_steps,
                   "ns_precision": w.ns_precision, "normuon": w.normuon, "parallelism": "single GPU",
                   "stream_groups": head["stream_groups"]},
        "step_ms": head["step_ms"],
        "ns_alg_gflop_per_step": head["ns_alg_gflop_per_step"],
        "ns_tflops_kernels": head.get("ns_tflops_kernels"),
        "pct_bf16_peak_step": head["ns_tflops_step"] / PEAK_BF16_TFLOPS * 100.0,
        "roofline": head.get("roofline"),
        "kernels": head["kernels"],
        "kernels_pass": "a second pass of the same steps with every launch on one stream (stream_groups=1), "
                        "each timed with HIP events; the timed region above runs the shipped stream-group "
                        "schedule without per-launch events",
        "per_config": others,
        "wall_s": head["wall_s"],
        "device": torch.cuda.get_device_name(0),
        "source_hash": _kernel_source_hash(),
    }
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    out["env"] = env_snapshot()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
