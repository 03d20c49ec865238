"""Host-side checks of bench.py's measurement tooling (no GPU): kernel-name
classification, the rocprofv3 trace and counter summarisers on synthetic
CSV files, the CPU-baseline leg (the oracle timed on a bounded sample) and
the refusal of multi-GPU runs."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

NAMES = {
    "muon::(anonymous namespace)::k_ns_big<256, 4, 0, false>(muon::MatDesc const*)": ("gram", "k_ns_big GRAM T=256 waves=8"),
    "muon::(anonymous namespace)::k_ns_big<256, 4, 1, false>(muon::MatDesc const*)": ("poly", "k_ns_big POLY T=256 waves=8"),
    "muon::(anonymous namespace)::k_ns_big<128, 2, 2, true>(muon::MatDesc const*)":
        ("update", "k_ns_big UPDATE T=128 waves=4 +rowstats"),
    "muon::(anonymous namespace)::k_ns_big<256, 4, 0, false, true>(muon::MatDesc const*)":
        ("gram", "k_ns_big GRAM T=256 waves=8 +nt"),
    "muon::(anonymous namespace)::k_ns_big<256, 4, 1, false, false>(muon::MatDesc const*)":
        ("poly", "k_ns_big POLY T=256 waves=8"),
    "muon::(anonymous namespace)::k_ns_big<256, 4, 2, true, false>(muon::MatDesc const*)":
        ("update", "k_ns_big UPDATE T=256 waves=8 +rowstats"),
    "muon::(anonymous namespace)::k_ns<float, 64, 2>(muon::MatDesc const*)": ("update", "k_ns<f32> UPDATE T=64"),
    "muon::(anonymous namespace)::k_momentum<__bf16>(muon::MatDesc const*)": ("momentum", "k_momentum"),
    "muon::(anonymous namespace)::k_apply<__bf16>(muon::MatDesc const*)": ("apply", "k_apply"),
    "muon::(anonymous namespace)::k_ns_small(muon::MatDesc const*)": ("ns_small", "k_ns_small"),
    "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)": ("copy", None),
}


def test_kernel_names_classify():
    for name, (cls, short) in NAMES.items():
        assert bench._kernel_class(name) == cls, name
        if short:
            assert bench._short_kernel(name) == short, name


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_from_synthetic_trace(tmp_path):
    upd = "muon::(anonymous namespace)::k_ns_big<256, 4, 2, false>(x)"
    mom = "muon::(anonymous namespace)::k_momentum<__bf16>(x)"
    rows = []
    for name, grid, dur_ns in ((upd, 1296, 150000), (upd, 1296, 140000), (upd, 432, 120000), (mom, 20736, 190000)):
        rows.append({"Kernel_Name": name, "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur_ns,
                     "Workgroup_Size_X": 512, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1,
                     "Grid_Size_X": 512 * grid, "Grid_Size_Y": 1, "Grid_Size_Z": 1})
    _write_csv(tmp_path / "run_kernel_trace.csv", rows)
    md = bench.trace_summary(str(tmp_path), "w", "cmd")
    lines = [ln for ln in md.splitlines() if ln.startswith("| k_")]
    # one row per (kernel, grid size), largest total time first
    assert lines[0].startswith("| k_ns_big UPDATE T=256 waves=8 | 1296 | 2 | 145.0 |")
    assert any(ln.startswith("| k_ns_big UPDATE T=256 waves=8 | 432 | 1 | 120.0 |") for ln in lines)
    assert any(ln.startswith("| k_momentum | 20736 | 1 | 190.0 |") for ln in lines)


def test_pmc_summary_scales_by_the_copy(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
    upd = "muon::(anonymous namespace)::k_ns_big<256, 4, 2, false>(x)"
    for counter, sub, copy_kib, upd_kib in (("FETCH_SIZE", "f", 524288.0, 1000.0), ("WRITE_SIZE", "w", 1048576.0, 300.0)):
        d = tmp_path / sub
        d.mkdir()
        rows = [{"Counter_Name": counter, "Kernel_Name": copy, "Grid_Size": 100, "Counter_Value": copy_kib},
                {"Counter_Name": counter, "Kernel_Name": upd, "Grid_Size": 1296, "Counter_Value": upd_kib},
                # a smaller-grid launch of the same kernel (a stream group's) is not the one reported
                {"Counter_Name": counter, "Kernel_Name": upd, "Grid_Size": 432, "Counter_Value": 7.0}]
        _write_csv(d / "run_counter_collection.csv", rows)
    t = bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), "w")
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    u = t["kernels"]["update"]
    assert u["fetch_bytes"] == pytest.approx(2.0 * 1000.0 * 1024)
    assert u["write_bytes"] == pytest.approx(300.0 * 1024)
    assert u["hbm_bytes_per_launch"] == pytest.approx(u["fetch_bytes"] + u["write_bytes"])


def test_lds_summary_ratios(tmp_path):
    upd = "muon::(anonymous namespace)::k_ns_big<256, 4, 2, false, false>(x)"
    mom = "muon::(anonymous namespace)::k_momentum<__bf16, false>(x)"
    rows = []
    for disp, (name, grid, vals) in enumerate((
            (upd, 1296, {"SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_ADDR_CONFLICT": 2.0, "SQ_LDS_IDX_ACTIVE": 1000.0,
                         "SQ_INSTS_LDS": 50.0}),
            (upd, 1296, {"SQ_LDS_BANK_CONFLICT": 30.0, "SQ_LDS_ADDR_CONFLICT": 4.0, "SQ_LDS_IDX_ACTIVE": 1000.0,
                         "SQ_INSTS_LDS": 70.0}),
            # a smaller-grid launch (a stream group's) is not the one reported
            (upd, 432, {"SQ_LDS_BANK_CONFLICT": 900.0, "SQ_LDS_ADDR_CONFLICT": 0.0, "SQ_LDS_IDX_ACTIVE": 1000.0,
                        "SQ_INSTS_LDS": 1.0}),
            (mom, 20736, {"SQ_LDS_BANK_CONFLICT": 0.0, "SQ_LDS_ADDR_CONFLICT": 0.0, "SQ_LDS_IDX_ACTIVE": 500.0,
                          "SQ_INSTS_LDS": 8.0}))):
        for c, v in vals.items():
            rows.append({"Dispatch_Id": disp, "Counter_Name": c, "Kernel_Name": name, "Grid_Size": grid,
                         "Counter_Value": v})
    _write_csv(tmp_path / "run_counter_collection.csv", rows)
    t = bench.lds_summary(str(tmp_path), 1)
    u = t["kernels"]["update"]
    assert u["dispatches"] == 2 and u["bank_conflict_pct"] == pytest.approx(2.0)
    assert u["addr_conflict_pct"] == pytest.approx(0.3) and u["lds_insts"] == pytest.approx(60.0)
    assert t["kernels"]["momentum"]["bank_conflict_pct"] == 0.0


def test_cpu_baseline_leg_reports_a_rate():
    r = bench.cpu_baseline(0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["ms_per_layer_step"] > 0
    assert "layer 0 of the 124M body" in r["sample"]


def test_bench_refuses_several_gpus():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
