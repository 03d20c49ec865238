"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

api.cpp, plan.cpp and schedule.cpp are compiled with g++ and
-fsanitize=address,undefined, linked with stub kernel launchers
(tests/native/launch_stubs.cpp) and the HIP runtime, and driven by
tests/native/abi_check.c: table validation, planning of the five workloads'
tables, argument checks of every entry point and the host schedules. Any
sanitizer report aborts the check program.

The planner's decisions are checked by tests/native/plan_check.cpp, built
against plan.cpp alone with the same sanitizers: every tile of every tiled
matrix listed exactly once in its group's Gram, polynomial and update lists,
each active matrix in exactly one Newton-Schulz kernel class, and the
stream-group count and per-group cache policies of the workloads' tables.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "muon_newton_schulz_04_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _have_toolchain():
    return (shutil.which("g++") and shutil.which("gcc") and
            os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")) and
            os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")))


@pytest.mark.skipif(not _have_toolchain(), reason="g++ / gcc / ROCm HIP runtime not available")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    inc = [f"-I{ROCM}/include", f"-I{ROOT}/include", "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src in ("api.cpp", "plan.cpp", "schedule.cpp"):
        o = str(tmp_path / (src + ".o"))
        subprocess.run(["g++", "-std=c++17", *san, *inc, "-c", os.path.join(CSRC, src), "-o", o], check=True)
        objs.append(o)
    o = str(tmp_path / "launch_stubs.o")
    subprocess.run(["g++", "-std=c++17", *san, *inc, "-c", os.path.join(NATIVE, "launch_stubs.cpp"), "-o", o],
                   check=True)
    objs.append(o)
    o = str(tmp_path / "abi_check.o")
    subprocess.run(["gcc", "-std=c99", "-Wall", *san, *inc, "-c", os.path.join(NATIVE, "abi_check.c"), "-o", o],
                   check=True)
    objs.append(o)
    exe = str(tmp_path / "abi_check")
    subprocess.run(["g++", *san, *objs, "-o", exe, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-lm"],
                   check=True)
    env = dict(os.environ)
    # leaks inside the HIP runtime's own initialisation are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all expectations hold" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


@pytest.mark.skipif(not _have_toolchain(), reason="g++ / ROCm headers not available")
def test_planner_decisions_under_asan_and_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    inc = [f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}", "-D__HIP_PLATFORM_AMD__"]
    exe = str(tmp_path / "plan_check")
    subprocess.run(["g++", "-std=c++17", *san, *inc, os.path.join(NATIVE, "plan_check.cpp"),
                    os.path.join(CSRC, "plan.cpp"), "-o", exe], check=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all expectations hold" in r.stdout
