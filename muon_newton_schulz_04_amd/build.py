"""Build libmuon.so in-tree with hipcc for gfx950.

Every call recompiles every source (so a stale library never survives a
source change) and links muon_newton_schulz_04_amd/libmuon.so.
Usage: python -m muon_newton_schulz_04_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmuon.so")
# compiler version and flags of the last build, next to the library (read by
# bench.py's environment record, which runs no compiler itself)
BUILD_INFO = os.path.join(PKG, "libmuon.build.txt")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "plan.cpp", "schedule.cpp", "kernels_elementwise.hip", "kernels_ns.hip",
           "kernels_ns_mfma.hip", "kernels_ns_small.hip", "kernels_ns_panel.hip", "static_scratch.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmuon)")


def _flags(src: str):
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]
    if src.endswith(".hip"):
        # packed fp32 math stays off; the kernels are written for scalar / float2 code
        return common + ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                         "-packed-fp32-ops", "-mllvm", "-disable-promote-alloca-to-lds"]
    return common + [f"--offload-arch={ARCH}"]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}",
           f"-Wl,--version-script={os.path.join(CSRC, 'libmuon.map')}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libmuon.so failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if OUT == os.path.join(PKG, "libmuon.so"):
        r = subprocess.run([cc, "--version"], capture_output=True, text=True)
        ver = " | ".join(x.strip() for x in r.stdout.splitlines() if "version" in x.lower())
        with open(BUILD_INFO, "w") as f:
            f.write(f"hipcc: {ver}\narch: {ARCH}\nflags (.hip): {' '.join(_flags('x.hip'))}\n")
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
