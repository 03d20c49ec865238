"""Properties of the gfx950 assembly of the kernels that load global memory
straight into LDS (CPU only: hipcc cross-compiles).

Those loads take their LDS address in M0, and the helper that issues them sets
M0 itself, in the same inline-asm block, right before the load. The compiler
reserves M0 and does not honour a clobber of it, so the helper is only safe
while the compiler keeps no M0 value of its own in these kernels. This test
compiles them with the library's own flags and checks, over the whole
assembly, that
  - every explicit M0 operand is the helper's `s_mov_b32 m0, s<N>`, and the
    next instruction is its direct-to-LDS buffer load;
  - every direct-to-LDS load is so preceded (none is the compiler's own);
  - no instruction that reads M0 implicitly (indirect register moves,
    messages, GWS / append / ordered-count LDS operations, global loads to
    LDS, parameter and interpolation loads) appears at all.
"""

import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from muon_newton_schulz_04_amd import build

SOURCES = ("kernels_ns_mfma.hip", "kernels_ns_panel.hip")

# mnemonics (prefixes) whose encodings read M0 without naming it
IMPLICIT_M0 = ("s_movrel", "v_movrel", "s_sendmsg", "s_ttracedata", "ds_gws", "ds_append", "ds_consume",
               "ds_ordered_count", "global_load_lds", "ds_param_load", "ds_direct_load", "v_interp",
               "lds_param_load", "lds_direct_load")
M0_WRITE = re.compile(r"^s_mov_b32\s+m0,\s*s\d+$")
LDS_DMA = re.compile(r"^buffer_load_dword\w*\s.*\blds$")
M0_OPERAND = re.compile(r"\bm0\b")


def _instructions(asm: str):
    """The instruction lines of an assembly listing, comments and directives
    stripped, labels and blank lines dropped."""
    out = []
    for line in asm.splitlines():
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        out.append(line)
    return out


def _compile(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = ([build.hipcc()] + build._flags(src) + ["--offload-device-only", "-S", os.path.join(build.CSRC, src),
                                                 "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    with open(out) as f:
        return f.read()


def check_m0_use(insts):
    """(pairs, problems): the number of helper pairs and a list of the lines
    that break the rules above."""
    problems = []
    pairs = 0
    for i, ins in enumerate(insts):
        if ins.startswith(IMPLICIT_M0):
            problems.append(f"implicit M0 reader: {ins}")
        if LDS_DMA.match(ins):
            if i == 0 or not M0_WRITE.match(insts[i - 1]):
                problems.append(f"LDS load without its own M0 write: {ins}")
            continue
        if M0_OPERAND.search(ins):
            if M0_WRITE.match(ins) and i + 1 < len(insts) and LDS_DMA.match(insts[i + 1]):
                pairs += 1
            else:
                problems.append(f"M0 use outside the helper: {ins}")
    return pairs, problems


def test_checker_flags_foreign_m0_use():
    """The checker itself: a listing with only helper pairs passes; a
    compiler-style M0 value, a bare LDS load and an implicit reader fail."""
    good = ["s_mov_b32 m0, s5", "buffer_load_dwordx4 v1, s[8:11], s2 offen lds", "s_waitcnt vmcnt(0)"]
    assert check_m0_use(good) == (1, [])
    for bad in (["s_mov_b32 m0, -1", "ds_read_b32 v0, v1"],
                ["buffer_load_dwordx4 v1, s[8:11], s2 offen lds"],
                ["s_mov_b32 m0, s5", "s_nop 0", "buffer_load_dwordx4 v1, s[8:11], s2 offen lds"],
                ["v_movrels_b32 v0, v1"],
                ["s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)"]):
        assert check_m0_use(bad)[1], bad


def _have_hipcc():
    try:
        return bool(build.hipcc())
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_m0_written_only_by_the_lds_load_helper(tmp_path):
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        listings = list(ex.map(lambda s: _compile(s, str(tmp_path)), SOURCES))
    for src, asm in zip(SOURCES, listings):
        pairs, problems = check_m0_use(_instructions(asm))
        assert pairs > 0, f"{src}: no direct-to-LDS loads found (the check would be vacuous)"
        assert not problems, f"{src}: " + "; ".join(problems[:10])
