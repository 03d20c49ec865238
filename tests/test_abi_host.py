"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load, export every function include/libmuon.h declares, and
validate tables before touching HIP; on a host without a GPU, muon_init must
fail cleanly with MUON_E_NO_DEVICE.
"""

import ctypes
import math
import os
import re

import pytest

from muon_newton_schulz_04_amd import binding as B
from workloads import custom_workload, get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmuon.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = B.load()
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B._SIGS), "binding and header disagree"


def test_struct_sizes_match_c_layout():
    assert ctypes.sizeof(B.muon_matrix) == 48
    assert ctypes.sizeof(B.muon_hparams) == 4 * 4 + 16 * 3 * 4 + 4 * 7
    assert ctypes.sizeof(B.muon_layout) == 8 + 8 + 8 * 4 + 8 + 8


def test_hparams_default_values():
    hp = B.muon_hparams_default()
    assert math.isclose(hp.momentum, 0.95, rel_tol=1e-7)
    assert hp.nesterov == 1 and hp.ns_steps == 5 and hp.ns_precision == B.MUON_NS_BF16
    for k in range(B.MUON_MAX_NS_STEPS):
        a, b, c = hp.ns_coeffs[k]
        assert (round(a, 4), round(b, 4), round(c, 4)) == (3.4445, -4.775, 2.0315)
    assert math.isclose(hp.ns_eps, 1e-7, rel_tol=1e-6)
    assert hp.normuon == 0 and math.isclose(hp.normuon_eps, 1e-10, rel_tol=1e-6)
    assert hp.stream_groups == 0  # the library chooses (one group for small steps, else three)


def _ws(entries, hp=None):
    return B.muon_workspace_bytes(entries, hp)


def test_workspace_bytes_arithmetic():
    # one 100 x 300 matrix (T = 128): canonical 100 x 300 -> padded 128 x 384, bf16
    w = custom_workload(50, [(100, 300, 1)])
    s, nbytes = _ws(w.entries, B.muon_hparams_default())
    assert s == B.MUON_OK
    x = 128 * 384 * 2
    a = 128 * 128 * 2
    assert nbytes >= 3 * x + 2 * a
    # fp32 mode stores the Newton-Schulz buffers as float32, on 64-tiles at
    # this size: padded 128 x 320
    s2, nbytes32 = _ws(w.entries, B.make_hparams(precision="fp32"))
    x32 = 128 * 320 * 4
    a32 = 128 * 128 * 4
    assert s2 == B.MUON_OK and nbytes32 >= 3 * x32 + 2 * a32
    # tile choice: a small fp32 matrix goes on 64-tiles (136 x 520 -> 192 x 576,
    # not 256 x 640 as 128-tiles would pad it); a bf16 256 x 1024 matrix is not
    # padded at all
    w2 = custom_workload(51, [(136, 520, 1)])
    s4, nb4 = _ws(w2.entries, B.make_hparams(precision="fp32"))
    assert s4 == B.MUON_OK
    assert 3 * 192 * 576 * 4 + 2 * 192 * 192 * 4 <= nb4 < 3 * 256 * 640 * 4 + 2 * 256 * 256 * 4
    w3 = custom_workload(52, [(256, 1024, 2)])
    s5, nb5 = _ws(w3.entries, B.muon_hparams_default())
    assert s5 == B.MUON_OK
    assert 2 * (3 * 256 * 1024 * 2 + 2 * 256 * 256 * 2) <= nb5 < 2 * (3 * 384 * 1024 * 2 + 2 * 384 * 384 * 2)
    # the 124M body: 48 padded 768^2 + 24 padded 768 x 3072 canonical matrices
    body = get_workload(1)
    s3, nb = _ws(body.entries, B.muon_hparams_default())
    x_elems = 48 * 768 * 768 + 24 * 768 * 3072
    assert s3 == B.MUON_OK and nb >= 3 * x_elems * 2 + 2 * 72 * 768 * 768 * 2


def test_validation_errors():
    hp = B.muon_hparams_default()
    M = B.muon_matrix
    assert _ws([M(0, 4, 1, 0, 1.0, 1.0, 0, 0)], hp)[0] == B.MUON_E_SHAPE
    assert _ws([M(4, 4, 0, 0, 1.0, 1.0, 0, 0)], hp)[0] == B.MUON_E_SHAPE
    assert _ws([M(4, 4, 1, -1, 1.0, 1.0, 0, 0)], hp)[0] == B.MUON_E_LAYOUT
    assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 0), M(4, 4, 1, 8, 1.0, 1.0, 0, 0)], hp)[0] == B.MUON_E_LAYOUT
    assert _ws([M(4, 4, 1, 0, float("nan"), 1.0, 0, 0)], hp)[0] == B.MUON_E_INVALID_ARG
    assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 7)], hp)[0] == B.MUON_E_INVALID_ARG
    assert "reserved" in B.muon_last_error()
    bad = B.muon_hparams_default()
    bad.ns_steps = 0
    assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 0)], bad)[0] == B.MUON_E_INVALID_ARG
    bad = B.muon_hparams_default()
    bad.momentum = 1.5
    assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 0)], bad)[0] == B.MUON_E_INVALID_ARG
    bad = B.muon_hparams_default()
    bad.ns_precision = 3
    assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 0)], bad)[0] == B.MUON_E_INVALID_ARG
    for groups in (5, -1):
        bad = B.muon_hparams_default()
        bad.stream_groups = groups
        assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 0)], bad)[0] == B.MUON_E_INVALID_ARG
    # adjacent (touching) entries are fine; empty table is fine
    assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 0), M(4, 4, 1, 16, 1.0, 1.0, 0, 0)], hp)[0] == B.MUON_OK
    assert _ws([], hp)[0] == B.MUON_OK
    # NULL hparams means the defaults
    assert _ws([M(4, 4, 1, 0, 1.0, 1.0, 0, 0)], None)[0] == B.MUON_OK


def test_status_strings():
    for s in range(-7, 1):
        assert B.muon_status_string(s)
    assert B.muon_status_string(-99) == "unknown status"


def test_init_without_gpu_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host has a GPU")
    w = custom_workload(51, [(8, 8, 1)])
    s, nbytes = _ws(w.entries, None)
    assert s == B.MUON_OK
    buf = (ctypes.c_ubyte * (nbytes + 256))()
    addr = (ctypes.addressof(buf) + 255) // 256 * 256
    s, h = B.muon_init(w.entries, None, addr, nbytes, 0)
    assert s == B.MUON_E_NO_DEVICE and not h.value
    # validation comes first: a bad table reports its own error, not the device
    s, h = B.muon_init([B.muon_matrix(0, 1, 1, 0, 1.0, 1.0, 0, 0)], None, addr, nbytes, 0)
    assert s == B.MUON_E_SHAPE
    # a null / misaligned workspace is rejected before the device is queried
    s, h = B.muon_init(w.entries, None, 0, nbytes, 0)
    assert s == B.MUON_E_WORKSPACE
    s, h = B.muon_init(w.entries, None, addr + 16, nbytes, 0)
    assert s == B.MUON_E_WORKSPACE


def test_null_handle_calls_are_safe():
    lib = B.load()
    assert lib.muon_step(None, None, None, None, 0, 0.1, -1.0, None) == B.MUON_E_INVALID_ARG
    assert lib.muon_reset(None, None, 0, None) == B.MUON_E_INVALID_ARG
    assert lib.muon_num_matrices(None) == 0
    lib.muon_destroy(None)


# ---- host-side schedules, pinned to the values the pages print ----

def test_wsd_schedule_matches_the_pages():
    # [P3] FlexAttention record: 1875 iterations, no warmup, warmdown 562 steps,
    # "the warmdown starts at step 1313 and falls linearly to 0"
    n, wd = 1875, 562
    assert n - wd == 1313
    assert B.muon_lr_wsd(0, n, 0, wd) == 1.0
    assert B.muon_lr_wsd(1312, n, 0, wd) == 1.0
    assert B.muon_lr_wsd(1313, n, 0, wd) == 1.0  # (n - it) / wd = 1 at the first warmdown step
    assert math.isclose(B.muon_lr_wsd(1874, n, 0, wd), 1.0 / wd, rel_tol=1e-6)  # last step: one step from 0
    assert all(B.muon_lr_wsd(i + 1, n, 0, wd) < B.muon_lr_wsd(i, n, 0, wd) for i in range(1313, 1874))
    # [P4] 50B run: 95367 iterations, warmdown 27247 ("about 28.6% of training")
    assert round(27247 / 95367 * 100, 1) == 28.6
    assert B.muon_lr_wsd(95367 - 27247 - 1, 95367, 0, 27247) == 1.0
    # halfway through the warmdown the multiplier is half (n - it = 13623 steps left of 27247)
    assert math.isclose(B.muon_lr_wsd(95367 - 13623, 95367, 0, 27247), 13623 / 27247, rel_tol=1e-6)
    # the Adam group's 500-step warmup: (it + 1) / 500
    assert math.isclose(B.muon_lr_wsd(0, 95367, 500, 27247), 1 / 500, rel_tol=1e-6)
    assert B.muon_lr_wsd(499, 95367, 500, 27247) == 1.0
    assert math.isnan(B.muon_lr_wsd(n, n, 0, wd)) and math.isnan(B.muon_lr_wsd(-1, n, 0, wd))


def test_cooldown_floor_schedule_matches_the_pages():
    # [P2] change 3: last 80% of the main phase decays to the 0.30 floor, the
    # 20 extension steps stay on the floor
    main, frac, floor = 1000, 0.80, 0.30
    assert B.muon_lr_cooldown_floor(0, main, frac, floor) == 1.0
    assert B.muon_lr_cooldown_floor(200, main, frac, floor) == 1.0  # 1 - 0.8 of the way in: still flat
    assert math.isclose(B.muon_lr_cooldown_floor(600, main, frac, floor), 0.30 + 0.70 * 0.5, rel_tol=1e-6)
    for s in range(main, main + 20):
        assert math.isclose(B.muon_lr_cooldown_floor(s, main, frac, floor), floor, rel_tol=1e-6)
    vals = [B.muon_lr_cooldown_floor(s, main, frac, floor) for s in range(200, main + 1)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))


def test_momentum_warmup_matches_the_pages():
    # [P3]: frac = min(step / 500, 1), momentum from 0.85 to 0.95
    assert math.isclose(B.muon_momentum_warmup(0, 500, 0.85, 0.95), 0.85, rel_tol=1e-6)
    assert math.isclose(B.muon_momentum_warmup(250, 500, 0.85, 0.95), 0.90, rel_tol=1e-6)
    assert math.isclose(B.muon_momentum_warmup(500, 500, 0.85, 0.95), 0.95, rel_tol=1e-6)
    assert math.isclose(B.muon_momentum_warmup(10000, 500, 0.85, 0.95), 0.95, rel_tol=1e-6)
    assert math.isnan(B.muon_momentum_warmup(-1, 500, 0.85, 0.95))
