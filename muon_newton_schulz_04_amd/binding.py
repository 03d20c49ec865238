"""ctypes binding of libmuon (include/libmuon.h), same names as the C ABI.

Argument marshalling only: every step of the Muon update runs in the HIP
kernels of libmuon.so. PyTorch is used for device memory and streams. The
library must be built first (python -m muon_newton_schulz_04_amd.build);
loading fails loudly if it is missing.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmuon.so")

MUON_OK = 0
MUON_E_INVALID_ARG = -1
MUON_E_SHAPE = -2
MUON_E_LAYOUT = -3
MUON_E_NO_DEVICE = -4
MUON_E_HIP = -5
MUON_E_STATE = -6
MUON_E_WORKSPACE = -7
MUON_E_HOST = -8

MUON_MAX_NS_STEPS = 16
MUON_STATIC_WORKSPACE_BYTES = 64 << 20
MUON_NS_BF16 = 0
MUON_NS_FP32 = 1
MUON_MOMENTUM_LERP = 0
MUON_MOMENTUM_HEAVY_BALL = 1

MUON_VIEW_XTILDE = 0
MUON_VIEW_NS_OUT = 1
MUON_VIEW_SUMSQ = 2
MUON_VIEW_SCALE = 3
MUON_VIEW_V = 4
MUON_VIEW_F = 5
MUON_VIEW_STATUS = 6
MUON_VIEW_GRAM = 7
MUON_VIEW_POLY = 8

MUON_KERNEL_MOMENTUM = 0
MUON_KERNEL_GRAM = 1
MUON_KERNEL_POLY = 2
MUON_KERNEL_UPDATE = 3
MUON_KERNEL_NORMUON = 4
MUON_KERNEL_APPLY = 5
MUON_KERNEL_NS_SMALL = 6
MUON_KERNEL_NS_PANEL = 7
MUON_KERNEL_COUNT = 8
KERNEL_NAMES = ["momentum", "gram", "poly", "update", "normuon", "apply", "ns_small", "ns_panel"]


class muon_matrix(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("count", ctypes.c_int64),
        ("offset", ctypes.c_int64),
        ("lr_mul", ctypes.c_float),
        ("wd_mul", ctypes.c_float),
        ("frozen", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class muon_hparams(ctypes.Structure):
    _fields_ = [
        ("momentum", ctypes.c_float),
        ("nesterov", ctypes.c_int32),
        ("momentum_kind", ctypes.c_int32),
        ("ns_steps", ctypes.c_int32),
        ("ns_coeffs", (ctypes.c_float * 3) * MUON_MAX_NS_STEPS),
        ("ns_eps", ctypes.c_float),
        ("ns_precision", ctypes.c_int32),
        ("normuon", ctypes.c_int32),
        ("normuon_beta2", ctypes.c_float),
        ("normuon_eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("stream_groups", ctypes.c_int32),
    ]


class muon_layout(ctypes.Structure):
    _fields_ = [
        ("x_offset", ctypes.c_int64),
        ("row_offset", ctypes.c_int64),
        ("m", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("ld", ctypes.c_int32),
        ("m_pad", ctypes.c_int32),
        ("transposed", ctypes.c_int32),
        ("active", ctypes.c_int32),
        ("stored_rows", ctypes.c_int32),
        ("stored_cols", ctypes.c_int32),
        ("param_offset", ctypes.c_int64),
        ("gram_offset", ctypes.c_int64),
    ]


class muon_work(ctypes.Structure):
    _fields_ = [
        ("flops", ctypes.c_double * MUON_KERNEL_COUNT),
        ("bytes", ctypes.c_double * MUON_KERNEL_COUNT),
        ("launches", ctypes.c_int64 * MUON_KERNEL_COUNT),
        ("active_elements", ctypes.c_int64),
    ]


_P = ctypes.c_void_p
_SIGS = {
    "muon_hparams_default": (None, [ctypes.POINTER(muon_hparams)]),
    "muon_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(muon_matrix), ctypes.c_int32,
                                            ctypes.POINTER(muon_hparams), ctypes.POINTER(ctypes.c_size_t)]),
    "muon_init": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.POINTER(muon_matrix), ctypes.c_int32,
                                 ctypes.POINTER(muon_hparams), _P, ctypes.c_size_t, ctypes.c_int32]),
    "muon_init_static": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.POINTER(muon_matrix), ctypes.c_int32,
                                        ctypes.POINTER(muon_hparams), ctypes.c_int32]),
    "muon_step": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, ctypes.c_float, ctypes.c_float, _P]),
    "muon_reset": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "muon_destroy": (None, [_P]),
    "muon_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "muon_last_error": (ctypes.c_char_p, [_P]),
    "muon_matrix_layout": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(muon_layout)]),
    "muon_num_matrices": (ctypes.c_int32, [_P]),
    "muon_debug_view": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_size_t)]),
    "muon_work_stats": (ctypes.c_int, [_P, ctypes.POINTER(muon_work)]),
    "muon_profile_enable": (ctypes.c_int, [_P, ctypes.c_int32]),
    "muon_profile_read": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                         ctypes.POINTER(ctypes.c_double)]),
    "muon_lr_wsd": (ctypes.c_float, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "muon_lr_cooldown_floor": (ctypes.c_float, [ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float]),
    "muon_momentum_warmup": (ctypes.c_float, [ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libmuon.so (after torch, so the library binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads torch's libamdhip64 first)

    if not os.path.exists(path):
        raise RuntimeError(f"libmuon.so not found at {path}; build it with "
                           "`python -m muon_newton_schulz_04_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# --- same-named thin wrappers ------------------------------------------------

def muon_hparams_default() -> muon_hparams:
    hp = muon_hparams()
    load().muon_hparams_default(ctypes.byref(hp))
    return hp


def muon_status_string(s: int) -> str:
    return load().muon_status_string(s).decode()


def muon_last_error(h=None) -> str:
    return load().muon_last_error(h).decode()


def muon_lr_wsd(it: int, num_iterations: int, warmup_iters: int, warmdown_iters: int) -> float:
    return load().muon_lr_wsd(it, num_iterations, warmup_iters, warmdown_iters)


def muon_lr_cooldown_floor(step: int, main_iterations: int, cooldown_frac: float, floor: float) -> float:
    return load().muon_lr_cooldown_floor(step, main_iterations, cooldown_frac, floor)


def muon_momentum_warmup(step: int, warmup_steps: int, start: float, end: float) -> float:
    return load().muon_momentum_warmup(step, warmup_steps, start, end)


def _table(entries) -> "ctypes.Array":
    arr = (muon_matrix * max(1, len(entries)))()
    for k, e in enumerate(entries):
        if isinstance(e, muon_matrix):
            arr[k] = e
        else:
            arr[k] = muon_matrix(int(e.rows), int(e.cols), int(e.count), int(e.offset), float(e.lr_mul),
                                 float(e.wd_mul), int(e.frozen), 0)
    return arr


def muon_workspace_bytes(entries, hp: Optional[muon_hparams]) -> tuple:
    tbl = _table(entries)
    out = ctypes.c_size_t(0)
    s = load().muon_workspace_bytes(tbl, len(entries), ctypes.byref(hp) if hp is not None else None,
                                    ctypes.byref(out))
    return s, out.value


def muon_init(entries, hp: Optional[muon_hparams], workspace_ptr: int, ws_bytes: int, device: int) -> tuple:
    tbl = _table(entries)
    h = _P()
    s = load().muon_init(ctypes.byref(h), tbl, len(entries), ctypes.byref(hp) if hp is not None else None,
                         _P(workspace_ptr), ws_bytes, device)
    return s, h


def muon_init_static(entries, hp: Optional[muon_hparams], device: int) -> tuple:
    tbl = _table(entries)
    h = _P()
    s = load().muon_init_static(ctypes.byref(h), tbl, len(entries), ctypes.byref(hp) if hp is not None else None,
                                device)
    return s, h


def muon_step(h, params_ptr: int, grads_ptr: int, mom_ptr: int, numel: int, lr: float, momentum_coef: float,
              stream_ptr: int) -> int:
    return load().muon_step(h, _P(params_ptr), _P(grads_ptr), _P(mom_ptr), numel, lr, momentum_coef,
                            _P(stream_ptr))


def muon_reset(h, mom_ptr: int, numel: int, stream_ptr: int) -> int:
    return load().muon_reset(h, _P(mom_ptr), numel, _P(stream_ptr))


def muon_destroy(h) -> None:
    load().muon_destroy(h)


def muon_num_matrices(h) -> int:
    return load().muon_num_matrices(h)


def muon_matrix_layout(h, index: int) -> muon_layout:
    out = muon_layout()
    s = load().muon_matrix_layout(h, index, ctypes.byref(out))
    if s != MUON_OK:
        raise ValueError(f"muon_matrix_layout({index}) failed: {muon_status_string(s)}")
    return out


def muon_debug_view(h, which: int) -> tuple:
    ptr = _P()
    nbytes = ctypes.c_size_t(0)
    s = load().muon_debug_view(h, which, ctypes.byref(ptr), ctypes.byref(nbytes))
    return s, (ptr.value or 0), nbytes.value


def muon_work_stats(h) -> muon_work:
    out = muon_work()
    s = load().muon_work_stats(h, ctypes.byref(out))
    if s != MUON_OK:
        raise ValueError(f"muon_work_stats failed: {muon_status_string(s)}")
    return out


def muon_profile_enable(h, on: int) -> int:
    return load().muon_profile_enable(h, on)


def muon_profile_read(h, kernel: int, clear: int = 0) -> tuple:
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    s = load().muon_profile_read(h, kernel, clear, ctypes.byref(n), ctypes.byref(ms))
    return s, n.value, ms.value


class MuonError(RuntimeError):
    pass


def check(status: int, h=None, what: str = "") -> None:
    if status != MUON_OK:
        raise MuonError(f"{what}: {muon_status_string(status)} ({muon_last_error(h)})")


# --- convenience: a handle that owns its torch workspace ---------------------

def make_hparams(momentum=0.95, nesterov=1, momentum_kind=MUON_MOMENTUM_LERP, ns_steps=5, coeffs=None,
                 ns_eps=1e-7, precision="bf16", normuon=0, normuon_beta2=0.95, normuon_eps=1e-10,
                 weight_decay=0.0, stream_groups=0) -> muon_hparams:
    hp = muon_hparams_default()
    hp.momentum = momentum
    hp.nesterov = nesterov
    hp.momentum_kind = momentum_kind
    hp.ns_steps = ns_steps
    if coeffs is not None:
        for k, (a, b, c) in enumerate(coeffs):
            hp.ns_coeffs[k][0], hp.ns_coeffs[k][1], hp.ns_coeffs[k][2] = a, b, c
    hp.ns_eps = ns_eps
    hp.ns_precision = MUON_NS_FP32 if precision == "fp32" else MUON_NS_BF16
    hp.normuon = normuon
    hp.normuon_beta2 = normuon_beta2
    hp.normuon_eps = normuon_eps
    hp.weight_decay = weight_decay
    hp.stream_groups = stream_groups
    return hp


class MuonHandle:
    """libmuon handle plus its device workspace (a torch uint8 tensor)."""

    def __init__(self, entries: Sequence, hp: muon_hparams, device: int = 0):
        import torch

        self.hp = hp
        self.entries = list(entries)
        s, nbytes = muon_workspace_bytes(self.entries, hp)
        check(s, None, "muon_workspace_bytes")
        self.ws_bytes = nbytes
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=f"cuda:{device}")
        s, h = muon_init(self.entries, hp, self.workspace.data_ptr(), self.ws_bytes, device)
        check(s, None, "muon_init")
        self.h = h
        self.device = device

    def step(self, params, grads, momentum, lr: float, momentum_coef: float = -1.0, stream=None) -> None:
        import torch

        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        numel = min(params.numel(), grads.numel(), momentum.numel())
        s = muon_step(self.h, params.data_ptr(), grads.data_ptr(), momentum.data_ptr(), numel, lr, momentum_coef,
                      st.cuda_stream)
        check(s, self.h, "muon_step")

    def reset(self, momentum=None, stream=None) -> None:
        import torch

        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        ptr = momentum.data_ptr() if momentum is not None else 0
        numel = momentum.numel() if momentum is not None else 0
        check(muon_reset(self.h, ptr, numel, st.cuda_stream), self.h, "muon_reset")

    def view(self, which: int, dtype):
        """A torch view of an internal buffer (valid once the stream work is done)."""
        s, ptr, nbytes = muon_debug_view(self.h, which)
        check(s, self.h, "muon_debug_view")
        off = ptr - self.workspace.data_ptr()
        if off < 0 or off + nbytes > self.workspace.numel():
            raise MuonError("debug view outside the workspace")
        return self.workspace[off:off + nbytes].view(dtype)

    def layout(self, index: int) -> muon_layout:
        return muon_matrix_layout(self.h, index)

    @property
    def num_matrices(self) -> int:
        return muon_num_matrices(self.h)

    def close(self) -> None:
        if getattr(self, "h", None):
            muon_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
