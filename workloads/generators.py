"""Seeded input generators (no optimizer arithmetic here).

Every number is drawn from NumPy's PCG64 seeded by
SeedSequence([config_id, purpose, step, matrix_index]), so any single
(sub-)matrix can be regenerated on its own: purpose 0 = initial parameters,
1 = gradients, 2 = the per-matrix gradient scale sigma. Values are drawn in
float64 and cast to float32 once; the GPU library and the oracle both consume
the same float32 arrays.

Gradient classes:
  iid        N(0, 0.1^2) entries (the tiny workload's N(0, 1e-2), read as a variance)
  spike      sigma*Z + (10*sigma/2) * A @ B.T, A in R^{rows x 4}, B in R^{cols x 4},
             Z, A, B i.i.d. N(0,1); sigma = 10^U(-4,-2) drawn once per matrix.
             The rank-4 term's entries have standard deviation 10*sigma.
  rank8      A @ B.T / sqrt(8) + 1e-6 * Z, A in R^{rows x 8}, B in R^{cols x 8}
  student_t  Student-t entries with 3 degrees of freedom
  zero       all zeros
  gauss      N(0, 1) entries (unit scale; used by small parity cases)
Initial parameters: N(0, 0.02^2) for every matrix.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PURPOSE_PARAMS = 0
PURPOSE_GRADS = 1
PURPOSE_SIGMA = 2


def _rng(config_id: int, purpose: int, step: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config_id, purpose, step, index])))


def matrix_sigma(config_id: int, index: int) -> float:
    r = _rng(config_id, PURPOSE_SIGMA, 0, index)
    return float(10.0 ** r.uniform(-4.0, -2.0))


def gen_matrix_grad(config_id: int, step: int, index: int, rows: int, cols: int, gclass: str) -> np.ndarray:
    """One float32 [rows, cols] gradient for sub-matrix `index` at `step`."""
    if gclass == "zero":
        return np.zeros((rows, cols), np.float32)
    r = _rng(config_id, PURPOSE_GRADS, step, index)
    if gclass == "iid":
        g = 0.1 * r.standard_normal((rows, cols))
    elif gclass == "gauss":
        g = r.standard_normal((rows, cols))
    elif gclass == "spike":
        sigma = matrix_sigma(config_id, index)
        z = r.standard_normal((rows, cols))
        a = r.standard_normal((rows, 4))
        b = r.standard_normal((cols, 4))
        g = sigma * z + (10.0 * sigma / 2.0) * (a @ b.T)
    elif gclass == "rank8":
        a = r.standard_normal((rows, 8))
        b = r.standard_normal((cols, 8))
        z = r.standard_normal((rows, cols))
        g = (a @ b.T) / np.sqrt(8.0) + 1e-6 * z
    elif gclass == "student_t":
        g = r.standard_t(3.0, (rows, cols))
    else:
        raise ValueError(f"unknown gradient class {gclass!r}")
    return np.ascontiguousarray(g, dtype=np.float32)


def gen_matrix_param(config_id: int, index: int, rows: int, cols: int) -> np.ndarray:
    r = _rng(config_id, PURPOSE_PARAMS, 0, index)
    return np.ascontiguousarray(0.02 * r.standard_normal((rows, cols)), dtype=np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill(workload, out: np.ndarray, fn) -> np.ndarray:
    subs = workload.submatrices()

    def work(item):
        gi, ei, _k, off, rows, cols = item
        e = workload.entries[ei]
        out[off:off + rows * cols] = fn(gi, e, rows, cols).reshape(-1)

    if len(subs) > 1 and workload.total > (1 << 20):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, subs))
    else:
        for item in subs:
            work(item)
    return out


def gen_grads(workload, step: int, out: np.ndarray | None = None) -> np.ndarray:
    """Flat float32 gradients of the whole workload at `step`."""
    if out is None:
        out = np.empty(workload.total, np.float32)
    return _fill(workload, out,
                 lambda gi, e, r, c: gen_matrix_grad(workload.config_id, step, gi, r, c, e.gclass))


def gen_params(workload, out: np.ndarray | None = None) -> np.ndarray:
    """Flat float32 initial parameters of the whole workload."""
    if out is None:
        out = np.empty(workload.total, np.float32)
    return _fill(workload, out, lambda gi, e, r, c: gen_matrix_param(workload.config_id, gi, r, c))


def gen_sigmas(workload) -> np.ndarray:
    return np.array([matrix_sigma(workload.config_id, gi) for gi, *_ in workload.submatrices()])
