"""Oracle for the Muon optimizer step — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy. Only tests/, the smoke check and the bench's
CPU-baseline leg may use it; the HIP library never does. It shares no code
with the HIP path.

Sources (cited by page title and section):
  [P4] "modded-nanogpt 50B-token 长时程训练实验解析：Muon vs Adam 与数据复用策略的实证对比",
       section "从源码看 Muon 的分布式正交化实现" (Muon's orthogonalization, from the
       source): the Newton-Schulz quintic, its coefficients, the Frobenius
       normalisation with eps 1e-7, the transpose to the short side, the
       heavy-ball + Nesterov momentum, the max(1, rows/cols)^0.5 scale and the
       update p <- p - lr * g; section "超参配置解析" (hyper-parameters): Muon lr
       0.02, momentum 0.95, Nesterov on, weight decay 0.
  [P2] "2025-10-27_FixMuonLR" record analysis, section "改动二" (change 2,
       the Muon step): the momentum buffer updated in place with lerp, the
       early qkvo reshape into four matrices, and NorMuon's second-moment
       statistic taken along the longer dimension with rsqrt scaling per lane;
       section "改动一" (change 1): per-matrix lr_mul / wd_mul.

Readings where the pages are silent or garbled:
  R1 lerp momentum m <- beta*m + (1-beta)*g (P2) as the default; the heavy-ball
     form of P4 is kept as an option. Both give the same NS input up to a
     positive scale, which the normalisation removes.
  R2 Nesterov blend u = (1-beta)*g + beta*m_new (lerp form) / u = g + beta*buf_new
     (heavy-ball form, P4).
  R3 The comparison lost in P4's "if G.size(0) G.size(1)" is read as ">":
     NS runs on X = u^T when rows > cols, so that X has rows <= cols.
  R4 s = 1/(||u||_F + 1e-7) from the float u; in the bf16 rounding contract
     s is folded into iteration 0 instead of rounding s*X to bf16.
  R5 The bf16 rounding contract: the input X~ is rounded once, then three
     rounding points per iteration, at the bf16 outputs of the three products
     of the factored iteration: A = X X^T, B = b A + c A^2 and X = a X + B X.
     Each product and sum is exact (float64 here); a X is added before the
     rounding of the new X. The folded variant (a I carried inside the
     rounded B) is kept beside it for comparison only.
  R6 NorMuon per row of the canonical (rows <= cols) frame: mean of squares
     over the longer dimension, v EMA with v0 = 0 and no bias correction,
     divide by sqrt(v)+eps, rescale to keep the Frobenius norm, 0/0 -> 0.
  R7 Decoupled weight decay p <- p*(1 - lr*lr_mul*wd*wd_mul) - ...; the shape
     scale uses the stored [R, C].
  R8 Frozen matrices: params, momentum and v untouched.

Parity unpinned (defined by this oracle alone, no page fixes them):
  - apply_update with weight decay != 0: the pages run Muon with wd = 0 only,
    so the decoupled form of R7 is a reading; with wd = 0 it is the pages'
    p <- p - lr * scale * O, which the pins do fix.
  - the NorMuon orientation for non-square matrices (R6): the pins fix the
    norm preservation, the equal-lanes identity and the statistics along the
    longer side, but "per row of the canonical frame" is a reading.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple

import numpy as np

# [P4] Muon source section: the quintic coefficients, eps and default step count.
NS_A, NS_B, NS_C = 3.4445, -4.7750, 2.0315
NS_EPS = 1e-7
NS_STEPS = 5

BF16_MAX = float.fromhex("0x1.fe00000000000p+127")  # largest finite bfloat16


def default_coeffs(steps: int = NS_STEPS) -> List[Tuple[float, float, float]]:
    return [(NS_A, NS_B, NS_C)] * steps


# ----------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even), written from the format:
# 8 significant bits, the float32 exponent range.
# ----------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(x)                       # |x| = f * 2**e, f in [0.5, 1)
        e = np.maximum(e, -125)                  # below 2**-126 the grid is uniform (subnormals)
        q = np.ldexp(1.0, e - 8)                 # spacing of the 8-bit significand grid
        r = np.rint(x / q) * q                   # np.rint rounds half to even
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
        r = np.where(np.isfinite(x), r, x)
    return r


def bf16_ulp(x) -> np.ndarray:
    """Spacing of the bfloat16 grid at the magnitude of x."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(1.0, e - 8)


# ----------------------------------------------------------------------------
# Momentum
# ----------------------------------------------------------------------------
def momentum_lerp(m, g, beta):
    """[P2] change 2: momentum_buffer.lerp_(grad, 1 - beta), i.e. beta*m + (1-beta)*g."""
    return beta * np.asarray(m, np.float64) + (1.0 - beta) * np.asarray(g, np.float64)


def nesterov_lerp(g, m_new, beta):
    """Nesterov blend for the lerp form: (1-beta)*g + beta*m_new (reading R2)."""
    return (1.0 - beta) * np.asarray(g, np.float64) + beta * np.asarray(m_new, np.float64)


def momentum_heavy_ball(buf, g, beta):
    """[P4] Muon source: buf.mul_(momentum).add_(g)."""
    return beta * np.asarray(buf, np.float64) + np.asarray(g, np.float64)


def nesterov_heavy_ball(g, buf_new, beta):
    """[P4] Muon source, Nesterov correction: g + momentum*buf."""
    return np.asarray(g, np.float64) + beta * np.asarray(buf_new, np.float64)


# ----------------------------------------------------------------------------
# Newton-Schulz orthogonalisation
# ----------------------------------------------------------------------------
def to_short_side(u: np.ndarray) -> Tuple[np.ndarray, bool]:
    """[P4] Muon source: transpose so the iteration runs on the shorter side (R3)."""
    if u.shape[0] > u.shape[1]:
        return u.T, True
    return u, False


def frobenius_scale(u, eps: float = NS_EPS) -> float:
    """[P4] Muon source: divide by (norm + eps) so the largest singular value is <= 1."""
    return 1.0 / (float(np.linalg.norm(np.asarray(u, np.float64))) + eps)


def ns_exact(X, s: float, coeffs: Sequence[Tuple[float, float, float]] = None) -> np.ndarray:
    """Quintic Newton-Schulz in float64, in the pages' notation ([P4] Muon source).

    X is in the short-side frame (rows <= cols); s is the normalising factor.
    Each iteration: A = X X^T, B = A X, X = a X + b B + c A B.
    """
    coeffs = default_coeffs() if coeffs is None else coeffs
    X = s * np.asarray(X, np.float64)
    for a, b, c in coeffs:
        A = X @ X.T
        B = A @ X
        X = a * X + b * B + c * (A @ B)
    return X


def ns_exact_factored(X, s: float, coeffs=None) -> np.ndarray:
    """The same iteration in the factored form a X + (b A + c A^2) X (exact arithmetic)."""
    coeffs = default_coeffs() if coeffs is None else coeffs
    X = s * np.asarray(X, np.float64)
    for a, b, c in coeffs:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def ns_bf16_contract(Xt, s: float, coeffs=None) -> np.ndarray:
    """bf16 rounding contract of the factored iteration (readings R4, R5).

    [P4] Muon source: the loop A = X X^T, B = A X, X = a X + b B + c A B,
    run in bf16. Grouping b A X + c A A X as (b A + c A^2) X gives the
    factored step A = X X^T; B = b A + c A^2; X = a X + B X, whose three
    products are the three rounding points here. Xt: the bf16-rounded
    short-side input (float64 array of bf16 values); s: the normalising
    factor, folded into iteration 0 (X = s Xt is never rounded itself).
    Products and sums are exact (float64); R() rounds to bf16:
      it 0:  A = R(s^2 Xt Xt^T);  B = R(b A + c A A);  X = R(a s Xt + s B Xt)
      it>0:  A = R(X X^T);        B = R(b A + c A A);  X = R(a X + B X)
    """
    coeffs = default_coeffs() if coeffs is None else coeffs
    X = np.asarray(Xt, np.float64)
    for k, (a, b, c) in enumerate(coeffs):
        g = (s * s) if k == 0 else 1.0      # iteration 0 sees s Xt
        A = bf16_round(g * (X @ X.T))
        Bm = bf16_round(b * A + c * (A @ A))
        h = s if k == 0 else 1.0
        X = bf16_round(h * (a * X + Bm @ X))
    return X


def ns_bf16_contract_folded(Xt, s: float, coeffs=None) -> np.ndarray:
    """The same iteration with a I folded into the rounded polynomial:
      A = R(g X X^T);  P = R(a I + b A + c A A);  X = R(h P X)
    (g = s^2, h = s in iteration 0, else 1). Equal to ns_bf16_contract in
    exact arithmetic; it rounds a + b A_ii + c (A A)_ii on the diagonal,
    where the bf16 grid is coarse. Not a gate of the library; kept to
    report how far the two placements of the a X term lie apart.
    """
    coeffs = default_coeffs() if coeffs is None else coeffs
    X = np.asarray(Xt, np.float64)
    eye = np.eye(X.shape[0])
    for k, (a, b, c) in enumerate(coeffs):
        g = (s * s) if k == 0 else 1.0
        A = bf16_round(g * (X @ X.T))
        P = bf16_round(a * eye + b * A + c * (A @ A))
        h = s if k == 0 else 1.0
        X = bf16_round(h * (P @ X))
    return X


# ----------------------------------------------------------------------------
# NorMuon and the parameter update
# ----------------------------------------------------------------------------
def normuon(O, v, beta2: float, eps: float):
    """[P2] change 2 (reshape timing): NorMuon's per-lane second moment (reading R6).

    O is in the short-side frame [m, n], m <= n; one lane per row.
    Returns (O_hat, v_new).
    """
    O = np.asarray(O, np.float64)
    r = (O * O).sum(axis=1) / O.shape[1]
    v_new = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * r
    d = np.sqrt(v_new) + eps
    Oh = O / d[:, None]
    num = float(np.linalg.norm(O))
    den = float(np.linalg.norm(Oh))
    if den == 0.0:
        return np.zeros_like(O), v_new
    return Oh * (num / den), v_new


def shape_scale(rows: int, cols: int) -> float:
    """[P4] Muon source: max(1, rows/cols)^0.5."""
    return math.sqrt(max(1.0, rows / cols))


def apply_update(p, O_stored, lr: float, lr_mul: float, wd: float, wd_mul: float, rows: int, cols: int):
    """[P4] p.data.add_(g, alpha=-lr) on the scaled update, with per-matrix
    lr_mul / wd_mul ([P2] change 1) and decoupled decay (reading R7)."""
    p = np.asarray(p, np.float64)
    decay = 1.0 - lr * lr_mul * wd * wd_mul
    return p * decay - lr * lr_mul * shape_scale(rows, cols) * np.asarray(O_stored, np.float64)


# ----------------------------------------------------------------------------
# Whole step over a table of matrices
# ----------------------------------------------------------------------------
def _entries(table) -> Iterable[Tuple[int, int, int, int, float, float, int]]:
    gi = 0
    for e in table:
        if isinstance(e, dict):
            rows, cols, count, off = e["rows"], e["cols"], e.get("count", 1), e["offset"]
            lr_mul, wd_mul, frozen = e.get("lr_mul", 1.0), e.get("wd_mul", 1.0), e.get("frozen", 0)
        else:
            rows, cols, count, off = e.rows, e.cols, e.count, e.offset
            lr_mul, wd_mul, frozen = e.lr_mul, e.wd_mul, e.frozen
        for k in range(count):
            yield gi, off + k * rows * cols, rows, cols, lr_mul, wd_mul, frozen
            gi += 1


class OracleMuon:
    """Float64 Muon over flat buffers laid out like the GPU library's.

    mode "bf16": NS under the bf16 rounding contract; mode "exact": float64 NS
    (the reference for the library's fp32 NS mode).
    """

    def __init__(self, table, total: int, *, momentum=0.95, nesterov=1, ns_steps=NS_STEPS,
                 coeffs=None, normuon=0, normuon_beta2=0.95, normuon_eps=1e-10,
                 weight_decay=0.0, momentum_kind="lerp", ns_eps=NS_EPS, mode="bf16"):
        self.table = list(table)
        self.total = int(total)
        self.beta = momentum
        self.nesterov = nesterov
        self.coeffs = list(coeffs) if coeffs is not None else default_coeffs(ns_steps)
        self.normuon = normuon
        self.beta2 = normuon_beta2
        self.neps = normuon_eps
        self.wd = weight_decay
        self.kind = momentum_kind
        self.ns_eps = ns_eps
        self.mode = mode
        self.m = np.zeros(self.total, np.float64)
        self.v = {}
        for gi, off, rows, cols, *_ in _entries(self.table):
            self.v[gi] = np.zeros(min(rows, cols), np.float64)
        self.record = {}

    def reset(self):
        self.m[:] = 0.0
        for k in self.v:
            self.v[k][:] = 0.0

    def step(self, params: np.ndarray, grads: np.ndarray, lr: float, beta: float | None = None,
             keep: Sequence[int] | None = None) -> np.ndarray:
        """One step; returns new float64 params. `keep` lists matrix indices
        whose intermediates are stored in self.record (u, xt, s, O, O_hat)."""
        beta = self.beta if beta is None else beta
        p_out = np.array(params, np.float64, copy=True)
        self.record = {}
        for gi, off, rows, cols, lr_mul, wd_mul, frozen in _entries(self.table):
            if frozen:
                continue
            sl = slice(off, off + rows * cols)
            g = np.asarray(grads[sl], np.float64).reshape(rows, cols)
            m = self.m[sl].reshape(rows, cols)
            if self.kind == "lerp":
                m_new = momentum_lerp(m, g, beta)
                u = nesterov_lerp(g, m_new, beta) if self.nesterov else m_new
            else:
                m_new = momentum_heavy_ball(m, g, beta)
                u = nesterov_heavy_ball(g, m_new, beta) if self.nesterov else m_new
            self.m[sl] = m_new.reshape(-1)
            X, transposed = to_short_side(u)
            s = frobenius_scale(u, self.ns_eps)
            if self.mode == "bf16":
                xt = bf16_round(X)
                O = ns_bf16_contract(xt, s, self.coeffs)
            else:
                xt = X
                O = ns_exact(X, s, self.coeffs)
            Oh = O
            if self.normuon:
                Oh, self.v[gi] = normuon(O, self.v[gi], self.beta2, self.neps)
            O_st = Oh.T if transposed else Oh
            p_out[sl] = apply_update(p_out[sl].reshape(rows, cols), O_st, lr, lr_mul, self.wd,
                                     wd_mul, rows, cols).reshape(-1)
            if keep is not None and gi in keep:
                self.record[gi] = dict(u=u, xt=xt, s=s, O=O, O_hat=Oh, transposed=transposed)
        return p_out


def rel_fro(a, b) -> float:
    """||a - b||_F / ||b||_F (0 if both are zero; inf if only b is zero)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = float(np.linalg.norm(b))
    nd = float(np.linalg.norm(a - b))
    if nb == 0.0:
        return 0.0 if nd == 0.0 else math.inf
    return nd / nb


__all__ = [
    "NS_A", "NS_B", "NS_C", "NS_EPS", "NS_STEPS", "default_coeffs",
    "bf16_round", "bf16_ulp",
    "momentum_lerp", "nesterov_lerp", "momentum_heavy_ball", "nesterov_heavy_ball",
    "to_short_side", "frobenius_scale", "ns_exact", "ns_exact_factored", "ns_bf16_contract",
    "ns_bf16_contract_folded", "normuon", "shape_scale", "apply_update", "OracleMuon", "rel_fro",
]
