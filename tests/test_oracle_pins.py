"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something other than itself: constants the
pages print (tests/golden/), closed forms from spectral theory, a library
routine (torch's bfloat16 cast, numpy's SVD), invariances the method has, or
brute force on tiny inputs. Each is chosen so that a plausible slip in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a missed
rounding point) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import custom_workload, gen_grads, get_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            vals[k] = float(v)
    return vals


def _p_scalar(x, steps=5, a=3.4445, b=-4.7750, c=2.0315):
    # Written independently of the oracle: the odd quintic applied to one number.
    for _ in range(steps):
        x = a * x + b * x * x * x + c * x * x * x * x * x
    return x


def _haar(n, rng):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


# ---------------------------------------------------------------------------
# Constants printed on the pages
# ---------------------------------------------------------------------------
def test_constants_match_pages():
    g = _golden("muon_constants.txt")
    assert (O.NS_A, O.NS_B, O.NS_C) == (g["ns_a"], g["ns_b"], g["ns_c"])
    assert O.NS_EPS == g["ns_eps"]
    assert O.NS_STEPS == g["ns_steps_used"]
    w = get_workload(1)
    assert w.lr == g["muon_lr"] and w.momentum == g["muon_momentum"] and w.weight_decay == g["weight_decay"]
    # GPT body of 12 layers, width 768: 12 * (4 d^2 + 4 d^2 + 4 d^2) = 84,934,656 matrix entries.
    d, L = int(g["gpt_n_embd"]), int(g["gpt_n_layer"])
    assert w.total == L * 12 * d * d == 84_934_656


# ---------------------------------------------------------------------------
# bfloat16 rounding against torch's float32 -> bfloat16 cast (library routine)
# ---------------------------------------------------------------------------
def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    parts = [
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3e38, -3.3e38, 0.0, -0.0],
                 np.float32),
    ]
    # exact ties: bf16 grid points plus half a grid step
    base = rng.integers(-(2 ** 15), 2 ** 15, 20_000).astype(np.int32) << 16
    tie = (base | 0x8000).view(np.float32)
    parts.append(tie[np.isfinite(tie)])
    x = np.concatenate(parts)
    ours = O.bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_round_hand_values():
    assert O.bf16_round(1 + 2 ** -8) == 1.0                 # tie -> even
    assert O.bf16_round(1 + 3 * 2 ** -8) == 1 + 2 ** -6      # tie -> even (upwards)
    assert O.bf16_round(1 + 2 ** -8 + 2 ** -20) == 1 + 2 ** -7
    assert O.bf16_ulp(1.0) == 2 ** -7


# ---------------------------------------------------------------------------
# Newton-Schulz: spectral closed form
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n", [(5, 5), (4, 9)])
def test_ns_exact_diagonal_closed_form(m, n):
    sig = np.array([1.0, 0.5, 0.1, 1e-2, 1e-3][:m])
    X = np.zeros((m, n))
    X[np.arange(m), np.arange(m)] = sig
    s = 1.0 / (math.sqrt(float((sig ** 2).sum())) + 1e-7)
    out = O.ns_exact(X, s)
    want = np.zeros((m, n))
    want[np.arange(m), np.arange(m)] = [_p_scalar(v * s) for v in sig]
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


def test_ns_exact_conjugated_closed_form():
    rng = np.random.default_rng(1)
    m, n = 7, 12
    U = _haar(m, rng)
    V = _haar(n, rng)[:, :m]
    sig = np.array([2.0, 1.0, 0.7, 0.3, 0.05, 0.01, 0.002])
    X = U @ np.diag(sig) @ V.T
    s = 1.0 / (np.linalg.norm(X) + 1e-7)
    out = O.ns_exact(X, s)
    want = U @ np.diag([_p_scalar(v * s) for v in sig]) @ V.T
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


def test_ns_matches_svd_polar_band():
    rng = np.random.default_rng(2)
    for m, n in [(3, 3), (4, 6), (6, 10)]:
        X = rng.standard_normal((m, n))
        s = O.frobenius_scale(X)
        out = O.ns_exact(X, s)
        U, sv, Vt = np.linalg.svd(X, full_matrices=False)
        D = U.T @ out @ Vt.T
        np.testing.assert_allclose(D - np.diag(np.diag(D)), 0.0, atol=1e-12)
        np.testing.assert_allclose(np.diag(D), [_p_scalar(v * s) for v in sv], atol=1e-12)
        # close to the polar factor U V^T: singular values land in NS's band
        big = sv * s >= 1e-2
        assert np.all(np.diag(D)[big] >= 0.68) and np.all(np.diag(D)[big] <= 1.135)


def test_ns_factored_form_equals_pages_form():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((6, 11))
    s = O.frobenius_scale(X)
    np.testing.assert_allclose(O.ns_exact_factored(X, s), O.ns_exact(X, s), atol=1e-12)


def test_ns_transpose_and_scale_invariance():
    rng = np.random.default_rng(4)
    G = rng.standard_normal((8, 8))
    a = O.ns_exact(G, O.frobenius_scale(G))
    b = O.ns_exact(G.T, O.frobenius_scale(G))
    np.testing.assert_allclose(b, a.T, atol=1e-12)
    c = O.ns_exact(1e3 * G, O.frobenius_scale(1e3 * G))
    np.testing.assert_allclose(c, a, atol=1e-6)  # eps 1e-7 breaks exact invariance slightly


# ---------------------------------------------------------------------------
# bf16 rounding contract
# ---------------------------------------------------------------------------
def _bf16_torch(x):
    return float(torch.tensor([x], dtype=torch.float64).to(torch.bfloat16).to(torch.float64)[0])


def test_bf16_contract_diagonal_recurrence():
    # Diagonal input: every product sum has one nonzero term, so the contract
    # reduces to a scalar recurrence per entry with the same rounding points.
    m, n = 6, 10
    rng = np.random.default_rng(5)
    u = np.zeros((m, n))
    u[np.arange(m), np.arange(m)] = rng.uniform(0.01, 1.0, m) * rng.choice([-1, 1], m)
    xt = O.bf16_round(u)
    s = 1.0 / (np.linalg.norm(u) + 1e-7)
    out = O.ns_bf16_contract(xt, s)
    fold = O.ns_bf16_contract_folded(xt, s)
    a, b, c = 3.4445, -4.7750, 2.0315
    for i in range(m):
        x = y = float(xt[i, i])
        for k in range(5):
            g = s * s if k == 0 else 1.0
            h = s if k == 0 else 1.0
            # four-point: A, B = b A + c A^2, X = a X + B X
            A = _bf16_torch(g * (x * x))
            Bv = _bf16_torch(b * A + c * (A * A))
            x = _bf16_torch(h * (a * x + Bv * x))
            # folded: P = a + b A + c A^2 rounded, X = P X
            Ay = _bf16_torch(g * (y * y))
            P = _bf16_torch(a + b * Ay + c * (Ay * Ay))
            y = _bf16_torch(h * (P * y))
        assert abs(out[i, i] - x) <= O.bf16_ulp(x), (i, out[i, i], x)
        assert abs(fold[i, i] - y) <= O.bf16_ulp(y), (i, fold[i, i], y)
    for r in (out, fold):
        off = r.copy()
        off[np.arange(m), np.arange(m)] = 0
        assert np.all(off == 0)


def _contract_scalar(Xt, s, steps=5, a=3.4445, b=-4.7750, c=2.0315):
    # The four-point contract written with Python loops over entries and torch's
    # float64 -> bfloat16 cast at each rounding point (independent of the
    # oracle's matrix code and of its rounding routine).
    m, n = len(Xt), len(Xt[0])
    X = [list(map(float, row)) for row in Xt]
    for k in range(steps):
        g = s * s if k == 0 else 1.0
        h = s if k == 0 else 1.0
        A = [[_bf16_torch(g * sum(X[i][t] * X[j][t] for t in range(n))) for j in range(m)] for i in range(m)]
        AA = [[sum(A[i][t] * A[t][j] for t in range(m)) for j in range(m)] for i in range(m)]
        Bm = [[_bf16_torch(b * A[i][j] + c * AA[i][j]) for j in range(m)] for i in range(m)]
        X = [[_bf16_torch(h * (a * X[i][j] + sum(Bm[i][t] * X[t][j] for t in range(m)))) for j in range(n)]
             for i in range(m)]
    return np.array(X)


@pytest.mark.parametrize("m,n,seed", [(2, 3, 20), (3, 5, 21), (3, 3, 22)])
def test_bf16_contract_matches_scalar_loops(m, n, seed):
    # Non-diagonal inputs: every rounding point, every term (a X included) and
    # every index of the contract is checked entry by entry.
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((m, n))
    xt = O.bf16_round(u)
    s = 1.0 / (np.linalg.norm(u) + 1e-7)
    want = _contract_scalar(xt, s)
    got = O.ns_bf16_contract(xt, s)
    np.testing.assert_array_equal(got, want)
    # each step's output lies on the bf16 grid and is not the exact iterate
    assert np.array_equal(O.bf16_round(got), got)
    assert O.rel_fro(got, O.ns_exact(xt, s)) > 0


def test_bf16_contract_misplaced_rounding_is_detected():
    # The two placements of the a X term differ on generic input by far more
    # than one bf16 ulp, so the scalar-loop pin above separates them.
    rng = np.random.default_rng(23)
    u = rng.standard_normal((3, 5))
    xt = O.bf16_round(u)
    s = 1.0 / (np.linalg.norm(u) + 1e-7)
    d = np.abs(O.ns_bf16_contract(xt, s) - O.ns_bf16_contract_folded(xt, s))
    assert d.max() > 0


def test_bf16_contract_close_to_exact():
    # The contract stays within a few percent of exact NS on the body's gradient
    # class, and so does the folded placement of a X.
    w = custom_workload(7, [(64, 192, 1, "spike"), (96, 96, 1, "iid")])
    g = gen_grads(w, 0)
    for _gi, _ei, _k, off, r, c in w.submatrices():
        u = g[off:off + r * c].reshape(r, c).astype(np.float64)
        X, _ = O.to_short_side(u)
        s = O.frobenius_scale(u)
        ex = O.ns_exact(X, s)
        e = O.rel_fro(O.ns_bf16_contract(O.bf16_round(X), s), ex)
        e2 = O.rel_fro(O.ns_bf16_contract_folded(O.bf16_round(X), s), ex)
        assert 1e-3 < e < 4e-2, e
        assert 1e-3 < e2 < 4e-2, e2


def test_rel_fro_hand_values():
    assert O.rel_fro(np.array([5.0, 12.0]) + np.array([3.0, 4.0]), np.array([5.0, 12.0])) == 5.0 / 13.0
    assert O.rel_fro(np.zeros((2, 2)), np.zeros((2, 2))) == 0.0
    assert O.rel_fro(np.ones(3), np.zeros(3)) == math.inf
    assert O.rel_fro(np.zeros(3), np.array([0.0, 3.0, 4.0])) == 1.0
    # a Frobenius norm over all entries, not a per-row or spectral norm
    a = np.array([[1.0, 0.0], [0.0, 0.0]])
    b = np.array([[0.0, 0.0], [0.0, 2.0]])
    assert O.rel_fro(a + b, b) == 0.5


def test_bf16_ulp_matches_next_bf16_value():
    # spacing = (next bfloat16 above x) - x, stepping the bit pattern with torch
    rng = np.random.default_rng(24)
    x = np.concatenate([np.abs(rng.standard_normal(5000)) * 10.0 ** rng.integers(-30, 30, 5000),
                        [1.0, 2.0, 3.0, 1e-39, 2.0 ** -126, 2.0 ** -133]]).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    nxt = (xb.view(torch.int16) + 1).view(torch.bfloat16)
    spacing = (nxt.double() - xb.double()).numpy()
    np.testing.assert_array_equal(O.bf16_ulp(xb.double().numpy()), spacing)


# ---------------------------------------------------------------------------
# Momentum
# ---------------------------------------------------------------------------
def test_momentum_closed_form_and_nesterov():
    rng = np.random.default_rng(6)
    beta = 0.95
    gs = [rng.standard_normal((3, 4)) for _ in range(6)]
    m = np.zeros((3, 4))
    for t, g in enumerate(gs, start=1):
        m = O.momentum_lerp(m, g, beta)
        closed = (1 - beta) * sum(beta ** (t - k) * gs[k - 1] for k in range(1, t + 1))
        np.testing.assert_allclose(m, closed, atol=1e-14)
        u = O.nesterov_lerp(g, m, beta)
        np.testing.assert_allclose(u, (1 - beta) * g + beta * closed, atol=1e-14)


def test_heavy_ball_equals_lerp_after_ns():
    w = custom_workload(8, [(12, 20, 2, "gauss"), (20, 12, 1, "gauss")], steps=4)
    outs = {}
    for kind in ("lerp", "heavy_ball"):
        # eps 0: the two forms differ by the factor 1-beta, which eps would otherwise see
        orc = O.OracleMuon(w.entries, w.total, mode="exact", momentum_kind=kind, ns_eps=0.0)
        p = np.zeros(w.total)
        for t in range(4):
            p = orc.step(p, gen_grads(w, t), lr=0.1)
        outs[kind] = p
    np.testing.assert_allclose(outs["heavy_ball"], outs["lerp"], atol=1e-12)


# ---------------------------------------------------------------------------
# Whole-step invariants
# ---------------------------------------------------------------------------
def test_zero_grads_give_zero_update_and_frozen_untouched():
    w = custom_workload(9, [(16, 16, 2, "zero"), (8, 24, 1, "gauss", 1.0, 1), (24, 8, 1, "zero")])
    for mode in ("bf16", "exact"):
        orc = O.OracleMuon(w.entries, w.total, mode=mode, normuon=1)
        p0 = np.arange(w.total, dtype=np.float64) * 1e-3
        p = orc.step(p0, gen_grads(w, 0), lr=0.05)
        assert np.all(np.isfinite(p))
        np.testing.assert_array_equal(p, p0)
        fz = w.entries[1]
        assert np.all(orc.m[fz.offset:fz.offset + fz.rows * fz.cols] == 0)


def test_step_transpose_invariance_exact():
    # A [R, C] matrix and its [C, R] transpose with transposed gradients get
    # transposed updates (non-square: the short-side frame is identical).
    rng = np.random.default_rng(10)
    R, C = 10, 26
    w = custom_workload(11, [(R, C, 1), (C, R, 1)])
    g = np.empty(w.total)
    G = rng.standard_normal((R, C))
    g[:R * C] = G.reshape(-1)
    g[R * C:] = G.T.reshape(-1)
    for mode in ("bf16", "exact"):
        orc = O.OracleMuon(w.entries, w.total, mode=mode, normuon=1)
        p = orc.step(np.zeros(w.total), g, lr=1.0)
        a = p[:R * C].reshape(R, C)
        b = p[R * C:].reshape(C, R)
        # shape scale differs: sqrt(max(1, C/R)) for the tall copy
        np.testing.assert_array_equal(b, a.T * math.sqrt(C / R)) if mode == "bf16" else \
            np.testing.assert_allclose(b, a.T * math.sqrt(C / R), atol=1e-12)


def test_normuon_norm_preserved_and_lanes_equalised():
    rng = np.random.default_rng(12)
    O_ = rng.standard_normal((5, 13)) * rng.uniform(0.1, 3.0, (5, 1))
    Oh, v = O.normuon(O_, np.zeros(5), 0.95, 1e-10)
    assert abs(np.linalg.norm(Oh) - np.linalg.norm(O_)) < 1e-12
    # after one step from v0 = 0 every lane (row over the longer side) has the same energy
    rn = np.linalg.norm(Oh, axis=1)
    np.testing.assert_allclose(rn, rn[0], rtol=1e-9)
    np.testing.assert_allclose(v, 0.05 * (O_ ** 2).mean(axis=1), rtol=1e-14)
    # rows of equal energy: NorMuon is the identity
    H = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1]], float)
    Oh2, _ = O.normuon(H, np.array([0.3, 0.3, 0.3]), 0.95, 1e-10)
    np.testing.assert_allclose(Oh2, H, atol=1e-12)


def test_normuon_lanes_follow_longer_side_for_tall_matrix():
    # Stored [R > C]: the lanes are the C stored columns (statistics over R).
    rng = np.random.default_rng(13)
    R, C = 12, 4
    w = custom_workload(14, [(R, C, 1, "gauss")])
    orc = O.OracleMuon(w.entries, w.total, mode="exact", normuon=1)
    g = rng.standard_normal(R * C) * np.repeat(rng.uniform(0.1, 5, R), C)
    p = orc.step(np.zeros(w.total), g, lr=1.0)
    upd = -p.reshape(R, C) / math.sqrt(R / C)
    cols = np.linalg.norm(upd, axis=0)
    np.testing.assert_allclose(cols, cols[0], rtol=1e-9)


def test_normuon_brute_force_tiny():
    O_ = [[0.5, -1.0, 2.0], [0.25, 0.0, -0.75]]
    v = [0.1, 0.2]
    beta2, eps = 0.9, 1e-10
    m, n = 2, 3
    v_new = [beta2 * v[i] + (1 - beta2) * sum(O_[i][j] ** 2 for j in range(n)) / n for i in range(m)]
    scaled = [[O_[i][j] / (math.sqrt(v_new[i]) + eps) for j in range(n)] for i in range(m)]
    num = math.sqrt(sum(x * x for row in O_ for x in row))
    den = math.sqrt(sum(x * x for row in scaled for x in row))
    want = [[x * num / den for x in row] for row in scaled]
    Oh, vv = O.normuon(np.array(O_), np.array(v), beta2, eps)
    np.testing.assert_allclose(Oh, want, rtol=1e-14)
    np.testing.assert_allclose(vv, v_new, rtol=1e-14)


def test_apply_update_hand_values():
    p = np.array([[1.0], [2.0], [3.0], [4.0]])
    Ost = np.array([[0.5], [-0.5], [1.0], [0.0]])
    # [4, 1]: shape scale sqrt(4) = 2; lr 0.1, lr_mul 3, wd 0.5, wd_mul 2 -> decay 1 - 0.3
    out = O.apply_update(p, Ost, 0.1, 3.0, 0.5, 2.0, 4, 1)
    want = p * 0.7 - 0.1 * 3.0 * 2.0 * Ost
    np.testing.assert_allclose(out, want, rtol=1e-15)
    assert O.shape_scale(3072, 768) == 2.0 and O.shape_scale(768, 3072) == 1.0


def test_oracle_step_matches_hand_composition():
    # One matrix, one step, composed by hand from the definitions.
    rng = np.random.default_rng(15)
    R, C = 9, 5
    g = rng.standard_normal(R * C)
    w = custom_workload(16, [(R, C, 1, "gauss", 1.5)])
    orc = O.OracleMuon(w.entries, w.total, mode="exact", momentum=0.9)
    p = orc.step(np.ones(w.total), g, lr=0.2)
    G = g.reshape(R, C)
    m = 0.1 * G
    u = 0.1 * G + 0.9 * m
    X = u.T
    Y = O.ns_exact(X, 1.0 / (np.linalg.norm(u) + 1e-7)).T
    want = 1.0 - 0.2 * 1.5 * math.sqrt(R / C) * Y
    np.testing.assert_allclose(p.reshape(R, C), want, atol=1e-14)
