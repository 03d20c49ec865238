"""GPU parity: libmuon (through its C ABI) against the CPU oracle.

Small cases run every stage against the oracle on every matrix; the full-size
workloads (124M body, 124M + NorMuon, the stress batch, the 1.5B body) run
in the same launch configuration the bench times and are checked on sampled
matrices plus properties that hold at any size.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from muon_newton_schulz_04_amd import binding as B
from workloads import custom_workload, gen_grads, gen_matrix_grad, get_workload

from _harness import GpuRun, assert_worst, check_stages, snapshot

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


RAGGED = [
    (200, 200, 2, "spike"),       # two 128-tiles per side, ragged tail
    (136, 520, 1, "spike"),       # wide
    (520, 136, 1, "spike"),       # tall -> transposed
    (40, 100, 1, "gauss"),        # small tile class (T = 64)
    (100, 40, 1, "gauss"),
    (64, 64, 3, "rank8"),
    (1, 7, 1, "gauss"),           # degenerate: a single row
    (7, 1, 1, "gauss"),           # a single column
    (130, 130, 1, "zero"),        # zero gradients -> zero update
    (96, 160, 1, "gauss", 1.0, 1),  # frozen
    (33, 257, 1, "student_t", 0.0),  # lr_mul 0: params unchanged, momentum advances
    (384, 768, 1, "spike", 2.0),  # several tiles, lr_mul 2
    (1000, 700, 1, "spike"),      # tall, 256-tiles with a padded edge (768 x 1024)
]


def _run_all_stages(w, steps, **hp):
    _say(f"[case] {w.name} hp={hp} steps={steps}")
    run = GpuRun(w, **hp)
    idx = [gi for gi, *_ in run.subs]
    orc_m = {gi: np.zeros((r, c)) for gi, _e, _k, _o, r, c in run.subs}
    p0 = run.params.cpu().numpy().copy()
    for t in range(steps):
        p_prev, v_prev = snapshot(run, idx)
        g = run.load_grads(t)
        run.step()
        rep = []
        worst = check_stages(run, t, idx, grads_host=g, p_prev=p_prev, v_prev=v_prev, orc_m=orc_m, report=rep)
        _say(f"  step {t}: {worst}")
        for r in sorted(rep, key=lambda x: -x[6])[:4]:
            _say(f"    NS gi={r[2]} [{r[3]},{r[4]}] {r[5]}: gpu-vs-contract {r[6]:.3e} contract-vs-exact {r[7]:.3e} "
                 f"gpu-vs-exact {r[8]:.3e}")
        assert_worst(worst, fp32=run.fp32)
        for gi, ei, _k, off, r, c in run.subs:
            e = w.entries[ei]
            if e.gclass == "zero" and not e.frozen:
                assert np.all(run.ns_out(gi) == 0)
            assert e.frozen or np.all(run.ns_out_padding(gi) == 0)
    p = run.params.cpu().numpy()
    mom = run.mom.cpu().numpy()
    for gi, ei, _k, off, r, c in run.subs:
        e = w.entries[ei]
        sl = slice(off, off + r * c)
        if e.frozen:
            assert np.array_equal(p[sl], p0[sl]) and np.all(mom[sl] == 0)
        elif e.lr_mul == 0.0 or (e.gclass == "zero" and w.weight_decay == 0.0):
            assert np.array_equal(p[sl], p0[sl])
            if e.gclass != "zero":
                assert np.any(mom[sl] != 0)
    assert np.all(run.scalars(B.MUON_VIEW_STATUS) == 0)
    return run


@pytest.mark.parametrize("normuon", [0, 1])
def test_ragged_bf16_all_stages(normuon):
    w = custom_workload(100 + normuon, RAGGED, steps=3, normuon=normuon, lr=0.05)
    _run_all_stages(w, 3)


def _random_table(seed, n_entries):
    """A seeded mixed table: small (1..64), medium and large sides in both
    orientations, 256-row panels, every gradient class, lr_mul 0.5 / 1 / 2 and
    some frozen entries, so that shapes meet every kernel class and edge case
    together in one plan."""
    rng = np.random.default_rng(seed)
    classes = ["spike", "gauss", "student_t", "rank8", "zero"]
    out = []
    for _ in range(n_entries):
        kind = rng.choice(["small", "medium", "large", "panel"], p=[0.35, 0.3, 0.2, 0.15])
        lo, hi = {"small": (1, 64), "medium": (65, 300), "large": (301, 800), "panel": (257, 1400)}[kind]
        a, b = int(rng.integers(lo, hi + 1)), int(rng.integers(lo if kind == "panel" else 1, hi + 1))
        if kind == "panel":
            a = 256  # and the other side > 256: one 256-row panel
        r, c = (a, b) if rng.random() < 0.5 else (b, a)
        out.append((r, c, int(rng.integers(1, 3)), str(rng.choice(classes, p=[0.3, 0.25, 0.2, 0.15, 0.1])),
                    float(rng.choice([0.5, 1.0, 2.0])), int(rng.random() < 0.1)))
    return out


@pytest.mark.parametrize("case, precision, normuon, groups", [(0, "bf16", 0, 3), (1, "bf16", 1, 3),
                                                            (2, "fp32", 1, 2), (3, "bf16", 0, 4)])
def test_random_mixed_tables_all_stages(case, precision, normuon, groups):
    shapes = _random_table(20261203 + case, 14)
    _say(f"[case] random table {case} ({precision}, normuon={normuon}, {groups} stream groups): {shapes}")
    w = custom_workload(170 + case, shapes, steps=2, ns_precision=precision, normuon=normuon, lr=0.05,
                        weight_decay=0.05 * normuon)
    _run_all_stages(w, 2, stream_groups=groups)


# matrices that are one 256-row panel (every iteration in one workgroup,
# A and B in LDS), next to one just beyond the panel kernel's limit
PANEL = [
    (256, 256, 2, "spike"),               # a single 256-column block
    (256, 990, 1, "spike"),               # n_pad 1024, Gram K trimmed to 992
    (990, 256, 1, "spike"),               # tall -> transposed
    (256, 4096, 1, "spike"),              # the largest panel: 16 column blocks
    (256, 4100, 1, "spike"),              # n_pad 4352: the tiled kernels
    (256, 768, 1, "rank8"),
    (256, 512, 1, "zero"),
    (256, 300, 1, "student_t", 0.0),      # lr_mul 0
    (300, 256, 1, "gauss", 1.0, 1),       # frozen
]


@pytest.mark.parametrize("normuon", [0, 1])
def test_panel_matrices_all_stages(normuon):
    w = custom_workload(150 + normuon, PANEL, steps=3, normuon=normuon, lr=0.05, weight_decay=0.05 * normuon)
    _run_all_stages(w, 3)


# every matrix on 128 / 256 tiles, decoupled weight decay with per-matrix
# lr_mul / wd_mul, ragged edges, transposed blocks, zero and frozen matrices
LARGE_TILES = [
    (200, 300, 1, "spike", 1.5, 0, 0.5),
    (300, 200, 1, "spike", 1.0, 0, 2.0),  # tall -> transposed
    (1000, 700, 1, "spike"),              # 256-tiles, transposed, padded edge
    (130, 130, 1, "zero"),
    (96, 160, 1, "gauss", 1.0, 1),        # frozen
    (65, 131, 1, "student_t", 0.0),       # lr_mul 0
    (129, 67, 2, "gauss"),                # odd widths: scalar edge path
    (300, 560, 1, "spike"),               # 128-tiles: last tile row leaves a wave's rows all padding
    (1100, 420, 1, "spike"),              # 256-tiles, transposed: edge waves with 0, 1 or 2 column blocks
    (300, 2100, 1, "spike"),              # long K on 128-tiles
    (700, 2100, 1, "spike"),              # long K on 256-tiles, padded edge
]


def test_long_thin_matrices_all_stages():
    # bf16 matrices whose short side is at most 64 but too long for the
    # one-workgroup kernel (padded long side > 512) run on the generic 64-tile
    # kernels, with K up to the whole long side: a single row of 2^20 (the
    # dimension limit), tall and wide thin matrices, and a zero one
    shapes = [(1, 1 << 20, 1, "gauss"), (3000, 20, 1, "spike"), (48, 1000, 2, "gauss"), (64, 700, 1, "rank8"),
              (2, 5000, 1, "zero")]
    w = custom_workload(114, shapes, steps=2, lr=0.05)
    _run_all_stages(w, 2)
    w2 = custom_workload(115, shapes[:3], steps=1, normuon=1, lr=0.05)
    _run_all_stages(w2, 1)


def _run_with_coeffs(w, steps, coeffs, sharp, **hp):
    _say(f"[case] {w.name} {len(coeffs)} NS iterations, sharp={sharp} hp={hp}")
    run = GpuRun(w, coeffs=coeffs, **hp)
    idx = [gi for gi, *_ in run.subs]
    orc_m = {gi: np.zeros((r, c)) for gi, _e, _k, _o, r, c in run.subs}
    for t in range(steps):
        p_prev, v_prev = snapshot(run, idx)
        g = run.load_grads(t)
        run.step()
        rep = []
        worst = check_stages(run, t, idx, grads_host=g, p_prev=p_prev, v_prev=v_prev, orc_m=orc_m, report=rep,
                             coeffs=coeffs, sharp=sharp)
        _say(f"  step {t}: {worst}")
        for r in sorted(rep, key=lambda x: -x[6]):
            _say(f"    NS gi={r[2]} [{r[3]},{r[4]}] {r[5]}: gpu-vs-contract {r[6]:.3e} contract-vs-exact {r[7]:.3e} "
                 f"gpu-vs-exact {r[8]:.3e}")
        assert_worst(worst, fp32=run.fp32)


STEP_SHAPES = [(400, 520, 1, "spike"), (200, 300, 1, "spike"), (48, 1000, 1, "gauss"), (64, 64, 2, "gauss"),
               (256, 640, 1, "spike")]


@pytest.mark.parametrize("ns_steps", [1, 10, 16])
def test_newton_schulz_step_counts(ns_steps):
    # The pages' quintic at one iteration (the first is also the last: s
    # scaling and the NorMuon row sums in the same update launch), at the
    # pages' signature default of 10 and at the maximum of 16, on 256-, 128-
    # and 64-tiles and the one-workgroup kernel. Beyond five iterations the
    # quintic does not converge, so only G3(b) (against exact NS) applies.
    w = custom_workload(116 + ns_steps, STEP_SHAPES, steps=2, normuon=1, ns_steps=ns_steps, lr=0.05)
    _run_with_coeffs(w, 2, O.default_coeffs(ns_steps), sharp=ns_steps <= 5)


@pytest.mark.parametrize("ns_steps", [10, 16])
def test_newton_schulz_step_counts_convergent_tail(ns_steps):
    # Five quintic iterations, then the cubic Newton-Schulz step (1.5, -0.5, 0),
    # which converges to the orthogonal factor: rounding noise stops growing,
    # so the GPU is held to the full G3(a) gate against the contract at 10 and
    # 16 iterations (per-iteration coefficients and the buffer ping-pong at
    # every count, sharply).
    coeffs = O.default_coeffs(5) + [(1.5, -0.5, 0.0)] * (ns_steps - 5)
    w = custom_workload(140 + ns_steps, STEP_SHAPES, steps=2, normuon=1, ns_steps=ns_steps, lr=0.05)
    _run_with_coeffs(w, 2, coeffs, sharp=True)


def test_stream_groups_give_identical_results():
    # the 9 tiled matrices split over 2, 3 or 4 streams, or all on the
    # caller's stream (also the library's own choice, 0, for a step this
    # small): the same kernels on the same tiles, so bit-identical
    w = custom_workload(110, LARGE_TILES + [(200, 300, 2, "spike"), (64, 64, 3, "rank8"), (256, 512, 2, "spike")],
                        steps=2, lr=0.05,
                        weight_decay=0.1, normuon=1)
    groups = (1, 0, 2, 3, 4)
    runs = [GpuRun(w, stream_groups=g) for g in groups]
    assert [int(B.muon_work_stats(r.H.h).launches[B.MUON_KERNEL_MOMENTUM]) for r in runs] == [1, 1, 2, 3, 4]
    for t in range(2):
        for r in runs:
            r.load_grads(t)
            r.step()
        for g, r in zip(groups[1:], runs[1:]):
            for name in ("params", "mom"):
                assert torch.equal(getattr(runs[0], name), getattr(r, name)), \
                    f"step {t}: {name} differs between one and {g} stream groups"
            assert torch.equal(runs[0].H.view(B.MUON_VIEW_NS_OUT, torch.bfloat16),
                               r.H.view(B.MUON_VIEW_NS_OUT, torch.bfloat16))


def test_step_captured_in_a_hip_graph_replays_like_eager():
    # muon_step allocates nothing, never synchronises and records no memset,
    # and its two-stream fork / join is event-based, so a caller can capture it
    # in a HIP graph; every replay must equal the eager step on the same state
    # (tiled, small and one-panel matrices: every kind of launch the step makes)
    w = custom_workload(111, LARGE_TILES + [(64, 64, 3, "rank8"), (256, 512, 2, "spike")], steps=1, lr=0.05,
                        weight_decay=0.1)
    run = GpuRun(w)
    run.load_grads(0)
    run.step()  # past the first-step paths
    eager_p, eager_m = run.params.clone(), run.mom.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        run.H.step(run.params, run.grads, run.mom, w.lr)
    torch.cuda.synchronize()
    # capture does not execute: restart both copies from the same state
    run.params.copy_(eager_p)
    run.mom.copy_(eager_m)
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        run.H.step(eager_p, run.grads, eager_m, w.lr)  # eager, same handle, other buffers
        torch.cuda.synchronize()
        assert torch.equal(run.params, eager_p), f"replay {r}: params differ from the eager step"
        assert torch.equal(run.mom, eager_m), f"replay {r}: momentum differs from the eager step"


def test_gram_and_polynomial_buffers_are_symmetric_and_consistent():
    # The large-tile kernels compute only upper tiles, and on a diagonal tile
    # only the 32 x 32 blocks on or above its diagonal; everything below is
    # written from the mirror image. So the last iteration's A and B must be
    # exactly symmetric, and B must be the bf16 polynomial b A + c A A of that
    # A (fp64 here, fp32 accumulation on the GPU).
    # Padded edges (700 -> 768 on 256-tiles, 200 / 300 -> 256 on 128-tiles)
    # must hold A = B = 0 there: edge waves skip the blocks that lie wholly in
    # the padding, so those values come from the epilogue alone.
    shapes = [(768, 768, 2, "spike"), (768, 3072, 1, "spike"), (3072, 768, 1, "gauss"),
              (300, 200, 1, "spike"), (200, 260, 1, "gauss"), (64, 64, 2, "rank8"),
              (1000, 700, 1, "spike"), (256, 1024, 1, "spike"), (2100, 700, 1, "spike")]
    w = custom_workload(112, shapes, steps=1, lr=0.02)
    run = GpuRun(w)
    run.load_grads(0)
    run.step()
    A_all = run.H.view(B.MUON_VIEW_GRAM, torch.bfloat16)
    P_all = run.H.view(B.MUON_VIEW_POLY, torch.bfloat16)
    _a, b, c = O.default_coeffs()[-1]
    checked = set()
    for gi, *_ in run.subs:
        L = run.lay[gi]
        if L.m_pad == 64 and L.ld <= 512:
            continue  # one-workgroup path: A and B' stay in LDS
        sz = L.m_pad * L.m_pad
        A = A_all[L.gram_offset:L.gram_offset + sz].view(L.m_pad, L.m_pad)
        P = P_all[L.gram_offset:L.gram_offset + sz].view(L.m_pad, L.m_pad)
        assert torch.equal(A, A.t().contiguous()), f"A of matrix {gi} not symmetric"
        assert torch.equal(P, P.t().contiguous()), f"B of matrix {gi} not symmetric"
        Af = A.float().cpu().numpy().astype(np.float64)
        Pf = P.float().cpu().numpy().astype(np.float64)
        assert np.all(Af[L.m:, :] == 0) and np.all(Pf[L.m:, :] == 0), f"matrix {gi}: padding not zero"
        An = Af[:L.m, :L.m]
        Pn = Pf[:L.m, :L.m]
        assert np.all(np.diag(An) >= 0)
        ref = O.bf16_round(b * An + c * (An @ An))
        err = np.linalg.norm(Pn - ref) / np.linalg.norm(ref)
        _say(f"  matrix {gi} [{L.m} x {L.n}] m_pad {L.m_pad}: B vs poly(A) {err:.2e}")
        assert err <= 5e-3
        checked.add(L.m_pad)
    assert {256, 768} <= checked  # one- and three-tile diagonals covered


def test_weight_decay_large_tiles_ragged():
    w = custom_workload(109, LARGE_TILES, steps=3, lr=0.05, weight_decay=0.1)
    _run_all_stages(w, 3)


def test_ragged_fp32_all_stages():
    w = custom_workload(102, RAGGED, steps=3, ns_precision="fp32", normuon=1, lr=0.05)
    _run_all_stages(w, 3)


def test_fp32_group_larger_than_the_mall():
    # one stream group writing 285 MB of X~ (more than the 256 MB MALL): the
    # momentum kernel stores X~ nontemporally, in the runs of the untransposed
    # matrices and in the transposed matrices' tiles; one matrix of each
    # orientation is checked against the oracle
    w = custom_workload(118, [(2048, 4352, 4, "spike"), (4352, 2048, 4, "gauss")], steps=2,
                        ns_precision="fp32", lr=0.05)
    _say(f"[case] {w.name}: {w.num_matrices} matrices, {w.total} elements, one stream group")
    run = GpuRun(w, stream_groups=1)
    sample = [1, 6]
    orc_m = {gi: np.zeros((run.subs[gi][4], run.subs[gi][5])) for gi in sample}
    for t in range(w.steps):
        p_prev, v_prev = snapshot(run, sample)
        g = run.load_grads(t)
        run.step()
        worst = check_stages(run, t, sample, grads_host=g, p_prev=p_prev, v_prev=v_prev, orc_m=orc_m)
        _say(f"  step {t}: {worst}")
        assert_worst(worst, fp32=True)


def test_bf16_group_whose_gram_output_exceeds_the_mall():
    # one stream group whose Gram output A (34 x 2048^2 bf16 = 285 MB) is larger
    # than the 256 MB MALL: the Gram and polynomial kernels store A and B, their
    # mirrors included, nontemporally (as the momentum kernel does X~). The
    # first and last matrix are checked against the oracle, and the last
    # iteration's A and B of both must still be exactly symmetric
    w = custom_workload(119, [(2048, 2048, 34, "spike")], steps=2, lr=0.05)
    _say(f"[case] {w.name}: {w.num_matrices} matrices, {w.total} elements, one stream group")
    run = GpuRun(w, stream_groups=1)
    sample = [0, 33]
    orc_m = {gi: np.zeros((run.subs[gi][4], run.subs[gi][5])) for gi in sample}
    for t in range(w.steps):
        p_prev, v_prev = snapshot(run, sample)
        g = run.load_grads(t)
        run.step()
        worst = check_stages(run, t, sample, grads_host=g, p_prev=p_prev, v_prev=v_prev, orc_m=orc_m)
        _say(f"  step {t}: {worst}")
        assert_worst(worst)
    A_all = run.H.view(B.MUON_VIEW_GRAM, torch.bfloat16)
    P_all = run.H.view(B.MUON_VIEW_POLY, torch.bfloat16)
    for gi in sample:
        L = run.lay[gi]
        sz = L.m_pad * L.m_pad
        A = A_all[L.gram_offset:L.gram_offset + sz].view(L.m_pad, L.m_pad)
        P = P_all[L.gram_offset:L.gram_offset + sz].view(L.m_pad, L.m_pad)
        assert torch.equal(A, A.t().contiguous()), f"A of matrix {gi} not symmetric"
        assert torch.equal(P, P.t().contiguous()), f"B of matrix {gi} not symmetric"
    assert np.all(run.scalars(B.MUON_VIEW_STATUS) == 0)


def test_heavy_ball_and_weight_decay_and_steps():
    # heavy-ball momentum, Nesterov off, decoupled weight decay, 7 NS steps with
    # a per-iteration coefficient schedule whose last step is the cubic
    # Newton-Schulz step (c = 0: the polynomial has no A A term)
    w = custom_workload(103, [(150, 300, 1, "gauss", 1.5), (300, 150, 1, "gauss")], steps=2,
                        weight_decay=0.1, nesterov=0, ns_steps=7, lr=0.03)
    coeffs = [(3.4445, -4.7750, 2.0315)] * 5 + [(2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]
    run = GpuRun(w, momentum_kind=B.MUON_MOMENTUM_HEAVY_BALL, coeffs=coeffs)
    orc = O.OracleMuon(w.entries, w.total, momentum=w.momentum, nesterov=0, coeffs=coeffs,
                       weight_decay=0.1, momentum_kind="heavy_ball", mode="bf16")
    for t in range(2):
        p_prev = run.params.cpu().numpy().astype(np.float64)
        g = run.load_grads(t)
        orc.step(p_prev, g, lr=w.lr, keep=[0, 1])
        run.step()
        for gi in (0, 1):
            _gi, ei, _k, off, R, C = run.subs[gi]
            e = w.entries[ei]
            assert O.rel_fro(run.mat(run.mom, gi), orc.m[off:off + R * C].reshape(R, C)) <= 1e-6
            xt = run.xtilde(gi)
            s = float(run.scalars(B.MUON_VIEW_SCALE)[gi])
            out = run.ns_out(gi)
            ref = O.ns_bf16_contract(xt, s, coeffs)
            ex = O.ns_exact(xt, s, coeffs)
            _say(f"  matrix {gi}: gpu-vs-contract {O.rel_fro(out, ref):.3e} gpu-vs-exact {O.rel_fro(out, ex):.3e} "
                 f"contract-vs-exact {O.rel_fro(ref, ex):.3e}")
            assert O.rel_fro(out, ref) <= 2e-2
            assert O.rel_fro(out, ex) <= O.rel_fro(ref, ex) + 5e-3
            tr = R > C
            want = O.apply_update(p_prev[off:off + R * C].reshape(R, C), out.T if tr else out, w.lr, e.lr_mul,
                                  0.1, e.wd_mul, R, C)
            assert O.rel_fro(run.mat(run.params, gi), want) <= 1e-6


def test_tiny_config_free_running_fp32():
    # the tiny d = 128 block in fp32 NS: free-running params and momentum vs the
    # float64 oracle over all steps
    w = get_workload(0)
    run = GpuRun(w)
    orc = O.OracleMuon(w.entries, w.total, momentum=w.momentum, mode="exact")
    p_or = run.params.cpu().numpy().astype(np.float64)
    for t in range(w.steps):
        g = run.load_grads(t)
        p_or = orc.step(p_or, g, lr=w.lr)
        run.step()
    p = run.params.cpu().numpy().astype(np.float64)
    m = run.mom.cpu().numpy().astype(np.float64)
    for gi, _ei, _k, off, r, c in run.subs:
        sl = slice(off, off + r * c)
        e_p = O.rel_fro(p[sl], p_or[sl])
        e_d = O.rel_fro(p[sl] - gen0(w)[sl], p_or[sl] - gen0(w)[sl])
        e_m = O.rel_fro(m[sl], orc.m[sl])
        _say(f"  tiny matrix {gi}: params {e_p:.2e} update {e_d:.2e} momentum {e_m:.2e}")
        assert e_p <= 1e-6 and e_m <= 1e-6 and e_d <= 1e-4


def test_per_call_schedules_free_running_fp32():
    # The library's schedule functions drive every step through muon_step's
    # per-call arguments: momentum warm-up 0.85 -> 0.95 over 4 steps
    # (momentum_coef) and the WSD learning rate with a 3-step warm-down (lr),
    # over 6 free-running fp32-NS steps on 64- and 128-tiles. Params and
    # momentum vs the float64 oracle stepped with the same per-step values.
    w = custom_workload(113, [(128, 128, 2, "gauss"), (96, 200, 1, "gauss"), (200, 96, 1, "gauss"),
                              (300, 260, 1, "gauss")], steps=6, ns_precision="fp32")
    run = GpuRun(w)
    orc = O.OracleMuon(w.entries, w.total, momentum=w.momentum, mode="exact")
    p0 = run.params.cpu().numpy().astype(np.float64)
    p_or = p0.copy()
    for t in range(6):
        beta = B.muon_momentum_warmup(t, 4, 0.85, 0.95)
        lr = 0.05 * B.muon_lr_wsd(t, 6, 0, 3)
        g = run.load_grads(t)
        p_or = orc.step(p_or, g, lr=lr, beta=beta)
        run.step(lr=lr, momentum_coef=beta)
    p = run.params.cpu().numpy().astype(np.float64)
    m = run.mom.cpu().numpy().astype(np.float64)
    for gi, _ei, _k, off, r, c in run.subs:
        sl = slice(off, off + r * c)
        e_p = O.rel_fro(p[sl], p_or[sl])
        e_d = O.rel_fro(p[sl] - p0[sl], p_or[sl] - p0[sl])
        e_m = O.rel_fro(m[sl], orc.m[sl])
        _say(f"  matrix {gi} [{r} x {c}]: params {e_p:.2e} update {e_d:.2e} momentum {e_m:.2e}")
        assert e_p <= 1e-6 and e_m <= 1e-6 and e_d <= 1e-4


_P0 = {}


def gen0(w):
    if w.name not in _P0:
        from workloads import gen_params
        _P0[w.name] = gen_params(w).astype(np.float64)
    return _P0[w.name]


def test_determinism_and_batch_independence():
    shapes = [(200, 200, 2, "spike"), (136, 520, 1, "spike"), (520, 136, 1, "spike"), (64, 64, 2, "rank8"),
              (256, 512, 1, "spike")]
    w = custom_workload(104, shapes, steps=2, normuon=1)
    r1, r2 = GpuRun(w), GpuRun(w)
    for t in range(2):
        g = gen_grads(w, t)
        for r in (r1, r2):
            r.load_grads(t, g)
            r.step()
    assert torch.equal(r1.params, r2.params) and torch.equal(r1.mom, r2.mom)
    # the same matrices in reversed table order give bit-identical per-matrix results
    rev = custom_workload(104, list(reversed(shapes)), steps=2, normuon=1)
    r3 = GpuRun(rev)
    sub_f = r1.subs
    sub_r = r3.subs
    # map: same (shape, gclass) occurrence order
    g_by_t = []
    for t in range(2):
        gf = gen_grads(w, t)
        gr = np.empty(rev.total, np.float32)
        for (gi, ei, k, off, R, C) in sub_f:
            j = _partner(w, rev, gi)
            _g2, _e2, _k2, off2, _R2, _C2 = sub_r[j]
            gr[off2:off2 + R * C] = gf[off:off + R * C]
        g_by_t.append(gr)
    pf = r1.params.cpu().numpy()
    r3.params.copy_(torch.from_numpy(_permute(w, rev, r1, gen0(w).astype(np.float32))))
    for t in range(2):
        r3.load_grads(t, g_by_t[t])
        r3.step()
    pr = r3.params.cpu().numpy()
    for (gi, ei, k, off, R, C) in sub_f:
        j = _partner(w, rev, gi)
        off2 = sub_r[j][3]
        assert np.array_equal(pf[off:off + R * C], pr[off2:off2 + R * C]), gi


def _partner(w, rev, gi):
    # index of matrix gi of w inside the reversed table
    counts = [e.count for e in w.entries]
    ei, k = 0, gi
    while k >= counts[ei]:
        k -= counts[ei]
        ei += 1
    rei = len(w.entries) - 1 - ei
    return sum(e.count for e in rev.entries[:rei]) + k


def _permute(w, rev, run, p):
    out = np.empty(rev.total, np.float32)
    for (gi, ei, k, off, R, C) in run.subs:
        j = _partner(w, rev, gi)
        off2 = rev.submatrices()[j][3]
        out[off2:off2 + R * C] = p[off:off + R * C]
    return out


def test_nonfinite_gradient_is_isolated_and_reported():
    w = custom_workload(105, [(128, 256, 1, "gauss"), (128, 256, 1, "gauss"), (200, 100, 1, "gauss")], steps=1)
    clean = GpuRun(w)
    dirty = GpuRun(w)
    g = gen_grads(w, 0)
    clean.load_grads(0, g)
    clean.step()
    g2 = g.copy()
    g2[5] = np.nan
    dirty.load_grads(0, g2)
    dirty.step()
    st = dirty.scalars(B.MUON_VIEW_STATUS)
    assert st[0] == 1 and st[1] == 0 and st[2] == 0
    pc, pd = clean.params.cpu().numpy(), dirty.params.cpu().numpy()
    n0 = 128 * 256
    assert np.array_equal(pc[n0:], pd[n0:])
    assert not np.all(np.isfinite(pd[:n0]))


def test_reset_zeroes_state_and_restarts():
    w = custom_workload(106, [(96, 200, 1, "gauss"), (200, 96, 1, "gauss"), (50, 50, 1, "gauss", 1.0, 1)],
                        steps=2, normuon=1)
    run = GpuRun(w)
    frozen_off = w.entries[2].offset
    run.mom[frozen_off:frozen_off + 2500] = 7.0  # the frozen matrix's momentum is never touched
    for t in range(2):
        run.load_grads(t)
        run.step()
    run.H.reset(run.mom)
    torch.cuda.synchronize()
    m = run.mom.cpu().numpy()
    assert np.all(m[:frozen_off] == 0) and np.all(m[frozen_off:frozen_off + 2500] == 7.0)
    assert np.all(run.H.view(B.MUON_VIEW_V, torch.float32).cpu().numpy() == 0)
    # a step after reset equals a first step from the same params
    fresh = GpuRun(w)
    fresh.params.copy_(run.params)
    fresh.mom[frozen_off:frozen_off + 2500] = 7.0
    g = gen_grads(w, 0)
    for r in (run, fresh):
        r.load_grads(0, g)
        r.step()
    assert torch.equal(run.params, fresh.params) and torch.equal(run.mom, fresh.mom)


def test_checkpoint_resume_is_bit_identical():
    # The optimizer state is the caller's momentum plus NorMuon's v in the
    # workspace (reset() after warm-up clears exactly these, per the
    # FixMuonLR record's change 2). k steps, a checkpoint of params,
    # momentum and v, a fresh handle and workspace restored from it, and k
    # more steps there must equal 2k uninterrupted steps bit for bit.
    shapes = [(768, 768, 2, "spike"), (300, 200, 1, "spike"), (64, 64, 3, "rank8"), (1000, 700, 1, "spike"),
              (48, 1000, 1, "gauss"), (96, 160, 1, "gauss", 1.0, 1)]
    w = custom_workload(120, shapes, steps=4, normuon=1, lr=0.05, weight_decay=0.1)
    k = 2
    ref, first = GpuRun(w), GpuRun(w)
    for t in range(k):
        g = gen_grads(w, t)
        for r in (ref, first):
            r.load_grads(t, g)
            r.step()
    ck_p, ck_m = first.params.clone(), first.mom.clone()
    ck_v = first.H.view(B.MUON_VIEW_V, torch.float32).clone()
    first.H.close()
    resumed = GpuRun(w)
    resumed.params.copy_(ck_p)
    resumed.mom.copy_(ck_m)
    resumed.H.view(B.MUON_VIEW_V, torch.float32).copy_(ck_v)
    torch.cuda.synchronize()
    for t in range(k, 2 * k):
        g = gen_grads(w, t)
        for r in (ref, resumed):
            r.load_grads(t, g)
            r.step()
    assert torch.equal(ref.params, resumed.params)
    assert torch.equal(ref.mom, resumed.mom)
    assert torch.equal(ref.H.view(B.MUON_VIEW_V, torch.float32), resumed.H.view(B.MUON_VIEW_V, torch.float32))
    assert torch.any(ref.H.view(B.MUON_VIEW_V, torch.float32) != 0)


def test_work_split_between_panel_small_and_tiled_kernels():
    # which kernel runs which matrix: 256-row panels up to n_pad 4096 in the
    # panel kernel (one launch per stream group that has any), 64-row
    # matrices with n_pad <= 512 in the small kernel, the rest tiled; the
    # algorithmic flops follow the matrices
    shapes = [(256, 1024, 3, "spike"), (2048, 256, 1, "spike"), (256, 4100, 1, "spike"), (64, 300, 2, "gauss"),
              (768, 768, 2, "spike"), (256, 512, 1, "gauss", 1.0, 1)]
    w = custom_workload(160, shapes, steps=1)

    def flops(m, n, steps=5):
        return steps * (m * (m + 1) * n + m * (m + 1) * m + 2 * m * m * n)

    for groups in (1, 3):
        H = B.MuonHandle(w.entries, B.make_hparams(stream_groups=groups))
        ws = B.muon_work_stats(H.h)
        panel = 3 * flops(256, 1024) + flops(256, 2048)
        small = 2 * flops(64, 300)
        tiled = flops(256, 4100) + 2 * flops(768, 768)
        assert ws.flops[B.MUON_KERNEL_NS_PANEL] == pytest.approx(panel, rel=1e-12)
        assert ws.flops[B.MUON_KERNEL_NS_SMALL] == pytest.approx(small, rel=1e-12)
        tiled_sum = sum(ws.flops[k] for k in (B.MUON_KERNEL_GRAM, B.MUON_KERNEL_POLY, B.MUON_KERNEL_UPDATE))
        assert tiled_sum == pytest.approx(tiled, rel=1e-12)
        assert ws.launches[B.MUON_KERNEL_NS_SMALL] == 1
        assert 1 <= ws.launches[B.MUON_KERNEL_NS_PANEL] <= groups
        del H


def test_empty_and_all_frozen_tables_are_noops():
    w = custom_workload(107, [(64, 64, 2, "gauss", 1.0, 1)], steps=1)
    run = GpuRun(w)
    p0 = run.params.clone()
    run.load_grads(0)
    run.step()
    assert torch.equal(run.params, p0) and torch.all(run.mom == 0)
    H = B.MuonHandle([], B.make_hparams())
    x = torch.zeros(4, device="cuda")
    H.step(x, x.clone(), x.clone(), 0.1)
    torch.cuda.synchronize()


def test_step_argument_errors():
    w = custom_workload(108, [(32, 48, 1, "gauss")], steps=1)
    run = GpuRun(w)
    lib = B.load()
    h = run.H.h
    st = torch.cuda.current_stream().cuda_stream
    p, g, m = run.params, run.grads, run.mom
    assert B.muon_step(h, p.data_ptr(), g.data_ptr(), m.data_ptr(), w.total - 1, 0.1, -1, st) == B.MUON_E_LAYOUT
    assert B.muon_step(h, p.data_ptr(), p.data_ptr(), m.data_ptr(), w.total, 0.1, -1, st) == B.MUON_E_INVALID_ARG
    assert B.muon_step(h, p.data_ptr(), g.data_ptr(), m.data_ptr(), w.total, float("nan"), -1, st) == \
        B.MUON_E_INVALID_ARG
    assert B.muon_step(h, p.data_ptr(), g.data_ptr(), m.data_ptr(), w.total, 0.1, 1.5, st) == B.MUON_E_INVALID_ARG
    assert B.muon_step(h, p.data_ptr() + 4, g.data_ptr(), m.data_ptr(), w.total - 4, 0.1, -1, st) in (
        B.MUON_E_LAYOUT,)
    assert "aligned" in B.muon_last_error(h) or "hold" in B.muon_last_error(h)
    assert lib.muon_num_matrices(h) == 1


# ---------------------------------------------------------------------------
# Full-size workloads, sampled
# ---------------------------------------------------------------------------
def _full_size(config_id, sample, steps=None, check_every=1):
    w = get_workload(config_id)
    steps = w.steps if steps is None else steps
    _say(f"[case] config {config_id} {w.name}: {w.num_matrices} matrices, {w.total} elements, {steps} steps")
    run = GpuRun(w)
    orc_m = {gi: np.zeros((run.subs[gi][4], run.subs[gi][5])) for gi in sample}
    rep = []
    for t in range(steps):
        p_prev, v_prev = snapshot(run, sample)
        g = run.load_grads(t)
        run.step()
        worst = check_stages(run, t, sample, grads_host=g, p_prev=p_prev, v_prev=v_prev, orc_m=orc_m, report=rep)
        _say(f"  step {t}: {worst}")
        assert_worst(worst, fp32=run.fp32)
    assert np.all(np.isfinite(run.params.cpu().numpy()))
    # per shape and gradient class, over the sampled matrices and all steps:
    # GPU vs the bf16 contract, the contract vs exact NS (the method's own
    # error) and GPU vs exact NS
    by = {}
    for _k, _t, _gi, R, C, gc, e3, ce, eex in rep:
        m = by.setdefault((R, C, gc), [0.0, 0.0, 0.0, 0])
        m[0], m[1], m[2], m[3] = max(m[0], e3), max(m[1], ce), max(m[2], eex), m[3] + 1
    for (R, C, gc), m in sorted(by.items()):
        _say(f"  NS table {w.name} [{R},{C}] {gc}: n={m[3]} gpu-vs-contract {m[0]:.3e} "
             f"contract-vs-exact {m[1]:.3e} gpu-vs-exact {m[2]:.3e}")
    return run


def test_gpt2_body_124m_sampled():
    # layer 0 and layer 11: qkvo x4, c_fc, c_proj (transposed)
    _full_size(1, sample=list(range(0, 6)) + list(range(66, 72)))


def test_gpt2_body_124m_normuon_sampled():
    _full_size(2, sample=list(range(0, 6)) + list(range(66, 72)))


@pytest.mark.timeout(900)
def test_stress_batch_all_matrices():
    w = get_workload(4)
    run = _full_size(4, sample=[gi for gi, *_ in get_workload(4).submatrices()])
    p = run.params.cpu().numpy()
    from workloads import gen_params
    p0 = gen_params(w)
    m = run.mom.cpu().numpy()
    for gi, ei, _k, off, r, c in run.subs:
        e = w.entries[ei]
        sl = slice(off, off + r * c)
        if e.frozen:
            assert np.array_equal(p[sl], p0[sl]) and np.all(m[sl] == 0)
        if e.gclass == "zero":
            assert np.array_equal(p[sl], p0[sl])


@pytest.mark.timeout(1200)
def test_scaled_body_1p5b_sampled():
    # layers 0, 23, 47: one qkvo matrix, c_fc and c_proj of each
    s = []
    for layer in (0, 23, 47):
        s += [6 * layer, 6 * layer + 4, 6 * layer + 5]
    _full_size(3, sample=s)
