"""muon_init_static (the library's static device workspace, no device
allocation) against muon_init with a caller workspace, through the C ABI.

Two handles in a row on one GPU, the second with a smaller table: each must
step exactly like an ordinary handle on the same inputs (the same kernels on
the same tiles, so params and momentum agree bit for bit), and a table larger
than the static workspace is rejected.
"""

import pytest
import torch

from muon_newton_schulz_04_amd import binding as B
from workloads import custom_workload, gen_grads, gen_params, get_workload

pytestmark = pytest.mark.gpu


def _step_both(w, steps):
    hp = B.make_hparams(normuon=w.normuon, ns_steps=w.ns_steps, weight_decay=w.weight_decay)
    s, nbytes = B.muon_workspace_bytes(w.entries, hp)
    assert s == B.MUON_OK and nbytes <= B.MUON_STATIC_WORKSPACE_BYTES
    ref = B.MuonHandle(w.entries, hp)
    s, h = B.muon_init_static(w.entries, hp, 0)
    B.check(s, None, "muon_init_static")
    try:
        p0 = torch.from_numpy(gen_params(w)).cuda()
        pa, pb = p0.clone(), p0.clone()
        ma, mb = torch.zeros_like(p0), torch.zeros_like(p0)
        st = torch.cuda.current_stream().cuda_stream
        for t in range(steps):
            g = torch.from_numpy(gen_grads(w, t)).cuda()
            ref.step(pa, g, ma, w.lr)
            B.check(B.muon_step(h, pb.data_ptr(), g.data_ptr(), mb.data_ptr(), w.total, w.lr, -1.0, st), h,
                    "muon_step")
            torch.cuda.synchronize()
            assert torch.equal(pa, pb), f"step {t}: params differ between the static and the caller workspace"
            assert torch.equal(ma, mb), f"step {t}: momentum differs between the static and the caller workspace"
        assert not torch.equal(pa, p0)
    finally:
        B.muon_destroy(h)
        ref.close()


def test_static_workspace_matches_caller_workspace():
    # large-tile, one-workgroup, 64-tile and padded-edge matrices with NorMuon
    first = custom_workload(130, [(768, 768, 2, "spike"), (300, 200, 1, "spike"), (64, 64, 3, "rank8"),
                                  (1000, 700, 1, "spike"), (48, 1000, 1, "gauss")], steps=2, normuon=1, lr=0.05)
    _step_both(first, 2)
    # the next call on the same GPU, with a smaller table: the array keeps the
    # previous contents, which muon_init_static clears where it must
    second = custom_workload(131, [(200, 200, 1, "spike"), (64, 64, 2, "gauss")], steps=2, lr=0.05)
    _step_both(second, 2)


def test_static_workspace_rejects_tables_beyond_its_size():
    w = get_workload(1)  # the 124M body needs about 649 MiB of workspace
    s, h = B.muon_init_static(w.entries, B.make_hparams(), 0)
    assert s == B.MUON_E_WORKSPACE and not h.value
    assert "static workspace" in B.muon_last_error()
