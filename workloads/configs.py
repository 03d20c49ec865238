"""The five Muon-step workloads, as matrix tables plus hyper-parameters.

Shapes follow the GPT-2-style body the pages train: per layer a fused
attention weight viewed as four [d, d] matrices (Q, K, V, O), an MLP
up-projection c_fc [d, 4d] and a down-projection c_proj [4d, d]
(page "modded-nanogpt 50B-token 长时程训练实验解析", GPTConfig in the section on
the hyper-parameters; page "2025-10-27_FixMuonLR" analysis, change 2, the
early qkvo reshape into four matrices).

Every table entry is a run of `count` contiguous row-major [rows, cols]
matrices starting at element `offset` of the flat parameter / gradient /
momentum buffers. Table order is layer-major: qkvo x4, c_fc, c_proj.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Sequence, Tuple


@dataclass(frozen=True)
class Entry:
    rows: int
    cols: int
    count: int
    offset: int
    lr_mul: float = 1.0
    wd_mul: float = 1.0
    frozen: int = 0
    name: str = ""
    gclass: str = "spike"  # gradient distribution class (see generators.py)


@dataclass
class Workload:
    config_id: int
    name: str
    entries: List[Entry]
    steps: int
    lr: float = 0.02
    momentum: float = 0.95
    nesterov: int = 1
    ns_steps: int = 5
    ns_precision: str = "bf16"  # "bf16" or "fp32"
    normuon: int = 0
    normuon_beta2: float = 0.95
    normuon_eps: float = 1e-10
    weight_decay: float = 0.0
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def total(self) -> int:
        if not self.entries:
            return 0
        return max(e.offset + e.rows * e.cols * e.count for e in self.entries)

    def submatrices(self) -> List[Tuple[int, int, int, int, int, int]]:
        """(global index, entry index, k within entry, offset, rows, cols)."""
        out = []
        gi = 0
        for ei, e in enumerate(self.entries):
            for k in range(e.count):
                out.append((gi, ei, k, e.offset + k * e.rows * e.cols, e.rows, e.cols))
                gi += 1
        return out

    @property
    def num_matrices(self) -> int:
        return sum(e.count for e in self.entries)

    @property
    def active_elements(self) -> int:
        return sum(e.rows * e.cols * e.count for e in self.entries if not e.frozen)


def _body(d: int, layers: int, gclass: str, cfc_lr_mul: float = 1.0) -> List[Entry]:
    entries = []
    off = 0
    for layer in range(layers):
        entries.append(Entry(d, d, 4, off, name=f"h{layer}.qkvo", gclass=gclass))
        off += 4 * d * d
        entries.append(Entry(d, 4 * d, 1, off, lr_mul=cfc_lr_mul, name=f"h{layer}.c_fc", gclass=gclass))
        off += 4 * d * d
        entries.append(Entry(4 * d, d, 1, off, name=f"h{layer}.c_proj", gclass=gclass))
        off += 4 * d * d
    return entries


def _stress() -> List[Entry]:
    entries = []
    off = 0
    classes = ("rank8", "student_t", "zero", "frozen")
    for shape, n in (((64, 64), 4096), ((256, 1024), 256)):
        r, c = shape
        for i in range(n):
            cls = classes[i % 4]
            frozen = 1 if cls == "frozen" else 0
            entries.append(
                Entry(
                    r, c, 1, off,
                    lr_mul=0.0 if frozen else 1.0,
                    frozen=frozen,
                    name=f"s{r}x{c}.{i}",
                    gclass="student_t" if frozen else cls,
                )
            )
            off += r * c
    return entries


def _make(config_id: int) -> Workload:
    if config_id == 0:
        return Workload(
            0, "tiny_d128", _body(128, 1, "iid"), steps=3, lr=0.02, ns_precision="fp32",
            description="one block d=128, i.i.d. N(0, 0.1^2) grads, fp32 NS, 3 steps",
        )
    if config_id == 1:
        return Workload(
            1, "gpt2_124m_body", _body(768, 12, "spike"), steps=10, lr=0.02,
            description="12 layers d=768, bf16 NS, sigma log-uniform grads + rank-4 spike, 10 steps",
        )
    if config_id == 2:
        return Workload(
            2, "gpt2_124m_body_normuon", _body(768, 12, "spike", cfc_lr_mul=2.0), steps=10, lr=0.03,
            normuon=1,
            description="124M body + NorMuon (beta2 0.95, eps 1e-10), lr 0.03, c_fc lr_mul 2",
        )
    if config_id == 3:
        return Workload(
            3, "body_1p5b_d1600", _body(1600, 48, "spike"), steps=5, lr=0.02,
            description="48 layers d=1600 (~1.5B-parameter body), bf16 NS, 5 steps",
        )
    if config_id == 4:
        return Workload(
            4, "stress_4096x64_256x256x1024", _stress(), steps=5, lr=0.02,
            description="4096 [64,64] + 256 [256,1024]: rank-8+1e-6 noise, Student-t(3), zero, frozen",
        )
    raise KeyError(config_id)


CONFIGS = {i: _make(i) for i in range(5)}


def get_workload(config_id: int) -> Workload:
    """A fresh copy of workload `config_id` (0..4)."""
    w = _make(config_id)
    return w


def custom_workload(
    config_id: int,
    shapes: Sequence[Tuple],
    steps: int = 3,
    **hp,
) -> Workload:
    """A workload from (rows, cols[, count[, gclass[, lr_mul[, frozen[, wd_mul]]]]]) tuples.

    Used for parity cases with ragged edges, degenerate shapes and mixed
    classes at sizes the oracle finishes in seconds.
    """
    entries = []
    off = 0
    for s in shapes:
        rows, cols = int(s[0]), int(s[1])
        count = int(s[2]) if len(s) > 2 else 1
        gclass = s[3] if len(s) > 3 else "spike"
        lr_mul = float(s[4]) if len(s) > 4 else 1.0
        frozen = int(s[5]) if len(s) > 5 else 0
        wd_mul = float(s[6]) if len(s) > 6 else 1.0
        entries.append(Entry(rows, cols, count, off, lr_mul=lr_mul, wd_mul=wd_mul, frozen=frozen,
                             name=f"m{len(entries)}", gclass=gclass))
        off += rows * cols * count
    return Workload(config_id, f"custom{config_id}", entries, steps=steps, **hp)


def with_hparams(w: Workload, **kw) -> Workload:
    return replace(w, **kw)
