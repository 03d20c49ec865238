"""Seeded synthetic workloads for the Muon optimizer step.

This package holds the five workload definitions (matrix tables and
hyper-parameters) and the seeded input generators. It holds none of the
optimizer's arithmetic: it only lays out matrices and draws numbers. Both the
tests / bench (which drive the HIP library) and the CPU oracle consume what it
produces; neither side imports the other.
"""

from .configs import (  # noqa: F401
    CONFIGS,
    Entry,
    Workload,
    get_workload,
    custom_workload,
)
from .generators import (  # noqa: F401
    gen_grads,
    gen_params,
    gen_sigmas,
    gen_matrix_grad,
    gen_matrix_param,
)
