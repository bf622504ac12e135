"""Seeded synthetic inputs shaped like the workloads of SAF3R's global attention.

This package is the only code shared by the CPU oracle and the HIP path.  It
draws random numbers and lays them out; it computes none of the method's
arithmetic (no key sets, no scores, no attention).
"""
from .gen import (  # noqa: F401
    ROLE_POSITION, ROLE_VERTICAL, ROLE_CORRESPONDENCE, ROLE_SCANNING, ROLE_DENSE,
    ROLE_CORR_STRIDE, ROLE_BROADCAST, ROLE_NAMES, Geometry, Workload, CONFIGS, config, make_inputs, make_layer,
    make_geometry_inputs, bf16_round, bf16_to_f32, sample_rows, make_front_loaded_dino,
    make_grouped_front_dino, layer_roles,
)
