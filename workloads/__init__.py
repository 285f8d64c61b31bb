"""Workload definitions and the seeded synthetic input generator.

This package holds no arithmetic of the draft-and-verify step itself: it only
names shapes and draws random inputs.  Both the CPU oracle (``oracle/``) and the
HIP path read their inputs from here, so neither depends on the other.
"""

from .configs import WORKLOADS, Workload, get_workload, scaled  # noqa: F401
from .gen import make_inputs, step_qkv, uniforms, bf16_round_bits, f32_to_bf16_bits  # noqa: F401
