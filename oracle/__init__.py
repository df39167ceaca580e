"""fp64 CPU oracle for the Mamba-3 SSM scan.  TEST INFRASTRUCTURE ONLY.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg.  Shares no code with the HIP library or its binding.
"""
from .mamba3_oracle import (  # noqa: F401
    zero_state, discretize, rot_pairs, prefill, decode_step,
    prefill_rotated_frame, prefill_complex, prefill_chunked,
    EXP_TRAPEZOID, DECAYED_TRAPEZOID, EXP_EULER, gated_rmsnorm, rank_down_projection,
    bc_rmsnorm,
)
from .mamba3_backward import prefill_backward, forward_torch  # noqa: F401
