"""Mamba-3 SSM scan (chunked prefill + recurrent decode) for MI355X (gfx950).

The computation lives in libmamba3.so (hand-written HIP kernels behind a C
ABI, include/mamba3.h); ``binding`` is its ctypes binding, with one Python
function per C entry point.  ``synthetic`` draws seeded inputs.
"""
from .binding import (  # noqa: F401
    M3Error, State, m3_dims, m3_state, m3_gate, m3_bcnorm, m3_grads, make_dims, lib, grad_shapes,
    m3_abi_version, m3_last_error, m3_state_bytes, m3_state_zero, m3_state_load,
    m3_state_readout, mamba3_prefill_workspace_bytes, mamba3_prefill, mamba3_decode_step,
    mamba3_prefill_gated, mamba3_decode_step_gated, mamba3_prefill_ex, mamba3_decode_step_ex,
    mamba3_prefill_backward_workspace_bytes, mamba3_prefill_backward, mamba3_prefill_noalloc,
)
