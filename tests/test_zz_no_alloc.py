"""mamba3_prefill_noalloc (the prefill for callers that cannot allocate: its
segment workspace lives in the library's own device scratch) against
mamba3_prefill with a caller workspace, through the C ABI: bit-identical
outputs and final states (the same kernels run on the same data), on two
calls in a row, the second with a smaller input, plus a fused-path size
that needs no workspace.  The oracle's 2e-2 bf16 bar is checked as well.
"""

import numpy as np
import pytest

import oracle
from state_space_sequence_prefill_amd import synthetic as syn

from m3_testlib import assert_parity, inputs_on_gpu, oracle_args, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import state_space_sequence_prefill_amd as m3  # noqa: E402


def W(**kw):
    return syn.WORKLOADS["tiny_siso_f32"].with_(**kw)


def run_both(w, seed):
    d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
    ex, tt = inputs_on_gpu(w, seed)
    T = w.seqlen
    outs = []
    for noalloc in (False, True):
        s = m3.State.empty(d)
        m3.m3_state_zero(d, s)
        y = torch.full((w.batch, T, w.heads, w.rank, w.headdim), float("nan"), dtype=tt["x"].dtype,
                       device="cuda")
        args = (d, T, tt["x"], tt["B"], tt["C"], tt["dt"], tt["lam"], tt["theta"], tt["A"], tt["D"], s, y)
        if noalloc:
            m3.mamba3_prefill_noalloc(*args)
        else:
            nws = m3.mamba3_prefill_workspace_bytes(d, T)
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
            m3.mamba3_prefill(*args, ws)
        torch.cuda.synchronize()
        outs.append((to_np(y), to_np(s.h), to_np(s.B_prev), to_np(s.x_prev)))
    return ex, outs


def check(w, seed):
    d = m3.make_dims(w.batch, w.heads, w.headdim, w.dstate, w.rank, w.chunk, w.io_dtype)
    need = m3.mamba3_prefill_workspace_bytes(d, w.seqlen)
    print(f"[noalloc {w.batch}x{w.heads} P{w.headdim} N{w.dstate} T{w.seqlen}] workspace {need} B", flush=True)
    ex, (ref, got) = run_both(w, seed)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    pairs = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    y_ref, _ = oracle.prefill(**oracle_args(ex, pairs))
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    assert_parity(np.moveaxis(got[0][bs, :, hs], 0, 1)[None], y_ref, w.io_dtype, "[noalloc] y", chain_axis=2,
                  token_axis=1)
    return need


def test_noalloc_matches_workspace_entry_point_twice():
    """Two calls in a row on the segment path, the second smaller (fewer
    chains, fewer tokens): the scratch keeps the first call's contents, which
    the second must not depend on."""
    big = W(batch=1, heads=4, headdim=64, dstate=128, rank=1, seqlen=64 * 48 + 5, chunk=64, io_dtype="bf16")
    small = W(batch=1, heads=2, headdim=32, dstate=64, rank=2, seqlen=32 * 30 + 3, chunk=32, io_dtype="bf16")
    assert check(big, 5100) > 0
    assert check(small, 5101) > 0


def test_noalloc_fused_path():
    """Many chains: one fused pass, no workspace, no scratch."""
    w = W(batch=2, heads=64, headdim=32, dstate=32, rank=1, seqlen=100, chunk=64, io_dtype="bf16")
    assert check(w, 5102) == 0
