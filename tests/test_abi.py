"""C-ABI tests that run without a GPU.

The library must load, export every function that include/mamba3.h
declares, and reject every host-detectable problem with the documented
status before it makes any HIP call (so these tests never touch a device).
"""

import ctypes
import os
import re

import pytest

from state_space_sequence_prefill_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mamba3.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libmamba3.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:m3|mamba3)_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version():
    # version 2 added m3_dims.disc (the discretisation rule); version 3 the
    # gated entry points and m3_gate; version 4 m3_bcnorm and the _ex calls;
    # version 5 the backward pass and m3_grads; version 6 mamba3_prefill_noalloc
    assert B.m3_abi_version() == 6


def test_dims_struct_matches_header():
    """The binding's m3_dims mirrors the header field by field (eight int32)."""
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "mamba3.h")).read()
    body = re.search(r"typedef struct \{([^}]*)\} m3_dims;", hdr).group(1)
    names = re.findall(r"(\w+)\s*[,;]", body.replace("int32_t", ""))
    assert names == [f for f, _ in B.m3_dims._fields_]
    assert ctypes.sizeof(B.m3_dims) == 32


def dims(**kw):
    base = dict(batch=2, heads=3, headdim=64, dstate=64, rank=1, chunk=64, io_dtype="bf16")
    base.update(kw)
    return B.make_dims(**base)


FAKE = 0x10000  # a 16-byte aligned non-NULL address; never dereferenced on the host


def fake_state():
    return B.m3_state(FAKE, FAKE, FAKE)


def call_prefill(d, seqlen=16, ptrs=None, state=None, ws=None, wsb=0):
    p = [FAKE] * 9 if ptrs is None else ptrs
    st = fake_state() if state is None else state
    return B.lib().mamba3_prefill(ctypes.byref(d), seqlen, *p[:8], ctypes.byref(st), p[8], ws, wsb, None)


def call_decode(d, ptrs=None, state=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    st = fake_state() if state is None else state
    return B.lib().mamba3_decode_step(ctypes.byref(d), *p[:8], ctypes.byref(st), p[8], None)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, B.M3_ERR_SHAPE), ("heads", -1, B.M3_ERR_SHAPE), ("headdim", 0, B.M3_ERR_SHAPE),
    ("dstate", 0, B.M3_ERR_SHAPE), ("rank", 0, B.M3_ERR_SHAPE), ("chunk", 0, B.M3_ERR_SHAPE),
    ("io_dtype", 7, B.M3_ERR_DTYPE), ("dstate", 15, B.M3_ERR_UNSUPPORTED),
    ("dstate", 512, B.M3_ERR_UNSUPPORTED), ("dstate", 48, B.M3_ERR_UNSUPPORTED),
    ("headdim", 48, B.M3_ERR_UNSUPPORTED), ("headdim", 256, B.M3_ERR_UNSUPPORTED),
    ("rank", 9, B.M3_ERR_UNSUPPORTED),
    ("chunk", 128, B.M3_ERR_UNSUPPORTED), ("chunk", 24, B.M3_ERR_UNSUPPORTED),
    ("disc", 3, B.M3_ERR_UNSUPPORTED), ("disc", -1, B.M3_ERR_UNSUPPORTED),
])
def test_prefill_rejects_bad_dims(field, value, status):
    d = dims(**{field: value})
    assert call_prefill(d) == status
    assert B.m3_last_error()


def test_prefill_tile_height_and_lds_limit():
    # The chunk length is a tile height (the chunked form gives the same result
    # for any chunk): where chunk x rank rows do not fit 160 KiB of LDS the
    # library tiles with half or a quarter of the chunk, so fp32 I/O with N =
    # 128 at a 64-token chunk (32-token tiles) and rank 4 with N = 128 at a
    # 64-token chunk (16-token tiles) are accepted (seqlen 0: checks only) ...
    assert call_prefill(dims(io_dtype="f32", dstate=128, chunk=64), seqlen=0) == B.M3_OK
    assert call_prefill(dims(rank=4, chunk=64, dstate=128), seqlen=0) == B.M3_OK
    assert call_prefill(dims(io_dtype="f32", dstate=128, headdim=128, chunk=64), seqlen=0) == B.M3_OK
    # ... and shapes whose rows fit no tile height are refused
    assert call_prefill(dims(io_dtype="f32", dstate=128, headdim=128, rank=4, chunk=16)) == B.M3_ERR_UNSUPPORTED
    assert call_prefill(dims(io_dtype="f32", dstate=256, headdim=64, chunk=16)) == B.M3_ERR_UNSUPPORTED


def _prefill_support(io, P, N, R, Q):
    d = B.make_dims(1, 1, P, N, R, Q, io)
    nbytes = ctypes.c_size_t()
    return B.lib().mamba3_prefill_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(nbytes)) == B.M3_OK


# fp32 sizes the prefill refuses at every chunk (mamba3.h lists them with
# their LDS / register arithmetic): N = 256 except P = 16 with ranks 1, 2,
# and P = 128 with N = 128 at ranks 3 to 8
F32_REFUSED = sorted([(P, 256, R) for P in (16, 32, 64, 128) for R in range(1, 9) if not (P == 16 and R <= 2)]
                     + [(128, 128, R) for R in range(3, 9)])


def test_prefill_support_is_monotone_in_chunk():
    """The chunk is a tile height: every (dtype, P, N, R) accepted at chunk 16
    is accepted at 32 and 64; bf16 accepts every P in {16, 32, 64, 128}, N in
    {16, ..., 256} and R in 1..8, and fp32 all but the listed sizes."""
    for io in ("bf16", "f32"):
        refused = []
        for P in (16, 32, 64, 128):
            for N in (16, 32, 64, 128, 256):
                for R in range(1, 9):
                    ok = [_prefill_support(io, P, N, R, Q) for Q in (16, 32, 64)]
                    if ok[0]:
                        assert ok[1] and ok[2], (io, P, N, R, ok)
                    if not any(ok):
                        refused.append((P, N, R))
        assert sorted(refused) == ([] if io == "bf16" else F32_REFUSED), (io, refused)


def test_decode_checks_dims():
    assert call_decode(dims(dstate=15)) == B.M3_ERR_UNSUPPORTED
    assert call_decode(dims(dstate=48)) == B.M3_ERR_UNSUPPORTED
    assert call_decode(dims(dstate=512)) == B.M3_ERR_UNSUPPORTED
    assert call_decode(dims(rank=9)) == B.M3_ERR_UNSUPPORTED
    assert call_decode(dims(headdim=256)) == B.M3_ERR_UNSUPPORTED
    assert call_decode(dims(io_dtype=5)) == B.M3_ERR_DTYPE


def _decode_support(io, P, N, R):
    d = B.make_dims(1, 1, P, N, R, 64, io)
    hb = ctypes.c_size_t()
    return B.lib().m3_state_bytes(ctypes.byref(d), ctypes.byref(hb), None, None) == B.M3_OK


def test_decode_support_set():
    """Decode serves every headdim in {16, 32, 64, 128}, dstate in {16, ...,
    256} and rank 1 to 8, except headdim 128 with dstate 256 at ranks above 4
    (the matrix-core kernel's 133 KiB of state staging rows plus the rank
    operands exceed 160 KiB of LDS, and the VALU kernel serves ranks <= 4)."""
    for io in ("bf16", "f32"):
        refused = [(P, N, R) for P in (16, 32, 64, 128) for N in (16, 32, 64, 128, 256) for R in range(1, 9)
                   if not _decode_support(io, P, N, R)]
        assert refused == [(128, 256, R) for R in (5, 6, 7, 8)], (io, refused)


@pytest.mark.parametrize("i", range(9))
def test_prefill_rejects_null_pointer(i):
    p = [FAKE] * 9
    p[i] = None
    assert call_prefill(dims(), ptrs=p) == B.M3_ERR_NULL


@pytest.mark.parametrize("i", range(9))
def test_decode_rejects_null_pointer(i):
    p = [FAKE] * 9
    p[i] = None
    assert call_decode(dims(), ptrs=p) == B.M3_ERR_NULL


@pytest.mark.parametrize("i", range(9))
def test_prefill_rejects_misaligned_pointer(i):
    p = [FAKE] * 9
    p[i] = FAKE + 4
    assert call_prefill(dims(), ptrs=p) == B.M3_ERR_ALIGN


@pytest.mark.parametrize("which", ["h", "B_prev", "x_prev"])
def test_state_pointer_checks(which):
    st = fake_state()
    setattr(st, which, None)
    assert call_prefill(dims(), state=st) == B.M3_ERR_NULL
    assert call_decode(dims(), state=st) == B.M3_ERR_NULL
    st = fake_state()
    setattr(st, which, FAKE + 8)
    assert call_prefill(dims(), state=st) == B.M3_ERR_ALIGN


def test_null_state_and_dims():
    d = dims()
    p = [FAKE] * 9
    assert B.lib().mamba3_prefill(None, 4, *p[:8], ctypes.byref(fake_state()), p[8], None, 0, None) == B.M3_ERR_NULL
    assert B.lib().mamba3_prefill(ctypes.byref(d), 4, *p[:8], None, p[8], None, 0, None) == B.M3_ERR_NULL


def test_negative_seqlen():
    assert call_prefill(dims(), seqlen=-1) == B.M3_ERR_SHAPE


def test_zero_seqlen_is_a_noop_before_any_hip_call():
    # no kernel is launched for an empty prompt; input pointers may be NULL
    assert call_prefill(dims(), seqlen=0, ptrs=[None] * 9) == B.M3_OK


def test_state_bytes():
    d = dims(batch=8, heads=32, headdim=64, dstate=128, rank=1)
    assert B.m3_state_bytes(d) == (8 * 32 * 64 * 128 * 4, 8 * 32 * 128 * 2, 8 * 32 * 64 * 2)
    d = dims(batch=256, heads=32, headdim=64, dstate=64, rank=4, io_dtype="f32")
    assert B.m3_state_bytes(d) == (256 * 32 * 64 * 64 * 4, 256 * 32 * 4 * 64 * 4, 256 * 32 * 4 * 64 * 4)


def test_workspace_plan():
    # many chains: one fused pass, no workspace
    assert B.mamba3_prefill_workspace_bytes(dims(batch=8, heads=32, dstate=128), 4096) == 0
    # few long chains: segment summaries
    n = B.mamba3_prefill_workspace_bytes(dims(batch=1, heads=32, dstate=128), 16384)
    assert n >= 8 * 32 * 64 * 128 * 4
    # short prompt of few chains: not worth splitting
    assert B.mamba3_prefill_workspace_bytes(dims(batch=1, heads=2), 64 * 3) == 0
    assert B.mamba3_prefill_workspace_bytes(dims(batch=1, heads=2), 0) == 0


def test_short_workspace_is_rejected():
    d = dims(batch=1, heads=32, dstate=128)
    need = B.mamba3_prefill_workspace_bytes(d, 16384)
    assert call_prefill(d, seqlen=16384, ws=FAKE, wsb=need - 1) == B.M3_ERR_WORKSPACE
    assert call_prefill(d, seqlen=16384, ws=None, wsb=need) == B.M3_ERR_NULL
    assert call_prefill(d, seqlen=16384, ws=FAKE + 4, wsb=need) == B.M3_ERR_ALIGN


def test_state_ops_validate():
    d = dims()
    st = fake_state()
    assert B.lib().m3_state_zero(ctypes.byref(d), None, None) == B.M3_ERR_NULL
    assert B.lib().m3_state_load(ctypes.byref(d), ctypes.byref(st), None, FAKE, FAKE, None) == B.M3_ERR_NULL
    assert B.lib().m3_state_readout(ctypes.byref(d), ctypes.byref(st), FAKE, FAKE + 2, FAKE, None) == B.M3_ERR_ALIGN
    bad = dims(dstate=7)
    assert B.lib().m3_state_zero(ctypes.byref(bad), ctypes.byref(st), None) == B.M3_ERR_UNSUPPORTED


def test_last_error_is_cleared_by_success():
    call_prefill(dims(dstate=15))
    assert "odd" in B.m3_last_error()
    B.m3_state_bytes(dims())
    assert B.m3_last_error() == ""


# ---------------------------------------------------------------------------
# gated entry points (output epilogue)
# ---------------------------------------------------------------------------

def test_gate_struct_matches_header():
    hdr = open(HEADER).read()
    body = re.search(r"typedef struct \{([^}]*)\} m3_gate;", hdr).group(1)
    names = re.findall(r"(\w+)\s*;", body)
    assert names == [f for f, _ in B.m3_gate._fields_]
    assert ctypes.sizeof(B.m3_gate) == 32


def call_prefill_gated(d, gate, seqlen=16, ptrs=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    g = None if gate is None else ctypes.byref(gate)
    return B.lib().mamba3_prefill_gated(ctypes.byref(d), seqlen, *p[:8], g, ctypes.byref(fake_state()), p[8],
                                        None, 0, None)


def call_decode_gated(d, gate, ptrs=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    g = None if gate is None else ctypes.byref(gate)
    return B.lib().mamba3_decode_step_gated(ctypes.byref(d), *p[:8], g, ctypes.byref(fake_state()), p[8], None)


@pytest.mark.parametrize("call", [call_prefill_gated, call_decode_gated])
def test_gate_argument_checks(call):
    d = dims()
    assert call(d, None) == B.M3_ERR_NULL
    assert call(d, B.m3_gate(None, FAKE, 1e-5)) == B.M3_ERR_NULL
    assert call(d, B.m3_gate(FAKE, None, 1e-5)) == B.M3_ERR_NULL
    assert call(d, B.m3_gate(FAKE + 2, FAKE, 1e-5)) == B.M3_ERR_ALIGN
    assert call(d, B.m3_gate(FAKE, FAKE + 4, 1e-5)) == B.M3_ERR_ALIGN
    assert call(d, B.m3_gate(FAKE, FAKE, -1e-5)) == B.M3_ERR_SHAPE
    assert call(d, B.m3_gate(FAKE, FAKE, float("nan"))) == B.M3_ERR_SHAPE
    assert "eps" in B.m3_last_error()
    assert call(d, B.m3_gate(FAKE, FAKE, 1e-5, FAKE + 4)) == B.M3_ERR_ALIGN
    assert "down" in B.m3_last_error()
    # the other arguments are still checked
    p = [FAKE] * 9
    p[8] = None
    assert call(d, B.m3_gate(FAKE, FAKE, 0.0), ptrs=p) == B.M3_ERR_NULL


def test_gated_prefill_needs_the_producer_consumer_kernel():
    """fp32 with N = P = 128 and rank 2 has no producer/consumer tiling at any
    chunk height; the plain prefill serves it, the gated one refuses it."""
    d = dims(io_dtype="f32", dstate=128, headdim=128, rank=2, chunk=16)
    ok = B.m3_gate(FAKE, FAKE, 1e-5)
    assert call_prefill(d, seqlen=0) == B.M3_OK
    assert call_prefill_gated(d, ok, seqlen=0) == B.M3_ERR_UNSUPPORTED
    # every bf16 shape the headline families use is served
    for r, n, c in ((1, 128, 64), (2, 128, 64), (4, 64, 64), (4, 128, 32)):
        assert call_prefill_gated(dims(rank=r, dstate=n, chunk=c), ok, seqlen=0) == B.M3_OK


def test_gated_zero_seqlen_is_a_noop():
    assert call_prefill_gated(dims(), B.m3_gate(FAKE, FAKE, 0.0), seqlen=0, ptrs=[None] * 9) == B.M3_OK


# ---------------------------------------------------------------------------
# _ex entry points (BC normalisation + optional epilogue)
# ---------------------------------------------------------------------------

def test_bcnorm_struct_matches_header():
    hdr = open(HEADER).read()
    body = re.search(r"typedef struct \{([^}]*)\} m3_bcnorm;", hdr).group(1)
    names = re.findall(r"(\w+)\s*;", body)
    assert names == [f for f, _ in B.m3_bcnorm._fields_]
    assert ctypes.sizeof(B.m3_bcnorm) == 24


def call_prefill_ex(d, bc, gate=None, seqlen=16, ptrs=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return B.lib().mamba3_prefill_ex(ctypes.byref(d), seqlen, *p[:8], None if bc is None else ctypes.byref(bc),
                                     None if gate is None else ctypes.byref(gate), ctypes.byref(fake_state()), p[8],
                                     None, 0, None)


def call_decode_ex(d, bc, gate=None, ptrs=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return B.lib().mamba3_decode_step_ex(ctypes.byref(d), *p[:8], None if bc is None else ctypes.byref(bc),
                                         None if gate is None else ctypes.byref(gate), ctypes.byref(fake_state()),
                                         p[8], None)


@pytest.mark.parametrize("call", [call_prefill_ex, call_decode_ex])
def test_bcnorm_argument_checks(call):
    d = dims()
    assert call(d, B.m3_bcnorm(None, FAKE, 1e-6)) == B.M3_ERR_NULL
    assert call(d, B.m3_bcnorm(FAKE, None, 1e-6)) == B.M3_ERR_NULL
    assert call(d, B.m3_bcnorm(FAKE + 4, FAKE, 1e-6)) == B.M3_ERR_ALIGN
    assert call(d, B.m3_bcnorm(FAKE, FAKE + 8, 1e-6)) == B.M3_ERR_ALIGN
    assert call(d, B.m3_bcnorm(FAKE, FAKE, -1.0)) == B.M3_ERR_SHAPE
    assert call(d, B.m3_bcnorm(FAKE, FAKE, float("nan"))) == B.M3_ERR_SHAPE
    assert "bcnorm.eps" in B.m3_last_error()
    # the gate is still checked, and the other arguments
    assert call(d, B.m3_bcnorm(FAKE, FAKE, 0.0), B.m3_gate(None, FAKE, 0.0)) == B.M3_ERR_NULL
    p = [FAKE] * 9
    p[1] = None
    assert call(d, B.m3_bcnorm(FAKE, FAKE, 0.0), ptrs=p) == B.M3_ERR_NULL


def test_prefill_ex_without_options_is_the_plain_call():
    d = dims()
    assert call_prefill_ex(d, None, seqlen=0, ptrs=[None] * 9) == B.M3_OK
    assert call_prefill_ex(dims(dstate=15), None) == B.M3_ERR_UNSUPPORTED


def test_bcnorm_prefill_support():
    ok = B.m3_bcnorm(FAKE, FAKE, 1e-6)
    # served: every bf16 shape of the headline families, with and without a gate
    for r, n, c in ((1, 128, 64), (2, 128, 64), (4, 64, 64), (4, 128, 32)):
        assert call_prefill_ex(dims(rank=r, dstate=n, chunk=c), ok, seqlen=0) == B.M3_OK
        assert call_prefill_ex(dims(rank=r, dstate=n, chunk=c), ok, B.m3_gate(FAKE, FAKE, 0.0), seqlen=0) == B.M3_OK
    # bf16 N = 64, P = 16: the norm's partial sums do not fit beside the tiles
    assert call_prefill_ex(dims(dstate=64, headdim=16), ok, seqlen=0) == B.M3_ERR_UNSUPPORTED
    assert call_prefill_ex(dims(dstate=64, headdim=16), None, seqlen=0) == B.M3_OK
    # fp32 shapes that only the single-role kernel serves
    assert call_prefill_ex(dims(io_dtype="f32", dstate=128, headdim=128, rank=2, chunk=16), ok,
                           seqlen=0) == B.M3_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------

def test_grads_struct_matches_header():
    hdr = open(HEADER).read()
    body = re.search(r"typedef struct \{([^}]*)\} m3_grads;", hdr).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\*\s*(\w+)\s*;", body)
    assert names == [f for f, _ in B.m3_grads._fields_] == list(B.GRAD_FIELDS)
    assert ctypes.sizeof(B.m3_grads) == 11 * 8


def call_backward(d, seqlen=32, ptrs=None, grads=None, ws=FAKE, wsb=1 << 40, dh=None, state=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    g = B.m3_grads(*([FAKE] * 11)) if grads is None else grads
    st = fake_state() if state is None else state
    return B.lib().mamba3_prefill_backward(ctypes.byref(d), seqlen, *p[:8], ctypes.byref(st), p[8], dh,
                                           ctypes.byref(g), ws, wsb, None)


def test_backward_workspace_size():
    d = dims(batch=2, heads=3, headdim=64, dstate=128, rank=1)
    n = B.mamba3_prefill_backward_workspace_bytes(d, 100)
    # 2 units of 64 tokens: two P x N slots per unit and one per chain, then
    # e^{lE}, (cos, sin) of the end angle, two pairs of unit sums, the chain sums
    small = 256 + 6 * 2 * 64 * 2 * 4 + 256 + 256 + 256
    assert n == 6 * (2 * 2 + 1) * 64 * 128 * 4 + small
    d4 = dims(batch=1, heads=1, headdim=64, dstate=64, rank=4)   # one unit of 16 tokens
    assert B.mamba3_prefill_backward_workspace_bytes(d4, 9) == 3 * 64 * 64 * 4 + 5 * 256
    assert B.mamba3_prefill_backward_workspace_bytes(d, 0) == 0


def test_backward_argument_checks():
    d = dims()
    for i in range(11):
        g = [FAKE] * 11
        g[i] = None
        assert call_backward(d, grads=B.m3_grads(*g)) == B.M3_ERR_NULL
        g[i] = FAKE + 4
        assert call_backward(d, grads=B.m3_grads(*g)) == B.M3_ERR_ALIGN
    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert call_backward(d, ptrs=p) == B.M3_ERR_NULL
    assert call_backward(d, dh=FAKE + 4) == B.M3_ERR_ALIGN
    assert call_backward(d, wsb=16) == B.M3_ERR_WORKSPACE
    assert call_backward(d, ws=None) == B.M3_ERR_NULL
    assert call_backward(d, seqlen=0) == B.M3_ERR_SHAPE
    assert call_backward(d, seqlen=-3) == B.M3_ERR_SHAPE
    st = fake_state()
    st.h = None
    assert call_backward(d, state=st) == B.M3_ERR_NULL
    assert B.lib().mamba3_prefill_backward(ctypes.byref(d), 8, *([FAKE] * 8), None, FAKE, None,
                                           ctypes.byref(B.m3_grads(*([FAKE] * 11))), FAKE, 1 << 40,
                                           None) == B.M3_ERR_NULL


def test_backward_size_limit():
    assert call_backward(dims(headdim=128, dstate=128)) == B.M3_ERR_UNSUPPORTED
    assert "8192" in B.m3_last_error()
    # the matrix-core tiles are 16 wide
    assert call_backward(dims(headdim=24, dstate=64)) == B.M3_ERR_UNSUPPORTED
    assert call_backward(dims(headdim=64, dstate=40)) == B.M3_ERR_UNSUPPORTED
    assert call_backward(dims(headdim=64, dstate=64, rank=8)) == B.M3_ERR_UNSUPPORTED


def call_prefill_noalloc(d, seqlen=16, ptrs=None, state=None):
    p = [FAKE] * 9 if ptrs is None else ptrs
    st = fake_state() if state is None else state
    return B.lib().mamba3_prefill_noalloc(ctypes.byref(d), seqlen, *p[:8], ctypes.byref(st), p[8], None)


def test_noalloc_checks_like_prefill():
    """mamba3_prefill_noalloc validates exactly like mamba3_prefill (no
    workspace argument to check), before any HIP call."""
    assert call_prefill_noalloc(dims(rank=9)) == B.M3_ERR_UNSUPPORTED
    assert call_prefill_noalloc(dims(), seqlen=-1) == B.M3_ERR_SHAPE
    assert call_prefill_noalloc(dims(), seqlen=0) == B.M3_OK
    for i in range(9):
        p = [FAKE] * 9
        p[i] = None
        assert call_prefill_noalloc(dims(), ptrs=p) == B.M3_ERR_NULL
    p = [FAKE] * 9
    p[3] = FAKE + 4
    assert call_prefill_noalloc(dims(), ptrs=p) == B.M3_ERR_ALIGN


def test_noalloc_rejects_workspace_beyond_scratch():
    """Few long chains whose segment workspace exceeds the 16 MiB scratch are
    refused with M3_ERR_UNSUPPORTED before any HIP call; the message says why."""
    d = dims(batch=1, heads=64, headdim=128, dstate=128, rank=1, chunk=64)
    nbytes = ctypes.c_size_t()
    assert B.lib().mamba3_prefill_workspace_bytes(ctypes.byref(d), 1 << 16, ctypes.byref(nbytes)) == B.M3_OK
    assert nbytes.value > 16 << 20
    assert call_prefill_noalloc(d, seqlen=1 << 16) == B.M3_ERR_UNSUPPORTED
    assert "scratch" in B.m3_last_error()
