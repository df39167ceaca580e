"""Shared helpers for the GPU parity tests: seeded inputs -> torch tensors on
the GPU and the matching exact fp64 arrays for the oracle."""

import numpy as np

from state_space_sequence_prefill_amd import synthetic as syn


def relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


def tol_for(io_dtype):
    """Relative L2 bounds: 2e-2 for bf16 I/O, 1e-5 for fp32 I/O."""
    return 2e-2 if io_dtype == "bf16" else 1e-5


def to_gpu(arr, io_dtype, key):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if key in syn.IO_KEYS and io_dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: values are already bf16-representable
    return t.cuda().contiguous()


def inputs_on_gpu(w, seed, long_memory=False, seqlen=None, zero_D=False, dt_scale=1.0, a_scale=1.0):
    """Returns (exact fp64 dict, torch dict) for workload w.  dt_scale and
    a_scale stretch dt (and the dt-scaled angles) and A, e.g. for strong decay."""
    raw = syn.draw(w, seed, long_memory=long_memory, seqlen=seqlen)
    if zero_D:
        raw["D"] = np.zeros_like(raw["D"])
    if dt_scale != 1.0:
        raw["dt"] = raw["dt"] * dt_scale
        raw["theta"] = raw["theta"] * dt_scale
    if a_scale != 1.0:
        raw["A"] = raw["A"] * a_scale
    ex = syn.as_exact(raw, w.io_dtype)
    tt = {k: to_gpu(v, w.io_dtype, k) for k, v in ex.items()}
    return ex, tt


def state_to_gpu(st, io_dtype):
    h, Bp, xp = st
    return (to_gpu(syn.round_io(h, "f32"), "f32", "h"),
            to_gpu(syn.round_io(Bp, io_dtype), io_dtype, "B"),
            to_gpu(syn.round_io(xp, io_dtype), io_dtype, "x"))


def exact_state(st, io_dtype):
    h, Bp, xp = st
    return (syn.round_io(h, "f32"), syn.round_io(Bp, io_dtype), syn.round_io(xp, io_dtype))


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def oracle_args(ex, pairs):
    """Slice the exact inputs down to the (b, h) chains in `pairs`, stacked on
    the head axis (batch = 1), for the oracle."""
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    return dict(
        x=np.moveaxis(ex["x"][bs, :, hs], 0, 1)[None],
        Bm=np.moveaxis(ex["B"][bs, :, hs], 0, 1)[None],
        Cm=np.moveaxis(ex["C"][bs, :, hs], 0, 1)[None],
        dt=ex["dt"][bs, :, hs].T[None],
        lam=ex["lam"][bs, :, hs].T[None],
        theta=np.moveaxis(ex["theta"][bs, :, hs], 0, 1)[None],
        A=ex["A"][hs],
        D=ex["D"][hs],
    )


def state_slice(st, pairs):
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    return tuple(s[bs, hs][None] for s in st)
