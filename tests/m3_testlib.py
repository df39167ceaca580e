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


# Regression guard for bf16 I/O, separate from the 2e-2 bar: about twice the
# largest pooled error the kernels showed on the seeded workloads (3.3e-3),
# so a change that loses precision fails here long before it reaches the bar.
BF16_GUARD = 7e-3
# Per-token bound, as a multiple of the bar: ||e_t|| <= TOKEN_FACTOR * bar *
# max(||ref_t||, 0.1 * median_t ||ref_t||) for every token t of every chain.  A
# fault confined to some tokens (say the first of each chunk) fails it even
# when the pooled norm hides it.
TOKEN_FACTOR = 4.0


# State-reset inputs (a token with dt = 1000 / |A|) give that token's input
# weights ~1000x the others', and with bf16 I/O the carried state enters the
# output product rounded to bf16 relative to that size: tokens shortly after a
# reset whose output is a small difference of two large terms see up to ~0.13
# relative error, and the pooled error up to 7.3e-3.  For such inputs the
# regression guard is off and the per-token bound is SPREAD_TOKEN_FACTOR x the
# bar (the pooled and per-chain bars are unchanged).
SPREAD_TOKEN_FACTOR = 10.0


def small_rows(pre, eps):
    """Rows of an epilogue's input (..., rows, P) whose RMS is below a tenth of
    the median row's and below 3 sqrt(eps): the normalisation lifts such a
    row to full size, so the bf16 rounding of the terms that nearly cancelled
    in it (say gamma C.B against D at a sequence's first token) returns
    amplified.  Returned as a boolean array over the rows."""
    rms = np.sqrt(np.mean(np.asarray(pre, dtype=np.float64) ** 2, axis=-1))
    return (rms < 0.1 * np.median(rms)) & (rms < 3.0 * np.sqrt(eps))


def assert_parity(got, ref, io_dtype, label, chain_axis, token_axis=None, tol=None, guard=True, token_factor=None,
                  spread=False, exclude=None):
    """Compare a GPU result with the oracle's: the pooled relative L2 error,
    the error of every chain (index along chain_axis) and, with token_axis,
    every token's relative error (the floor keeps near-zero rows meaningful).
    `exclude` (boolean, broadcastable to the leading axes of got up to the
    token and chain axes) marks rows held only to the pooled bar (see
    small_rows).  Prints all three; returns the pooled error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite values"
    bar = tol_for(io_dtype) if tol is None else tol
    pooled_all = relerr(got, ref)
    nex = 0
    if exclude is not None and np.any(exclude):
        ex = np.asarray(exclude, dtype=bool)
        ex = ex.reshape(ex.shape + (1,) * (got.ndim - ex.ndim))
        nex = int(np.sum(exclude))
        assert pooled_all <= bar, f"{label}: pooled {pooled_all:.3e} with the {nex} small rows"
        got = np.where(ex, 0.0, got)
        ref = np.where(ex, 0.0, ref)
    pooled = relerr(got, ref)
    g = np.moveaxis(got, chain_axis, 0).reshape(got.shape[chain_axis], -1)
    r = np.moveaxis(ref, chain_axis, 0).reshape(ref.shape[chain_axis], -1)
    rn = np.linalg.norm(r, axis=1)
    per_chain = np.linalg.norm(g - r, axis=1) / np.where(rn > 0, rn, 1.0)
    msg = f"{label}: pooled {pooled:.3e}, worst chain {per_chain.max():.3e}"
    if nex:
        msg += f" ({nex} small rows held to the pooled bar only: pooled with them {pooled_all:.3e})"
    worst_tok = None
    if token_axis is not None:
        ax = [chain_axis, token_axis]
        gt = np.moveaxis(got, ax, [0, 1])
        rt = np.moveaxis(ref, ax, [0, 1])
        gt = gt.reshape(gt.shape[0], gt.shape[1], -1)
        rt = rt.reshape(rt.shape[0], rt.shape[1], -1)
        en = np.linalg.norm(gt - rt, axis=2)
        tn = np.linalg.norm(rt, axis=2)
        floor = 0.1 * np.median(tn, axis=1, keepdims=True)
        rel_tok = en / np.maximum(np.maximum(tn, floor), 1e-300)
        worst_tok = float(rel_tok.max())
        ci, ti = np.unravel_index(int(rel_tok.argmax()), rel_tok.shape)
        msg += f", worst token {worst_tok:.3e} (chain {ci}, token {ti})"
    print(msg, flush=True)
    assert pooled <= bar, msg
    assert per_chain.max() <= bar, msg
    if spread and io_dtype == "bf16":
        guard = False
        token_factor = SPREAD_TOKEN_FACTOR if token_factor is None else token_factor
    if worst_tok is not None:
        assert worst_tok <= (TOKEN_FACTOR if token_factor is None else token_factor) * bar, msg
    if guard and io_dtype == "bf16" and tol is None:
        assert pooled <= BF16_GUARD, msg
    return pooled


def to_gpu(arr, io_dtype, key):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if key in syn.IO_KEYS and io_dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: values are already bf16-representable
    return t.cuda().contiguous()


def inputs_on_gpu(w, seed, long_memory=False, seqlen=None, zero_D=False, dt_scale=1.0, a_scale=1.0,
                  resets=(), big_angles=0.0, degenerate=False):
    """Returns (exact fp64 dict, torch dict) for workload w.  dt_scale and
    a_scale stretch dt (and the dt-scaled angles) and A, e.g. for strong decay.
    resets: (token, log_decay) pairs; that token's dt is set so that dt * A
    equals log_decay in every chain (a state reset; its angle is left as
    drawn).  big_angles > 0 adds a one-signed angle of big_angles * U(1, 2)
    radians per (token, pair), so chunk-local angle sums run to thousands of
    radians.  degenerate: the method's boundary cases in one input: no
    rotation at all in the even heads (theta = 0), every 7th token without
    step (dt = 0: no decay and zero input weights), and the trapezoid weight
    at its ends (lam = 0 on every 5th token, lam = 1 on every 3rd)."""
    raw = syn.draw(w, seed, long_memory=long_memory, seqlen=seqlen)
    if degenerate:
        raw["theta"][:, :, 0::2, :] = 0.0
        raw["dt"][:, 0::7, :] = 0.0
        raw["lam"][:, 0::5, :] = 0.0
        raw["lam"][:, 0::3, :] = 1.0
    if zero_D:
        raw["D"] = np.zeros_like(raw["D"])
    if dt_scale != 1.0:
        raw["dt"] = raw["dt"] * dt_scale
        raw["theta"] = raw["theta"] * dt_scale
    if a_scale != 1.0:
        raw["A"] = raw["A"] * a_scale
    for t, ld in resets:
        raw["dt"][:, t, :] = ld / raw["A"][None, :]
    if big_angles:
        rng = np.random.default_rng(seed + 12345)
        raw["theta"] = raw["theta"] + big_angles * rng.uniform(1.0, 2.0, size=raw["theta"].shape)
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
