"""Seeded synthetic inputs for the Mamba-3 scan.

This module draws random numbers and nothing else: it holds none of the
scan's arithmetic, and both the GPU path's tests/benchmark and the CPU oracle
receive exactly the arrays it produces.

Workload shapes and distributions (per token-head unless noted):
    x, B, C  ~ N(0, 1)
    dt       = softplus(N(-2, 0.5))
    lam      = sigmoid(N(0, 1))
    theta    = U(-pi, pi) * dt          (per state pair; angle already scaled by dt)
    A        = -exp(U(-1, 1))           per head   ("long memory": -exp(U(-5, -3)))
    D        ~ N(0, 1)                  per head
Draw order with numpy's PCG64 generator: x, B, C, dt_raw, lam_raw, theta_raw,
A_raw, D.  The output gate (``draw_gate``, its own seed) draws z ~ N(0, 1)
(same layout as x, or without the rank axis when the ranks are folded) and
then the per-head channel weights ~ U(0.5, 1.5); the rank down-projection
(``draw_down``, its own seed) draws weights ~ U(-1, 1) per (head, rank,
channel); the BC normalisation (``draw_bcnorm``, its own seed) draws the
channel weights of B, then of C, ~ U(0.5, 1.5) per (head, state channel).  Values are drawn in float64 and then cast to the I/O dtype by
round-to-nearest-even; the exact cast values are what every consumer sees.

The named workloads mirror the pages' 1.5B-scale Mamba-3 layers (32 heads of
head dimension 64, state 128 SISO or 64 with rank-4 MIMO, 4K and 16K token
prompts, batched decode).
"""

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    headdim: int
    dstate: int
    rank: int
    seqlen: int
    chunk: int
    io_dtype: str  # "f32" or "bf16"

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny_siso_f32": Workload("tiny_siso_f32", 1, 1, 16, 16, 1, 64, 16, "f32"),
    "siso_1p5b_t4096": Workload("siso_1p5b_t4096", 8, 32, 64, 128, 1, 4096, 64, "bf16"),
    "mimo_r4_t4096": Workload("mimo_r4_t4096", 8, 32, 64, 64, 4, 4096, 64, "bf16"),
    "decode_mimo_r4_n64": Workload("decode_mimo_r4_n64", 256, 32, 64, 64, 4, 1, 64, "bf16"),
    "decode_siso_n128": Workload("decode_siso_n128", 256, 32, 64, 128, 1, 1, 64, "bf16"),
    "long_siso_t16384": Workload("long_siso_t16384", 1, 32, 64, 128, 1, 16384, 64, "bf16"),
}


def _softplus(v):
    return np.logaddexp(0.0, v)


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def draw(w: Workload, seed: int, long_memory: bool = False, seqlen=None):
    """Draw fp64 inputs for workload ``w``.

    Returns a dict of float64 numpy arrays with the library's layouts:
    x (b,T,H,R,P), B, C (b,T,H,R,N), dt, lam (b,T,H), theta (b,T,H,N/2),
    A, D (H,).  ``seqlen`` overrides w.seqlen.
    """
    T = w.seqlen if seqlen is None else seqlen
    b, H, R, P, N = w.batch, w.heads, w.rank, w.headdim, w.dstate
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, T, H, R, P))
    Bm = rng.standard_normal((b, T, H, R, N))
    Cm = rng.standard_normal((b, T, H, R, N))
    dt = _softplus(rng.normal(-2.0, 0.5, (b, T, H)))
    lam = _sigmoid(rng.standard_normal((b, T, H)))
    theta = rng.uniform(-np.pi, np.pi, (b, T, H, N // 2)) * dt[..., None]
    if long_memory:
        A = -np.exp(rng.uniform(-5.0, -3.0, H))
    else:
        A = -np.exp(rng.uniform(-1.0, 1.0, H))
    D = rng.standard_normal(H)
    return {"x": x, "B": Bm, "C": Cm, "dt": dt, "lam": lam, "theta": theta, "A": A, "D": D}


def draw_gate(w: Workload, seed: int, seqlen=None, decode: bool = False, folded: bool = False):
    """Gate input z (b,T,H,R,P), or (b,H,R,P) for a decode step (no R axis
    when ``folded``: the ranks are folded by the down-projection), and the
    per-head channel weights (H,P) of the output epilogue, fp64."""
    T = w.seqlen if seqlen is None else seqlen
    b, H, R, P = w.batch, w.heads, w.rank, w.headdim
    rng = np.random.default_rng(seed)
    lead = (b,) if decode else (b, T)
    z = rng.standard_normal(lead + ((H, P) if folded else (H, R, P)))
    weight = rng.uniform(0.5, 1.5, (H, P))
    return z, weight


def draw_bcnorm(w: Workload, seed: int):
    """BC-normalisation channel weights of B and of C, (H,N) each, fp64."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 1.5, (w.heads, w.dstate)), rng.uniform(0.5, 1.5, (w.heads, w.dstate))


def draw_down(w: Workload, seed: int):
    """Rank down-projection weights (H,R,P), fp64."""
    rng = np.random.default_rng(seed)
    return rng.uniform(-1.0, 1.0, (w.heads, w.rank, w.headdim))


def draw_gate_torch(w: Workload, seed: int, device="cuda", seqlen=None, folded: bool = False):
    """``draw_gate``'s distributions on the device (z in the I/O dtype,
    weights fp32), for timing runs; with ``folded`` also the down-projection
    weights (returned third)."""
    import torch

    T = w.seqlen if seqlen is None else seqlen
    b, H, R, P = w.batch, w.heads, w.rank, w.headdim
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    io = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    shape = (b, T, H, P) if folded else (b, T, H, R, P)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(io)
    weight = torch.rand((H, P), generator=g, device=device, dtype=torch.float32) + 0.5
    if not folded:
        return z, weight
    down = torch.rand((H, R, P), generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0
    return z, weight, down


def draw_state(w: Workload, seed: int, scale: float = 1.0):
    """A random non-zero state (h, B_prev, x_prev), all N(0, scale^2), fp64."""
    b, H, R, P, N = w.batch, w.heads, w.rank, w.headdim, w.dstate
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((b, H, P, N)),
            rng.standard_normal((b, H, R, N)),
            rng.standard_normal((b, H, R, P)))


def round_io(a: np.ndarray, io_dtype: str) -> np.ndarray:
    """Round fp64 values to the I/O dtype (round-to-nearest-even), back as fp64.

    The rounding is done bit-wise in numpy so that no GPU library is needed:
    bf16 keeps the top 16 bits of the fp32 pattern after adding the RNE bias.
    """
    f = np.asarray(a, dtype=np.float32)
    if io_dtype == "f32":
        return f.astype(np.float64)
    if io_dtype != "bf16":
        raise ValueError(io_dtype)
    u = f.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


IO_KEYS = ("x", "B", "C")
F32_KEYS = ("dt", "lam", "theta", "A", "D")


def as_exact(inputs: dict, io_dtype: str) -> dict:
    """Return the exact values the library sees: x, B, C rounded to the I/O
    dtype, dt/lam/theta/A/D rounded to fp32 (all as float64 arrays)."""
    out = {}
    for k, v in inputs.items():
        out[k] = round_io(v, io_dtype) if k in IO_KEYS else round_io(v, "f32")
    return out


def draw_torch(w: Workload, seed: int, device="cuda", seqlen=None, long_memory: bool = False):
    """Same distributions and layouts as ``draw``, drawn directly on the device
    with torch's generator (for timing runs, where the values do not matter
    but their distribution and size do).  x, B, C are cast to the I/O dtype
    (round-to-nearest-even); dt, lam, theta, A, D are fp32."""
    import torch

    T = w.seqlen if seqlen is None else seqlen
    b, H, R, P, N = w.batch, w.heads, w.rank, w.headdim, w.dstate
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    io = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    f32 = torch.float32

    def normal(shape, mean=0.0, std=1.0):
        return torch.randn(shape, generator=g, device=device, dtype=f32) * std + mean

    def uniform(shape, lo, hi):
        return torch.rand(shape, generator=g, device=device, dtype=f32) * (hi - lo) + lo

    x = normal((b, T, H, R, P)).to(io)
    Bm = normal((b, T, H, R, N)).to(io)
    Cm = normal((b, T, H, R, N)).to(io)
    dt = torch.nn.functional.softplus(normal((b, T, H), -2.0, 0.5))
    lam = torch.sigmoid(normal((b, T, H)))
    theta = uniform((b, T, H, N // 2), -torch.pi, torch.pi) * dt[..., None]
    A = -torch.exp(uniform((H,), -5.0, -3.0) if long_memory else uniform((H,), -1.0, 1.0))
    D = normal((H,))
    return {"x": x, "B": Bm, "C": Cm, "dt": dt.contiguous(), "lam": lam.contiguous(),
            "theta": theta.contiguous(), "A": A, "D": D}
