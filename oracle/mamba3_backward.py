"""Gradients of the Mamba-3 scan: plain, slow, fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY, like mamba3_oracle.py: only the tests, the package
smoke check and the benchmark's CPU-baseline leg may use it; it shares no
code with the HIP library or its binding.

What it computes: the exact gradients of the scan defined in
mamba3_oracle.py (lilting.ch Mamba-3 article, "アーキテクチャ改善" 1-3: the
exponential-trapezoid update, the rotating state, the rank-R coupling)
with respect to every input, for a scalar loss
    L = sum_t <dy_t, y_t> + <dh_final, h_T>
given the output cotangent dy and, optionally, that of the final state.
The pages train these layers (their models are trained end to end) but
print no backward pass; the plainest definition of one is the derivative
of the forward definition itself.  Here the forward definition is written
token by token with torch fp64 CPU tensors, and torch's reverse-mode
automatic differentiation (a library routine, used as one step) takes the
derivatives.  The forward written here is pinned to mamba3_oracle.prefill,
and the derivatives to central finite differences, by the tests.

The pending pair of the final state is a copy of the last token's (B, x),
so its cotangent adds to dB and dx of that token; callers fold it in.
"""
import numpy as np

from .mamba3_oracle import EXP_TRAPEZOID, DECAYED_TRAPEZOID, EXP_EULER


def _torch():
    import torch
    return torch


def _discretize_t(dt, lam, A, disc):
    """(alpha, beta, gamma) per token in torch, the same rules as the
    forward oracle's discretize (lilting.ch, "1. 指数台形離散化")."""
    torch = _torch()
    alpha = torch.exp(dt * A)
    if disc == EXP_TRAPEZOID:
        return alpha, (1.0 - lam) * dt, lam * dt
    if disc == DECAYED_TRAPEZOID:
        return alpha, alpha * (1.0 - lam) * dt, lam * dt
    if disc == EXP_EULER:
        return alpha, torch.zeros_like(dt), dt
    raise ValueError(f"unknown discretisation rule {disc}")


def _rot_pairs_t(v, ang):
    """Rotate adjacent pairs (2j, 2j+1) of the last axis by ang[..., j]."""
    torch = _torch()
    a, b = v[..., 0::2], v[..., 1::2]
    c, s = torch.cos(ang), torch.sin(ang)
    return torch.stack((a * c - b * s, a * s + b * c), dim=-1).flatten(-2)


def forward_torch(x, Bm, Cm, dt, lam, theta, A, D, h0, Bp0, xp0, disc=EXP_TRAPEZOID):
    """The definition in torch: y (batch, T, H, R, P) and h_T (batch, H, P, N)."""
    torch = _torch()
    h, Bp, xp = h0, Bp0, xp0
    ys = []
    for t in range(x.shape[1]):
        alpha, beta, gamma = _discretize_t(dt[:, t], lam[:, t], A[None, :], disc)
        G = alpha[..., None, None] * h + beta[..., None, None] * torch.einsum("bhrp,bhrn->bhpn", xp, Bp)
        h = _rot_pairs_t(G, theta[:, t][:, :, None, :])
        h = h + gamma[..., None, None] * torch.einsum("bhrp,bhrn->bhpn", x[:, t], Bm[:, t])
        ys.append(torch.einsum("bhpn,bhrn->bhrp", h, Cm[:, t]) + D[None, :, None, None] * x[:, t])
        Bp, xp = Bm[:, t], x[:, t]
    return torch.stack(ys, dim=1), h


def prefill_backward(x, Bm, Cm, dt, lam, theta, A, D, state, dy, dh_final=None, disc=EXP_TRAPEZOID):
    """Gradients of L = <dy, y> + <dh_final, h_T> for a prefill from `state`.

    Arrays as in mamba3_oracle.prefill; state = (h, B_prev, x_prev).
    Returns a dict of fp64 numpy arrays: dx, dB, dC (like x, B, C), ddt,
    dlam (batch, T, H), dtheta (batch, T, H, N/2), dA, dD (H,), dh0, dB_prev,
    dx_prev (like the state's parts).
    """
    torch = _torch()
    f = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    leaves = {"x": f(x), "B": f(Bm), "C": f(Cm), "dt": f(dt), "lam": f(lam), "theta": f(theta), "A": f(A),
              "D": f(D), "h0": f(state[0]), "Bp0": f(state[1]), "xp0": f(state[2])}
    L = leaves
    y, hT = forward_torch(L["x"], L["B"], L["C"], L["dt"], L["lam"], L["theta"], L["A"], L["D"], L["h0"], L["Bp0"],
                          L["xp0"], disc)
    loss = (y * torch.tensor(np.asarray(dy, dtype=np.float64))).sum()
    if dh_final is not None:
        loss = loss + (hT * torch.tensor(np.asarray(dh_final, dtype=np.float64))).sum()
    grads = torch.autograd.grad(loss, list(leaves.values()), allow_unused=True)
    names = {"x": "dx", "B": "dB", "C": "dC", "dt": "ddt", "lam": "dlam", "theta": "dtheta", "A": "dA", "D": "dD",
             "h0": "dh0", "Bp0": "dB_prev", "xp0": "dx_prev"}
    out = {}
    for (k, leaf), g in zip(leaves.items(), grads):
        out[names[k]] = np.zeros(leaf.shape) if g is None else g.detach().numpy()
    return out
