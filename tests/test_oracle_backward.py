"""Pins of the backward oracle (oracle/mamba3_backward.py), CPU only.

The gradients come from reverse-mode differentiation of a torch transcript
of the definition; they are pinned to things other than themselves: the
transcript's forward against the numpy definition (mamba3_oracle.prefill),
directional central finite differences of the numpy definition, and two
closed forms (dD and dC_t = h_t^T dy_t with h_t from the numpy recurrence).
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

DISCS = [oracle.EXP_TRAPEZOID, oracle.DECAYED_TRAPEZOID, oracle.EXP_EULER]


def relerr(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (n if n > 0 else 1.0))


def case(seed, b=1, T=5, H=2, R=2, P=3, N=4):
    rng = np.random.default_rng(seed)
    inp = dict(
        x=rng.standard_normal((b, T, H, R, P)),
        Bm=rng.standard_normal((b, T, H, R, N)),
        Cm=rng.standard_normal((b, T, H, R, N)),
        dt=np.log1p(np.exp(rng.normal(-1.0, 0.5, (b, T, H)))),
        lam=1.0 / (1.0 + np.exp(-rng.standard_normal((b, T, H)))),
        theta=rng.uniform(-2.0, 2.0, (b, T, H, N // 2)),
        A=-np.exp(rng.uniform(-1.0, 1.0, H)),
        D=rng.standard_normal(H),
    )
    state = (rng.standard_normal((b, H, P, N)), rng.standard_normal((b, H, R, N)), rng.standard_normal((b, H, R, P)))
    dy = rng.standard_normal((b, T, H, R, P))
    dh = rng.standard_normal((b, H, P, N))
    return inp, state, dy, dh


@pytest.mark.parametrize("disc", DISCS)
def test_torch_transcript_matches_numpy_definition(disc):
    inp, state, _, _ = case(1)
    y_ref, (h_ref, _, _) = oracle.prefill(**inp, state=state, disc=disc)
    t = {k: torch.tensor(v) for k, v in inp.items()}
    y, h = oracle.forward_torch(t["x"], t["Bm"], t["Cm"], t["dt"], t["lam"], t["theta"], t["A"], t["D"],
                                *(torch.tensor(s) for s in state), disc=disc)
    assert relerr(y.numpy(), y_ref) < 1e-14
    assert relerr(h.numpy(), h_ref) < 1e-14


def loss_numpy(inp, state, dy, dh, disc):
    y, (h, _, _) = oracle.prefill(**inp, state=state, disc=disc)
    return float(np.sum(y * dy) + np.sum(h * dh))


GRAD_OF = {"x": "dx", "Bm": "dB", "Cm": "dC", "dt": "ddt", "lam": "dlam", "theta": "dtheta", "A": "dA", "D": "dD"}
STATE_GRAD = ("dh0", "dB_prev", "dx_prev")


@pytest.mark.parametrize("disc", DISCS)
def test_gradients_match_central_differences(disc):
    """<grad, v> against (L(p + e v) - L(p - e v)) / 2e of the numpy
    definition, for a random direction v in every input and state part."""
    inp, state, dy, dh = case(2)
    g = oracle.prefill_backward(**inp, state=state, dy=dy, dh_final=dh, disc=disc)
    rng = np.random.default_rng(3)
    eps = 1e-6
    for name in list(GRAD_OF) + list(range(3)):
        if isinstance(name, str):
            v = rng.standard_normal(inp[name].shape)
            plus = dict(inp, **{name: inp[name] + eps * v})
            minus = dict(inp, **{name: inp[name] - eps * v})
            fd = (loss_numpy(plus, state, dy, dh, disc) - loss_numpy(minus, state, dy, dh, disc)) / (2 * eps)
            an = float(np.sum(g[GRAD_OF[name]] * v))
        else:
            v = rng.standard_normal(state[name].shape)
            sp = tuple(s + eps * v if i == name else s for i, s in enumerate(state))
            sm = tuple(s - eps * v if i == name else s for i, s in enumerate(state))
            fd = (loss_numpy(inp, sp, dy, dh, disc) - loss_numpy(inp, sm, dy, dh, disc)) / (2 * eps)
            an = float(np.sum(g[STATE_GRAD[name]] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_closed_forms_dD_and_dC():
    """dD_h = sum over tokens and ranks of <dy, x>; dC_t = h_t^T dy_t with
    h_t from the numpy recurrence (prefixes of the sequence)."""
    inp, state, dy, _ = case(4, T=4)
    g = oracle.prefill_backward(**inp, state=state, dy=dy)
    assert relerr(g["dD"], np.einsum("bthrp,bthrp->h", dy, inp["x"])) < 1e-13
    for t in range(inp["x"].shape[1]):
        pre = {k: (v[:, :t + 1] if v.ndim >= 3 else v) for k, v in inp.items()}
        _, (h_t, _, _) = oracle.prefill(**pre, state=state)
        assert relerr(g["dC"][:, t], np.einsum("bhpn,bhrp->bhrn", h_t, dy[:, t])) < 1e-12


def test_no_output_cotangent_no_gradient():
    inp, state, dy, _ = case(5)
    g = oracle.prefill_backward(**inp, state=state, dy=np.zeros_like(dy))
    assert all(np.all(v == 0) for v in g.values())
