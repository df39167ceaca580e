"""Pins for the fp64 oracle (CPU only).

The pages print no worked example and no code, so the oracle is pinned to
things other than itself: hand-worked tiny cases (tests/golden), a library
IIR filter (scipy.signal.lfilter) for constant coefficients, explicit
transition-matrix products built with scipy.linalg.expm, the textbook Mamba-2
(exponential Euler, SSD) quadratic form for lam = 1, a geometric-series closed
form, norm preservation of pure rotations, MIMO superposition, linearity and
state hand-off.  The last block plants plausible mistakes in the oracle and
checks that at least one pin catches each of them.
"""

import json
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.signal

import oracle
from oracle import mamba3_oracle as OM

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seed, b=2, T=19, H=2, R=1, P=3, N=4, state=True, A_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, T, H, R, P))
    Bm = rng.standard_normal((b, T, H, R, N))
    Cm = rng.standard_normal((b, T, H, R, N))
    dt = np.logaddexp(0.0, rng.normal(-1.0, 0.5, (b, T, H)))
    lam = 1.0 / (1.0 + np.exp(-rng.standard_normal((b, T, H))))
    th = rng.uniform(-np.pi, np.pi, (b, T, H, N // 2)) * dt[..., None]
    A = -A_scale * np.exp(rng.uniform(-1, 1, H))
    D = rng.standard_normal(H)
    st = None
    if state:
        st = (rng.standard_normal((b, H, P, N)), rng.standard_normal((b, H, R, N)),
              rng.standard_normal((b, H, R, P)))
    return dict(x=x, Bm=Bm, Cm=Cm, dt=dt, lam=lam, theta=th, A=A, D=D), st


def relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (n if n > 0 else 1.0)


# ---------------------------------------------------------------------------
# Pin functions (return an error; the tests and the mutation checks share them)
# ---------------------------------------------------------------------------

def pin_hand_worked():
    """Max abs error over the hand-worked golden cases."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    worst = 0.0
    for c in cases:
        x = np.array(c["x"])[None, :, None]          # (1,T,1,R,P)
        Bm = np.array(c["B"])[None, :, None]
        Cm = np.array(c["C"])[None, :, None]
        dt = np.array(c["dt"])[None, :, None]
        lam = np.array(c["lam"])[None, :, None]
        th = np.array(c["theta"])[None, :, None]
        A = np.array(c["A"])
        D = np.array(c["D"])
        st = (np.array(c["h0"])[None, None], np.array(c["B_prev0"])[None, None],
              np.array(c["x_prev0"])[None, None])
        y, (h, _, _) = oracle.prefill(x, Bm, Cm, dt, lam, th, A, D, st)
        worst = max(worst, np.abs(y[0, :, 0] - np.array(c["y"])).max(),
                    np.abs(h[0, 0] - np.array(c["h_final"])).max())
    return worst


def _coefs(disc, dt0, lam0, A0):
    """(alpha, beta, gamma) of each rule for constant parameters, written out
    from the rule's description (lilting.ch Mamba-3 article, "1. 指数台形離散化"
    and the table "Mamba-2とMamba-3の比較")."""
    alpha = np.exp(dt0 * A0)
    if disc == oracle.EXP_TRAPEZOID:      # both inputs weighted, neither decayed
        return alpha, (1 - lam0) * dt0, lam0 * dt0
    if disc == oracle.DECAYED_TRAPEZOID:  # previous input carried through the transition
        return alpha, alpha * (1 - lam0) * dt0, lam0 * dt0
    return alpha, 0.0, dt0                # exponential Euler: current input only


def pin_lfilter(lam_value=None, theta_zero=False, seed=7, disc=0):
    """Constant dt, lam, theta and A: each complex pair of each state row is a
    first-order complex IIR filter of the (time-varying) input u_t = b_t x_t:
        z_t = a z_{t-1} + gamma u_t + beta e^{i theta} u_{t-1},  a = alpha e^{i theta}
    evaluated with scipy.signal.lfilter.  Fresh state."""
    rng = np.random.default_rng(seed)
    T, P, N, R = 23, 3, 6, 2
    x = rng.standard_normal((1, T, 1, R, P))
    Bm = rng.standard_normal((1, T, 1, R, N))
    Cm = rng.standard_normal((1, T, 1, R, N))
    dt0 = 0.37
    lam0 = 0.3 if lam_value is None else lam_value
    th0 = np.zeros(N // 2) if theta_zero else rng.uniform(-np.pi, np.pi, N // 2) * dt0
    A = np.array([-0.8])
    D = np.array([0.6])
    dt = np.full((1, T, 1), dt0)
    lam = np.full((1, T, 1), lam0)
    th = np.broadcast_to(th0, (1, T, 1, N // 2)).copy()
    y, (h, _, _) = oracle.prefill(x, Bm, Cm, dt, lam, th, A, D, disc=disc)

    alpha, beta, gamma = _coefs(disc, dt0, lam0, A[0])
    b = Bm[0, :, 0, :, 0::2] + 1j * Bm[0, :, 0, :, 1::2]          # (T,R,N/2)
    c = Cm[0, :, 0, :, 0::2] + 1j * Cm[0, :, 0, :, 1::2]
    u = np.einsum("trp,trj->tpj", x[0, :, 0], b)                   # (T,P,N/2)
    z = np.zeros((T, P, N // 2), dtype=np.complex128)
    for j in range(N // 2):
        e = np.exp(1j * th0[j])
        for p in range(P):
            z[:, p, j] = scipy.signal.lfilter([gamma, beta * e], [1.0, -alpha * e], u[:, p, j])
    y_ref = np.real(np.einsum("trj,tpj->trp", np.conj(c), z)) + D[0] * x[0, :, 0]
    h_ref = np.empty((P, N))
    h_ref[:, 0::2] = z[-1].real
    h_ref[:, 1::2] = z[-1].imag
    return max(relerr(y[0, :, 0], y_ref), relerr(h[0, 0], h_ref))


def _rot_matrix(ang):
    """Block-diagonal N x N rotation, each 2x2 block = expm of the generator of
    multiplication by i on (re, im): [[0, -1], [1, 0]] * angle."""
    blocks = [scipy.linalg.expm(np.array([[0.0, -a], [a, 0.0]])) for a in ang]
    return scipy.linalg.block_diag(*blocks)


def pin_transition_bruteforce(seed=3):
    """Unrolled recurrence with explicit N x N transition matrices:
    h_t = F(t,0) h_0 + sum_{s=1..t} F(t,s) (beta_s R_s u_{s-1} + gamma_s u_s),
    F(t,s) = prod_{k=s+1..t} alpha_k R_k, u_0 = pending input."""
    pr, st = rand_problem(seed, b=1, T=6, H=1, R=2, P=2, N=4)
    y, (h, _, _) = oracle.prefill(**pr, state=st)
    T = 6
    x, Bm, Cm = pr["x"][0, :, 0], pr["Bm"][0, :, 0], pr["Cm"][0, :, 0]
    dt, lam, th = pr["dt"][0, :, 0], pr["lam"][0, :, 0], pr["theta"][0, :, 0]
    A, D = pr["A"][0], pr["D"][0]
    h0, Bp0, xp0 = st[0][0, 0], st[1][0, 0], st[2][0, 0]
    alpha = np.exp(dt * A)
    beta = (1 - lam) * dt
    gamma = lam * dt
    Rm = [_rot_matrix(th[t]) for t in range(T)]
    # u[s] for s = 0..T: u[0] is the pending input, u[s] = token s-1 (1-based step s)
    u = [xp0.T @ Bp0] + [x[t].T @ Bm[t] for t in range(T)]       # (P,N) each
    worst = 0.0
    for t in range(1, T + 1):
        def F(t_, s_):
            M = np.eye(4)
            for k in range(s_ + 1, t_ + 1):
                M = alpha[k - 1] * Rm[k - 1] @ M
            return M
        ht = (F(t, 0) @ h0.T).T
        for s in range(1, t + 1):
            v = beta[s - 1] * (Rm[s - 1] @ u[s - 1].T).T + gamma[s - 1] * u[s]
            ht = ht + (F(t, s) @ v.T).T
        yt = Cm[t - 1] @ ht.T + D * x[t - 1]                         # (R,P)
        worst = max(worst, relerr(y[0, t - 1, 0], yt))
        if t == T:
            worst = max(worst, relerr(h[0, 0], ht))
    return worst


def pin_mamba2_ssd(seed=11, disc=0):
    """lam = 1 and theta = 0: Mamba-2's exponential-Euler SSM (the pages'
    comparison table), whose output has the textbook structured-masked form
    y = (L o C B^T) x + D x,  L[t,s] = exp(sum_{k=s+1..t} dt_k A) dt_s, s <= t,
    for a fresh state.  The exponential-Euler rule gives that form for any lam."""
    pr, _ = rand_problem(seed, b=1, T=17, H=2, R=2, P=3, N=4, state=False)
    if disc != oracle.EXP_EULER:
        pr["lam"][:] = 1.0
    pr["theta"][:] = 0.0
    y, _ = oracle.prefill(**pr, disc=disc)
    worst = 0.0
    for hd in range(2):
        dt = pr["dt"][0, :, hd]
        a = dt * pr["A"][hd]
        cs = np.cumsum(a)
        T = len(dt)
        L = np.zeros((T, T))
        for t in range(T):
            for s in range(t + 1):
                L[t, s] = np.exp(cs[t] - cs[s]) * dt[s]
        Cm = pr["Cm"][0, :, hd]
        Bm = pr["Bm"][0, :, hd]
        x = pr["x"][0, :, hd]
        G = np.einsum("trn,sqn->trsq", Cm, Bm)
        y_ref = np.einsum("ts,trsq,sqp->trp", L, G, x) + pr["D"][hd] * x
        worst = max(worst, relerr(y[0, :, hd], y_ref))
    return worst


def pin_geometric_series(disc=0):
    """Constant dt, lam, B, x; theta = 0; fresh state.  u = x B^T:
    h_1 = gamma u;  h_t = alpha h_{t-1} + (beta + gamma) u, so
    h_t = alpha^{t-1} gamma u + (beta + gamma) u (1 - alpha^{t-1}) / (1 - alpha),
    where beta + gamma = dt for Mamba-3's rule and dt (lam + (1 - lam) alpha) for
    the decayed (textbook) trapezoid."""
    T, P, N = 9, 2, 2
    dt0, lam0, A0 = 0.5, 0.35, -0.9
    xv = np.array([1.5, -0.5])
    bv = np.array([0.25, 2.0])
    x = np.broadcast_to(xv, (1, T, 1, 1, P)).copy()
    Bm = np.broadcast_to(bv, (1, T, 1, 1, N)).copy()
    Cm = np.zeros((1, T, 1, 1, N))
    dt = np.full((1, T, 1), dt0)
    lam = np.full((1, T, 1), lam0)
    th = np.zeros((1, T, 1, 1))
    worst = 0.0
    alpha = np.exp(dt0 * A0)
    u = np.outer(xv, bv)
    for t in range(1, T + 1):
        _, (h, _, _) = oracle.prefill(x[:, :t], Bm[:, :t], Cm[:, :t], dt[:, :t], lam[:, :t],
                                      th[:, :t], np.array([A0]), np.array([0.0]), disc=disc)
        _, beta, gamma = _coefs(disc, dt0, lam0, A0)
        ref = alpha ** (t - 1) * gamma * u + (beta + gamma) * u * (1 - alpha ** (t - 1)) / (1 - alpha)
        worst = max(worst, relerr(h[0, 0], ref))
    return worst


def pin_pure_rotation(seed=5):
    """A = 0 (no decay), x = 0, zero pending: the state only rotates, so
    ||h_t||_F = ||h_0||_F and y_t[r] = RotPairs(h_0, Phi_t) . C_t[r] with
    Phi_t = sum_{k<=t} theta_k (closed form through complex exponentials)."""
    pr, st = rand_problem(seed, b=1, T=15, H=1, R=2, P=3, N=6)
    pr["A"][:] = 0.0
    pr["x"][:] = 0.0
    st = (st[0], np.zeros_like(st[1]), np.zeros_like(st[2]))
    y, _ = oracle.prefill(**pr, state=st)
    h0 = st[0][0, 0]
    z0 = h0[:, 0::2] + 1j * h0[:, 1::2]
    Phi = np.cumsum(pr["theta"][0, :, 0], axis=0)                     # (T,N/2)
    worst = 0.0
    for t in range(15):
        zt = z0 * np.exp(1j * Phi[t])[None, :]
        _, (h, _, _) = oracle.prefill(**{k: (v[:, :t + 1] if v.ndim > 1 else v) for k, v in pr.items()},
                                      state=st)
        worst = max(worst, abs(np.linalg.norm(h[0, 0]) - np.linalg.norm(h0)) / np.linalg.norm(h0))
        c = pr["Cm"][0, t, 0, :, 0::2] + 1j * pr["Cm"][0, t, 0, :, 1::2]
        yt = np.real(np.einsum("rj,pj->rp", np.conj(c), zt))
        worst = max(worst, relerr(y[0, t, 0], yt))
    return worst


ALL_PINS = {
    "hand_worked": (pin_hand_worked, 1e-12),
    "lfilter": (pin_lfilter, 1e-12),
    "lfilter_lam1": (lambda: pin_lfilter(lam_value=1.0), 1e-12),
    "lfilter_lam0_theta0": (lambda: pin_lfilter(lam_value=0.0, theta_zero=True), 1e-12),
    "transition_bruteforce": (pin_transition_bruteforce, 1e-12),
    "mamba2_ssd": (pin_mamba2_ssd, 1e-12),
    "geometric_series": (pin_geometric_series, 1e-12),
    "pure_rotation": (pin_pure_rotation, 1e-12),
    # the two other discretisation rules
    "lfilter_decayed_trapezoid": (lambda: pin_lfilter(disc=oracle.DECAYED_TRAPEZOID), 1e-12),
    "lfilter_exp_euler": (lambda: pin_lfilter(disc=oracle.EXP_EULER), 1e-12),
    "geometric_series_decayed_trapezoid": (lambda: pin_geometric_series(disc=oracle.DECAYED_TRAPEZOID), 1e-12),
    "mamba2_ssd_exp_euler_any_lam": (lambda: pin_mamba2_ssd(disc=oracle.EXP_EULER), 1e-12),
}


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name):
    fn, tol = ALL_PINS[name]
    assert fn() < tol


# ---------------------------------------------------------------------------
# Agreement of the formulations, chunked algebra, structure
# ---------------------------------------------------------------------------

DISCS = [0, 1, 2]  # EXP_TRAPEZOID, DECAYED_TRAPEZOID, EXP_EULER


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("R,P,N", [(1, 1, 2), (1, 4, 6), (3, 2, 4), (4, 3, 8)])
def test_formulations_agree(R, P, N, disc):
    pr, st = rand_problem(100 + R * 10 + N, b=2, T=21, H=2, R=R, P=P, N=N)
    y0, s0 = oracle.prefill(**pr, state=st, disc=disc)
    for f in (oracle.prefill_rotated_frame, oracle.prefill_complex):
        y1, s1 = f(**pr, state=st, disc=disc)
        assert relerr(y1, y0) < 1e-12
        for a, b in zip(s1, s0):
            assert relerr(a, b) < 1e-12


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("T", [1, 7, 37, 64])
@pytest.mark.parametrize("Q", [1, 5, 16, 64, 100])
def test_chunked_matches_sequential(T, Q, disc):
    pr, st = rand_problem(T * 7 + Q, b=1, T=T, H=2, R=2, P=3, N=4)
    y0, s0 = oracle.prefill(**pr, state=st, disc=disc)
    y1, s1 = oracle.prefill_chunked(**pr, state=st, chunk=Q, disc=disc)
    assert relerr(y1, y0) < 1e-11
    for a, b in zip(s1, s0):
        assert relerr(a, b) < 1e-11


def test_chunked_long_memory():
    """Weak decay (A ~ -exp(U(-5,-3))) so the carried state dominates."""
    pr, st = rand_problem(77, b=1, T=50, H=2, R=1, P=2, N=4, A_scale=np.exp(-4.0))
    y0, s0 = oracle.prefill(**pr, state=st)
    y1, s1 = oracle.prefill_chunked(**pr, state=st, chunk=16)
    assert relerr(y1, y0) < 1e-11
    assert relerr(s1[0], s0[0]) < 1e-11


def test_lambda_zero_is_shifted_euler():
    """lam = 0, theta = 0: h_t = alpha_t h_{t-1} + dt_t u_{t-1}, i.e. the lam = 1
    (Euler) recurrence driven by the inputs shifted one token later, with the
    pending pair as the first shifted-in token.  D = 0."""
    pr, st = rand_problem(21, b=1, T=12, H=2, R=2, P=3, N=4)
    pr["theta"][:] = 0.0
    pr["D"][:] = 0.0
    p0 = dict(pr)
    p0["lam"] = np.zeros_like(pr["lam"])
    y0, s0 = oracle.prefill(**p0, state=st)
    p1 = dict(pr)
    p1["lam"] = np.ones_like(pr["lam"])
    p1["x"] = np.concatenate([st[2][:, None], pr["x"][:, :-1]], axis=1)
    p1["Bm"] = np.concatenate([st[1][:, None], pr["Bm"][:, :-1]], axis=1)
    st1 = (st[0], np.zeros_like(st[1]), np.zeros_like(st[2]))
    y1, s1 = oracle.prefill(**p1, state=st1)
    assert relerr(y0, y1) < 1e-12
    assert relerr(s0[0], s1[0]) < 1e-12


def test_theta_zero_real_pairs_decouple():
    """theta = 0: the recurrence is real and every state column evolves on its
    own, so the output is the sum over columns of one-column (N = 2 with the
    partner column zeroed) runs, minus the skip term counted once per extra run."""
    pr, st = rand_problem(31, b=1, T=11, H=1, R=2, P=2, N=6)
    pr["theta"][:] = 0.0
    y, s = oracle.prefill(**pr, state=st)
    acc = np.zeros_like(y)
    hacc = np.zeros_like(s[0])
    for n in range(6):
        mask = np.zeros(6)
        mask[n] = 1.0
        p = dict(pr)
        p["Bm"] = pr["Bm"] * mask
        p["Cm"] = pr["Cm"] * mask
        stn = (st[0] * mask, st[1] * mask, st[2])
        yn, sn = oracle.prefill(**p, state=stn)
        acc += yn
        hacc += sn[0]
    acc -= 5 * pr["D"][None, None, :, None, None] * pr["x"]
    assert relerr(acc, y) < 1e-12
    assert relerr(hacc, s[0]) < 1e-12


def test_mimo_superposition():
    """MIMO rank R: the shared state is the sum of the states driven by each
    input rank, and each output rank reads it with its own C:
    y_r = sum_r' SISO(x_r', B_r', C_r) + D x_r."""
    pr, st = rand_problem(41, b=1, T=13, H=2, R=3, P=2, N=4)
    y, _ = oracle.prefill(**pr, state=None)
    for r in range(3):
        acc = pr["D"][None, None, :, None] * pr["x"][:, :, :, r]
        for rp in range(3):
            p = dict(pr)
            p["x"] = pr["x"][:, :, :, rp:rp + 1]
            p["Bm"] = pr["Bm"][:, :, :, rp:rp + 1]
            p["Cm"] = pr["Cm"][:, :, :, r:r + 1]
            p["D"] = np.zeros_like(pr["D"])
            ys, _ = oracle.prefill(**p)
            acc = acc + ys[:, :, :, 0]
        assert relerr(y[:, :, :, r], acc) < 1e-12


def test_rank_one_equals_siso_shapes():
    pr, st = rand_problem(43, b=2, T=9, H=2, R=1, P=4, N=4)
    y, s = oracle.prefill(**pr, state=st)
    assert y.shape == (2, 9, 2, 1, 4)
    assert s[0].shape == (2, 2, 4, 4) and s[1].shape == (2, 2, 1, 4) and s[2].shape == (2, 2, 1, 4)


def test_linearity():
    """Output and final state are linear in (x, h_0, x_prev) for fixed B, C, dt,
    lam, theta."""
    pr, st = rand_problem(51, b=1, T=10, H=2, R=2, P=2, N=4)
    pr2, st2 = rand_problem(52, b=1, T=10, H=2, R=2, P=2, N=4)
    a, c = 0.7, -1.3
    pmix = dict(pr)
    pmix["x"] = a * pr["x"] + c * pr2["x"]
    stmix = (a * st[0] + c * st2[0], st[1], a * st[2] + c * st2[2])
    p2 = dict(pr)
    p2["x"] = pr2["x"]
    st2b = (st2[0], st[1], st2[2])
    y1, s1 = oracle.prefill(**pr, state=st)
    y2, s2 = oracle.prefill(**p2, state=st2b)
    ym, sm = oracle.prefill(**pmix, state=stmix)
    assert relerr(ym, a * y1 + c * y2) < 1e-12
    assert relerr(sm[0], a * s1[0] + c * s2[0]) < 1e-12


def test_split_prefill_handoff():
    """prefill(T1) -> state -> prefill(T2) equals prefill(T1 + T2)."""
    pr, st = rand_problem(61, b=2, T=20, H=2, R=2, P=3, N=4)
    y, s = oracle.prefill(**pr, state=st)
    first = {k: (v[:, :7] if v.ndim > 1 else v) for k, v in pr.items()}
    second = {k: (v[:, 7:] if v.ndim > 1 else v) for k, v in pr.items()}
    ya, sa = oracle.prefill(**first, state=st)
    yb, sb = oracle.prefill(**second, state=sa)
    assert relerr(np.concatenate([ya, yb], axis=1), y) < 1e-12
    for u, v in zip(sb, s):
        assert relerr(u, v) < 1e-12


def test_prefill_then_decode_equals_longer_prefill():
    pr, st = rand_problem(71, b=2, T=12, H=2, R=2, P=3, N=4)
    y, s = oracle.prefill(**pr, state=st)
    first = {k: (v[:, :9] if v.ndim > 1 else v) for k, v in pr.items()}
    _, cur = oracle.prefill(**first, state=st)
    for t in range(9, 12):
        yt, cur = oracle.decode_step(pr["x"][:, t], pr["Bm"][:, t], pr["Cm"][:, t], pr["dt"][:, t],
                                     pr["lam"][:, t], pr["theta"][:, t], pr["A"], pr["D"], cur)
        assert relerr(yt, y[:, t]) < 1e-12
    for u, v in zip(cur, s):
        assert relerr(u, v) < 1e-12


def test_empty_sequence_is_noop():
    pr, st = rand_problem(81, b=1, T=0, H=2, R=1, P=2, N=4)
    for f in (oracle.prefill, oracle.prefill_rotated_frame, oracle.prefill_complex,
              lambda **k: oracle.prefill_chunked(**k, chunk=16)):
        y, s = f(**pr, state=st)
        assert y.shape[1] == 0
        for u, v in zip(s, st):
            assert np.array_equal(u, v)


def test_textbook_trapezoid_reading_differs():
    """The decayed-endpoint trapezoid (previous input also multiplied by alpha)
    is a different method: at constant inputs its increments are
    dt (lam + (1 - lam) alpha) u instead of dt u.  The geometric-series pin
    separates the two readings."""
    alpha, lam0, dt0 = np.exp(-0.45), 0.35, 0.5
    assert abs(dt0 * (lam0 + (1 - lam0) * alpha) - dt0) > 1e-3


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------

def _bad_rot_sign(v, ang):
    return OM.__dict__["_orig_rot"](v, -np.asarray(ang))


def _bad_rot_halves(v, ang):
    """Pairs (j, j + N/2) instead of adjacent (2j, 2j+1)."""
    n = v.shape[-1] // 2
    a, b = v[..., :n], v[..., n:]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty(np.broadcast_shapes(v.shape), dtype=np.float64)
    out[..., :n] = c * a - s * b
    out[..., n:] = s * a + c * b
    return out


def _bad_disc_decayed(dt, lam, A, disc=0):
    a, b, g = OM.__dict__["_orig_disc"](dt, lam, A, disc)
    return a, b * a, g


def _bad_disc_swapped(dt, lam, A, disc=0):
    a, b, g = OM.__dict__["_orig_disc"](dt, lam, A, disc)
    return a, g, b


def _bad_step_unrotated_pending(h, Bp, xp, x_t, B_t, C_t, dt_t, lam_t, th_t, A, D, disc=0):
    alpha, beta, gamma = OM.discretize(dt_t, lam_t, A, disc)
    h = OM.rot_pairs(alpha[..., None, None] * h, th_t[:, :, None, :])
    h = h + beta[..., None, None] * OM._outer_sum(xp, Bp) + gamma[..., None, None] * OM._outer_sum(x_t, B_t)
    y = np.einsum("bhpn,bhrn->bhrp", h, C_t) + D[None, :, None, None] * x_t
    return h, y


def _bad_step_no_skip(h, Bp, xp, x_t, B_t, C_t, dt_t, lam_t, th_t, A, D, disc=0):
    return OM.__dict__["_orig_step"](h, Bp, xp, x_t, B_t, C_t, dt_t, lam_t, th_t, A, 0.0 * D, disc)


def _bad_step_transposed_readout(h, Bp, xp, x_t, B_t, C_t, dt_t, lam_t, th_t, A, D, disc=0):
    alpha, beta, gamma = OM.discretize(dt_t, lam_t, A, disc)
    G = alpha[..., None, None] * h + beta[..., None, None] * OM._outer_sum(xp, Bp)
    h = OM.rot_pairs(G, th_t[:, :, None, :]) + gamma[..., None, None] * OM._outer_sum(x_t, B_t)
    Crot = OM.rot_pairs(C_t, th_t[:, :, None, :])      # reads C in the wrong frame
    y = np.einsum("bhpn,bhrn->bhrp", h, Crot) + D[None, :, None, None] * x_t
    return h, y


def _bad_disc_ignored(dt, lam, A, disc=0):
    return OM.__dict__["_orig_disc"](dt, lam, A)


MUTANTS = {
    "discretisation_rule_ignored": ("discretize", _bad_disc_ignored),
    "rotation_sign": ("rot_pairs", _bad_rot_sign),
    "rotation_pairing": ("rot_pairs", _bad_rot_halves),
    "decayed_previous_input": ("discretize", _bad_disc_decayed),
    "lambda_swapped": ("discretize", _bad_disc_swapped),
    "pending_not_rotated": ("_step", _bad_step_unrotated_pending),
    "skip_term_dropped": ("_step", _bad_step_no_skip),
    "readout_wrong_frame": ("_step", _bad_step_transposed_readout),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    attr, bad = MUTANTS[mutant]
    monkeypatch.setitem(OM.__dict__, "_orig_rot", OM.rot_pairs)
    monkeypatch.setitem(OM.__dict__, "_orig_disc", OM.discretize)
    monkeypatch.setitem(OM.__dict__, "_orig_step", OM._step)
    monkeypatch.setattr(OM, attr, bad)
    caught = [name for name, (fn, tol) in ALL_PINS.items() if not fn() < tol]
    assert caught, f"planted mistake {mutant!r} passed every pin"


# ---------------------------------------------------------------------------
# Output epilogue: pre-gate grouped RMSNorm
# ---------------------------------------------------------------------------

def test_gated_rmsnorm_worked_example():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "gated_rmsnorm_worked.json")))
    y = np.array(g["y"])[None, None, :]           # (H=1, R=1, P=2)
    z = np.array(g["z"])[None, None, :]
    w = np.array(g["weight"])[None, :]
    out = oracle.gated_rmsnorm(y, z, w, g["eps"])
    assert np.max(np.abs(out[0, 0] - np.array(g["out"]))) < g["tolerance"]


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.3])
def test_gated_rmsnorm_matches_torch(eps):
    """torch's rms_norm and silu (an independent implementation) on random rows."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    b, T, H, R, P = 2, 3, 4, 2, 16
    y = rng.standard_normal((b, T, H, R, P))
    z = rng.standard_normal((b, T, H, R, P)) * 3
    w = rng.standard_normal((H, P))
    out = oracle.gated_rmsnorm(y, z, w, eps)
    ty, tz, tw = (torch.from_numpy(a) for a in (y, z, w))
    ref = torch.stack([torch.nn.functional.rms_norm(ty[:, :, h], (P,), weight=tw[h], eps=eps)
                       for h in range(H)], dim=2) * torch.nn.functional.silu(tz)
    assert relerr(out, ref.numpy()) < 1e-13


def test_gated_rmsnorm_scale_invariant():
    """With eps = 0 the output does not change when a row of y is scaled."""
    rng = np.random.default_rng(6)
    y = rng.standard_normal((5, 3, 2, 8))
    z = rng.standard_normal((5, 3, 2, 8))
    w = rng.standard_normal((3, 8))
    c = rng.uniform(0.1, 10.0, (5, 3, 2, 1))
    assert relerr(oracle.gated_rmsnorm(c * y, z, w, 0.0), oracle.gated_rmsnorm(y, z, w, 0.0)) < 1e-13


def _bad_gate_post(y, z, weight, eps):
    """Gate applied before the norm (post-gate RMSNorm)."""
    z = np.asarray(z, dtype=np.float64)
    g = np.asarray(y, dtype=np.float64) * z / (1 + np.exp(-z))
    return np.asarray(weight)[:, None, :] * g / np.sqrt(np.mean(g * g, axis=-1, keepdims=True) + eps)


def _bad_gate_axis(y, z, weight, eps):
    """Normalised over the ranks instead of the channels of a row."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    ms = np.mean(y * y, axis=-2, keepdims=True)
    return np.asarray(weight)[:, None, :] * y / np.sqrt(ms + eps) * z / (1 + np.exp(-z))


@pytest.mark.parametrize("bad", [_bad_gate_post, _bad_gate_axis])
def test_gated_rmsnorm_pins_catch_planted_mistake(bad, monkeypatch):
    monkeypatch.setattr(oracle, "gated_rmsnorm", bad)
    caught = 0
    for fn in (test_gated_rmsnorm_worked_example, lambda: test_gated_rmsnorm_matches_torch(1e-5)):
        try:
            fn()
        except AssertionError:
            caught += 1
    assert caught > 0


# ---------------------------------------------------------------------------
# MIMO rank down-projection (read-out of the R rank outputs to P channels)
# ---------------------------------------------------------------------------

def _down_example():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rank_down_worked.json")))
    return g, np.array(g["y"])[None, :, :], np.array(g["down"])[None, :, :]   # (H=1, R=2, P=2)


def test_rank_down_worked_example():
    g, y, down = _down_example()
    s = oracle.rank_down_projection(y, down)
    assert np.max(np.abs(s[0] - np.array(g["s"]))) < g["tolerance"]
    out = oracle.gated_rmsnorm(s[:, None, :], np.array(g["z"])[None, None, :], np.array(g["weight"])[None, :],
                               g["eps"])
    assert np.max(np.abs(out[0, 0] - np.array(g["out"]))) < g["tolerance"]


def test_rank_down_special_cases():
    """One-hot weights pick one rank; unit weights sum the ranks (numpy's sum)."""
    rng = np.random.default_rng(21)
    b, T, H, R, P = 2, 3, 3, 4, 8
    y = rng.standard_normal((b, T, H, R, P))
    for r0 in range(R):
        onehot = np.zeros((H, R, P))
        onehot[:, r0, :] = 1.0
        assert np.array_equal(oracle.rank_down_projection(y, onehot), y[..., r0, :])
    assert relerr(oracle.rank_down_projection(y, np.ones((H, R, P))), np.sum(y, axis=-2)) < 1e-15


def test_rank_down_matches_torch_einsum():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(22)
    y = rng.standard_normal((2, 5, 3, 4, 16))
    down = rng.standard_normal((3, 4, 16))
    ref = torch.einsum("bthrp,hrp->bthp", torch.from_numpy(y), torch.from_numpy(down)).numpy()
    assert relerr(oracle.rank_down_projection(y, down), ref) < 1e-14


def _bad_down_transposed(y, down):
    """Weights indexed [h, p, r] (only defined when R == P)."""
    down = np.asarray(down, dtype=np.float64)
    return np.sum(np.swapaxes(down, -1, -2)[None] * np.asarray(y, dtype=np.float64), axis=-2)


def _bad_down_rank_shift(y, down):
    """Rank r weighted by rank r+1's weights."""
    down = np.roll(np.asarray(down, dtype=np.float64), 1, axis=1)
    return np.sum(down * np.asarray(y, dtype=np.float64), axis=-2)


@pytest.mark.parametrize("bad", [_bad_down_transposed, _bad_down_rank_shift])
def test_rank_down_pins_catch_planted_mistake(bad, monkeypatch):
    monkeypatch.setattr(oracle, "rank_down_projection", bad)
    with pytest.raises(AssertionError):
        test_rank_down_worked_example()


# ---------------------------------------------------------------------------
# BC normalisation (RMSNorm of B and C rows before the scan)
# ---------------------------------------------------------------------------

def test_bc_rmsnorm_worked_example():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "bc_rmsnorm_worked.json")))
    v = np.array(g["v"])[None, None, :]      # (H=1, R=1, N=4)
    w = np.array(g["weight"])[None, :]
    for case in g["cases"]:
        out = oracle.bc_rmsnorm(v, w, case["eps"])
        assert np.max(np.abs(out[0, 0] - np.array(case["out"]))) < case["tolerance"]


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_bc_rmsnorm_matches_torch(eps):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(31)
    b, T, H, R, N = 2, 3, 4, 2, 32
    v = rng.standard_normal((b, T, H, R, N)) * 2.5
    w = rng.standard_normal((H, N))
    out = oracle.bc_rmsnorm(v, w, eps)
    tv, tw = torch.from_numpy(v), torch.from_numpy(w)
    ref = torch.stack([torch.nn.functional.rms_norm(tv[:, :, h], (N,), weight=tw[h], eps=eps) for h in range(H)],
                      dim=2)
    assert relerr(out, ref.numpy()) < 1e-13


def test_bc_rmsnorm_unit_rows_and_weights_are_identity():
    """Rows that already have unit RMS, unit weights and eps = 0: the prefill
    with normalised B and C equals the plain prefill."""
    rng = np.random.default_rng(32)
    b, T, H, R, P, N = 1, 9, 2, 2, 4, 6
    Bm = rng.standard_normal((b, T, H, R, N))
    Cm = rng.standard_normal((b, T, H, R, N))
    Bm /= np.sqrt(np.mean(Bm * Bm, axis=-1, keepdims=True))
    Cm /= np.sqrt(np.mean(Cm * Cm, axis=-1, keepdims=True))
    ones = np.ones((H, N))
    assert relerr(oracle.bc_rmsnorm(Bm, ones, 0.0), Bm) < 1e-15
    assert relerr(oracle.bc_rmsnorm(Cm, ones, 0.0), Cm) < 1e-15


def test_bc_rmsnorm_scale_invariant():
    rng = np.random.default_rng(33)
    v = rng.standard_normal((5, 3, 2, 16))
    w = rng.standard_normal((3, 16))
    c = rng.uniform(0.01, 100.0, (5, 3, 2, 1))
    assert relerr(oracle.bc_rmsnorm(c * v, w, 0.0), oracle.bc_rmsnorm(v, w, 0.0)) < 1e-13


def _bad_bc_axis(v, weight, eps):
    """Normalised over the ranks instead of the state channels."""
    v = np.asarray(v, dtype=np.float64)
    return np.asarray(weight)[:, None, :] * v / np.sqrt(np.mean(v * v, axis=-2, keepdims=True) + eps)


def _bad_bc_eps_outside(v, weight, eps):
    """eps added to the root instead of the mean square."""
    v = np.asarray(v, dtype=np.float64)
    return np.asarray(weight)[:, None, :] * v / (np.sqrt(np.mean(v * v, axis=-1, keepdims=True)) + eps)


@pytest.mark.parametrize("bad", [_bad_bc_axis, _bad_bc_eps_outside])
def test_bc_rmsnorm_pins_catch_planted_mistake(bad, monkeypatch):
    monkeypatch.setattr(oracle, "bc_rmsnorm", bad)
    caught = 0
    for fn in (test_bc_rmsnorm_worked_example, lambda: test_bc_rmsnorm_matches_torch(0.5)):
        try:
            fn()
        except AssertionError:
            caught += 1
    assert caught > 0
