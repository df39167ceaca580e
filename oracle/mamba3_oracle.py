"""Mamba-3 SSM layer scan: plain, slow, fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library and its
Python binding never import, call or link it, and this module imports nothing
from them: the two share no code, constants or helpers.

Sources (web pages on Mamba-3; none prints an equation, so the update below is
the library's stated definition, and each ingredient is tied to the passage
that describes it):

* lilting.ch, "Together AIがMamba-3を発表、長文推論でTransformer比約7倍の速度と
  複素数値SSM", section "アーキテクチャ改善":
  - "1. 指数台形離散化" and its table of discretisation methods: Mamba-3's
    discretisation is second order and mixes the current input with the
    previous one, where Mamba-2's exponential-Euler rule is first order.
  - "2. 複素数値状態" and its state-type table: N real state dimensions
    are N/2 complex ones; the complex transition is realised as block-diagonal
    2x2 rotations applied to real vectors (the "RoPE trick").
  - "3. MIMO SSM": rank-r coupling of input and output channels.
  - table "Mamba-2とMamba-3の比較": exponential Euler (Mamba-2) vs
    exponential trapezoid (Mamba-3).
* perforder.com, "Mamba-3解剖：複素数SSMとMIMOが拓く線形モデルの極北", section on
  complex-valued updates and RoPE-like rotation.

Definition (per batch row b and head h, independently).  State: h (P x N,
real), pending B_prev (R x N) and x_prev (R x P).  For every token t:

    alpha = exp(dt_t * A_h)
    beta  = (1 - lam_t) * dt_t
    gamma = lam_t * dt_t
    G     = alpha * h + beta * sum_r outer(x_prev[r], B_prev[r])
    h     = RotPairs(G, theta_t) + gamma * sum_r outer(x_t[r], B_t[r])
    y_t[r] = h @ C_t[r] + D_h * x_t[r]
    (B_prev, x_prev) = (B_t, x_t)

RotPairs rotates each adjacent pair of state columns (2j, 2j+1) by the angle
theta_t[j]: (a, b) -> (a cos - b sin, a sin + b cos), i.e. multiplication of
the complex number a + i b by exp(i theta).  theta is the per-token angle
(already scaled by dt), shared by all P rows and all R ranks.  A fresh
sequence starts from h = 0 and a zero pending pair.

Readings adopted where the pages are silent (all listed in the design notes):
the previous-input term is rotated but not decayed; the state is exported in
the lab frame; pairs are adjacent columns with index 2j the real part; dt,
lam, theta, A, D are shared by the R ranks.

Layouts (numpy float64 arrays, any values; inputs are used exactly as given):
    x     (batch, T, H, R, P)
    Bm,Cm (batch, T, H, R, N)
    dt, lam (batch, T, H)
    theta (batch, T, H, N/2)
    A, D  (H,)
    state: (h (batch, H, P, N), B_prev (batch, H, R, N), x_prev (batch, H, R, P))

Five formulations are provided.  ``prefill`` is the definition above and is
the one the parity tests compare against.  ``prefill_rotated_frame`` writes
the same recurrence the way the pages describe the RoPE trick (cumulative
angles applied to B and C, state kept unrotated); ``prefill_complex`` uses
complex128 numbers; ``prefill_chunked`` is the chunked (block) algebra that a
parallel prefill evaluates; ``decode_step`` is one token of the definition.
"""

import numpy as np

__all__ = [
    "zero_state",
    "discretize",
    "rot_pairs",
    "prefill",
    "decode_step",
    "prefill_rotated_frame",
    "prefill_complex",
    "prefill_chunked",
]


def zero_state(batch, H, P, N, R):
    """Fresh-sequence state: h = 0 and a zero pending (B_prev, x_prev)."""
    return (
        np.zeros((batch, H, P, N)),
        np.zeros((batch, H, R, N)),
        np.zeros((batch, H, R, P)),
    )


# Discretisation rules (the integers are the library's m3_disc values).
EXP_TRAPEZOID = 0      # Mamba-3's rule (the default)
DECAYED_TRAPEZOID = 1  # textbook trapezoid: the previous input decays with the state
EXP_EULER = 2          # Mamba-2's first-order rule


def discretize(dt, lam, A, disc=EXP_TRAPEZOID):
    """Per-token coefficients (alpha, beta, gamma) of the update
    h = Rot(theta)(alpha h + beta u_prev) + gamma u.

    lilting.ch Mamba-3 article, "1. 指数台形離散化" and its table of
    discretisation methods, and the table "Mamba-2とMamba-3の比較":
    * EXP_TRAPEZOID (Mamba-3): second order, the current input weighted by
      lam*dt and the previous one by (1-lam)*dt; the state decays by exp(dt*A).
    * DECAYED_TRAPEZOID: the textbook trapezoid, where the previous input is
      carried through the transition too: beta = exp(dt*A) (1-lam) dt.
    * EXP_EULER (Mamba-2): first order, current input only: beta = 0,
      gamma = dt (lam is ignored).
    dt, lam: (..., H); A: (H,).  Returns arrays of shape (..., H).
    """
    alpha = np.exp(dt * A)
    if disc == EXP_TRAPEZOID:
        beta = (1.0 - lam) * dt
        gamma = lam * dt
    elif disc == DECAYED_TRAPEZOID:
        beta = alpha * (1.0 - lam) * dt
        gamma = lam * dt
    elif disc == EXP_EULER:
        beta = np.zeros_like(alpha)
        gamma = dt * np.ones_like(alpha)
    else:
        raise ValueError(f"unknown discretisation {disc!r}")
    return alpha, beta, gamma


def rot_pairs(v, ang):
    """Rotate adjacent pairs (2j, 2j+1) of the last axis of v by ang[..., j].

    lilting.ch Mamba-3 article, "2. 複素数値状態": the complex transition is a
    block-diagonal matrix of 2x2 rotations applied to a real vector.
    (a, b) -> (a cos - b sin, a sin + b cos).  ang broadcasts against
    v[..., ::2].
    """
    a = v[..., 0::2]
    b = v[..., 1::2]
    c = np.cos(ang)
    s = np.sin(ang)
    out = np.empty(np.broadcast_shapes(v.shape), dtype=np.float64)
    out[..., 0::2] = c * a - s * b
    out[..., 1::2] = s * a + c * b
    return out


def _outer_sum(x, Bm):
    """sum_r outer(x[..., r, :], Bm[..., r, :]) -> (..., P, N)  (rank-R input)."""
    return np.einsum("...rp,...rn->...pn", x, Bm)


def _unpack(x, Bm):
    batch, T, H, R, P = x.shape
    N = Bm.shape[-1]
    if N % 2:
        raise ValueError("state size N must be even (N/2 complex pairs)")
    return batch, T, H, R, P, N


def _init(state, batch, H, P, N, R):
    if state is None:
        return zero_state(batch, H, P, N, R)
    h, Bp, xp = state
    return (np.array(h, dtype=np.float64, copy=True),
            np.array(Bp, dtype=np.float64, copy=True),
            np.array(xp, dtype=np.float64, copy=True))


def _step(h, Bp, xp, x_t, B_t, C_t, dt_t, lam_t, th_t, A, D, disc=EXP_TRAPEZOID):
    """One token of the definition; all arrays carry leading (batch, H)."""
    alpha, beta, gamma = discretize(dt_t, lam_t, A, disc)
    G = alpha[..., None, None] * h + beta[..., None, None] * _outer_sum(xp, Bp)
    h = rot_pairs(G, th_t[:, :, None, :])
    h = h + gamma[..., None, None] * _outer_sum(x_t, B_t)
    y = np.einsum("bhpn,bhrn->bhrp", h, C_t) + D[None, :, None, None] * x_t
    return h, y


def prefill(x, Bm, Cm, dt, lam, theta, A, D, state=None, disc=EXP_TRAPEZOID):
    """The definition, token by token in the lab frame.

    Returns y (batch, T, H, R, P) and the final state (h, B_prev, x_prev).
    T = 0 returns an empty y and the initial state unchanged.
    """
    batch, T, H, R, P, N = _unpack(x, Bm)
    h, Bp, xp = _init(state, batch, H, P, N, R)
    y = np.zeros((batch, T, H, R, P))
    for t in range(T):
        h, y[:, t] = _step(h, Bp, xp, x[:, t], Bm[:, t], Cm[:, t],
                           dt[:, t], lam[:, t], theta[:, t], A, D, disc)
        Bp, xp = np.array(Bm[:, t], dtype=np.float64), np.array(x[:, t], dtype=np.float64)
    return y, (h, Bp, xp)


def decode_step(x, Bm, Cm, dt, lam, theta, A, D, state, disc=EXP_TRAPEZOID):
    """One recurrent step for one new token per (batch, head).

    x (batch, H, R, P); Bm, Cm (batch, H, R, N); dt, lam (batch, H);
    theta (batch, H, N/2).  Returns y (batch, H, R, P) and the new state.
    """
    batch, H, R, P = x.shape
    N = Bm.shape[-1]
    h, Bp, xp = _init(state, batch, H, P, N, R)
    h, y = _step(h, Bp, xp, x, Bm, Cm, dt, lam, theta, A, D, disc)
    return y, (h, np.array(Bm, dtype=np.float64), np.array(x, dtype=np.float64))


def prefill_rotated_frame(x, Bm, Cm, dt, lam, theta, A, D, state=None, disc=EXP_TRAPEZOID):
    """Same recurrence written with cumulative angles on B and C.

    lilting.ch Mamba-3 article, "2. 複素数値状態" (RoPE trick) and perforder.com
    "Mamba-3解剖", section on RoPE-like rotation: the state is kept in a
    rotating frame g_t = Rot(-Phi_t) h_t, Phi_t = sum_{k<=t} theta_k, and the
    rotation moves onto B and C as Btil_t = Rot(-Phi_t) B_t,
    Ctil_t = Rot(-Phi_t) C_t.  Then
        g_t = alpha g_{t-1} + beta Btil_{t-1} x_{t-1} + gamma Btil_t x_t,
        y_t = Ctil_t^T g_t + D x_t,
    which is the plain real recurrence of the pages' formula on rotated B/C.
    At t = 0, Phi = 0, so g_0 = h_0 and the pending B is used unrotated.
    The final lab-frame state is Rot(Phi_T) g_T.
    """
    batch, T, H, R, P, N = _unpack(x, Bm)
    g, Bp_til, xp = _init(state, batch, H, P, N, R)
    Phi = np.zeros((batch, H, N // 2))
    y = np.zeros((batch, T, H, R, P))
    for t in range(T):
        Phi = Phi + theta[:, t]
        B_til = rot_pairs(Bm[:, t], -Phi[:, :, None, :])
        C_til = rot_pairs(Cm[:, t], -Phi[:, :, None, :])
        alpha, beta, gamma = discretize(dt[:, t], lam[:, t], A, disc)
        g = (alpha[..., None, None] * g
             + beta[..., None, None] * _outer_sum(xp, Bp_til)
             + gamma[..., None, None] * _outer_sum(x[:, t], B_til))
        y[:, t] = np.einsum("bhpn,bhrn->bhrp", g, C_til) + D[None, :, None, None] * x[:, t]
        Bp_til, xp = B_til, np.array(x[:, t], dtype=np.float64)
    h = rot_pairs(g, Phi[:, :, None, :])
    Bp = Bm[:, T - 1] if T > 0 else (state[1] if state is not None else Bp_til)
    return y, (h, np.array(Bp, dtype=np.float64), xp)


def prefill_complex(x, Bm, Cm, dt, lam, theta, A, D, state=None, disc=EXP_TRAPEZOID):
    """Same recurrence in complex128 arithmetic.

    lilting.ch Mamba-3 article, "2. 複素数値状態" and its state-type table: N
    real state dimensions are N/2 complex ones, each carrying an amplitude and
    a phase.  Pair j is z_j = h[:, 2j] + i h[:, 2j+1] (likewise b_j, c_j), and
        z_t = exp(i theta_t) (alpha z_{t-1} + beta sum_r x_prev[r] b_prev[r])
              + gamma sum_r x_t[r] b_t[r],
        y_t[r] = Re sum_j conj(c_j[r]) z_j + D x_t[r].
    """
    batch, T, H, R, P, N = _unpack(x, Bm)
    h, Bp, xp = _init(state, batch, H, P, N, R)

    def cplx(v):
        return v[..., 0::2] + 1j * v[..., 1::2]

    z = cplx(h)                      # (b, H, P, N/2)
    bp = cplx(Bp)                    # (b, H, R, N/2)
    y = np.zeros((batch, T, H, R, P))
    for t in range(T):
        alpha, beta, gamma = discretize(dt[:, t], lam[:, t], A, disc)
        rot = np.exp(1j * theta[:, t])[:, :, None, :]          # (b, H, 1, N/2)
        bt = cplx(Bm[:, t])
        ct = cplx(Cm[:, t])
        pend = np.einsum("bhrp,bhrj->bhpj", xp, bp)
        cur = np.einsum("bhrp,bhrj->bhpj", x[:, t], bt)
        z = rot * (alpha[..., None, None] * z + beta[..., None, None] * pend) \
            + gamma[..., None, None] * cur
        y[:, t] = np.real(np.einsum("bhrj,bhpj->bhrp", np.conj(ct), z)) \
            + D[None, :, None, None] * x[:, t]
        bp, xp = bt, np.array(x[:, t], dtype=np.float64)
    h_out = np.empty((batch, H, P, N))
    h_out[..., 0::2] = z.real
    h_out[..., 1::2] = z.imag
    Bp_out = np.empty((batch, H, R, N))
    Bp_out[..., 0::2] = bp.real
    Bp_out[..., 1::2] = bp.imag
    return y, (h_out, Bp_out, xp)


def prefill_chunked(x, Bm, Cm, dt, lam, theta, A, D, state=None, chunk=64, disc=EXP_TRAPEZOID):
    """Chunked (block) evaluation of the same recurrence.

    This is the "dual", matmul-shaped form that lets a parallel prefill use
    matrix units (lilting.ch Mamba-3 article, section on SSM history: Mamba-2
    restructured the scan so attention-style GPU kernels apply).  Within a
    chunk of tokens c0..e (local index), with inclusive local sums
    cs_t = sum_{k=c0..t} dt_k A and phi_t = sum_{k=c0..t} theta_k,
    Btil_s = Rot(-phi_s) B_s and Ctil_t = Rot(-phi_t) C_t:

      M[t, s] = gamma_s e^{cs_t - cs_s} + [s < t] beta_{s+1} e^{cs_t - cs_{s+1}}
      y_t = e^{cs_t} Ctil_t . h + sum_{s<=t} M[t, s] (Ctil_t . Btil_s) x_s
            + beta_{c0} e^{cs_t - cs_{c0}} (Ctil_t . B_prev) x_prev + D x_t
      g_e = e^{cs_e} h + sum_s M[e, s] x_s (x) Btil_s
            + beta_{c0} e^{cs_e - cs_{c0}} x_prev (x) B_prev
      h  <- Rot(phi_e) g_e;   (B_prev, x_prev) <- (B_e, x_e)

    where h is the lab-frame state before the chunk and the "lookback" pair
    (B_prev, x_prev) is the last token of the previous chunk (unrotated: its
    local angle is 0).  Loops over (batch, head) and chunks; dense Q x Q mask.
    """
    batch, T, H, R, P, N = _unpack(x, Bm)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    h0, Bp0, xp0 = _init(state, batch, H, P, N, R)
    y = np.zeros((batch, T, H, R, P))
    h_out = np.empty_like(h0)
    Bp_out = np.empty_like(Bp0)
    xp_out = np.empty_like(xp0)
    for b in range(batch):
        for hd in range(H):
            h = h0[b, hd].copy()
            Bp = Bp0[b, hd].copy()
            xp = xp0[b, hd].copy()
            for c0 in range(0, T, chunk):
                e = min(c0 + chunk, T)
                L = e - c0
                a = dt[b, c0:e, hd] * A[hd]
                cs = np.cumsum(a)
                _, beta, gamma = discretize(dt[b, c0:e, hd], lam[b, c0:e, hd], A[hd], disc)
                phi = np.cumsum(theta[b, c0:e, hd], axis=0)           # (L, N/2)
                Bt = rot_pairs(Bm[b, c0:e, hd], -phi[:, None, :])    # (L, R, N)
                Ct = rot_pairs(Cm[b, c0:e, hd], -phi[:, None, :])
                xs = x[b, c0:e, hd]                                  # (L, R, P)
                M = np.zeros((L, L))
                for t in range(L):
                    for s in range(t + 1):
                        M[t, s] = gamma[s] * np.exp(cs[t] - cs[s])
                        if s < t:
                            M[t, s] += beta[s + 1] * np.exp(cs[t] - cs[s + 1])
                S = np.einsum("trn,sqn->trsq", Ct, Bt)               # (L,R,L,R)
                y_intra = np.einsum("ts,trsq,sqp->trp", M, S, xs)
                look = beta[0] * np.exp(cs - cs[0])                  # (L,)
                y_look = np.einsum("t,trn,qn,qp->trp", look, Ct, Bp, xp)
                y_off = np.exp(cs)[:, None, None] * np.einsum("trn,pn->trp", Ct, h)
                y[b, c0:e, hd] = y_intra + y_look + y_off + D[hd] * xs
                w = M[L - 1]                                          # weights at chunk end
                g = (np.exp(cs[L - 1]) * h
                     + np.einsum("s,sqp,sqn->pn", w, xs, Bt)
                     + look[L - 1] * np.einsum("qp,qn->pn", xp, Bp))
                h = rot_pairs(g, phi[L - 1][None, :])
                Bp = np.array(Bm[b, e - 1, hd], dtype=np.float64)
                xp = np.array(x[b, e - 1, hd], dtype=np.float64)
            h_out[b, hd], Bp_out[b, hd], xp_out[b, hd] = h, Bp, xp
    return y, (h_out, Bp_out, xp_out)


def bc_rmsnorm(v, weight, eps):
    """BC normalisation: RMSNorm of the input and output projections B and C.

    ai-flow-lab.com Mamba-3 summary, section "実装とカーネル最適化" (BC/QK
    normalisation: the QKNorm of attention carried over to the SSM's B and C),
    and lilting.ch Mamba-3 article, the paragraph on other changes (a QKNorm
    layer added for training stability) and the comparison table's
    normalisation row.  Each (token, head, rank) row of N state channels is
    normalised by its root mean square and scaled per channel by the head's
    weight, before the scan uses it (and so before any rotation):
        out[..., h, r, n] = weight[h, n] * v[..., h, r, n] / sqrt(mean_n v[..., h, r, :]^2 + eps)
    v: (..., H, R, N); weight: (H, N); eps: scalar >= 0.
    """
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return np.asarray(weight, dtype=np.float64)[:, None, :] * v / np.sqrt(ms + eps)


def rank_down_projection(y, down):
    """MIMO read-out: the R rank outputs of a (token, head) folded into one row
    of P channels.

    lilting.ch Mamba-3 article, "3. MIMO SSM" (channels enter one rank-r SSM
    and leave it as channels again, coupled through an r-dimensional
    subspace): the rank-r output is brought back to the P channels by a
    learned per-(head, rank, channel) weight, channel by channel:
        s[..., h, p] = sum_r down[h, r, p] * y[..., h, r, p]
    y: (..., H, R, P); down: (H, R, P).  Returns (..., H, P).
    """
    y = np.asarray(y, dtype=np.float64)
    down = np.asarray(down, dtype=np.float64)
    s = np.zeros(y.shape[:-2] + y.shape[-1:])
    for r in range(y.shape[-2]):
        s = s + down[:, r, :] * y[..., r, :]
    return s


def gated_rmsnorm(y, z, weight, eps):
    """Output epilogue: pre-gate grouped RMSNorm of the scan output.

    ai-flow-lab.com Mamba-3 summary, section "実装とカーネル最適化" (a grouped
    RMSNorm placed before the output gate), and lilting.ch Mamba-3 article,
    table "Mamba-2とMamba-3の比較" (normalisation row).  Each (token, head,
    rank) row of P output channels is one group; it is normalised by its root
    mean square, scaled per channel by the head's weight, then multiplied by
    the gate's SiLU:
        out[..., h, r, p] = weight[h, p] * y[..., h, r, p] / sqrt(mean_p y[..., h, r, :]^2 + eps)
                            * z[..., h, r, p] * sigmoid(z[..., h, r, p])
    y, z: (..., H, R, P); weight: (H, P); eps: scalar >= 0.
    """
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    ms = np.mean(y * y, axis=-1, keepdims=True)
    silu = z / (1.0 + np.exp(-z))
    return np.asarray(weight, dtype=np.float64)[:, None, :] * y / np.sqrt(ms + eps) * silu
