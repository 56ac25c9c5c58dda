"""fp64 CPU oracle for the Mamba-3 SSM core.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module.  The HIP library never calls it and shares no code with
it.  Everything here is deliberately plain: a token-by-token loop in float64,
vectorised only over the independent (batch, head) pairs.

Sources (web pages on Mamba-3; cited by title and section):
  [CH]  "Znakomstvo s Mamba-3 ..." (chernovdev.ru), sec. 1 "Exponential-
        trapezoidal discretisation" -- the one displayed three-term recurrence;
        sec. 2 "Complex-valued SSMs and the RoPE trick" -- cumulative
        data-dependent rotations of B and C; sec. 3 "MIMO" -- B_t in R^{N x R},
        x_t in R^{P x R}, the state update becomes a matrix product.
  [PB]  "La dualita: Mamba-2 e Mamba-3" (book.paithon.it), sec. "State Space
        Duality" -- scalar-times-identity transition, masked-attention form
        Y = (M o C B^T) X; sec. "Mamba-3" -- the lambda family (lambda = 1 is
        Euler / Mamba-2, lambda = 1/2 the trapezoid), complex SSM of size N/2 ==
        real SSM of size N with 2x2 rotation blocks scaled by the decay, and
        MIMO as a sum of R outer products on an unchanged state.

Readings where the pages are silent (each listed in the design notes):
  * beta_t uses step t's own lambda, Delta and decay; Delta multiplies B
    explicitly (the displayed recurrence), not folded into B.
  * Fresh start: h_{-1} = 0 and B_{-1} x_{-1} = 0.  Continuation passes the
    carry (h, rotated B_{t-1}, x_{t-1}, cumulative angle).
  * Rotation pairs are adjacent state entries (2j, 2j+1); the rotated input is
    Btil = R(Phi)^T B with R(phi) = [[cos, -sin], [sin, cos]]; Phi is the
    inclusive cumulative angle (Phi_t includes theta_t).  The carried B_{t-1}
    keeps the rotation of its own step.  The returned state is the real state
    in this rotated frame.
  * y_t = h_t^T Ctil_t uses the state after the update; there is no D skip.
  * MIMO ranks share Delta, lambda, the decay and the rotation; no 1/R factor.

Parity: every function here is pinned by the not-gpu tests in
tests/test_oracle_pins.py (closed forms, special cases, brute force, an
independent complex-arithmetic recurrence, order of accuracy, hand-computed
values of the comparator and of the normalisation).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(a):
    return None if a is None else np.asarray(a, dtype=F64)


def rotate_pairs(v: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of ``v`` by -phi.

    v: [..., R, N];  phi: [..., N/2] (broadcast over R).  Returns R(phi)^T v
    pairwise: out[2j] = cos*v[2j] + sin*v[2j+1], out[2j+1] = -sin*v[2j] +
    cos*v[2j+1]  ([CH] sec. 2; [PB] sec. "Mamba-3", 2x2 rotation blocks).
    """
    c = np.cos(phi)[..., None, :]
    s = np.sin(phi)[..., None, :]
    v0 = v[..., 0::2]
    v1 = v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape), dtype=F64)
    out[..., 0::2] = c * v0 + s * v1
    out[..., 1::2] = -s * v0 + c * v1
    return out


def angles_from_rates(dt, omega):
    """Per-token rotation angles from rates: theta[..., h, j] = Delta[..., h] *
    omega[..., j].

    [PB] sec. "Mamba-3": the rotation angle depends on the data because the
    step Delta is selective, i.e. the angle of a token is its step times a
    rate.  The rates omega are given per token and state pair and shared by
    the heads (the workloads draw them that way).  dt [..., H]; omega [..., J]
    -> theta [..., H, J] in float64 (the product of two fp32 values is exact).
    """
    dt = _f64(dt)
    omega = _f64(omega)
    return dt[..., :, None] * omega[..., None, :]


def softplus(z):
    """softplus(z) = log(1 + exp(z)), evaluated without overflow.  The positive
    step Delta is the softplus of its raw value (the workloads draw Delta that
    way)."""
    return np.logaddexp(0.0, _f64(z))


def rms_norm(v, weight=None, eps=0.0):
    """RMS normalisation over the last axis: v / sqrt(mean(v^2) + eps), times an
    optional per-element gain ``weight`` (broadcast over the leading axes).

    [CH] sec. "Architecture and normalisation": B and C are RMS-normalised, by
    analogy with QK normalisation in Transformers.  For B, C of shape
    [..., R, N] each rank column (an N-vector) is normalised on its own.  A
    row of zeros is returned as zeros (a reading: with eps = 0 the quotient
    is undefined there; with eps > 0 it is zero anyway).
    """
    v = _f64(v)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    den = np.sqrt(ms + eps)
    # a row of zeros stays zero (also with eps = 0, where 0/0 is undefined)
    out = np.divide(v, den, out=np.zeros_like(v), where=ms > 0)
    if weight is not None:
        out = out * _f64(weight)
    return out


def prologue(B, C, dt, *, bc_norm=False, B_norm_w=None, C_norm_w=None, eps=0.0,
             B_bias=None, C_bias=None, dt_softplus=False, dt_bias=None):
    """The steps just before the SSM core, applied to raw projections.

    [CH] sec. "Architecture and normalisation": RMS normalisation of B and C
    (``rms_norm`` per (token, head, rank) over N, gains ``B_norm_w``,
    ``C_norm_w`` [N]), then learnable head-specific biases added after the
    normalisation (``B_bias``, ``C_bias`` [H, R, N]); [CA] "Normalizzazioni"
    and "Addio convoluzione corta" (biases on B and C after BCNorm).  The
    step: Delta = softplus(dt + dt_bias[h]) when ``dt_softplus`` (dt_bias [H]
    or None), else Delta = dt as given.
    B, C [..., H, R, N] (token axes first); dt [..., H].  Returns float64
    (B, C, Delta) ready for :func:`ssm_reference`.
    """
    B, C, dt = _f64(B), _f64(C), _f64(dt)
    if bc_norm:
        B = rms_norm(B, B_norm_w, eps)
        C = rms_norm(C, C_norm_w, eps)
    if B_bias is not None:
        B = B + _f64(B_bias)
    if C_bias is not None:
        C = C + _f64(C_bias)
    if dt_softplus:
        dt = softplus(dt if dt_bias is None else dt + _f64(dt_bias))
    return B, C, dt


def coefficients(dt, lam, A):
    """alpha = exp(Delta A), beta = (1 - lambda) Delta alpha, gamma = lambda Delta
    ([CH] sec. 1, displayed recurrence).  dt, lam: [..., H]; A: [H], or an A
    per token of the same shape as dt ([PB] sec. "Mamba-3": the decay rate may
    itself depend on the token)."""
    alpha = np.exp(dt * A)
    beta = (1.0 - lam) * dt * alpha
    gamma = lam * dt
    return alpha, beta, gamma


def ssm_step(h, Bp, xp, phi, x_t, B_t, C_t, dt_t, lam_t, A, theta_t):
    """One token of the exponential-trapezoidal MIMO recurrence.

    h: [Bt,H,N,P]; Bp: [Bt,H,R,N] (rotated B of the previous token);
    xp: [Bt,H,R,P]; phi: [Bt,H,N/2] or None; x_t: [Bt,H,R,P];
    B_t, C_t: [Bt,H,R,N]; dt_t, lam_t: [Bt,H]; A: [H]; theta_t: [Bt,H,N/2] or None.

    h_t = alpha h_{t-1} + beta Btil_{t-1} x_{t-1}^T + gamma Btil_t x_t^T with
    u = sum_r Btil[:, r] x[:, r]^T ([CH] sec. 1 and sec. 3; [PB] "Mamba-3");
    Y_t = h_t^T Ctil_t.  Returns (y_t [Bt,H,R,P], h, Btil_t, x_t, phi).
    """
    alpha, beta, gamma = coefficients(dt_t, lam_t, A)
    if theta_t is not None:
        phi = phi + theta_t
        Bt_r = rotate_pairs(B_t, phi)
        Ct_r = rotate_pairs(C_t, phi)
    else:
        Bt_r, Ct_r = B_t, C_t
    u_prev = np.einsum("bhrn,bhrp->bhnp", Bp, xp)
    u_cur = np.einsum("bhrn,bhrp->bhnp", Bt_r, x_t)
    h = (alpha[..., None, None] * h + beta[..., None, None] * u_prev
         + gamma[..., None, None] * u_cur)
    y_t = np.einsum("bhnp,bhrn->bhrp", h, Ct_r)
    return y_t, h, Bt_r, x_t, phi


def ssm_reference(x, B, C, dt, lam, A, theta=None, h0=None, Bprev_rot=None,
                  xprev=None, phi0=None, omega=None):
    """Sequential fp64 oracle of the whole sequence (prefill semantics).

    x [Bt,L,H,R,P]; B, C [Bt,L,H,R,N]; dt, lam [Bt,L,H]; A [H] or per token
    [Bt,L,H]; theta [Bt,L,H,N/2] or None, or instead omega [Bt,L,N/2] (rates:
    theta = :func:`angles_from_rates`); carry-in (all optional, zeros if None):
    h0 [Bt,H,N,P], Bprev_rot [Bt,H,R,N], xprev [Bt,H,R,P], phi0 [Bt,H,N/2].
    Returns dict(y [Bt,L,H,R,P], h [Bt,H,N,P], Bprev_rot [Bt,H,R,N],
    xprev [Bt,H,R,P], phi [Bt,H,N/2] or None), all float64.
    """
    x, B, C, dt, lam, A = map(_f64, (x, B, C, dt, lam, A))
    if omega is not None:
        assert theta is None, "give theta or omega, not both"
        theta = angles_from_rates(dt, omega)
    theta = _f64(theta)
    Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    h = np.zeros((Bt, H, N, P)) if h0 is None else _f64(h0).copy()
    Bp = np.zeros((Bt, H, R, N)) if Bprev_rot is None else _f64(Bprev_rot).copy()
    xp = np.zeros((Bt, H, R, P)) if xprev is None else _f64(xprev).copy()
    phi = None
    if theta is not None:
        phi = np.zeros((Bt, H, N // 2)) if phi0 is None else _f64(phi0).copy()
    y = np.zeros((Bt, L, H, R, P))
    for t in range(L):
        th = None if theta is None else theta[:, t]
        A_t = A if A.ndim == 1 else A[:, t]
        y[:, t], h, Bp, xp, phi = ssm_step(h, Bp, xp, phi, x[:, t], B[:, t], C[:, t],
                                           dt[:, t], lam[:, t], A_t, th)
    return dict(y=y, h=h, Bprev_rot=Bp, xprev=xp, phi=phi)


def decode_reference(h, Bprev_rot, xprev, phi, x, B, C, dt, lam, A, theta=None, omega=None):
    """One decode step against a resident state: the same token update as the
    prefill loop.  Shapes as in :func:`ssm_step` (no time axis); A is [H] or
    one per (batch, head) [Bt,H]; omega [Bt,N/2] (rates) instead of theta.
    Returns dict(y, h, Bprev_rot, xprev, phi)."""
    if omega is not None:
        assert theta is None, "give theta or omega, not both"
        theta = angles_from_rates(dt, omega)
    y, h2, Bp, xp, ph = ssm_step(_f64(h), _f64(Bprev_rot), _f64(xprev), _f64(phi),
                                 _f64(x), _f64(B), _f64(C), _f64(dt), _f64(lam),
                                 _f64(A), _f64(theta))
    return dict(y=y, h=h2, Bprev_rot=Bp, xprev=xp, phi=ph)


def ssm_backward(x, B, C, dt, lam, A, theta=None, h0=None, Bprev_rot=None, xprev=None, phi0=None,
                 dy=None, dh_final=None):
    """Gradients of a loss through the sequential recurrence (reverse mode),
    float64.  The loss reaches the core through y (upstream gradient dy, the
    shape of y) and the final state h (dh_final [Bt,H,N,P], optional); the
    carry-out (rotated B, x, angle) is not differentiated.

    The pages print no backward pass; this is the plain adjoint of the
    token loop of :func:`ssm_reference` ([CH] sec. 1-3), derived here.
    With g_t = dloss/dh_t (the adjoint state) and u_t = sum_r Btil_t[r] x_t[r]^T:
        g_t   = Ctil_t dy_t^T + alpha_{t+1} g_{t+1}    (g_{L-1} adds dh_final)
        du_t  = gamma_t g_t + beta_{t+1} g_{t+1}         (beta_L := 0)
        dBtil_t[r] = du_t x_t[r],  dx_t[r] = du_t^T Btil_t[r],  dCtil_t[r] = h_t dy_t[r]
        dalpha_t = <g_t, h_{t-1}>,  dbeta_t = <g_t, u_{t-1}>,  dgamma_t = <g_t, u_t>
    then through alpha = exp(Delta A), beta = (1 - lambda) Delta alpha,
    gamma = lambda Delta; through the rotation Btil = R(Phi)^T B (a pair's
    angle gradient is dBtil_0 Btil_1 - dBtil_1 Btil_0, summed over ranks and
    over B and C), and Phi_t = Phi_{-1} + sum_{s<=t} theta_s (so dtheta is the
    reverse cumulative sum of dPhi, and dphi0 its total).  The carry-in
    enters as h_{-1} = h0 and u_{-1} = sum_r Bprev_rot[r] xprev[r]^T.
    Returns dict(dx, dB, dC, ddt, dlam, dA (shape of A), dtheta (or None),
    dh0, dBprev_rot, dxprev, dphi0 (or None)).
    """
    x, B, C, dt, lam, A = map(_f64, (x, B, C, dt, lam, A))
    theta = _f64(theta)
    Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    dy = np.zeros_like(x) if dy is None else _f64(dy)
    h = np.zeros((Bt, H, N, P)) if h0 is None else _f64(h0).copy()
    Bp = np.zeros((Bt, H, R, N)) if Bprev_rot is None else _f64(Bprev_rot).copy()
    xp = np.zeros((Bt, H, R, P)) if xprev is None else _f64(xprev).copy()
    per_tok = A.ndim != 1
    # ---- forward, keeping every state and the rotated inputs
    phi = None
    if theta is not None:
        phi = np.zeros((Bt, H, N // 2)) if phi0 is None else _f64(phi0).copy()
        Phi = phi[:, None] + np.cumsum(theta, axis=1)          # [Bt,L,H,N/2]
        Br, Cr = rotate_pairs(B, Phi), rotate_pairs(C, Phi)
    else:
        Br, Cr = B, C
    hs = np.zeros((L + 1, Bt, H, N, P))  # hs[t + 1] = h_t, hs[0] = h_{-1}
    hs[0] = h
    us = np.zeros((L + 1, Bt, H, N, P))  # us[t + 1] = u_t, us[0] = u_{-1}
    us[0] = np.einsum("bhrn,bhrp->bhnp", Bp, xp)
    al = np.zeros((Bt, L, H))
    be = np.zeros((Bt, L, H))
    ga = np.zeros((Bt, L, H))
    for t in range(L):
        A_t = A if not per_tok else A[:, t]
        a_, b_, g_ = coefficients(dt[:, t], lam[:, t], A_t)
        al[:, t], be[:, t], ga[:, t] = a_, b_, g_
        us[t + 1] = np.einsum("bhrn,bhrp->bhnp", Br[:, t], x[:, t])
        hs[t + 1] = (a_[..., None, None] * hs[t] + b_[..., None, None] * us[t]
                     + g_[..., None, None] * us[t + 1])
    # ---- reverse
    g_next = np.zeros((Bt, H, N, P)) if dh_final is None else _f64(dh_final).copy()
    a_next = np.zeros((Bt, H))
    b_next = np.zeros((Bt, H))
    dx = np.zeros_like(x)
    dBr = np.zeros_like(Br)
    dCr = np.zeros_like(Cr)
    dal = np.zeros((Bt, L, H))
    dbe = np.zeros((Bt, L, H))
    dga = np.zeros((Bt, L, H))
    g_after = None  # g_{t+1}
    for t in range(L - 1, -1, -1):
        g_t = np.einsum("bhrn,bhrp->bhnp", Cr[:, t], dy[:, t])
        if t == L - 1:
            g_t = g_t + g_next  # dh_final
        else:
            g_t = g_t + a_next[..., None, None] * g_after
        dCr[:, t] = np.einsum("bhnp,bhrp->bhrn", hs[t + 1], dy[:, t])
        du = ga[:, t][..., None, None] * g_t
        if t < L - 1:
            du = du + b_next[..., None, None] * g_after
        dBr[:, t] = np.einsum("bhnp,bhrp->bhrn", du, x[:, t])
        dx[:, t] = np.einsum("bhnp,bhrn->bhrp", du, Br[:, t])
        dal[:, t] = np.einsum("bhnp,bhnp->bh", g_t, hs[t])
        dbe[:, t] = np.einsum("bhnp,bhnp->bh", g_t, us[t])
        dga[:, t] = np.einsum("bhnp,bhnp->bh", g_t, us[t + 1])
        a_next, b_next, g_after = al[:, t], be[:, t], g_t
    g0 = g_after  # g_0
    dh0 = al[:, 0][..., None, None] * g0
    du_m1 = be[:, 0][..., None, None] * g0
    dBprev = np.einsum("bhnp,bhrp->bhrn", du_m1, xp)
    dxprev = np.einsum("bhnp,bhrn->bhrp", du_m1, Bp)
    # ---- scalars: alpha = exp(dt A), beta = (1 - lam) dt alpha, gamma = lam dt
    A_full = A[None, None, :] if not per_tok else A
    ddt = dal * A_full * al + dbe * ((1 - lam) * al + A_full * be) + dga * lam
    dlam = -dbe * dt * al + dga * dt
    dA_tok = dt * (dal * al + dbe * be)
    dA = dA_tok if per_tok else dA_tok.sum(axis=(0, 1))
    # ---- rotation
    dtheta = dphi0 = None
    if theta is not None:
        c = np.cos(Phi)[..., None, :]
        s_ = np.sin(Phi)[..., None, :]

        def unrot(dv):  # dv [.., R, N] in the rotated frame -> input frame
            out = np.empty_like(dv)
            out[..., 0::2] = c * dv[..., 0::2] - s_ * dv[..., 1::2]
            out[..., 1::2] = s_ * dv[..., 0::2] + c * dv[..., 1::2]
            return out

        dB = unrot(dBr)
        dC = unrot(dCr)
        dPhi = (dBr[..., 0::2] * Br[..., 1::2] - dBr[..., 1::2] * Br[..., 0::2]
                + dCr[..., 0::2] * Cr[..., 1::2] - dCr[..., 1::2] * Cr[..., 0::2]).sum(axis=-2)  # [Bt,L,H,N/2]
        dtheta = np.flip(np.cumsum(np.flip(dPhi, axis=1), axis=1), axis=1)
        dphi0 = dPhi.sum(axis=1)
    else:
        dB, dC = dBr, dCr
    return dict(dx=dx, dB=dB, dC=dC, ddt=ddt, dlam=dlam, dA=dA, dtheta=dtheta, dh0=dh0,
                dBprev_rot=dBprev, dxprev=dxprev, dphi0=dphi0)


def rope_angles_cumsum(theta, phi0=None):
    """Inclusive cumulative angle Phi_t = Phi_{-1} + sum_{s<=t} theta_s along the
    sequence axis ([CH] sec. 2: rotations aggregated over all time steps).
    theta [Bt,L,H,J]; phi0 [Bt,H,J] or None."""
    th = _f64(theta)
    out = np.cumsum(th, axis=1)
    if phi0 is not None:
        out = out + _f64(phi0)[:, None]
    return out


def dual_reference(x, B, C, dt, lam, A, theta=None, h0=None, Bprev_rot=None,
                   xprev=None, phi0=None, omega=None):
    """Materialised masked-attention (SSD dual) form, O(L^2) per (b, h).

    [PB] sec. "State Space Duality": with a scalar-times-identity transition the
    recurrence equals Y = (M o C B^T) X with a causal decay mask.  For the
    three-term recurrence the mask follows by unrolling the recurrence (our
    derivation): with Lambda_t = sum_{k<=t} Delta_k A_k (A [H], or [Bt,L,H] per token),
        M[t, j] = exp(Lambda_t - Lambda_j) * (gamma_j + (1 - lambda_{j+1}) Delta_{j+1})  (j < t)
        M[t, t] = gamma_t,   M[t, j] = 0 (j > t),
    broadcast over the R x R rank blocks, plus the carried-in state
    H' = h0 + (1 - lambda_0) Delta_0 Btil_{-1} x_{-1}^T read out with decay
    exp(Lambda_t - Lambda_{-1}).  Rotations as in :func:`rotate_pairs`.
    Returns y [Bt,L,H,R,P] (float64).
    """
    x, B, C, dt, lam, A = map(_f64, (x, B, C, dt, lam, A))
    if omega is not None:
        theta = angles_from_rates(dt, omega)
    Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    if theta is not None:
        phi = rope_angles_cumsum(theta, phi0)  # [Bt,L,H,N/2]
        Bt_r = rotate_pairs(B, phi)
        Ct_r = rotate_pairs(C, phi)
    else:
        Bt_r, Ct_r = B, C
    logA = dt * A  # [Bt,L,H]
    Lam = np.cumsum(logA, axis=1)
    gamma = lam * dt
    nxt = np.zeros_like(dt)
    nxt[:, :-1] = (1.0 - lam[:, 1:]) * dt[:, 1:]
    delta = gamma + nxt
    y = np.zeros((Bt, L, H, R, P))
    tri = np.tril(np.ones((L, L), dtype=bool), k=-1)
    for b in range(Bt):
        for hh in range(H):
            lam_v = Lam[b, :, hh]
            diff = lam_v[:, None] - lam_v[None, :]
            M = np.where(tri, np.exp(np.where(tri, diff, 0.0)) * delta[b, None, :, hh], 0.0)
            M[np.arange(L), np.arange(L)] = gamma[b, :, hh]
            Cm = Ct_r[b, :, hh].reshape(L * R, N)
            Bm = Bt_r[b, :, hh].reshape(L * R, N)
            G = Cm @ Bm.T
            Mb = np.kron(M, np.ones((R, R)))
            Y = (Mb * G) @ x[b, :, hh].reshape(L * R, P)
            Hin = np.zeros((N, P))
            if h0 is not None:
                Hin += _f64(h0)[b, hh]
            if Bprev_rot is not None and xprev is not None:
                Hin += (1.0 - lam[b, 0, hh]) * dt[b, 0, hh] * (
                    _f64(Bprev_rot)[b, hh].T @ _f64(xprev)[b, hh])
            dec = np.exp(lam_v)  # exp(Lambda_t - Lambda_{-1})
            Y += (dec[:, None, None] * (Ct_r[b, :, hh] @ Hin)).reshape(L * R, P)
            y[b, :, hh] = Y.reshape(L, R, P)
    return y


def rel_l2(a, b) -> float:
    """Relative L2 error ||a - b|| / ||b|| in float64 (the parity metric); the
    plain ||a - b|| when b is all zeros.  Shapes must match exactly."""
    assert np.shape(a) == np.shape(b), (np.shape(a), np.shape(b))
    a = np.asarray(a, dtype=F64)
    b = np.asarray(b, dtype=F64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0))
