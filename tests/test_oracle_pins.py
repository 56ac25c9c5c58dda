"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a closed
form, an independently written special-case recurrence (Mamba-2 / Euler, the
complex-diagonal SSM), brute-force impulse responses, an order-of-accuracy
law, rotation periodicity, linearity, and the carry convention.
"""
import dataclasses

import numpy as np
import pytest

from oracle import m3_oracle as orc
from tests.fixtures import Shape, make_inputs



def _tiny(Bt=2, L=24, H=3, P=5, N=6, R=1, rope=False, seed=7, **kw):
    return make_inputs(Shape(Bt, L, H, P, N, R, "f32", rope), seed, **kw)


# ---------------------------------------------------------------- P-cf
def test_closed_form_scalar_constant_inputs():
    """N=P=R=1, theta=0, constant Delta, lambda, x=B=C=1:
    h_0 = gamma and h_t = alpha^t gamma + (beta+gamma)(1-alpha^t)/(1-alpha)."""
    L, dtv, lamv, Av = 50, 0.3, 0.7, -1.3
    ones = np.ones((1, L, 1, 1, 1))
    dt = np.full((1, L, 1), dtv)
    lam = np.full((1, L, 1), lamv)
    A = np.array([Av])
    out = orc.ssm_reference(ones, ones, ones, dt, lam, A)
    a = np.exp(dtv * Av)
    beta = (1 - lamv) * dtv * a
    gamma = lamv * dtv
    t = np.arange(L)
    h = a ** t * gamma + (beta + gamma) * (1 - a ** t) / (1 - a)
    np.testing.assert_allclose(out["y"][0, :, 0, 0, 0], h, rtol=1e-12, atol=0)
    np.testing.assert_allclose(out["h"][0, 0, 0, 0], h[-1], rtol=1e-12)


# ---------------------------------------------------------------- P-E
def _mamba2_loop(x, B, C, dt, A):
    """Independently written exponential-Euler (Mamba-2) recurrence, one (b,h)
    at a time with explicit loops: h = exp(dt A) h + dt B x^T; y = h^T C."""
    Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    y = np.zeros((Bt, L, H, R, P))
    hs = np.zeros((Bt, H, N, P))
    for b in range(Bt):
        for hh in range(H):
            h = np.zeros((N, P))
            for t in range(L):
                a = np.exp(dt[b, t, hh] * A[hh])
                upd = np.zeros((N, P))
                for r in range(R):
                    upd += np.outer(B[b, t, hh, r], x[b, t, hh, r])
                h = a * h + dt[b, t, hh] * upd
                for r in range(R):
                    y[b, t, hh, r] = C[b, t, hh, r] @ h
            hs[b, hh] = h
    return y, hs


@pytest.mark.parametrize("R", [1, 3])
def test_lambda_one_is_mamba2_euler(R):
    d = _tiny(R=R, lam_const=1.0)
    out = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"])
    y2, h2 = _mamba2_loop(*(np.float64(d[k]) for k in ("x", "B", "C", "dt")), np.float64(d["A"]))
    assert orc.rel_l2(out["y"], y2) <= 1e-12
    assert orc.rel_l2(out["h"], h2) <= 1e-12


# ---------------------------------------------------------------- P-D
@pytest.mark.parametrize("R,rope,carry", [(1, False, False), (2, True, False), (1, True, True), (4, False, True)])
def test_dual_form_equals_loop(R, rope, carry):
    d = _tiny(L=40, R=R, rope=rope, h0=carry, carry=carry)
    loop = orc.ssm_reference(**{k: d[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta",
                                                   "h0", "Bprev_rot", "xprev", "phi0")})
    dual = orc.dual_reference(**{k: d[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta",
                                                    "h0", "Bprev_rot", "xprev", "phi0")})
    assert orc.rel_l2(dual, loop["y"]) <= 1e-10


def test_impulse_responses_equal_mask_times_gram():
    """Brute force: the loop's response to unit impulses e_(j, r') equals the
    transfer matrix T[(t,r),(j,r')] = M[t,j] * <Ctil_{t,r}, Btil_{j,r'}>."""
    L, R, N = 12, 2, 4
    d = _tiny(Bt=1, L=L, H=1, P=1, N=N, R=R, rope=True, seed=11)
    T_imp = np.zeros((L * R, L * R))
    for j in range(L):
        for r in range(R):
            x = np.zeros((1, L, 1, R, 1))
            x[0, j, 0, r, 0] = 1.0
            out = orc.ssm_reference(x, d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"])
            T_imp[:, j * R + r] = out["y"][0, :, 0, :, 0].reshape(L * R)
    # independent scalar loops over (t, j) for the mask and the gram
    dt = np.float64(d["dt"][0, :, 0])
    lam = np.float64(d["lam"][0, :, 0])
    A = float(d["A"][0])
    phi = np.cumsum(np.float64(d["theta"][0, :, 0]), axis=0)  # [L, N/2]

    def rot(v, ang):
        out = np.empty(N)
        for q in range(N // 2):
            c, s = np.cos(ang[q]), np.sin(ang[q])
            out[2 * q] = c * v[2 * q] + s * v[2 * q + 1]
            out[2 * q + 1] = -s * v[2 * q] + c * v[2 * q + 1]
        return out

    T = np.zeros((L * R, L * R))
    for t in range(L):
        for j in range(t + 1):
            if j == t:
                m = lam[t] * dt[t]
            else:
                decay = np.exp(A * dt[j + 1:t + 1].sum())
                m = decay * (lam[j] * dt[j] + (1 - lam[j + 1]) * dt[j + 1])
            for r in range(R):
                for rr in range(R):
                    c = rot(np.float64(d["C"][0, t, 0, r]), phi[t])
                    b = rot(np.float64(d["B"][0, j, 0, rr]), phi[j])
                    T[t * R + r, j * R + rr] = m * (c @ b)
    assert np.max(np.abs(T_imp - T)) <= 1e-12 * max(1.0, np.max(np.abs(T)))


# ---------------------------------------------------------------- P-C
def test_rope_equals_complex_diagonal_recurrence():
    """Complex state z in C^{N/2 x P}: z_t = alpha e^{i theta_t} (z_{t-1} +
    (1-lambda)Delta b_{t-1} x_{t-1}^T) + lambda Delta b_t x_t^T, b = B_{2j} + i B_{2j+1};
    y = Re(sum_j conj(c_j) z_j).  Must equal the RoPE loop, and the oracle's
    returned state must equal e^{-i Phi} z pairwise."""
    d = _tiny(L=30, R=2, N=8, rope=True, h0=False, carry=False, seed=3)
    out = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"])
    x, B, C, dt, lam, A, th = (np.float64(d[k]) for k in ("x", "B", "C", "dt", "lam", "A", "theta"))
    Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    bc = B[..., 0::2] + 1j * B[..., 1::2]
    cc = C[..., 0::2] + 1j * C[..., 1::2]
    y = np.zeros((Bt, L, H, R, P))
    zfin = np.zeros((Bt, H, N // 2, P), dtype=complex)
    for b in range(Bt):
        for hh in range(H):
            z = np.zeros((N // 2, P), dtype=complex)
            for t in range(L):
                a = np.exp(dt[b, t, hh] * A[hh]) * np.exp(1j * th[b, t, hh])  # [N/2]
                prev = np.zeros((N // 2, P), dtype=complex)
                if t > 0:
                    prev = sum(np.outer(bc[b, t - 1, hh, r], x[b, t - 1, hh, r]) for r in range(R))
                cur = sum(np.outer(bc[b, t, hh, r], x[b, t, hh, r]) for r in range(R))
                z = a[:, None] * (z + (1 - lam[b, t, hh]) * dt[b, t, hh] * prev) \
                    + lam[b, t, hh] * dt[b, t, hh] * cur
                for r in range(R):
                    y[b, t, hh, r] = np.real(np.conj(cc[b, t, hh, r]) @ z)
            zfin[b, hh] = z
    assert orc.rel_l2(out["y"], y) <= 1e-10
    w = np.exp(-1j * out["phi"])[..., None] * zfin
    h_c = np.empty((Bt, H, N, P))
    h_c[:, :, 0::2] = w.real
    h_c[:, :, 1::2] = w.imag
    assert orc.rel_l2(out["h"], h_c) <= 1e-10


# ---------------------------------------------------------------- P-S
@pytest.mark.parametrize("rope,R", [(False, 1), (True, 2)])
def test_split_resume_and_decode_chain(rope, R):
    d = _tiny(L=33, R=R, rope=rope, h0=True, carry=True, seed=5)
    keys = ("x", "B", "C", "dt", "lam", "theta")
    whole = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"],
                              d["h0"], d["Bprev_rot"], d["xprev"], d["phi0"])
    rng = np.random.default_rng(1)
    for k in sorted(set(rng.integers(1, 32, size=3).tolist())):
        sl1 = {n: (None if d[n] is None else d[n][:, :k]) for n in keys}
        sl2 = {n: (None if d[n] is None else d[n][:, k:]) for n in keys}
        a = orc.ssm_reference(A=d["A"], h0=d["h0"], Bprev_rot=d["Bprev_rot"], xprev=d["xprev"],
                              phi0=d["phi0"], **sl1)
        b = orc.ssm_reference(A=d["A"], h0=a["h"], Bprev_rot=a["Bprev_rot"], xprev=a["xprev"],
                              phi0=a["phi"], **sl2)
        y = np.concatenate([a["y"], b["y"]], axis=1)
        assert orc.rel_l2(y, whole["y"]) <= 1e-12
        assert orc.rel_l2(b["h"], whole["h"]) <= 1e-12
    # decode chained token by token
    st = dict(h=d["h0"], Bprev_rot=d["Bprev_rot"], xprev=d["xprev"], phi=d["phi0"])
    ys = []
    for t in range(d["x"].shape[1]):
        th = None if d["theta"] is None else d["theta"][:, t]
        st = orc.decode_reference(st["h"], st["Bprev_rot"], st["xprev"], st["phi"],
                                  d["x"][:, t], d["B"][:, t], d["C"][:, t], d["dt"][:, t],
                                  d["lam"][:, t], d["A"], th)
        ys.append(st["y"])
    assert orc.rel_l2(np.stack(ys, axis=1), whole["y"]) <= 1e-12
    assert orc.rel_l2(st["h"], whole["h"]) <= 1e-12


# ---------------------------------------------------------------- per-token A
def _A_tok(d, seed=3):
    """A per token in [-16, -1], drawn like the per-head A."""
    Bt, L, H = d["dt"].shape
    u = np.random.default_rng(seed).random((Bt, L, H))
    return -np.exp(u * np.log(16.0))


def test_per_token_A_constant_in_time_is_the_per_head_A():
    d = _tiny(L=30, R=2, rope=True, h0=True, carry=True, seed=21)
    Bt, L, H = d["dt"].shape
    A_tok = np.broadcast_to(np.float64(d["A"])[None, None, :], (Bt, L, H)).copy()
    args = {k: d[k] for k in ("x", "B", "C", "dt", "lam", "theta", "h0", "Bprev_rot", "xprev", "phi0")}
    a = orc.ssm_reference(A=d["A"], **args)
    b = orc.ssm_reference(A=A_tok, **args)
    for k in ("y", "h", "Bprev_rot", "phi"):
        assert np.array_equal(a[k], b[k])


def test_per_token_A_impulse_responses():
    """Brute force with a decay rate per token: the loop's response to unit
    impulses equals scalar loops over (t, j) for the mask (decay the product of
    exp(Delta_s A_s) over j < s <= t) times the Gram entries."""
    L, R, N = 10, 2, 4
    d = _tiny(Bt=1, L=L, H=1, P=1, N=N, R=R, rope=False, seed=17)
    A_tok = _A_tok(d)
    T_imp = np.zeros((L * R, L * R))
    for j in range(L):
        for r in range(R):
            x = np.zeros((1, L, 1, R, 1))
            x[0, j, 0, r, 0] = 1.0
            out = orc.ssm_reference(x, d["B"], d["C"], d["dt"], d["lam"], A_tok)
            T_imp[:, j * R + r] = out["y"][0, :, 0, :, 0].reshape(L * R)
    dt = np.float64(d["dt"][0, :, 0])
    lam = np.float64(d["lam"][0, :, 0])
    a = A_tok[0, :, 0]
    T = np.zeros((L * R, L * R))
    for t in range(L):
        for j in range(t + 1):
            if j == t:
                m = lam[t] * dt[t]
            else:
                decay = 1.0
                for s_ in range(j + 1, t + 1):
                    decay *= np.exp(dt[s_] * a[s_])
                m = decay * (lam[j] * dt[j] + (1 - lam[j + 1]) * dt[j + 1])
            for r in range(R):
                for rr in range(R):
                    T[t * R + r, j * R + rr] = m * (np.float64(d["C"][0, t, 0, r]) @ np.float64(d["B"][0, j, 0, rr]))
    assert np.max(np.abs(T_imp - T)) <= 1e-12 * max(1.0, np.max(np.abs(T)))


@pytest.mark.parametrize("R,rope", [(1, False), (2, True)])
def test_per_token_A_dual_form_and_decode_chain(R, rope):
    d = _tiny(L=35, R=R, rope=rope, h0=True, carry=True, seed=23)
    A_tok = _A_tok(d, seed=5)
    args = {k: d[k] for k in ("x", "B", "C", "dt", "lam", "theta", "h0", "Bprev_rot", "xprev", "phi0")}
    loop = orc.ssm_reference(A=A_tok, **args)
    assert orc.rel_l2(orc.dual_reference(A=A_tok, **args), loop["y"]) <= 1e-10
    st = dict(h=d["h0"], Bprev_rot=d["Bprev_rot"], xprev=d["xprev"], phi=d["phi0"])
    ys = []
    for t in range(d["x"].shape[1]):
        th = None if d["theta"] is None else d["theta"][:, t]
        st = orc.decode_reference(st["h"], st["Bprev_rot"], st["xprev"], st["phi"], d["x"][:, t], d["B"][:, t],
                                  d["C"][:, t], d["dt"][:, t], d["lam"][:, t], A_tok[:, t], th)
        ys.append(st["y"])
    assert orc.rel_l2(np.stack(ys, axis=1), loop["y"]) <= 1e-12
    assert orc.rel_l2(st["h"], loop["h"]) <= 1e-12


# ---------------------------------------------------------------- P-ord
@pytest.mark.parametrize("lamv,order", [(0.5, 2.0), (1.0, 1.0), (0.0, 1.0)])
def test_order_of_accuracy(lamv, order):
    """dh/ds = a h + u(s), u = sin(w s), h(0) = 0, exact
    h(s) = Im[(e^{iws} - e^{as}) / (iw - a)].  The lambda-scheme with alpha inside
    beta is second order at lambda = 1/2 and first order at lambda in {0, 1}."""
    a, w, S = -1.5, 3.0, 2.0
    exact = np.imag((np.exp(1j * w * S) - np.exp(a * S)) / (1j * w - a))
    errs, hs = [], []
    for n in (40, 80, 160, 320):
        dtv = S / n
        t = np.arange(n + 1)
        u = np.sin(w * dtv * t)
        x = u.reshape(1, n + 1, 1, 1, 1)
        ones = np.ones_like(x)
        out = orc.ssm_reference(x, ones, ones, np.full((1, n + 1, 1), dtv),
                                np.full((1, n + 1, 1), lamv), np.array([a]))
        errs.append(abs(out["y"][0, -1, 0, 0, 0] - exact))
        hs.append(dtv)
    slope = np.polyfit(np.log(hs), np.log(errs), 1)[0]
    assert abs(slope - order) <= 0.2, slope


# ---------------------------------------------------------------- P-rot
@pytest.mark.parametrize("m", [2, 3, 5])
def test_rotation_periodicity(m):
    """A = 0 (no decay), theta = 2 pi / m, one impulse at t = 0: the readout
    repeats every m steps; m = 2 flips the sign every step."""
    L, N, P = 4 * m + 3, 4, 2
    rng = np.random.default_rng(m)
    x = np.zeros((1, L, 1, 1, P))
    x[0, 0, 0, 0] = rng.standard_normal(P)
    B = np.broadcast_to(rng.standard_normal(N), (1, L, 1, 1, N)).copy()
    C = np.broadcast_to(rng.standard_normal(N), (1, L, 1, 1, N)).copy()
    dt = np.full((1, L, 1), 0.4)
    lam = np.full((1, L, 1), 0.6)
    theta = np.full((1, L, 1, N // 2), 2 * np.pi / m)
    y = orc.ssm_reference(x, B, C, dt, lam, np.array([0.0]), theta)["y"][0, :, 0, 0]
    for t in range(1, L - m):
        np.testing.assert_allclose(y[t + m], y[t], atol=1e-12)
    if m == 2:
        for t in range(1, L - 1):
            np.testing.assert_allclose(y[t + 1], -y[t], atol=1e-12)


# ---------------------------------------------------------------- P-mimo
def test_mimo_is_sum_of_siso():
    R = 3
    d = _tiny(L=20, R=R, rope=True, seed=9)
    out = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"])
    h_sum = 0.0
    for rp in range(R):
        h_sum = h_sum + orc.ssm_reference(d["x"][..., rp:rp + 1, :], d["B"][..., rp:rp + 1, :],
                                          d["C"][..., rp:rp + 1, :], d["dt"], d["lam"], d["A"],
                                          d["theta"])["h"]
    assert orc.rel_l2(out["h"], h_sum) <= 1e-12
    for r in range(R):
        y_r = 0.0
        for rp in range(R):
            y_r = y_r + orc.ssm_reference(d["x"][..., rp:rp + 1, :], d["B"][..., rp:rp + 1, :],
                                          d["C"][..., r:r + 1, :], d["dt"], d["lam"], d["A"],
                                          d["theta"])["y"][..., 0, :]
        assert orc.rel_l2(out["y"][..., r, :], y_r) <= 1e-12


# ---------------------------------------------------------------- P-lin
def test_linearity_and_norms():
    d = _tiny(L=18, R=2, rope=True, h0=True, seed=4)
    x2 = np.random.default_rng(0).standard_normal(d["x"].shape)
    f = lambda x, h0: orc.ssm_reference(x, d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"], h0)
    y1 = f(d["x"], None)["y"]
    y2 = f(x2, None)["y"]
    y12 = f(d["x"] + 2.5 * x2, None)["y"]
    assert orc.rel_l2(y12, y1 + 2.5 * y2) <= 1e-12
    yh = f(np.zeros_like(x2), d["h0"])["y"]
    yboth = f(d["x"], d["h0"])["y"]
    assert orc.rel_l2(yboth, y1 + yh) <= 1e-12
    v = np.random.default_rng(1).standard_normal((5, 3, 8))
    ang = np.random.default_rng(2).standard_normal((5, 4)) * 10
    rv = orc.rotate_pairs(v, ang)
    np.testing.assert_allclose(rv[..., 0::2] ** 2 + rv[..., 1::2] ** 2,
                               v[..., 0::2] ** 2 + v[..., 1::2] ** 2, rtol=1e-12)
    z = _tiny(L=5, lam_const=0.0)
    y0 = orc.ssm_reference(z["x"], z["B"], z["C"], z["dt"], z["lam"], z["A"])["y"][:, 0]
    assert np.all(y0 == 0.0)


def test_rope_angles_cumsum_brute_force():
    rng = np.random.default_rng(3)
    th = rng.standard_normal((2, 9, 3, 4))
    p0 = rng.standard_normal((2, 3, 4))
    out = orc.rope_angles_cumsum(th, p0)
    for b in range(2):
        for h in range(3):
            for j in range(4):
                acc = p0[b, h, j]
                for t in range(9):
                    acc += th[b, t, h, j]
                    assert abs(out[b, t, h, j] - acc) <= 1e-13


def test_oracle_golden_regression():
    """Stored oracle outputs (written by tests/golden/make_golden.py, which calls
    only the oracle) still reproduce: guards later edits of the oracle."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    with open(path) as f:
        g = json.load(f)
    from tests.fixtures import make_inputs as mk
    s = Shape(**g["shape"])
    d = mk(s, g["seed"], h0=True, carry=True)
    out = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"],
                            d["h0"], d["Bprev_rot"], d["xprev"], d["phi0"])
    np.testing.assert_allclose(out["y"].ravel()[: len(g["y_head"])], g["y_head"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["h"].ravel()[: len(g["h_head"])], g["h_head"], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- chunk algebra
@pytest.mark.parametrize("R,Q,rope", [(1, 8, False), (2, 4, True), (4, 5, True)])
def test_chunked_shifted_state_decomposition(R, Q, rope):
    """The chunked form the GPU kernel evaluates, written out with numpy on the
    CPU: per chunk, intra-chunk masked product, readout of the carried shifted
    state H' = h_end + (1 - lambda_{end+1}) Delta_{end+1} u_end, and the
    inter-chunk update H'_c = exp(Lambda_end) H'_{c-1} + sum_j w_j Btil_j x_j^T.
    Must equal the sequential loop (pins the chunk decomposition)."""
    d = _tiny(L=23, R=R, rope=rope, h0=True, carry=True, seed=12)
    ref = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"],
                            d["h0"], d["Bprev_rot"], d["xprev"], d["phi0"])
    x, B, C, dt, lam, A = (np.float64(d[k]) for k in ("x", "B", "C", "dt", "lam", "A"))
    Bt, L, H, _, P = x.shape
    N = B.shape[-1]
    if rope:
        phi = orc.rope_angles_cumsum(d["theta"], d["phi0"])
        Br, Cr = orc.rotate_pairs(B, phi), orc.rotate_pairs(C, phi)
    else:
        Br, Cr = B, C
    y = np.zeros_like(x)
    hfin = np.zeros((Bt, H, N, P))
    for b in range(Bt):
        for hh in range(H):
            Hs = np.float64(d["h0"][b, hh]) + (1 - lam[b, 0, hh]) * dt[b, 0, hh] * (
                np.float64(d["Bprev_rot"][b, hh]).T @ np.float64(d["xprev"][b, hh]))
            for s in range(0, L, Q):
                e = min(s + Q, L)
                lg = dt[b, s:e, hh] * A[hh]
                Lam = np.cumsum(lg)
                gam = lam[b, s:e, hh] * dt[b, s:e, hh]
                nd = np.zeros(e - s)
                nd[:-1] = (1 - lam[b, s + 1:e, hh]) * dt[b, s + 1:e, hh]
                if e < L:
                    nd[-1] = (1 - lam[b, e, hh]) * dt[b, e, hh]
                dl = gam + nd
                rows = (e - s) * R
                tok = np.repeat(np.arange(e - s), R)
                Cm = Cr[b, s:e, hh].reshape(rows, N)
                Bm = Br[b, s:e, hh].reshape(rows, N)
                Xm = x[b, s:e, hh].reshape(rows, P)
                ti, tj = tok[:, None], tok[None, :]
                M = np.where(tj < ti, np.exp(Lam[ti] - Lam[tj]) * dl[tj], 0.0)
                M = np.where(tj == ti, gam[ti], M)
                Y = (M * (Cm @ Bm.T)) @ Xm + np.exp(Lam[tok])[:, None] * (Cm @ Hs)
                y[b, s:e, hh] = Y.reshape(e - s, R, P)
                w = np.exp(Lam[-1] - Lam[tok]) * dl[tok]
                Hs = np.exp(Lam[-1]) * Hs + Bm.T @ (w[:, None] * Xm)
            hfin[b, hh] = Hs
    assert orc.rel_l2(y, ref["y"]) <= 1e-12
    assert orc.rel_l2(hfin, ref["h"]) <= 1e-12


# ---------------------------------------------------------------- comparator
def test_rel_l2_hand_computed_values():
    """The parity metric itself: ||a - b|| / ||b|| on hand-computed cases.  A
    comparator that returned 0, or normalised by anything but ||b||, fails."""
    a, b = np.array([3.0, 4.0]), np.array([0.0, 5.0])
    assert abs(orc.rel_l2(a, b) - np.sqrt(10.0) / 5.0) <= 1e-15      # ||(3,-1)|| / 5
    assert abs(orc.rel_l2(b, a) - np.sqrt(10.0) / 5.0) <= 1e-15      # ||a|| = 5 as well
    assert abs(orc.rel_l2(2.0 * b, b) - 1.0) <= 1e-15
    assert abs(orc.rel_l2(np.array([1.0, 1.0, 1.0, 1.0]), np.array([0.0, 2.0, 0.0, 0.0])) - 1.0) <= 1e-15
    assert orc.rel_l2(b, b) == 0.0
    # scale invariance, and every element counts (2-D input is flattened)
    m_a = np.array([[1.0, 2.0], [3.0, 4.0]])
    m_b = np.array([[1.0, 2.0], [3.0, 5.0]])
    assert abs(orc.rel_l2(m_a, m_b) - 1.0 / np.sqrt(39.0)) <= 1e-15
    assert abs(orc.rel_l2(1e-30 * m_a, 1e-30 * m_b) - 1.0 / np.sqrt(39.0)) <= 1e-14
    assert abs(orc.rel_l2(1e30 * m_a, 1e30 * m_b) - 1.0 / np.sqrt(39.0)) <= 1e-14
    # zero reference: the plain norm of the difference
    assert abs(orc.rel_l2(np.array([3.0, 4.0]), np.zeros(2)) - 5.0) <= 1e-15
    # mismatched shapes are an error, not a broadcast
    with pytest.raises(AssertionError):
        orc.rel_l2(np.zeros(3), np.zeros((3, 1)))


# ---------------------------------------------------------------- angles from rates
def test_angles_from_rates_scalar_loop_and_semantics():
    rng = np.random.default_rng(5)
    dt = rng.random((2, 3, 4)).astype(np.float32)
    om = rng.standard_normal((2, 3, 5)).astype(np.float32)
    th = orc.angles_from_rates(dt, om)
    assert th.shape == (2, 3, 4, 5) and th.dtype == np.float64
    for b in range(2):
        for t in range(3):
            for h in range(4):
                for j in range(5):
                    assert th[b, t, h, j] == float(dt[b, t, h]) * float(om[b, t, j])
    # fp32 rounding of the exact product is the fp32 product
    assert np.array_equal(th.astype(np.float32), dt[..., None] * om[:, :, None, :])
    # a constant rate c gives cumulative angles c * (running sum of Delta)
    d = _tiny(Bt=1, L=9, H=2, N=4, rope=True, seed=3)
    om_c = np.full((1, 9, 2), 0.37)
    phi = orc.rope_angles_cumsum(orc.angles_from_rates(d["dt"], om_c))
    np.testing.assert_allclose(phi[0, :, 1, 0], 0.37 * np.cumsum(np.float64(d["dt"][0, :, 1])), rtol=1e-13)
    # the oracle given omega equals the oracle given the angles
    a = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"], omega=d["omega"])
    b = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"],
                          orc.angles_from_rates(d["dt"], d["omega"]))
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["h"], b["h"])


# ---------------------------------------------------------------- prologue
def test_softplus_identities():
    z = np.linspace(-30.0, 30.0, 121)
    sp = orc.softplus(z)
    np.testing.assert_allclose(sp - orc.softplus(-z), z, rtol=0, atol=1e-13)   # sp(z) - sp(-z) = z
    np.testing.assert_allclose(np.expm1(sp), np.exp(z), rtol=1e-12)            # e^sp(z) = 1 + e^z
    assert abs(orc.softplus(0.0) - np.log(2.0)) <= 1e-16
    assert orc.softplus(800.0) == 800.0 and np.isfinite(orc.softplus(-800.0))
    assert np.all(sp > 0) and np.all(np.diff(sp) > 0)


def test_rms_norm_hand_computed_and_invariants():
    # (3, 4): mean square 12.5
    out = orc.rms_norm(np.array([3.0, 4.0]))
    np.testing.assert_allclose(out, [3.0 / np.sqrt(12.5), 4.0 / np.sqrt(12.5)], rtol=1e-15)
    # eps enters under the root: ones(4) with eps 3 -> 1 / sqrt(1 + 3) = 1/2
    np.testing.assert_allclose(orc.rms_norm(np.ones(4), eps=3.0), 0.5, rtol=1e-15)
    # each row (last axis) on its own: RMS 1, sign and positive scale
    rng = np.random.default_rng(9)
    v = rng.standard_normal((3, 2, 4, 6)) * rng.random((3, 2, 4, 1)) * 50.0
    n = orc.rms_norm(v)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orc.rms_norm(-v), -n, rtol=1e-15)
    np.testing.assert_allclose(orc.rms_norm(v * 7.5), n, rtol=1e-13)
    # gain: elementwise along the normalised axis
    w = rng.random(6) + 0.5
    np.testing.assert_allclose(orc.rms_norm(v, w), n * w, rtol=1e-14)


def test_prologue_norm_bias_softplus():
    s = Shape(2, 7, 3, 4, 6, 2, "f32", True)
    d = make_inputs(s, 21)
    rng = np.random.default_rng(22)
    bB, bC = rng.standard_normal((3, 2, 6)), rng.standard_normal((3, 2, 6))
    wB = rng.random(6) + 0.5
    dtb = rng.standard_normal(3)
    B2, C2, dt2 = orc.prologue(d["B"], d["C"], d["dt_raw"], bc_norm=True, B_norm_w=wB, eps=1e-6,
                               B_bias=bB, C_bias=bC, dt_softplus=True, dt_bias=dtb)
    # bias added after the norm: removing it leaves RMS-normalised rows (times the gain)
    un = (B2 - bB) / wB
    rms_raw = np.sqrt(np.mean(np.float64(d["B"]) ** 2, axis=-1))
    np.testing.assert_allclose(np.sqrt(np.mean(un ** 2, axis=-1)), rms_raw / np.sqrt(rms_raw ** 2 + 1e-6), rtol=1e-12)
    rms_c = np.sqrt(np.mean(np.float64(d["C"]) ** 2, axis=-1))
    np.testing.assert_allclose(np.sqrt(np.mean((C2 - bC) ** 2, axis=-1)), rms_c / np.sqrt(rms_c ** 2 + 1e-6),
                               rtol=1e-12)
    # the head bias is per (head, rank, element), broadcast over batch and token
    np.testing.assert_allclose((C2 - orc.rms_norm(d["C"], eps=1e-6))[1, 4], bC, rtol=1e-13)
    # Delta = softplus(raw + bias[h]); without softplus Delta is passed through
    np.testing.assert_allclose(np.log(np.expm1(dt2)), np.float64(d["dt_raw"]) + dtb, rtol=1e-10, atol=1e-12)
    _, _, dt3 = orc.prologue(d["B"], d["C"], d["dt"])
    assert np.array_equal(dt3, np.float64(d["dt"]))
    # through the whole core: with the norm on, a positive per-row scale of the
    # raw B and C changes nothing
    sc = rng.random((2, 7, 3, 2, 1)) * 10 + 0.1
    outs = []
    for k in (1.0, sc):
        Bq, Cq, dq = orc.prologue(d["B"] * k, d["C"] * k, d["dt_raw"], bc_norm=True, B_bias=bB, C_bias=bC,
                                  dt_softplus=True)
        outs.append(orc.ssm_reference(d["x"], Bq, Cq, dq, d["lam"], d["A"], omega=d["omega"]))
    assert orc.rel_l2(outs[1]["y"], outs[0]["y"]) <= 1e-12


def test_rms_norm_zero_rows_stay_zero():
    v = np.zeros((2, 5))
    v[1] = [1.0, -2.0, 0.5, 0.0, 3.0]
    for eps in (0.0, 1e-6):
        out = orc.rms_norm(v, eps=eps)
        assert np.array_equal(out[0], np.zeros(5))
        np.testing.assert_allclose(out[1], v[1] / np.sqrt(np.mean(v[1] ** 2) + eps), rtol=1e-15)


# ---------------------------------------------------------------- backward
def _loss(d, dy, dhf, **over):
    a = {k: d[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta", "h0", "Bprev_rot", "xprev", "phi0")}
    a.update(over)
    out = orc.ssm_reference(**a)
    return float(np.sum(dy * out["y"]) + np.sum(dhf * out["h"])), out


def _bwd_case(rope=True, carry=True, a_tok=False, seed=41, L=7, R=2):
    s = Shape(1, L, 2, 3, 4, R, "f32", rope)
    d = {k: (None if v is None else np.float64(v)) for k, v in make_inputs(s, seed, h0=carry, carry=carry).items()}
    rng = np.random.default_rng(seed + 1)
    if a_tok:
        d["A"] = -np.exp(rng.random((1, L, 2)) * np.log(16.0))
    if rope:
        d["theta"] = d["theta"] * 20.0  # angles of order one per token
    dy = rng.standard_normal(d["x"].shape)
    dhf = rng.standard_normal((1, 2, 4, 3))
    return d, dy, dhf, rng


@pytest.mark.parametrize("rope,carry,a_tok", [(True, True, False), (False, False, False), (True, True, True),
                                              (False, True, True)])
def test_backward_matches_finite_differences(rope, carry, a_tok):
    """Directional derivatives of loss = <dy, y> + <dh_final, h_final> by
    central differences (fp64, step 1e-6) against <gradient, direction>, for
    every differentiated input."""
    d, dy, dhf, rng = _bwd_case(rope, carry, a_tok)
    g = orc.ssm_backward(**{k: d[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta", "h0", "Bprev_rot",
                                              "xprev", "phi0")}, dy=dy, dh_final=dhf)
    names = [("x", "dx"), ("B", "dB"), ("C", "dC"), ("dt", "ddt"), ("lam", "dlam"), ("A", "dA")]
    if rope:
        names += [("theta", "dtheta"), ("phi0", "dphi0")]
    if carry:
        names += [("h0", "dh0"), ("Bprev_rot", "dBprev_rot"), ("xprev", "dxprev")]
    eps = 1e-6
    for inp, gname in names:
        v = rng.standard_normal(d[inp].shape)
        lp, _ = _loss(d, dy, dhf, **{inp: d[inp] + eps * v})
        lm, _ = _loss(d, dy, dhf, **{inp: d[inp] - eps * v})
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(g[gname] * v))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (inp, fd, an)


def test_backward_elementwise_step_gradient():
    """Every element of dDelta and dlambda by central differences (the
    scalars that reach the decay, the trapezoid weights and the next token)."""
    d, dy, dhf, _ = _bwd_case(True, True, False, seed=43, L=5, R=1)
    g = orc.ssm_backward(**{k: d[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta", "h0", "Bprev_rot",
                                              "xprev", "phi0")}, dy=dy, dh_final=dhf)
    eps = 1e-6
    for inp, gname in (("dt", "ddt"), ("lam", "dlam")):
        for idx in np.ndindex(*d[inp].shape):
            v = np.zeros_like(d[inp])
            v[idx] = 1.0
            lp, _ = _loss(d, dy, dhf, **{inp: d[inp] + eps * v})
            lm, _ = _loss(d, dy, dhf, **{inp: d[inp] - eps * v})
            assert abs((lp - lm) / (2 * eps) - g[gname][idx]) <= 1e-7 * max(1.0, abs(g[gname][idx])), (inp, idx)


def test_backward_homogeneity_identities():
    """y and h_final are linear in (x, h0, xprev) jointly, y is linear in C
    (h_final does not depend on C), and without a carried B both are linear
    in B: so <grad, input> returns the loss (or its y part)."""
    d, dy, dhf, _ = _bwd_case(True, True, False, seed=47)
    args = {k: d[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta", "h0", "Bprev_rot", "xprev", "phi0")}
    g = orc.ssm_backward(**args, dy=dy, dh_final=dhf)
    loss, out = _loss(d, dy, dhf)
    lin = np.sum(g["dx"] * d["x"]) + np.sum(g["dh0"] * d["h0"]) + np.sum(g["dxprev"] * d["xprev"])
    assert abs(lin - loss) <= 1e-11 * max(1.0, abs(loss))
    assert abs(np.sum(g["dC"] * d["C"]) - np.sum(dy * out["y"])) <= 1e-11 * max(1.0, abs(loss))
    d2, dy2, dhf2, _ = _bwd_case(True, False, False, seed=48)
    args2 = {k: d2[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta")}
    g2 = orc.ssm_backward(**args2, dy=dy2, dh_final=dhf2)
    loss2, _ = _loss(d2, dy2, dhf2)
    assert abs(np.sum(g2["dB"] * d2["B"]) - loss2) <= 1e-11 * max(1.0, abs(loss2))


@pytest.mark.parametrize("R,Q,rope,a_tok", [(1, 4, True, False), (2, 3, True, False), (1, 5, False, True),
                                            (4, 2, True, True)])
def test_chunked_backward_decomposition(R, Q, rope, a_tok):
    """The chunked backward the GPU kernel evaluates, written out with numpy:
    a forward chunk walk keeps the shifted state entering each chunk; a
    reverse chunk walk carries the adjoint G of that state and per chunk
    forms the two Gram matrices C B^T and dY X^T, the masked products
    dX = S1^T dY + w B G, dB = S2^T C + w X G^T, dC = S2 B + E dY H^T, the
    adjoint G <- D G + C^T E dY, and the scalar gradients through the mask,
    the readout decay E, the column weights w and the chunk decay D.  Must
    equal the token-loop adjoint."""
    L = 11
    s = Shape(1, L, 2, 3, 4, R, "f32", rope)
    d = {k: (None if v is None else np.float64(v)) for k, v in make_inputs(s, 61 + R + Q, h0=True, carry=True).items()}
    rng = np.random.default_rng(62)
    if a_tok:
        d["A"] = -np.exp(rng.random((1, L, 2)) * np.log(16.0))
    dy = rng.standard_normal(d["x"].shape)
    dhf = rng.standard_normal((1, 2, 4, 3))
    ref = orc.ssm_backward(**{k: d[k] for k in ("x", "B", "C", "dt", "lam", "A", "theta", "h0", "Bprev_rot",
                                                "xprev", "phi0")}, dy=dy, dh_final=dhf)
    x, B, C, dt, lam = (d[k] for k in ("x", "B", "C", "dt", "lam"))
    Afull = d["A"] if a_tok else np.broadcast_to(d["A"][None, None, :], dt.shape)
    Bt_, _, H, _, P = x.shape
    N = B.shape[-1]
    if rope:
        Phi = orc.rope_angles_cumsum(d["theta"], d["phi0"])
        Br, Cr = orc.rotate_pairs(B, Phi), orc.rotate_pairs(C, Phi)
    else:
        Br, Cr = B, C
    dx = np.zeros_like(x)
    dBr = np.zeros_like(B)
    dCr = np.zeros_like(C)
    ddt = np.zeros_like(dt)
    dlam = np.zeros_like(dt)
    dA = np.zeros_like(dt)
    for hh in range(H):
        b = 0
        a = dt[b, :, hh] * Afull[b, :, hh]
        chunks = [(s0, min(s0 + Q, L)) for s0 in range(0, L, Q)]

        def scal(s0, e):
            Lam = np.cumsum(a[s0:e])
            gam = lam[b, s0:e, hh] * dt[b, s0:e, hh]
            nd = np.zeros(e - s0)
            nd[:-1] = (1 - lam[b, s0 + 1:e, hh]) * dt[b, s0 + 1:e, hh]
            if e < L:
                nd[-1] = (1 - lam[b, e, hh]) * dt[b, e, hh]
            return Lam, gam, gam + nd

        # forward walk: shifted state entering each chunk
        u_m1 = d["Bprev_rot"][b, hh].T @ d["xprev"][b, hh]
        Hs = d["h0"][b, hh] + (1 - lam[b, 0, hh]) * dt[b, 0, hh] * u_m1
        Hin = []
        for s0, e in chunks:
            Hin.append(Hs)
            Lam, gam, dl = scal(s0, e)
            tok = np.repeat(np.arange(e - s0), R)
            w = np.exp(Lam[-1] - Lam[tok]) * dl[tok]
            Bm = Br[b, s0:e, hh].reshape(-1, N)
            Xm = x[b, s0:e, hh].reshape(-1, P)
            Hs = np.exp(Lam[-1]) * Hs + Bm.T @ (w[:, None] * Xm)

        def turn(G_, H_):
            # per pair q: <G, J H> over the pair's two rows, J the derivative of the
            # pair rotation at angle 0 (J (v0, v1) = (v1, -v0))
            return np.sum(G_[0::2] * H_[1::2] - G_[1::2] * H_[0::2], axis=1)
        Tq = turn(dhf[b, hh], Hs)  # Hs is now the final state
        # reverse walk
        G = dhf[b, hh].copy()
        for c in range(len(chunks) - 1, -1, -1):
            s0, e = chunks[c]
            n = e - s0
            Lam, gam, dl = scal(s0, e)
            tok = np.repeat(np.arange(n), R)
            Cm = Cr[b, s0:e, hh].reshape(-1, N)
            Bm = Br[b, s0:e, hh].reshape(-1, N)
            Xm = x[b, s0:e, hh].reshape(-1, P)
            dYm = dy[b, s0:e, hh].reshape(-1, P)
            Hc = Hin[c]
            ti, tj = tok[:, None], tok[None, :]
            Mt = np.where(tj < ti, np.exp(Lam[ti] - Lam[tj]) * dl[tj], 0.0)
            Mt = np.where(tj == ti, gam[ti], Mt)
            E = np.exp(Lam)
            w = np.exp(Lam[-1] - Lam) * dl
            D = np.exp(Lam[-1])
            G1 = Cm @ Bm.T
            G2 = dYm @ Xm.T
            S1, S2 = Mt * G1, Mt * G2
            BG = Bm @ G
            dYH = dYm @ Hc.T
            dx[b, s0:e, hh] = (S1.T @ dYm + w[tok][:, None] * BG).reshape(n, R, P)
            dBr[b, s0:e, hh] = (S2.T @ Cm + w[tok][:, None] * (Xm @ G.T)).reshape(n, R, N)
            dCr[b, s0:e, hh] = (S2 @ Bm + E[tok][:, None] * dYH).reshape(n, R, N)
            # token-level scalar gradients
            dMr = G1 * G2
            dM = np.zeros((n, n))
            np.add.at(dM, (ti.repeat(n * R, 1), tj.repeat(n * R, 0)), dMr)
            dE = np.bincount(tok, weights=np.sum(dYH * Cm, axis=1), minlength=n)
            dw = np.bincount(tok, weights=np.sum(BG * Xm, axis=1), minlength=n)
            dD = np.sum(G * Hc)
            T, J = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
            Mtok = np.where(J < T, np.exp(Lam[T] - Lam[J]) * dl[J], 0.0)
            dLam = (np.sum(dM * Mtok, axis=1) - np.sum(dM * Mtok, axis=0) + dE * E - dw * w)
            dLam[-1] += np.sum(dw * w) + dD * D
            ddl = np.sum(np.where(T > J, dM * np.exp(Lam[T] - Lam[J]), 0.0), axis=0) + dw * np.exp(Lam[-1] - Lam)
            dgam = np.diag(dM) + ddl
            da = np.flip(np.cumsum(np.flip(dLam)))
            dtt = dt[b, s0:e, hh]
            ddt[b, s0:e, hh] += da * Afull[b, s0:e, hh] + dgam * lam[b, s0:e, hh]
            dA[b, s0:e, hh] += da * dtt
            dlam[b, s0:e, hh] += dgam * dtt
            # delta_t's next-token term: tokens s0+1..e-1 here, token e in the next chunk
            ddt[b, s0 + 1:e, hh] += ddl[:-1] * (1 - lam[b, s0 + 1:e, hh])
            dlam[b, s0 + 1:e, hh] -= ddl[:-1] * dt[b, s0 + 1:e, hh]
            if e < L:
                ddt[b, e, hh] += ddl[-1] * (1 - lam[b, e, hh])
                dlam[b, e, hh] -= ddl[-1] * dt[b, e, hh]
            G = D * G + Cm.T @ (E[tok][:, None] * dYm)
            if rope:
                # a common extra rotation of every token from s0 on changes only the
                # state carried across s0: dtheta at a chunk start is
                # <dh_final, J h_final> - <G, J H> with H the shifted state entering
                # the chunk and G its adjoint (no running sum over later tokens)
                assert np.allclose(ref["dtheta"][b, s0, hh], Tq - turn(G, Hc), rtol=1e-10, atol=1e-12)
                if c == 0:
                    assert np.allclose(ref["dphi0"][b, hh], Tq - turn(G, Hc), rtol=1e-10, atol=1e-12)
        # carry-in: H'_{-1} = h0 + kappa u_{-1}, kappa = (1 - lam_0) Delta_0, and
        # G is now the adjoint of H'_{-1}
        assert orc.rel_l2(G, ref["dh0"][b, hh]) <= 1e-12
        dkap = np.sum(G * u_m1)
        ddt[b, 0, hh] += dkap * (1 - lam[b, 0, hh])
        dlam[b, 0, hh] -= dkap * dt[b, 0, hh]
        kap = (1 - lam[b, 0, hh]) * dt[b, 0, hh]
        assert orc.rel_l2((kap * G @ d["xprev"][b, hh].T).T, ref["dBprev_rot"][b, hh]) <= 1e-12
        assert orc.rel_l2((kap * G.T @ d["Bprev_rot"][b, hh].T).T, ref["dxprev"][b, hh]) <= 1e-12
    assert orc.rel_l2(dx, ref["dx"]) <= 1e-12
    assert orc.rel_l2(ddt, ref["ddt"]) <= 1e-12
    assert orc.rel_l2(dlam, ref["dlam"]) <= 1e-12
    assert orc.rel_l2(dA if a_tok else dA.sum(axis=(0, 1)), ref["dA"]) <= 1e-12
    if rope:
        c_, s_ = np.cos(Phi)[..., None, :], np.sin(Phi)[..., None, :]
        for dv, key in ((dBr, "dB"), (dCr, "dC")):
            dr = np.empty_like(dv)
            dr[..., 0::2] = c_ * dv[..., 0::2] - s_ * dv[..., 1::2]
            dr[..., 1::2] = s_ * dv[..., 0::2] + c_ * dv[..., 1::2]
            assert orc.rel_l2(dr, ref[key]) <= 1e-12
    else:
        assert orc.rel_l2(dBr, ref["dB"]) <= 1e-12
        assert orc.rel_l2(dCr, ref["dC"]) <= 1e-12
