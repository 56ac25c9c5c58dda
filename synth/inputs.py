"""Seeded synthetic inputs for the Mamba-3 SSM core.

This module is shared by the fp64 oracle tests and the HIP-path tests: it only
draws random tensors and rounds them to the storage precision. It holds none
of the method's arithmetic (no decay, no trapezoid weights, no rotation, no
recurrence), so neither side can borrow the other's maths from here.

Distributions (the workloads described for the Mamba-3 core):
  x ~ N(0,1);  B, C ~ N(0,1)/sqrt(N);  Delta = softplus(z - 4), z ~ N(0,1)
  (the raw z - 4 is returned too, for callers that form Delta themselves);
  lambda = sigmoid(z'), z' ~ N(0,1);  A = -exp(U(0, ln 16)) one scalar per
  head;  rotation rates omega ~ N(0,1) per token and state pair, shared by
  all heads (the angles theta = Delta * omega are the method's arithmetic and
  are formed by the oracle or on the device, not here);  decode state
  h0 ~ N(0, 0.1^2).
Draw order is fixed: x, B, C, z_Delta, z_lambda, u_A, omega, h0, then carry.
bf16 tensors are drawn in fp32 and rounded to nearest-even, so both sides
receive identical bits.
"""
from __future__ import annotations

import dataclasses
import numpy as np

SEED_BASE = 20260000


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values that are already bf16-exact."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Shape:
    Bt: int
    L: int
    H: int
    P: int
    N: int
    R: int
    dtype: str  # "f32" or "bf16": storage of x, B, C (and y)
    rope: bool


# The five workloads: tiny fp32 SISO, SISO real, RoPE SISO, RoPE MIMO prefill,
# and the RoPE MIMO decode step (L is the number of decode steps there).
CONFIGS = {
    0: Shape(Bt=1, L=256, H=4, P=16, N=16, R=1, dtype="f32", rope=False),
    1: Shape(Bt=8, L=4096, H=32, P=64, N=128, R=1, dtype="bf16", rope=False),
    2: Shape(Bt=8, L=4096, H=32, P=64, N=64, R=1, dtype="bf16", rope=True),
    3: Shape(Bt=4, L=8192, H=32, P=64, N=64, R=4, dtype="bf16", rope=True),
    4: Shape(Bt=256, L=1000, H=32, P=64, N=64, R=4, dtype="bf16", rope=True),
}


def _softplus(z):
    return np.where(z > 20.0, z, np.log1p(np.exp(np.minimum(z, 20.0))))


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _normal(rng, shape, scale=1.0):
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)


def make_inputs(s: Shape, seed: int, *, h0: bool = False, carry: bool = False,
                lam_const: float | None = None, omega_zero: bool = False) -> dict:
    """Draw one batch of prefill inputs of shape ``s``.

    Returns fp32 numpy arrays (bf16-exact where ``s.dtype == 'bf16'``):
    x [Bt,L,H,R,P]; B, C [Bt,L,H,R,N]; dt, lam [Bt,L,H]; dt_raw [Bt,L,H]
    (dt = softplus(dt_raw) in fp32); A [H]; omega [Bt,L,N/2] or None (RoPE
    shapes only); optional h0 [Bt,H,N,P] and carry-in Bprev_rot [Bt,H,R,N]
    (fp32), xprev [Bt,H,R,P] (storage dtype), phi0 [Bt,H,N/2].
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    rnd = bf16_round if s.dtype == "bf16" else (lambda a: a.astype(np.float32))
    x = rnd(_normal(rng, (s.Bt, s.L, s.H, s.R, s.P)))
    B = rnd(_normal(rng, (s.Bt, s.L, s.H, s.R, s.N), 1.0 / np.sqrt(s.N)))
    C = rnd(_normal(rng, (s.Bt, s.L, s.H, s.R, s.N), 1.0 / np.sqrt(s.N)))
    z_dt = _normal(rng, (s.Bt, s.L, s.H))
    z_lam = _normal(rng, (s.Bt, s.L, s.H))
    u_A = rng.random(size=(s.H,), dtype=np.float32)
    dt_raw = (z_dt - np.float32(4.0)).astype(np.float32)
    dt = _softplus(dt_raw).astype(np.float32)
    lam = _sigmoid(z_lam).astype(np.float32)
    if lam_const is not None:
        lam = np.full_like(lam, np.float32(lam_const))
    A = (-np.exp(u_A * np.float32(np.log(16.0)))).astype(np.float32)
    omega = None
    if s.rope:
        omega = _normal(rng, (s.Bt, s.L, s.N // 2))
        if omega_zero:
            omega = np.zeros_like(omega)
    out = dict(x=x, B=B, C=C, dt=dt, dt_raw=dt_raw, lam=lam, A=A, omega=omega,
               h0=None, Bprev_rot=None, xprev=None, phi0=None)
    if h0:
        out["h0"] = _normal(rng, (s.Bt, s.H, s.N, s.P), 0.1)
    if carry:
        out["Bprev_rot"] = _normal(rng, (s.Bt, s.H, s.R, s.N), 1.0 / np.sqrt(s.N))
        out["xprev"] = rnd(_normal(rng, (s.Bt, s.H, s.R, s.P)))
        if s.rope:
            out["phi0"] = _normal(rng, (s.Bt, s.H, s.N // 2), 3.0)
    return out


def make_decode_inputs(s: Shape, steps: int, seed: int) -> dict:
    """Decode workload: random resident state h0 ~ N(0, 0.1^2), zero carry,
    and ``steps`` single-token inputs drawn like the prefill tensors with L=steps.

    Per-step tensors carry a leading step axis: x [steps,Bt,H,R,P], B, C
    [steps,Bt,H,R,N], dt, lam [steps,Bt,H], omega [steps,Bt,N/2] or None.
    """
    one = make_inputs(dataclasses.replace(s, L=steps), seed, h0=True)
    tr = lambda a: None if a is None else np.ascontiguousarray(np.moveaxis(a, 1, 0))
    return dict(
        h0=one["h0"], A=one["A"],
        x=tr(one["x"]), B=tr(one["B"]), C=tr(one["C"]),
        dt=tr(one["dt"]), lam=tr(one["lam"]), omega=tr(one["omega"]),
    )


def config_inputs(cfg: int, **kw) -> dict:
    return make_inputs(CONFIGS[cfg], SEED_BASE + cfg, **kw)
