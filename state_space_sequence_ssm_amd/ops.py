"""Thin torch binding of the C ABI: the same three entry points, marshalling
device tensors into the argument structures.  Every step of the computation
runs in the HIP kernels of libm3ssm.so; torch only provides device memory
and the current stream.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib


class M3Error(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {_lib.status_string(code)} ({code})")
        self.code = code


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.M3_BF16
    if t.dtype == torch.float32:
        return _lib.M3_F32
    raise TypeError(f"unsupported input dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _prologue(pro, H, R, N, bc_norm, bc_eps, B_norm_w, C_norm_w, B_bias, C_bias, dt_softplus, dt_bias):
    """Fill the m3_prologue of an argument structure (steps fused in front of
    the core: B / C RMS normalisation, head biases, Delta = softplus)."""
    f32 = torch.float32
    pro.bc_norm = 1 if bc_norm else 0
    pro.dt_softplus = 1 if dt_softplus else 0
    pro.bc_eps = float(bc_eps)
    pro.B_norm_w = _ptr(B_norm_w, f32, (N,), "B_norm_w")
    pro.C_norm_w = _ptr(C_norm_w, f32, (N,), "C_norm_w")
    pro.B_bias = _ptr(B_bias, f32, (H, R, N), "B_bias")
    pro.C_bias = _ptr(C_bias, f32, (H, R, N), "C_bias")
    pro.dt_bias = _ptr(dt_bias, f32, (H,), "dt_bias")


def m3_ssm_prefill(x, B, C, dt, lam, A, theta=None, h0=None, Bprev_rot=None, xprev=None, phi0=None,
                   *, y=None, h_final=None, Bprev_rot_out=None, xprev_out=None, phi_out=None,
                   want_state=True, want_carry=False, chunk=0, workspace=None, omega=None, A_tok=None,
                   head_major=False, noalloc=False, bc_norm=False, bc_eps=1e-6, B_norm_w=None, C_norm_w=None,
                   B_bias=None, C_bias=None, dt_softplus=False, dt_bias=None, stream=None):
    """Chunked prefill.  Shapes: x [Bt,L,H,R,P], B/C [Bt,L,H,R,N] (bf16 or fp32),
    dt/lam [Bt,L,H] fp32, A [H] fp32, theta [Bt,L,H,N/2] fp32 or None (or
    instead omega [Bt,L,N/2] fp32: rates shared by the heads, theta = dt * omega
    formed on chip); A_tok [Bt,L,H] fp32: A per token (then
    A may be None); optional
    carry-in h0 [Bt,H,N,P], Bprev_rot [Bt,H,R,N], xprev [Bt,H,R,P], phi0 [Bt,H,N/2].
    Output tensors are allocated when not given.  workspace: a uint8 device
    tensor of at least prefill_workspace_bytes(...) bytes, None to allocate one
    when the library asks for it, or False to run without (unsplit).  Returns
    a dict with y and, as requested, h_final and the carry-out (Bprev_rot,
    xprev, phi).  head_major: x, B, C and y are [Bt,H,L,R,.] instead.
    noalloc: call m3_ssm_prefill_noalloc (the library's static scratch in
    place of a workspace; workspace must then be None).
    Prologue (computed on chip; B, C and dt are then the raw projections):
    bc_norm / bc_eps / B_norm_w, C_norm_w [N]: RMS normalisation of each B and
    C row; B_bias, C_bias [H,R,N]: head biases added after it; dt_softplus /
    dt_bias [H]: Delta = softplus(dt + dt_bias)."""
    if head_major:
        Bt, H, L, R, P = x.shape
    else:
        Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    big = (lambda D: (Bt, H, L, R, D)) if head_major else (lambda D: (Bt, L, H, R, D))
    f32 = torch.float32
    if y is None:
        y = torch.empty_like(x)
    if want_state and h_final is None:
        h_final = torch.empty((Bt, H, N, P), device=x.device, dtype=f32)
    if want_carry:
        if Bprev_rot_out is None:
            Bprev_rot_out = torch.empty((Bt, H, R, N), device=x.device, dtype=f32)
        if xprev_out is None:
            xprev_out = torch.empty((Bt, H, R, P), device=x.device, dtype=x.dtype)
        if (theta is not None or omega is not None) and phi_out is None:
            phi_out = torch.empty((Bt, H, N // 2), device=x.device, dtype=f32)
    a = _lib.PrefillArgs()
    a.Bt, a.L, a.H, a.P, a.N, a.R, a.chunk = Bt, L, H, P, N, R, chunk
    a.in_dtype = _dtype_code(x)
    a.layout = 1 if head_major else 0
    a.x = _ptr(x, x.dtype, big(P), "x")
    a.B = _ptr(B, x.dtype, big(N), "B")
    a.C = _ptr(C, x.dtype, big(N), "C")
    a.dt = _ptr(dt, f32, (Bt, L, H), "dt")
    a.lam = _ptr(lam, f32, (Bt, L, H), "lam")
    a.A = _ptr(A, f32, (H,), "A")
    a.A_tok = _ptr(A_tok, f32, (Bt, L, H), "A_tok")
    a.theta = _ptr(theta, f32, (Bt, L, H, N // 2), "theta")
    a.omega = _ptr(omega, f32, (Bt, L, N // 2), "omega")
    a.h0 = _ptr(h0, f32, (Bt, H, N, P), "h0")
    a.Bprev_rot = _ptr(Bprev_rot, f32, (Bt, H, R, N), "Bprev_rot")
    a.xprev = _ptr(xprev, x.dtype, (Bt, H, R, P), "xprev")
    a.phi0 = _ptr(phi0, f32, (Bt, H, N // 2), "phi0")
    a.y = _ptr(y, x.dtype, big(P), "y")
    a.h_final = _ptr(h_final, f32, (Bt, H, N, P), "h_final")
    a.Bprev_rot_out = _ptr(Bprev_rot_out, f32, (Bt, H, R, N), "Bprev_rot_out")
    a.xprev_out = _ptr(xprev_out, x.dtype, (Bt, H, R, P), "xprev_out")
    a.phi_out = _ptr(phi_out, f32, (Bt, H, N // 2), "phi_out")
    _prologue(a.pro, H, R, N, bc_norm, bc_eps, B_norm_w, C_norm_w, B_bias, C_bias, dt_softplus, dt_bias)
    lib = _lib.load()
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        rc = lib.m3_ssm_prefill_noalloc(ctypes.byref(a), _stream(stream))
        if rc != _lib.M3_OK:
            raise M3Error(rc, "m3_ssm_prefill_noalloc")
        return dict(y=y, h=h_final, Bprev_rot=Bprev_rot_out, xprev=xprev_out, phi=phi_out)
    if workspace is not False:
        need = lib.m3_ssm_prefill_workspace_size(ctypes.byref(a))
        if need > 0:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            a.workspace = _ptr(workspace, torch.uint8, None, "workspace")
            a.workspace_bytes = workspace.numel()
    rc = lib.m3_ssm_prefill(ctypes.byref(a), _stream(stream))
    if rc != _lib.M3_OK:
        raise M3Error(rc, "m3_ssm_prefill")
    return dict(y=y, h=h_final, Bprev_rot=Bprev_rot_out, xprev=xprev_out, phi=phi_out)


def m3_ssm_prefill_backward(x, B, C, dt, lam, A, theta=None, h0=None, Bprev_rot=None, xprev=None, phi0=None,
                            *, dy, dh_final=None, A_tok=None, want_carry_grads=False, workspace=None,
                            out=None, stream=None):
    """Gradients of the prefill for upstream dy [Bt,L,H,R,P] (bf16) and
    dh_final [Bt,H,N,P] (fp32, optional).  Forward inputs as for
    m3_ssm_prefill (bf16, token-major).  Returns a dict with dx, dB, dC (bf16),
    ddt, dlam (fp32 [Bt,L,H]), dA ([H], or [Bt,L,H] with A_tok), dtheta (with
    theta) and, with want_carry_grads, dh0, dBprev_rot, dxprev, dphi0.  `out`:
    optional dict of preallocated gradient tensors (any subset of those keys)."""
    Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    f32, dev = torch.float32, x.device
    given = out
    out = dict(dx=torch.empty_like(x), dB=torch.empty_like(B), dC=torch.empty_like(C),
               ddt=torch.empty((Bt, L, H), device=dev, dtype=f32), dlam=torch.empty((Bt, L, H), device=dev, dtype=f32),
               dA=torch.empty((Bt, L, H) if A_tok is not None else (H,), device=dev, dtype=f32),
               dtheta=None if theta is None else torch.empty_like(theta),
               dh0=None, dBprev_rot=None, dxprev=None, dphi0=None)
    if want_carry_grads:
        out["dh0"] = torch.empty((Bt, H, N, P), device=dev, dtype=f32)
        if Bprev_rot is not None:
            out["dBprev_rot"] = torch.empty((Bt, H, R, N), device=dev, dtype=f32)
            out["dxprev"] = torch.empty((Bt, H, R, P), device=dev, dtype=x.dtype)
        if theta is not None:
            out["dphi0"] = torch.empty((Bt, H, N // 2), device=dev, dtype=f32)
    for k, v in (given or {}).items():
        out[k] = v
    a = _lib.BackwardArgs()
    a.Bt, a.L, a.H, a.P, a.N, a.R = Bt, L, H, P, N, R
    a.in_dtype = _dtype_code(x)
    big = lambda D: (Bt, L, H, R, D)  # noqa: E731
    a.x = _ptr(x, x.dtype, big(P), "x")
    a.B = _ptr(B, x.dtype, big(N), "B")
    a.C = _ptr(C, x.dtype, big(N), "C")
    a.dt = _ptr(dt, f32, (Bt, L, H), "dt")
    a.lam = _ptr(lam, f32, (Bt, L, H), "lam")
    a.A = _ptr(A, f32, (H,), "A")
    a.A_tok = _ptr(A_tok, f32, (Bt, L, H), "A_tok")
    a.theta = _ptr(theta, f32, (Bt, L, H, N // 2), "theta")
    a.h0 = _ptr(h0, f32, (Bt, H, N, P), "h0")
    a.Bprev_rot = _ptr(Bprev_rot, f32, (Bt, H, R, N), "Bprev_rot")
    a.xprev = _ptr(xprev, x.dtype, (Bt, H, R, P), "xprev")
    a.phi0 = _ptr(phi0, f32, (Bt, H, N // 2), "phi0")
    a.dy = _ptr(dy, x.dtype, big(P), "dy")
    a.dh_final = _ptr(dh_final, f32, (Bt, H, N, P), "dh_final")
    shapes = dict(dx=big(P), dB=big(N), dC=big(N), ddt=(Bt, L, H), dlam=(Bt, L, H),
                  dA=(Bt, L, H) if A_tok is not None else (H,), dtheta=(Bt, L, H, N // 2), dh0=(Bt, H, N, P),
                  dBprev_rot=(Bt, H, R, N), dxprev=(Bt, H, R, P), dphi0=(Bt, H, N // 2))
    for k in ("dx", "dB", "dC", "dxprev"):
        setattr(a, k, _ptr(out[k], x.dtype, shapes[k], k))
    for k in ("ddt", "dlam", "dA", "dtheta", "dh0", "dBprev_rot", "dphi0"):
        setattr(a, k, _ptr(out[k], f32, shapes[k], k))
    lib = _lib.load()
    need = lib.m3_ssm_prefill_backward_workspace_size(ctypes.byref(a))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    a.workspace = _ptr(workspace, torch.uint8, None, "workspace")
    a.workspace_bytes = workspace.numel()
    rc = lib.m3_ssm_prefill_backward(ctypes.byref(a), _stream(stream))
    if rc != _lib.M3_OK:
        raise M3Error(rc, "m3_ssm_prefill_backward")
    return out


def backward_workspace_bytes(Bt, L, H, P, N, R, rope=False):
    """Bytes of the workspace m3_ssm_prefill_backward needs for this shape."""
    a = _lib.BackwardArgs()
    a.Bt, a.L, a.H, a.P, a.N, a.R = Bt, L, H, P, N, R
    a.theta = 1 if rope else None  # only NULL-ness is read
    return _lib.load().m3_ssm_prefill_backward_workspace_size(ctypes.byref(a))


def prefill_workspace_bytes(Bt, L, H, P, N, R, dtype=torch.bfloat16, rope=False):
    """Bytes of the optional prefill workspace for this shape (0: none used)."""
    a = _lib.PrefillArgs()
    a.Bt, a.L, a.H, a.P, a.N, a.R = Bt, L, H, P, N, R
    a.in_dtype = _lib.M3_BF16 if dtype == torch.bfloat16 else _lib.M3_F32
    a.theta = 1 if rope else None  # only NULL-ness is read
    return _lib.load().m3_ssm_prefill_workspace_size(ctypes.byref(a))


def m3_ssm_decode_step(h, phi, Bprev_rot, xprev, x, B, C, dt, lam, A, theta=None, *, y=None, A_tok=None,
                       omega=None, bc_norm=False, bc_eps=1e-6, B_norm_w=None, C_norm_w=None, B_bias=None,
                       C_bias=None, dt_softplus=False, dt_bias=None, stream=None):
    """One decode token.  In/out (updated in place): h [Bt,H,N,P] fp32,
    phi [Bt,H,N/2] fp32 (None iff theta None), Bprev_rot [Bt,H,R,N] fp32,
    xprev [Bt,H,R,P].  Inputs x [Bt,H,R,P], B/C [Bt,H,R,N], dt/lam [Bt,H],
    A [H] (or A_tok [Bt,H]: this token's A; then A may be None), theta
    [Bt,H,N/2] or None (or omega [Bt,N/2]: rates shared by the heads, theta =
    dt * omega).  The prologue arguments are those of m3_ssm_prefill.
    Returns y [Bt,H,R,P]."""
    Bt, H, R, P = x.shape
    N = B.shape[-1]
    f32 = torch.float32
    if y is None:
        y = torch.empty_like(x)
    a = _lib.DecodeArgs()
    a.Bt, a.H, a.P, a.N, a.R = Bt, H, P, N, R
    a.in_dtype = _dtype_code(x)
    a.h = _ptr(h, f32, (Bt, H, N, P), "h")
    a.phi = _ptr(phi, f32, (Bt, H, N // 2), "phi")
    a.Bprev_rot = _ptr(Bprev_rot, f32, (Bt, H, R, N), "Bprev_rot")
    a.xprev = _ptr(xprev, x.dtype, (Bt, H, R, P), "xprev")
    a.x = _ptr(x, x.dtype, (Bt, H, R, P), "x")
    a.B = _ptr(B, x.dtype, (Bt, H, R, N), "B")
    a.C = _ptr(C, x.dtype, (Bt, H, R, N), "C")
    a.dt = _ptr(dt, f32, (Bt, H), "dt")
    a.lam = _ptr(lam, f32, (Bt, H), "lam")
    a.A = _ptr(A, f32, (H,), "A")
    a.A_tok = _ptr(A_tok, f32, (Bt, H), "A_tok")
    a.theta = _ptr(theta, f32, (Bt, H, N // 2), "theta")
    a.omega = _ptr(omega, f32, (Bt, N // 2), "omega")
    a.y = _ptr(y, x.dtype, (Bt, H, R, P), "y")
    _prologue(a.pro, H, R, N, bc_norm, bc_eps, B_norm_w, C_norm_w, B_bias, C_bias, dt_softplus, dt_bias)
    rc = _lib.load().m3_ssm_decode_step(ctypes.byref(a), _stream(stream))
    if rc != _lib.M3_OK:
        raise M3Error(rc, "m3_ssm_decode_step")
    return y


def m3_rope_angles_cumsum(theta, phi0=None, *, phi=None, stream=None):
    """Inclusive cumulative angles phi = phi0 + cumsum(theta, dim=1).
    theta [Bt,L,H,J] fp32; phi0 [Bt,H,J] or None.  Returns phi [Bt,L,H,J]."""
    Bt, L, H, J = theta.shape
    if phi is None:
        phi = torch.empty_like(theta)
    pt = _ptr(theta, torch.float32, (Bt, L, H, J), "theta")
    pp = _ptr(phi0, torch.float32, (Bt, H, J), "phi0")
    po = _ptr(phi, torch.float32, (Bt, L, H, J), "phi")
    rc = _lib.load().m3_rope_angles_cumsum(pt, pp, po, Bt, L, H, J, _stream(stream))
    if rc != _lib.M3_OK:
        raise M3Error(rc, "m3_rope_angles_cumsum")
    return phi
