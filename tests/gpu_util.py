"""Helpers for the GPU parity tests: move seeded numpy inputs to the device
with the right storage dtype, call the library with NaN-filled outputs (so a
value the kernels never wrote cannot pass), and run the oracle on the same
bits, for all (batch, head) units or a sample of them."""
from __future__ import annotations

import numpy as np
import torch

from oracle import m3_oracle as orc

# Relative-L2 bars: fp32 inputs 2e-3, bf16 inputs 2e-2 (outputs and states).
TOL = {"f32": 2e-3, "bf16": 2e-2}
NAN = float("nan")


def dev(a, dtype=torch.float32):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def storage_dtype(s):
    return torch.bfloat16 if s.dtype == "bf16" else torch.float32


def to_device(d, s):
    st = storage_dtype(s)
    out = {}
    for k, v in d.items():
        if v is None:
            out[k] = None
        elif k in ("x", "B", "C", "xprev"):
            out[k] = dev(v, st)
        else:
            out[k] = dev(v)
    return out


def host(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def angle_diff(a, b):
    """Elementwise distance of two angle arrays modulo 2*pi."""
    d = np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)
    return np.abs(np.arctan2(np.sin(d), np.cos(d)))


def nan_like(t):
    return torch.full_like(t, NAN)


def prefill(ops, x, B, C, dt, lam, A, theta=None, h0=None, Bprev_rot=None, xprev=None, phi0=None, *,
            carry=True, head_major=False, **kw):
    """m3_ssm_prefill with every output preallocated and NaN-filled."""
    if head_major:
        Bt, H, L, R, P = x.shape
    else:
        Bt, L, H, R, P = x.shape
    N = B.shape[-1]
    f32 = dict(device=x.device, dtype=torch.float32)
    out = dict(y=nan_like(x), h_final=torch.full((Bt, H, N, P), NAN, **f32))
    if carry:
        out["Bprev_rot_out"] = torch.full((Bt, H, R, N), NAN, **f32)
        out["xprev_out"] = torch.full((Bt, H, R, P), NAN, device=x.device, dtype=x.dtype)
        if theta is not None or kw.get("omega") is not None:
            out["phi_out"] = torch.full((Bt, H, N // 2), NAN, **f32)
    return ops.m3_ssm_prefill(x, B, C, dt, lam, A, theta, h0, Bprev_rot, xprev, phi0, want_carry=carry,
                              head_major=head_major, **out, **kw)


def prefill_d(ops, dd, carry=True, **kw):
    """prefill() on a dict of device inputs (carry-in taken from it when present)."""
    return prefill(ops, dd["x"], dd["B"], dd["C"], dd["dt"], dd["lam"], dd["A"], dd.get("theta"), dd.get("h0"),
                   dd.get("Bprev_rot"), dd.get("xprev"), dd.get("phi0"), carry=carry, **kw)


def decode(ops, st, x, B, C, dt, lam, A, theta=None, **kw):
    """One m3_ssm_decode_step on the in/out state dict ``st`` with a NaN-filled y."""
    return ops.m3_ssm_decode_step(st["h"], st["phi"], st["Bprev_rot"], st["xprev"], x, B, C, dt, lam, A, theta,
                                  y=nan_like(x), **kw)


def sample_units(units, ranges=8, per_range=2):
    """(batch*head) unit indices spread over ``ranges`` equal ranges of the
    unit axis, ``per_range`` at scattered offsets in each.  The prefill deals
    its workgroups so that each of the 8 XCDs walks one such range."""
    out = []
    w = max(units // ranges, 1)
    for r in range(ranges):
        for k in range(per_range):
            off = (7 * r + 13 * k + 3 + k * (w // 2)) % w
            u = min(r * w + off, units - 1)
            if u not in out:
                out.append(u)
    return out


def pick_units(d, units, H):
    """Sub-problem with one batch item whose heads are the sampled (b, h) units:
    prefill-shaped inputs [Bt, L, H, ...] -> [1, L, k, ...]; [Bt, H, ...] carries
    -> [1, k, ...]; A [H] -> [k]."""
    bs = [u // H for u in units]
    hs = [u % H for u in units]
    out = {}
    for k, v in d.items():
        if v is None or k in ("omega", "dt_raw"):
            out[k] = None if k != "dt_raw" else v
            continue
        if k == "A":
            out[k] = v[hs]
        elif k in ("h0", "Bprev_rot", "xprev", "phi0"):
            out[k] = np.stack([v[b, h] for b, h in zip(bs, hs)])[None]
        else:  # [Bt, L, H, ...]
            out[k] = np.stack([v[b, :, h] for b, h in zip(bs, hs)], axis=1)[None]
    return out


def oracle_units(d, units, H):
    """The oracle on the sampled units only (results carry the unit on the head axis)."""
    s = pick_units(d, units, H)
    return orc.ssm_reference(**{k: s.get(k) for k in ("x", "B", "C", "dt", "lam", "A", "theta", "h0",
                                                       "Bprev_rot", "xprev", "phi0")})


def oracle_prefill(d, sel_b=None, sel_h=None):
    """Run the oracle, optionally on a subset of (batch, head) units."""
    def pick(a, kind):
        if a is None:
            return None
        if sel_b is not None and kind != "h":
            a = a[sel_b]
        if sel_h is not None:
            if kind == "bl":   # [Bt, L, H, ...]
                a = a[:, :, sel_h]
            elif kind == "h":  # [H]
                a = a[sel_h]
            else:              # [Bt, H, ...]
                a = a[:, sel_h]
        return a
    kinds = dict(x="bl", B="bl", C="bl", dt="bl", lam="bl", theta="bl", A="h",
                 h0="bh", Bprev_rot="bh", xprev="bh", phi0="bh")
    args = {k: pick(d.get(k), kinds[k]) for k in kinds}
    return orc.ssm_reference(**args)
