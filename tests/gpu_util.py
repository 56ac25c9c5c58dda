"""Helpers for the GPU parity tests: move seeded numpy inputs to the device
with the right storage dtype and run the oracle on the same bits."""
from __future__ import annotations

import numpy as np
import torch

from oracle import m3_oracle as orc

# Relative-L2 bars: fp32 inputs 2e-3, bf16 inputs 2e-2 (outputs and states).
TOL = {"f32": 2e-3, "bf16": 2e-2}


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
    args = {k: pick(d[k], kinds[k]) for k in kinds}
    return orc.ssm_reference(**args)
