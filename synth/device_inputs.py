"""Seeded synthetic inputs drawn on the GPU with torch (same distributions as
synth.inputs), for workloads too large to draw on the host: the benchmark
and the full-size decode chain.  Like synth.inputs it only draws random
tensors; it holds none of the method's arithmetic (the angles theta of the
decode stream are the fp32 product Delta * omega of two drawn tensors, the
input recipe of the rotating workloads, and are checked bit for bit against
the oracle's angles_from_rates by the tests that use them).

Distributions: x ~ N(0,1); B, C ~ N(0,1)/sqrt(N); Delta = softplus(z - 4);
lambda = sigmoid(z'); A = -exp(U(0, ln 16)) per head; omega ~ N(0,1) per
token and state pair, shared by the heads; decode state h0 ~ N(0, 0.1^2).
"""
from __future__ import annotations

import math

import torch


def prefill_inputs(Bt, L, H, P, N, R, rope, seed, device="cuda", dtype=torch.bfloat16):
    """One prefill batch resident on the device: x [Bt,L,H,R,P], B, C
    [Bt,L,H,R,N] (dtype), dt, dt_raw, lam, A_tok [Bt,L,H], A [H], and with
    rope omega [Bt,L,N/2] and theta [Bt,L,H,N/2] (fp32)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    x = torch.randn((Bt, L, H, R, P), generator=g, device=device, dtype=f32).to(dtype)
    B = (torch.randn((Bt, L, H, R, N), generator=g, device=device, dtype=f32) / math.sqrt(N)).to(dtype)
    C = (torch.randn((Bt, L, H, R, N), generator=g, device=device, dtype=f32) / math.sqrt(N)).to(dtype)
    dt_raw = (torch.randn((Bt, L, H), generator=g, device=device) - 4.0).contiguous()
    dt = torch.nn.functional.softplus(dt_raw).contiguous()
    lam = torch.sigmoid(torch.randn((Bt, L, H), generator=g, device=device)).contiguous()
    A = (-torch.exp(torch.rand((H,), generator=g, device=device) * math.log(16.0))).contiguous()
    theta = om = None
    if rope:
        om = torch.randn((Bt, L, N // 2), generator=g, device=device)
        theta = (dt[:, :, :, None] * om[:, :, None, :]).contiguous()
    a_tok = (-torch.exp(torch.rand((Bt, L, H), generator=g, device=device) * math.log(16.0))).contiguous()
    return dict(x=x, B=B, C=C, dt=dt, dt_raw=dt_raw, lam=lam, A=A, theta=theta, omega=om, A_tok=a_tok)


class DecodeStream:
    """Per-step decode inputs drawn on the device in a fixed order from one
    seeded generator: the initial state first, then step by step x, B, C
    (dtype), z_Delta, z_lambda and omega.  theta = Delta * omega (fp32)."""

    def __init__(self, Bt, H, P, N, R, seed, device="cuda", dtype=torch.bfloat16):
        self.shape = (Bt, H, P, N, R)
        self.device, self.dtype = device, dtype
        self.g = torch.Generator(device=device)
        self.g.manual_seed(seed)
        g = self.g
        self.A = (-torch.exp(torch.rand((H,), generator=g, device=device) * math.log(16.0))).contiguous()
        self.h0 = (torch.randn((Bt, H, N, P), generator=g, device=device) * 0.1).contiguous()

    def step(self):
        Bt, H, P, N, R = self.shape
        g, dev, f32 = self.g, self.device, torch.float32
        x = torch.randn((Bt, H, R, P), generator=g, device=dev, dtype=f32).to(self.dtype)
        B = (torch.randn((Bt, H, R, N), generator=g, device=dev, dtype=f32) / math.sqrt(N)).to(self.dtype)
        C = (torch.randn((Bt, H, R, N), generator=g, device=dev, dtype=f32) / math.sqrt(N)).to(self.dtype)
        dt = torch.nn.functional.softplus(torch.randn((Bt, H), generator=g, device=dev) - 4.0).contiguous()
        lam = torch.sigmoid(torch.randn((Bt, H), generator=g, device=dev)).contiguous()
        om = torch.randn((Bt, N // 2), generator=g, device=dev)
        theta = (dt[:, :, None] * om[:, None, :]).contiguous()
        return dict(x=x, B=B, C=C, dt=dt, lam=lam, omega=om, theta=theta)
