"""Benchmark of the Mamba-3 SSM core on one MI355X.

Headline (value): prefill tokens/s of the SISO real-valued prefill, batch 8 x
L 4096, H 32, P 64, N 128, R 1, bf16 inputs, fp32 state, chunk 64.  The same
JSON line also carries the MIMO decode step (B=256, H 32, N=P=64, R=4, 1000
sequential steps, us/step), the RoPE SISO and RoPE MIMO prefills, the
roofline of each kernel (algorithmic bytes and flops over the measured
average launch time), and the fp64 oracle timed on the host cores.

Inputs are synthetic and seeded, drawn on the device with the distributions
of the workloads (x ~ N(0,1); B, C ~ N(0,1)/sqrt(N); Delta = softplus(N(0,1)-4);
lambda = sigmoid(N(0,1)); A = -exp(U(0, ln 16)); theta = Delta * omega,
omega ~ N(0,1) per token and pair; decode state ~ N(0, 0.1^2)) and are
resident in HBM before timing starts.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps S]
                       [--no-cpu-baseline] [--only prefill|decode|all|headline|pmc]
                       [--group base|variants]
       python bench.py --report-trace PREFIX          (rocprofv3 kernel trace -> markdown)
       python bench.py --report-pmc FETCH_PREFIX WRITE_PREFIX [FETCH_PREFIX WRITE_PREFIX ...]
       python bench.py --report-counters PREFIX [PREFIX ...]   (memory-pipe counters -> markdown)

--only headline times the headline workload alone (its own rows in a kernel
trace).  --only pmc runs the counter workload of one --group: a plain device
copy of known size (the scale for FETCH_SIZE / WRITE_SIZE), then a few
untimed launches of each workload of the group ("base": the five workloads
and the decode control at Bt=512; "variants": the prefill lines with angles
as rates and A per token; "prologue": the prefill lines with the prologue
fused).  Within a group every workload runs a distinct
kernel symbol or grid, so counter rows map to workloads.  PREFIX is the
rocprofv3 output prefix (-d DIR -o NAME gives DIR/NAME).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + decode µs/step (B=256); % MFMA peak / % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 MFMA
Q_ROWS = 64                    # (token, rank) rows per chunk tile


def prefill_shapes():
    # (name, Bt, L, H, P, N, R, rope)
    return {
        "siso_real": (8, 4096, 32, 64, 128, 1, False),
        "siso_rope": (8, 4096, 32, 64, 64, 1, True),
        "mimo_rope": (4, 8192, 32, 64, 64, 4, True),
    }


DECODE_SHAPE = (256, 32, 64, 64, 4)  # Bt, H, P, N, R
# control: twice the batch, so the resident state (268 MB) exceeds the 256 MB Infinity Cache
DECODE_SHAPE_BIG = (512, 32, 64, 64, 4)
DECODE_BIG_STEPS = 200
# the decode at higher MIMO rank, the B=256 shape otherwise: rank-R update and
# readout (4 R N P flops per unit) against the same 32 KB state stream
DECODE_RANKS = {"decode_r8": (256, 32, 64, 64, 8), "decode_r16": (256, 32, 64, 64, 16)}
DECODE_RANK_STEPS = 200
COPY_BYTES = 1 << 30                 # plain copy used to scale the HBM counters

# prefill lines beside the plain workloads: (line name, workload, mode)
# mode "pro": the prologue fused in front of the core -- raw B, C (RMS
# normalisation with gains, head biases), raw step (softplus with a head bias)
# and, with RoPE, angles as rates
VARIANTS = [("siso_rope_omega", "siso_rope", "omega"), ("mimo_rope_omega", "mimo_rope", "omega"),
            ("siso_real_atok", "siso_real", "atok"), ("siso_real_prologue", "siso_real", "pro"),
            ("siso_rope_prologue", "siso_rope", "pro"), ("mimo_rope_prologue", "mimo_rope", "pro")]


def ANGLES_GRID(Bt, H, J):
    """Threads launched by the angle scan: 256 per 32 (head, pair) columns per batch item."""
    return Bt * ((H * J // 4 + 7) // 8) * 256


def prefill_kernel_name(Bt, L, H, P, N, R, rope, state_only=False, pro=False):
    """Kernel symbol (as rocprofv3 prints it) that runs a bf16 prefill shape."""
    return (f"m3::pc::prefill_pc_kernel<{N}, {P}, {int(math.log2(R))}, {'true' if rope else 'false'}, "
            f"{'true' if state_only else 'false'}, {'true' if pro else 'false'}>")


def prefill_split(Bt, L, H, P, N, R, rope, cus=256):
    """Whether the library splits the sequences of this bf16 shape in two (the
    rule of m3_ssm_prefill_workspace_size): fewer than half as many units as
    compute units and at least 8 chunks."""
    return 2 * Bt * H <= cus and L >= 8 * (64 // R)


def prefill_two_part(Bt, L, H, P, N, R, rope, cus=256):
    """Whether a split also walks the first half's state in two parts at once
    (the first half has at least 8 chunks)."""
    Q = 64 // R
    half = ((L + 1) // 2 + Q - 1) // Q * Q
    return prefill_split(Bt, L, H, P, N, R, rope, cus) and half >= 8 * Q


COMBINE_KERNEL = "m3::(anonymous namespace)::split_combine_kernel"


def decode_kernel_name(Bt, H, P, N, R):
    # bf16 decode steps run on the matrix cores (rank bound 4 or 16 in registers)
    return f"m3::dmma::decode_mma_kernel<{N}, {P}, {4 if R <= 4 else 16}>"


def decode_grid(N, P):
    """Threads per launch of the matrix-core decode: one workgroup of
    64 max(1, N P / 4096) threads per (batch, head)."""
    return 64 * max(1, (N // 16) * (P // 16) // 16)


def prefill_unit_kernels(key, shp, pro=False):
    """(unit key, kernel symbol, grid in threads) of the launches of one
    prefill call; a split prefill is several launches (the state-only walk of
    the first half, in two parts joined by the combine kernel when it is long
    enough, then both halves)."""
    Bt, L, H, P, N, R, rope = shp
    out = []
    if prefill_split(*shp):
        two = prefill_two_part(*shp)
        out.append((key, prefill_kernel_name(*shp, state_only=True, pro=pro), (2 if two else 1) * Bt * H * 512))
        if two:
            out.append((key, COMBINE_KERNEL, Bt * H * 256))  # grid x; y = 8 parts
        out.append((key, prefill_kernel_name(*shp, pro=pro), 2 * Bt * H * 512))
    else:
        out.append((key, prefill_kernel_name(*shp, pro=pro), Bt * H * 512))
    return out


def unit_kernels():
    """(unit key, kernel symbol, launch grid in threads) of every timed launch
    of the plain workloads."""
    out = []
    for name, shp in prefill_shapes().items():
        out += prefill_unit_kernels("prefill_" + name, shp)
    Bt, H, P, N, R = DECODE_SHAPE
    out.append(("decode", decode_kernel_name(Bt, H, P, N, R), Bt * H * decode_grid(N, P)))
    Bt, H, P, N, R = DECODE_SHAPE_BIG
    out.append(("decode_bt512", decode_kernel_name(Bt, H, P, N, R), Bt * H * decode_grid(N, P)))
    Bt, L, H, P, N, R, _ = prefill_shapes()["siso_rope"]
    out.append(("angles", "m3::angles_cumsum_kernel", ANGLES_GRID(Bt, H, N // 2)))
    return out


# counter groups of the variant lines: within a group every line runs
# distinct kernels (symbol and grid), so counter rows map to lines
GROUPS = {"variants": [v for v in VARIANTS if v[2] != "pro"], "prologue": [v for v in VARIANTS if v[2] == "pro"]}
# counter groups with no prefill variant: the decode at rank 8 and at rank 16
# (one kernel symbol and grid, so a run each) and the three backward lines
OTHER_GROUPS = ("decode_r8", "decode_r16", "backward")
ALL_GROUPS = ("base",) + tuple(GROUPS) + OTHER_GROUPS


def variant_unit_kernels(group=None):
    """unit_kernels() of the variant lines of `group` (all when None): the
    kernels of their workloads, compiled with the prologue for mode "pro"."""
    out = []
    for line, wl, mode in (VARIANTS if group is None else GROUPS[group]):
        out += prefill_unit_kernels("prefill_" + line, prefill_shapes()[wl], pro=mode == "pro")
    return out


def backward_split(Bt, L, H, P, N, R, rope, cus=256):
    """Split chunk of the library's backward for this shape, 0 when it does
    not split (the rule of m3_ssm_prefill_backward_workspace_size): at most
    half as many units as compute units and at least 8 chunks."""
    Q = 64 // R
    nch = (L + Q - 1) // Q
    if 2 * Bt * H > cus or nch < 8:
        return 0
    return min(max((nch * 11 + 10) // 20, 4), nch - 4)


SPLIT_JOIN_KERNEL = "m3::bw::split_join_kernel"


def backward_unit_kernels():
    """(unit key, kernel symbol, grid x in threads) of the backward lines: one
    512-thread workgroup per (batch, head), or with the split the pre and main
    launches (two segments in grid y) and the joining kernel; the per-head dA
    reduction is a few hundred bytes and left out."""
    out = []
    for name, shp in prefill_shapes().items():
        Bt, L, H, P, N, R, rope = shp
        cm = backward_split(*shp)
        if cm:
            out += [("backward_" + name, backward_kernel_name(rope, N, P, 1), Bt * H * 512),
                    ("backward_" + name, backward_kernel_name(rope, N, P, 2), Bt * H * 512),
                    ("backward_" + name, SPLIT_JOIN_KERNEL, (Bt * cm * (64 // R) if rope else 1) * 256)]
        else:
            out.append(("backward_" + name, backward_kernel_name(rope, N, P), Bt * H * 512))
    return out


def group_units(group):
    """(unit key, kernel symbol, grid) of every counted launch of a counter group."""
    if group == "base":
        return unit_kernels()
    if group in GROUPS:
        return variant_unit_kernels(group)
    if group in DECODE_RANKS:
        Bt, H, P, N, R = DECODE_RANKS[group]
        return [(group, decode_kernel_name(Bt, H, P, N, R), Bt * H * decode_grid(N, P))]
    if group == "backward":
        return backward_unit_kernels()
    raise ValueError(group)


def prefill_algo(Bt, L, H, P, N, R, rope, omega=False, a_tok=False, pro=False):
    """Algorithmic bytes (each input read once, each output written once) and
    MFMA flops (chunked-scan count 2L[Q R^2 (N+P) + 2 R N P] per (b,h), Q = 64/R).
    omega: the angles come as rates per token shared by the heads; a_tok: A is
    given per token; pro: the prologue's gains [2][N], biases [2][H][R][N] and
    step biases [H] are read too."""
    bf, f4 = 2, 4
    tok = Bt * L * H
    byts = tok * R * (P + 2 * N) * bf + tok * 2 * f4 + (tok if a_tok else H) * f4   # x, B, C, dt, lam, A
    if pro:
        byts += (2 * N + 2 * H * R * N + H) * f4
    if rope:
        byts += (Bt * L if omega else tok) * (N // 2) * f4        # omega or theta
    byts += tok * R * P * bf                                      # y
    byts += Bt * H * N * P * f4                                   # h_final
    Q = Q_ROWS // R
    flops = Bt * H * 2 * L * (Q * R * R * (N + P) + 2 * R * N * P)
    return byts, flops


def backward_algo(Bt, L, H, P, N, R, rope):
    """Algorithmic bytes and MFMA flops of the backward: x, B, C, dy (bf16),
    Delta, lambda (and theta) read once; dx, dB, dC (bf16), dDelta, dlambda
    (and dtheta) written once; A and dA per head.  Flops per chunk of Q
    tokens (64 rows) and (b, h): the two Gram products, S1^T dY, B G, S2^T C,
    X G^T, S2 B, dY H^T, the adjoint update and the forward state walk,
    2 * 64 * (3 * 64 N + 2 * 64 P + 5 N P)."""
    bf, f4 = 2, 4
    tok = Bt * L * H
    byts = (tok * R * (2 * P + 2 * N) * bf      # x, dy, B, C read
            + tok * R * (P + 2 * N) * bf        # dx, dB, dC written
            + 2 * tok * 2 * f4                  # Delta, lambda read; their gradients written
            + 2 * Bt * H * N * P * f4           # dh_final read, dh0 written
            + 2 * H * f4)                       # A read, dA written
    if rope:
        byts += 2 * tok * (N // 2) * f4        # theta read, dtheta written
    chunks = Bt * H * ((L + (64 // R) - 1) // (64 // R))
    flops = chunks * 2 * 64 * (3 * 64 * N + 2 * 64 * P + 5 * N * P)
    return byts, flops


def backward_kernel_name(rope, N, P, mode=0):
    """Backward kernel symbol: mode 0 the whole walk, 1 and 2 the split's pre
    and main launches."""
    return f"m3::bw::backward_kernel<{N}, {P}, {'true' if rope else 'false'}, {mode}>"


def time_backward(torch, ops, inp, steps, warmup):
    """Average duration of the backward of one prefill workload (gradients of
    every input; upstream dy drawn N(0,1) in bf16, dh_final N(0,1))."""
    g = torch.Generator(device="cuda")
    g.manual_seed(20260300)
    x = inp["x"]
    Bt, L, H, R, P = x.shape
    N = inp["B"].shape[-1]
    dy = torch.randn(x.shape, generator=g, device="cuda").to(torch.bfloat16)
    dhf = torch.randn((Bt, H, N, P), generator=g, device="cuda")
    out = ops.m3_ssm_prefill_backward(x, inp["B"], inp["C"], inp["dt"], inp["lam"], inp["A"], inp["theta"],
                                      dy=dy, dh_final=dhf)
    ws = torch.empty(ops.backward_workspace_bytes(Bt, L, H, P, N, R, rope=inp["theta"] is not None),
                     dtype=torch.uint8, device="cuda")

    def run():
        ops.m3_ssm_prefill_backward(x, inp["B"], inp["C"], inp["dt"], inp["lam"], inp["A"], inp["theta"], dy=dy,
                                    dh_final=dhf, workspace=ws, out=out)

    for _ in range(max(warmup, 1)):
        run()
    torch.cuda.synchronize()
    return replay_ms(torch, [run] * steps)


def decode_algo(Bt, H, P, N, R, rope):
    bf, f4 = 2, 4
    u = Bt * H
    byts = u * (2 * N * P * f4            # state read + write
                + R * (P + 2 * N) * bf    # x, B, C
                + 2 * R * N * f4          # rotated B carry read + write
                + 2 * R * P * bf          # x carry read + write
                + 2 * f4                  # dt, lam
                + R * P * bf)             # y
    if rope:
        byts += u * (3 * (N // 2) * f4)   # phi read + write, theta
    flops = u * (2 * 2 * R * N * P + 3 * N * P + 2 * R * N * P)
    return byts, flops


def gen_prefill(torch, Bt, L, H, P, N, R, rope, seed):
    from synth.device_inputs import prefill_inputs
    return prefill_inputs(Bt, L, H, P, N, R, rope, seed)


def time_prefill(torch, ops, inp, steps, warmup, mode="", flushed=True):
    hm = mode == "hm"  # x, B, C, y head-major [Bt, H, L, R, .]
    if hm:
        inp = dict(inp)
        for k in ("x", "B", "C"):
            inp[k] = inp[k].permute(0, 2, 1, 3, 4).contiguous()
    y = torch.empty_like(inp["x"])
    if hm:
        Bt, H, L, R, P = inp["x"].shape
    else:
        Bt, L, H, R, P = inp["x"].shape
    N = inp["B"].shape[-1]
    hf = torch.empty((Bt, H, N, P), device="cuda", dtype=torch.float32)

    # the optional workspace (sequence split when the units leave compute units idle)
    nws = ops.prefill_workspace_bytes(Bt, L, H, P, N, R, dtype=inp["x"].dtype, rope=inp["theta"] is not None)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else False

    theta, omega = (None, inp["omega"]) if mode in ("omega", "pro") else (inp["theta"], None)
    A, a_tok = (None, inp["A_tok"]) if mode == "atok" else (inp["A"], None)
    dt, pro = inp["dt"], {}
    if mode == "pro":  # raw step and pre-norm B, C; gains and biases drawn on the device
        g = torch.Generator(device="cuda")
        g.manual_seed(20260200)
        R_ = inp["x"].shape[3]
        dt = inp["dt_raw"]
        pro = dict(bc_norm=True, bc_eps=1e-6, dt_softplus=True,
                   B_norm_w=torch.rand((N,), generator=g, device="cuda") + 0.5,
                   C_norm_w=torch.rand((N,), generator=g, device="cuda") + 0.5,
                   B_bias=torch.randn((H, R_, N), generator=g, device="cuda") * 0.3,
                   C_bias=torch.randn((H, R_, N), generator=g, device="cuda") * 0.3,
                   dt_bias=torch.randn((H,), generator=g, device="cuda") * 0.5)

    def run():
        ops.m3_ssm_prefill(inp["x"], inp["B"], inp["C"], dt, inp["lam"], A, theta,
                           y=y, h_final=hf, workspace=ws, omega=omega, A_tok=a_tok, head_major=hm, **pro)

    for _ in range(max(warmup, 1)):
        run()
    torch.cuda.synchronize()
    ms = replay_ms(torch, [run] * steps)
    return ms, ms, (flushed_ms(torch, run) if flushed else None)


FLUSH_BYTES = 1 << 30  # four times the 256 MB Infinity Cache
FLUSHED_RUNS = 51


def flushed_ms(torch, run):
    """Median duration of single launches, each after a 1 GiB read that
    evicts the Infinity Cache, timed by HIP events on the launch stream.  The
    eviction reads rather than writes: a written buffer leaves dirty lines
    whose write-back to HBM overlaps the timed launch."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    acc = torch.zeros((), dtype=torch.float32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(FLUSHED_RUNS)]
    for e0, e1 in ev:
        acc += buf.sum()
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    del buf
    return statistics.median(e0.elapsed_time(e1) for e0, e1 in ev)


def time_angles(torch, ops, Bt, L, H, J, steps, warmup, seed):
    """Mean per-launch duration (ms) of the cumulative-angle scan and its
    algorithmic bytes (theta read once, phi written once, phi0 read once)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    theta = torch.randn((Bt, L, H, J), generator=g, device="cuda") * 0.05
    phi0 = torch.randn((Bt, H, J), generator=g, device="cuda")
    phi = torch.empty_like(theta)
    for _ in range(warmup):
        ops.m3_rope_angles_cumsum(theta, phi0, phi=phi)
    torch.cuda.synchronize()
    ms = replay_ms(torch, [lambda: ops.m3_rope_angles_cumsum(theta, phi0, phi=phi)] * steps)
    return ms, 2 * theta.numel() * 4 + phi0.numel() * 4


WARM_S = 0.06  # sustained untimed work before timing: the clocks ramp for ~25 ms


def replay_ms(torch, launches):
    """Average duration of the launches (callables, in order) on the GPU: they
    are captured once in a HIP graph, so no host work sits between kernels,
    replayed untimed until WARM_S of sustained work has passed (the GPU clocks
    ramp up under load), then replayed once between two HIP events on the
    replay stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for launch in launches:
                launch()
        t0 = time.perf_counter()
        while True:  # untimed replays
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= WARM_S:
                break
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / len(launches)


def time_decode(torch, ops, Bt, H, P, N, R, steps, warmup, seed, flushed=True):
    """Per-step time of `steps` sequential decode steps (each with its own
    token's inputs), captured in one graph; and the median of single steps,
    each after a 1 GiB read that evicts the Infinity Cache (the state then
    comes from HBM, not from the cache)."""
    from synth.device_inputs import DecodeStream
    gen = DecodeStream(Bt, H, P, N, R, seed)
    S = steps + warmup
    toks = [gen.step() for _ in range(S)]
    h = gen.h0
    phi = torch.zeros((Bt, H, N // 2), device="cuda")
    Bp = torch.zeros((Bt, H, R, N), device="cuda")
    xp = torch.zeros((Bt, H, R, P), device="cuda", dtype=torch.bfloat16)
    y = torch.empty((Bt, H, R, P), device="cuda", dtype=torch.bfloat16)

    def step(t):
        d = toks[t]
        ops.m3_ssm_decode_step(h, phi, Bp, xp, d["x"], d["B"], d["C"], d["dt"], d["lam"], gen.A, d["theta"], y=y)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    # the whole sequence of steps (each with its own token's inputs) is one graph
    per_step = replay_ms(torch, [(lambda t=t: step(t)) for t in range(warmup, warmup + steps)])
    ok = bool(torch.isfinite(h).all())
    ev = flushed_ms(torch, lambda: step(warmup)) if flushed else None
    return per_step, ev, ok


def _cpu_prefill_worker(item):
    """One sequence (all 32 heads, L 4096) of the headline workload through the
    oracle, single-threaded; returns its wall time."""
    import dataclasses
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass
    from oracle import m3_oracle as orc
    from synth.inputs import CONFIGS, SEED_BASE, make_inputs
    s = dataclasses.replace(CONFIGS[1], Bt=1)
    d = make_inputs(s, SEED_BASE + 1 + 1000 * item)
    t0 = time.perf_counter()
    orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"])
    return time.perf_counter() - t0


def _cpu_decode_worker(args):
    """`steps` oracle decode steps of the decode workload on `nb` of its batch
    items (all 32 heads), single-threaded; returns the wall time of the steps."""
    part, nb, steps = args
    import dataclasses
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass
    import numpy as np
    from oracle import m3_oracle as orc
    from synth.inputs import CONFIGS, SEED_BASE, make_inputs
    s = dataclasses.replace(CONFIGS[4], Bt=nb, L=steps)
    d = make_inputs(s, SEED_BASE + 4 + 1000 * part, h0=True)
    th = orc.angles_from_rates(d["dt"], d["omega"])
    h, R, N, P, H = d["h0"], s.R, s.N, s.P, s.H
    Bp = np.zeros((nb, H, R, N))
    xp = np.zeros((nb, H, R, P))
    phi = np.zeros((nb, H, N // 2))
    t0 = time.perf_counter()
    for t in range(steps):
        r = orc.decode_reference(h, Bp, xp, phi, d["x"][:, t], d["B"][:, t], d["C"][:, t], d["dt"][:, t],
                                 d["lam"][:, t], d["A"], th[:, t])
        h, Bp, xp, phi = r["h"], r["Bprev_rot"], r["xprev"], r["phi"]
    return time.perf_counter() - t0


CPU_WORKERS_MAX = 16  # the host-core share of one GPU on the benchmark boxes
CPU_DECODE_STEPS = 10


def cpu_baseline():
    """The fp64 oracle, as it stands, on a bounded sample of two workloads, in
    a pool of single-threaded worker processes (one per host core, at most
    CPU_WORKERS_MAX).  Run before anything touches the GPU: the workers are
    started from a process that has not initialised it.
    Prefill: one sequence of the headline workload per worker (all 32 heads,
    L 4096), tokens/s = all the sample's tokens / wall time.  Decode:
    CPU_DECODE_STEPS steps of the B=256 decode workload, its 256 batch items
    shared among the workers, s/step = wall time / steps."""
    import multiprocessing as mp
    workers = max(1, min(os.cpu_count() or 1, CPU_WORKERS_MAX))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        t0 = time.perf_counter()
        per = pool.map(_cpu_prefill_worker, range(workers))
        wall = time.perf_counter() - t0
        Bt4 = DECODE_SHAPE[0]
        parts = [(i, Bt4 // workers + (1 if i < Bt4 % workers else 0), CPU_DECODE_STEPS) for i in range(workers)]
        t1 = time.perf_counter()
        dper = pool.map(_cpu_decode_worker, [p for p in parts if p[1] > 0])
        dwall = time.perf_counter() - t1
    L = 4096
    return dict(value=workers * L / wall, unit="tokens/s", cores=workers, kind="oracle",
                sample=f"{workers} sequences x L={L} x H=32 of the SISO real prefill (P=64, N=128), one per "
                       f"single-threaded worker process, fp64 numpy token loop, {wall:.1f} s wall "
                       f"(per sequence {min(per):.1f}-{max(per):.1f} s); decode: {CPU_DECODE_STEPS} steps of "
                       f"B=256 H=32 P=N=64 R=4 over the same workers, {dwall:.1f} s wall",
                seconds=wall, decode_s_per_step=dwall / CPU_DECODE_STEPS,
                decode_step_seconds_per_worker=max(dper) / CPU_DECODE_STEPS)


def kernel_source_hash():
    """Hash of the kernel sources' code: comments and whitespace are dropped, so
    that a change of wording leaves the profiled figures valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "state_space_sequence_ssm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            h.update(f.encode() + b"\0" + " ".join(code.split()).encode())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")


def traffic_for(unit_key):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, if it was taken on the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    tag = "traffic-json:"
    if tag not in text:
        return None
    t = json.loads(text.split(tag, 1)[1].strip().splitlines()[0])
    if t.get("source_hash") != kernel_source_hash():
        return None
    e = t.get("units", {}).get(unit_key)
    return None if e is None else e["bytes_per_launch"]


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name):
    """Kernel symbol without its argument list (the last parenthesised group)."""
    name = name.replace("void ", "")
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        if name[i] == ")":
            depth += 1
        elif name[i] == "(":
            depth -= 1
            if depth == 0:
                return name[:i]
    return name


def report_trace(prefix):
    """Per-dispatch durations of the m3 kernels from a rocprofv3 kernel trace."""
    import statistics
    rows = _csv_rows(prefix + "_kernel_trace.csv")
    grp, meta = {}, {}
    for r in rows:
        if "m3::" not in r["Kernel_Name"]:
            continue
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]))
        grp.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
        meta[key] = (r["Workgroup_Size_X"], r["LDS_Block_Size"], r["VGPR_Count"], r["Accum_VGPR_Count"],
                     r["SGPR_Count"], r["Scratch_Size"])
    units = {}
    for cgroup in ALL_GROUPS:  # launches of several lines on one symbol and grid share a row
        for u, k, g in group_units(cgroup):
            if u not in units.get((k, g), ""):
                units[(k, g)] = units[(k, g)] + " / " + u if (k, g) in units else u
    lines = ["| unit | kernel | grid (threads) | block | calls | avg us | median us | min us | max us "
             "| LDS B | arch VGPR | acc VGPR | SGPR | scratch |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for (k, g), v in sorted(grp.items(), key=lambda kv: -sum(kv[1])):
        wg, lds, vg, ag, sg, sc = meta[(k, g)]
        lines.append(f"| {units.get((k, g), '-')} | `{k}` | {g} | {wg} | {len(v)} | {statistics.mean(v):.1f} "
                     f"| {statistics.median(v):.1f} | {min(v):.1f} | {max(v):.1f} | {lds} | {vg} | {ag} | {sg} "
                     f"| {sc} |")
    try:
        stats = _csv_rows(prefix + "_kernel_stats.csv")
        lines += ["", "`--stats` summary (m3 kernels, all grids of one symbol merged):", "",
                  "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in stats:
            if "m3::" in r["Name"]:
                lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} "
                             f"| {int(r['MinNs']) / 1e3:.1f} | {int(r['MaxNs']) / 1e3:.1f} |")
    except OSError:
        pass
    print("\n".join(lines))


def algo_bytes():
    """Algorithmic bytes per call of every counted unit."""
    algo = {}
    for name, shp in prefill_shapes().items():
        algo["prefill_" + name] = prefill_algo(*shp)[0]
    for line, wl, mode in VARIANTS:
        shp = prefill_shapes()[wl]
        algo["prefill_" + line] = prefill_algo(*shp, omega=mode == "omega" or (mode == "pro" and shp[-1]),
                                               a_tok=mode == "atok", pro=mode == "pro")[0]
    algo["decode"] = decode_algo(*DECODE_SHAPE, True)[0]
    algo["decode_bt512"] = decode_algo(*DECODE_SHAPE_BIG, True)[0]
    for key, shp in DECODE_RANKS.items():
        algo[key] = decode_algo(*shp, True)[0]
    for name, shp in prefill_shapes().items():
        algo["backward_" + name] = backward_algo(*shp)[0]
    Bt, L, H, P, N, R, _ = prefill_shapes()["siso_rope"]
    algo["angles"] = 2 * Bt * L * H * (N // 2) * 4 + Bt * H * (N // 2) * 4
    return algo


def report_pmc(groups):
    """HBM bytes per launch of each timed kernel: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled by what the same counter reads for the plain
    copy of COPY_BYTES in the counter workload.  `groups`: (group, fetch
    prefix, write prefix) of each counter run."""
    def per_kernel(prefix, counter):
        acc = {}
        for r in _csv_rows(prefix + "_counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
            acc.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    def copy_value(acc):
        cands = [(k, v) for k, v in acc.items() if "neg_kernel" in k[0]]
        k, v = max(cands, key=lambda kv: max(kv[1]))
        return k[0], sum(v) / len(v)

    def find(acc, k, g):  # the counter file gives the total grid: 2-D launches match by name
        if (k, g) in acc:
            return acc[(k, g)]
        hits = [v for (kk, _), v in acc.items() if kk == k]
        return hits[0] if len(hits) == 1 else None

    algo = algo_bytes()
    units, lines, scales = {}, [], {}
    rows = ["| unit | kernel | dispatches | FETCH_SIZE B | WRITE_SIZE B | scaled HBM B per launch "
            "| algorithmic B per launch | ratio |", "|---|---|---|---|---|---|---|---|"]
    for group, fp, wp in groups:
        fetch = per_kernel(fp, "FETCH_SIZE")
        write = per_kernel(wp, "WRITE_SIZE")
        cname, cf = copy_value(fetch)
        _, cw = copy_value(write)
        sf, sw = COPY_BYTES / cf, COPY_BYTES / cw
        scales[group] = (sf, sw)
        lines.append(f"Group {group}: a plain elementwise copy (negation) of {COPY_BYTES} B reads FETCH_SIZE = "
                     f"{cf:.4g} B and WRITE_SIZE = {cw:.4g} B, so the factors are {sf:.4f} (fetch) and "
                     f"{sw:.4f} (write).")
        for unit, k, g in group_units(group):
            fv, wv = find(fetch, k, g), find(write, k, g)
            if not fv or not wv:
                continue
            f_avg, w_avg = sum(fv) / len(fv), sum(wv) / len(wv)
            tot = f_avg * sf + w_avg * sw
            e = units.setdefault(unit, {"bytes_per_launch": 0, "fetch_bytes": 0, "write_bytes": 0})
            e["bytes_per_launch"] += round(tot)  # per call of the entry point (all its launches)
            e["fetch_bytes"] += round(f_avg * sf)
            e["write_bytes"] += round(w_avg * sw)
            rows.append(f"| {unit} | `{k}` | {len(fv)} | {f_avg:.4g} | {w_avg:.4g} | {tot:.4g} | {algo[unit]:.4g} "
                        f"| {tot / algo[unit]:.3f} |")
    lines += [""] + rows
    lines += ["", "Per call of the entry point (a split prefill is several launches):", "",
              "| unit | HBM bytes per call | algorithmic bytes | ratio |", "|---|---|---|---|"]
    for unit, e in units.items():
        lines.append(f"| {unit} | {e['bytes_per_launch']:.4g} | {algo[unit]:.4g} | {e['bytes_per_launch'] / algo[unit]:.3f} |")
    lines += ["", "traffic-json: " + json.dumps({"source_hash": kernel_source_hash(), "units": units,
                                                 "scales": scales})]
    print("\n".join(lines))


# Memory-pipe counters of the prefill kernels (one rocprofv3 pass each, within
# the per-block limits): what the vector memory path is doing per cycle.
COUNTER_PASSES = {
    "ta": ["TA_BUSY_avr", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "GRBM_GUI_ACTIVE"],
    "tcp": ["TCP_PENDING_STALL_CYCLES_sum", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum",
            "TCP_GATE_EN1_sum", "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_BUSY_CU_CYCLES",
            "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"],
}


def report_counters(prefixes):
    """Per-dispatch averages of the memory-pipe counters of every timed kernel,
    and derived ratios: TA busy share, L2 read latency per request (cycles),
    share of CU cycles the vector L1 holds pending requests, LDS bank-conflict
    cycles per LDS-active cycle."""
    vals = {}
    for prefix in prefixes:
        for r in _csv_rows(prefix + "_counter_collection.csv"):
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
            vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}
    lines = ["| unit | kernel | counter | average per dispatch |", "|---|---|---|---|"]
    derived = ["| unit | TA busy (% of GPU cycles, avg over TA) | TA address stalled by TC (cycles / CU / GPU cycle) "
               "| L2 read latency (cycles / request) | vector-L1 pending stall (cycles / CU / GPU cycle) "
               "| LDS bank-conflict / LDS-active cycles |", "|---|---|---|---|---|---|"]
    seen = set()
    for unit, k, g in [u for grp in ALL_GROUPS for u in group_units(grp)]:
        a = avg.get((k, g)) or next((v for (kk, _), v in avg.items() if kk == k), None)
        if a is None or (k, g) in seen:
            continue
        seen.add((k, g))
        for c in sorted(a):
            lines.append(f"| {unit} | `{k}` | {c} | {a[c]:.4g} |")
        gui = a.get("GRBM_GUI_ACTIVE", float("nan")) / XCDS
        cus = SIMDS // 4

        def ratio(n, d):
            return f"{n / d:.3g}" if n == n and d and d == d else "-"
        derived.append(
            f"| {unit} | {ratio(100 * a.get('TA_BUSY_avr', float('nan')), gui)} "
            f"| {ratio(a.get('TA_ADDR_STALLED_BY_TC_CYCLES_sum', float('nan')), gui * cus)} "
            f"| {ratio(a.get('TCP_TCC_READ_REQ_LATENCY_sum', float('nan')), a.get('TCP_TCC_READ_REQ_sum', 0))} "
            f"| {ratio(a.get('TCP_PENDING_STALL_CYCLES_sum', float('nan')), gui * cus)} "
            f"| {ratio(a.get('SQ_LDS_BANK_CONFLICT', float('nan')), a.get('SQ_LDS_IDX_ACTIVE', 0))} |")
    print("\n".join(derived + [""] + lines))


SIMDS = 1024  # 256 CUs x 4 SIMDs
XCDS = 8


def report_mfma(prefix):
    """MFMA counters of each timed kernel: bf16 flops executed (MOPS_BF16 x 512)
    against the algorithmic count, and MFMA-busy cycles as a share of the
    SIMD cycles of the dispatch (the MfmaUtil expression of rocprofv3)."""
    acc = {}
    for r in _csv_rows(prefix + "_counter_collection.csv"):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
        acc.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    algo = {"prefill_" + name: prefill_algo(*shp)[1] for name, shp in prefill_shapes().items()}
    for name, shp in prefill_shapes().items():
        algo["backward_" + name] = backward_algo(*shp)[1]
    algo["decode"] = decode_algo(*DECODE_SHAPE, True)[1]
    algo["decode_bt512"] = decode_algo(*DECODE_SHAPE_BIG, True)[1]
    for key, shp in DECODE_RANKS.items():
        algo[key] = decode_algo(*shp, True)[1]
    lines = ["| unit | kernel | dispatches | bf16 MFMA flops per launch (counter) | algorithmic flops per call "
             "| MFMA busy (% of SIMD cycles) |", "|---|---|---|---|---|---|"]
    seen = set()
    for unit, k, g in [u for grp in ALL_GROUPS for u in group_units(grp)]:
        if unit not in algo or (k, g) in seen or "combine" in k:
            continue
        seen.add((k, g))
        hits = acc.get((k, g)) or next((v for (kk, _), v in acc.items() if kk == k), None)
        if not hits or "SQ_VALU_MFMA_BUSY_CYCLES" not in hits:
            continue
        n = len(hits["SQ_VALU_MFMA_BUSY_CYCLES"])
        mops = sum(hits.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])) / n * 512
        busy = sum(hits["SQ_VALU_MFMA_BUSY_CYCLES"]) / n
        gui = sum(hits["GRBM_GUI_ACTIVE"]) / n / XCDS
        lines.append(f"| {unit} | `{k}` | {n} | {mops:.4g} | {algo[unit]:.4g} | {100 * busy / (gui * SIMDS):.1f} |")
    print("\n".join(lines))


def pmc_workload(torch, ops, group):
    """Untimed launches for counter collection (see the module docstring)."""
    # same-dtype copy_ becomes a DMA transfer, so the plain copy kernel is an
    # elementwise negation: it reads COPY_BYTES and writes COPY_BYTES
    a = torch.ones(COPY_BYTES // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()
    if group in DECODE_RANKS:
        print(f"# counter workload: {group}", file=sys.stderr, flush=True)
        time_decode(torch, ops, *DECODE_RANKS[group], 3, 1, seed=20260104, flushed=False)
        torch.cuda.synchronize()
        print("# counter workload done", file=sys.stderr, flush=True)
        return
    if group == "backward":
        for i, (name, shp) in enumerate(prefill_shapes().items()):
            print(f"# counter workload: backward {name}", file=sys.stderr, flush=True)
            inp = gen_prefill(torch, *shp, seed=20260300 + i)
            time_backward(torch, ops, inp, 2, 0)
            del inp
            torch.cuda.empty_cache()
        torch.cuda.synchronize()
        print("# counter workload done", file=sys.stderr, flush=True)
        return
    if group == "base":
        runs = [(name, shp, "") for name, shp in prefill_shapes().items()]
    else:
        runs = [(line, prefill_shapes()[wl], mode) for line, wl, mode in GROUPS[group]]
    for i, (name, shp, mode) in enumerate(runs):
        print(f"# counter workload: prefill {name}", file=sys.stderr, flush=True)
        inp = gen_prefill(torch, *shp, seed=20260100 + i)
        time_prefill(torch, ops, inp, 2, 0, mode, flushed=False)
        del inp
        torch.cuda.empty_cache()
    if group == "base":
        Bt, L, H, P, N, R, _ = prefill_shapes()["siso_rope"]
        time_angles(torch, ops, Bt, L, H, N // 2, 2, 0, seed=20260110)
        for shp in (DECODE_SHAPE, DECODE_SHAPE_BIG):
            print(f"# counter workload: decode {shp}", file=sys.stderr, flush=True)
            time_decode(torch, ops, *shp, 3, 1, seed=20260104, flushed=False)
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    print("# counter workload done", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=("all", "prefill", "decode", "headline", "backward", "pmc"), default="all")
    ap.add_argument("--group", choices=ALL_GROUPS, default="base")
    ap.add_argument("--report-trace", metavar="PREFIX")
    ap.add_argument("--report-pmc", nargs="+", metavar="GROUP FETCH_PREFIX WRITE_PREFIX")
    ap.add_argument("--report-mfma", metavar="PREFIX")
    ap.add_argument("--report-counters", nargs="+", metavar="PREFIX")
    args = ap.parse_args()
    if args.report_trace:
        report_trace(args.report_trace)
        return
    if args.report_pmc:
        a = args.report_pmc
        if len(a) % 3:
            ap.error("--report-pmc takes GROUP FETCH_PREFIX WRITE_PREFIX triples")
        report_pmc([tuple(a[i:i + 3]) for i in range(0, len(a), 3)])
        return
    if args.report_mfma:
        report_mfma(args.report_mfma)
        return
    if args.report_counters:
        report_counters(args.report_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU path is "
              "not built: (batch, head) units shard with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    # the CPU baseline's worker processes start before anything touches the GPU
    cpu = None
    if args.only == "all" and not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
        print(f"# cpu baseline: {cpu['value']:.0f} tokens/s on {cpu['cores']} cores, "
              f"decode {cpu['decode_s_per_step']:.3f} s/step", file=sys.stderr, flush=True)

    import torch

    from state_space_sequence_ssm_amd import ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.only == "pmc":
        pmc_workload(torch, ops, args.group)
        return

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded, device-generated, resident in HBM)"}
    results = {}
    if args.only in ("all", "prefill", "headline"):
        runs = [(name, shp, "") for name, shp in prefill_shapes().items()]
        # the RoPE workloads also with their angles given as rates (theta = dt * omega on
        # chip), and the headline workload with A given per token
        runs += [(line, prefill_shapes()[wl], mode) for line, wl, mode in VARIANTS]
        if args.only == "headline":
            runs = runs[:1]
        for i, (name, shp, mode) in enumerate(runs):
            Bt, L, H, P, N, R, rope = shp
            inp = gen_prefill(torch, Bt, L, H, P, N, R, rope, seed=20260100 + i)
            torch.cuda.synchronize()
            ms, launch_ms, flushed = time_prefill(torch, ops, inp, args.steps, args.warmup, mode)
            byts, flops = prefill_algo(*shp, omega=mode == "omega" or (mode == "pro" and rope),
                                       a_tok=mode == "atok", pro=mode == "pro")
            angles = "RoPE, angles from rates" if (mode == "omega" or (mode == "pro" and rope)) else (
                "RoPE" if rope else "real")
            if mode == "atok":
                angles += ", A per token"
            if mode == "pro":
                angles += ", prologue fused (B/C RMS norm with gains and head biases, Delta = softplus(raw + bias))"
            res = dict(workload=f"prefill {name}: Bt={Bt} L={L} H={H} P={P} N={N} R={R} "
                                f"{angles} bf16 chunk {Q_ROWS // R}",
                       tokens_per_s=Bt * L / (ms * 1e-3), ms_per_step=ms, kernel_ms=launch_ms,
                       gbs=byts / (launch_ms * 1e-3) / 1e9, tflops=flops / (launch_ms * 1e-3) / 1e12,
                       bytes=byts, flops=flops, flushed_ms=flushed)
            res["hbm_frac"] = res["gbs"] / HBM_PEAK_GBS
            res["traffic"] = traffic_for("prefill_" + name)
            res["mfma_frac"] = res["tflops"] / MFMA_BF16_PEAK_TFS
            res["roofline_frac"] = max(byts / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFS * 1e12)) / (
                launch_ms * 1e-3)
            results[name] = res
            print(f"# {res['workload']}: {ms:.3f} ms/step, {res['tokens_per_s']:.3e} tok/s, "
                  f"{res['gbs']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% HBM), "
                  f"{res['tflops']:.1f} TFLOP/s ({100 * res['mfma_frac']:.2f}% MFMA); "
                  f"{flushed:.3f} ms per launch after an Infinity Cache eviction", file=sys.stderr, flush=True)
            del inp
            torch.cuda.empty_cache()
    if args.only in ("all", "prefill", "backward"):
        for i, (name, shp) in enumerate(prefill_shapes().items()):
            Bt, L, H, P, N, R, rope = shp
            inp = gen_prefill(torch, Bt, L, H, P, N, R, rope, seed=20260400 + i)
            ms = time_backward(torch, ops, inp, max(args.steps // 5, 3), max(args.warmup // 5, 1))
            byts, flops = backward_algo(*shp)
            res = dict(workload=f"backward {name}: Bt={Bt} L={L} H={H} P={P} N={N} R={R} "
                                f"{'RoPE' if rope else 'real'} bf16, gradients of x, B, C, Delta, lambda, A"
                                f"{', theta' if rope else ''}",
                       tokens_per_s=Bt * L / (ms * 1e-3), ms_per_step=ms, gbs=byts / (ms * 1e-3) / 1e9,
                       tflops=flops / (ms * 1e-3) / 1e12, bytes=byts, flops=flops,
                       kernel=backward_kernel_name(rope, N, P, 2 if backward_split(*shp) else 0),
                       traffic=traffic_for("backward_" + name))
            res["hbm_frac"] = res["gbs"] / HBM_PEAK_GBS
            res["mfma_frac"] = res["tflops"] / MFMA_BF16_PEAK_TFS
            results["backward_" + name] = res
            print(f"# {res['workload']}: {ms:.3f} ms, {res['tokens_per_s']:.3e} tok/s, {res['gbs']:.0f} GB/s "
                  f"({100 * res['hbm_frac']:.1f}% HBM), {res['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
            del inp
            torch.cuda.empty_cache()
    if args.only in ("all", "prefill"):
        Bt, L, H, P, N, R, _ = prefill_shapes()["siso_rope"]
        ms, byts = time_angles(torch, ops, Bt, L, H, N // 2, args.steps, args.warmup, seed=20260110)
        results["angles"] = dict(workload=f"cumulative angles: theta [{Bt},{L},{H},{N // 2}] fp32",
                                 kernel_ms=ms, gbs=byts / (ms * 1e-3) / 1e9, bytes=byts,
                                 hbm_frac=byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 traffic=traffic_for("angles"))
        print(f"# {results['angles']['workload']}: {ms * 1e3:.1f} us, {results['angles']['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
    if args.only in ("all", "decode"):
        lines = [("decode", DECODE_SHAPE, args.decode_steps),
                 ("decode_bt512", DECODE_SHAPE_BIG, min(DECODE_BIG_STEPS, args.decode_steps))]
        lines += [(k, shp, min(DECODE_RANK_STEPS, args.decode_steps)) for k, shp in DECODE_RANKS.items()]
        for key, shp, nsteps in lines:
            Bt, H, P, N, R = shp
            per_step, ev, ok = time_decode(torch, ops, Bt, H, P, N, R, nsteps, 20, seed=20260104)
            byts, flops = decode_algo(Bt, H, P, N, R, True)
            state_mb = Bt * H * N * P * 4 / 1e6
            results[key] = dict(
                workload=f"decode MIMO RoPE: Bt={Bt} H={H} P={P} N={N} R={R} bf16 inputs, fp32 state "
                         f"({state_mb:.0f} MB), {nsteps} sequential steps",
                us_per_step=per_step * 1e3, kernel_us=per_step * 1e3, gbs=byts / (per_step * 1e-3) / 1e9,
                hbm_frac=byts / (per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, bytes=byts, flops=flops, finite=ok,
                us_after_cache_eviction=ev * 1e3,
                gbs_after_cache_eviction=byts / (ev * 1e-3) / 1e9,
                tflops=flops / (per_step * 1e-3) / 1e12,
                kernel=decode_kernel_name(Bt, H, P, N, R),
                traffic=traffic_for(key))
            print(f"# {key}: {per_step * 1e3:.1f} us/step, {results[key]['gbs']:.0f} GB/s "
                  f"({100 * results[key]['hbm_frac']:.1f}% HBM, {results[key]['tflops']:.1f} TFLOP/s on the "
                  f"matrix cores); {ev * 1e3:.1f} us per single step after an "
                  f"Infinity Cache eviction", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()

    head = results.get("siso_real")
    if head is not None:
        out["value"] = head["tokens_per_s"]
        out["unit"] = "tokens/s"
        out["ms_per_step"] = head["ms_per_step"]
        out["config"] = {"workload": head["workload"], "global_batch": 8, "seq_len": 4096}
        tr = traffic_for("prefill_siso_real")
        out["roofline"] = {"bound": "hbm", "achieved": head["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": head["hbm_frac"], "traffic": tr,
                           "kernel": prefill_kernel_name(*prefill_shapes()["siso_real"]),
                           "split": prefill_split(*prefill_shapes()["siso_real"]),
                           "algorithmic_bytes_per_launch": head["bytes"],
                           "mfma_tflops": head["tflops"], "mfma_frac": head["mfma_frac"],
                           "ms_after_cache_eviction": head["flushed_ms"]}
    elif "decode" in results:
        dres = results["decode"]
        out["value"] = dres["us_per_step"]
        out["unit"] = "us/step"
        out["higher_is_better"] = False
        out["ms_per_step"] = dres["us_per_step"] * 1e-3
        out["config"] = {"workload": dres["workload"]}
    if "decode" in results:
        dres = results["decode"]
        out["decode"] = dres
        # the rate that the state streams from HBM: the slower of the graph-replayed
        # steps (state possibly resident in the Infinity Cache between steps) and
        # single steps after an eviction
        hbm_gbs = min(dres["gbs"], dres["gbs_after_cache_eviction"])
        out["decode_roofline"] = {"bound": "hbm", "achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": hbm_gbs / HBM_PEAK_GBS, "traffic": traffic_for("decode"),
                                  "kernel": decode_kernel_name(*DECODE_SHAPE),
                                  "achieved_graph_replay": dres["gbs"],
                                  "achieved_after_cache_eviction": dres["gbs_after_cache_eviction"]}
    for key in ["decode_bt512"] + list(DECODE_RANKS):
        if key in results:
            out[key] = results[key]
    for name in prefill_shapes():
        if "backward_" + name in results:
            out["backward_" + name] = results["backward_" + name]
    for k in ["siso_rope", "mimo_rope"] + [line for line, _, _ in VARIANTS]:
        if k in results:
            out["prefill_" + k] = results[k]
    if "angles" in results:
        out["angles"] = results["angles"]
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
