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
                       [--no-cpu-baseline] [--only prefill|decode|all|pmc]
       python bench.py --report-trace PREFIX          (rocprofv3 kernel trace -> markdown)
       python bench.py --report-pmc FETCH_PREFIX WRITE_PREFIX   (HBM counters -> markdown)

--only pmc runs the counter workload: a plain device copy of known size (the
scale for FETCH_SIZE / WRITE_SIZE), then two launches of each prefill kernel
and three decode steps, untimed.  PREFIX is the rocprofv3 output prefix
(-d DIR -o NAME gives DIR/NAME).
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
COPY_BYTES = 1 << 30                 # plain copy used to scale the HBM counters


def ANGLES_GRID(Bt, H, J):
    """Threads launched by the angle scan: 256 per 32 (head, pair) columns per batch item."""
    return Bt * ((H * J // 4 + 7) // 8) * 256


def prefill_kernel_name(Bt, L, H, P, N, R, rope, state_only=False):
    """Kernel symbol (as rocprofv3 prints it) that runs a bf16 prefill shape."""
    return (f"m3::pc::prefill_pc_kernel<{N}, {P}, {int(math.log2(R))}, {'true' if rope else 'false'}, "
            f"{'true' if state_only else 'false'}>")


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
    return f"m3::decode_step_kernel<m3::bf16_t, {N}, {P}, {4 if R <= 4 else 16}>"


def unit_kernels():
    """(unit key, kernel symbol, launch grid in threads) of every timed launch;
    a split prefill is several launches of one unit (the state-only walk of
    the first half, in two parts joined by the combine kernel when it is long
    enough, then both halves)."""
    out = []
    for name, shp in prefill_shapes().items():
        Bt, L, H, P, N, R, rope = shp
        if prefill_split(*shp):
            two = prefill_two_part(*shp)
            out.append(("prefill_" + name, prefill_kernel_name(*shp, state_only=True), (2 if two else 1) * Bt * H * 512))
            if two:
                out.append(("prefill_" + name, COMBINE_KERNEL, Bt * H * 256))  # grid x; y = 8 parts
            out.append(("prefill_" + name, prefill_kernel_name(*shp), 2 * Bt * H * 512))
        else:
            out.append(("prefill_" + name, prefill_kernel_name(*shp), Bt * H * 512))
    Bt, H, P, N, R = DECODE_SHAPE
    out.append(("decode", decode_kernel_name(Bt, H, P, N, R), Bt * H * 256))
    Bt, L, H, P, N, R, _ = prefill_shapes()["siso_rope"]
    out.append(("angles", "m3::angles_cumsum_kernel", ANGLES_GRID(Bt, H, N // 2)))
    return out


def prefill_algo(Bt, L, H, P, N, R, rope, omega=False, a_tok=False):
    """Algorithmic bytes (each input read once, each output written once) and
    MFMA flops (chunked-scan count 2L[Q R^2 (N+P) + 2 R N P] per (b,h), Q = 64/R).
    omega: the angles come as rates per token shared by the heads; a_tok: A is
    given per token."""
    bf, f4 = 2, 4
    tok = Bt * L * H
    byts = tok * R * (P + 2 * N) * bf + tok * 2 * f4 + (tok if a_tok else H) * f4   # x, B, C, dt, lam, A
    if rope:
        byts += (Bt * L if omega else tok) * (N // 2) * f4        # omega or theta
    byts += tok * R * P * bf                                      # y
    byts += Bt * H * N * P * f4                                   # h_final
    Q = Q_ROWS // R
    flops = Bt * H * 2 * L * (Q * R * R * (N + P) + 2 * R * N * P)
    return byts, flops


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
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dev, bf, f32 = "cuda", torch.bfloat16, torch.float32
    x = torch.randn((Bt, L, H, R, P), generator=g, device=dev, dtype=f32).to(bf)
    B = (torch.randn((Bt, L, H, R, N), generator=g, device=dev, dtype=f32) / math.sqrt(N)).to(bf)
    C = (torch.randn((Bt, L, H, R, N), generator=g, device=dev, dtype=f32) / math.sqrt(N)).to(bf)
    dt = torch.nn.functional.softplus(torch.randn((Bt, L, H), generator=g, device=dev) - 4.0).contiguous()
    lam = torch.sigmoid(torch.randn((Bt, L, H), generator=g, device=dev)).contiguous()
    A = (-torch.exp(torch.rand((H,), generator=g, device=dev) * math.log(16.0))).contiguous()
    theta = om = None
    if rope:
        om = torch.randn((Bt, L, N // 2), generator=g, device=dev)
        theta = (dt[:, :, :, None] * om[:, :, None, :]).contiguous()
    a_tok = (-torch.exp(torch.rand((Bt, L, H), generator=g, device=dev) * math.log(16.0))).contiguous()
    return dict(x=x, B=B, C=C, dt=dt, lam=lam, A=A, theta=theta, omega=om, A_tok=a_tok)


def time_prefill(torch, ops, inp, steps, warmup, mode=""):
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

    theta, omega = (None, inp["omega"]) if mode == "omega" else (inp["theta"], None)
    A, a_tok = (None, inp["A_tok"]) if mode == "atok" else (inp["A"], None)

    def run():
        ops.m3_ssm_prefill(inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], A, theta,
                           y=y, h_final=hf, workspace=ws, omega=omega, A_tok=a_tok, head_major=hm)

    for _ in range(max(warmup, 1)):
        run()
    torch.cuda.synchronize()
    ms = replay_ms(torch, [run] * steps)
    return ms, ms, flushed_ms(torch, run)


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


def time_decode(torch, ops, Bt, H, P, N, R, steps, warmup, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dev, bf, f32 = "cuda", torch.bfloat16, torch.float32
    S = steps + warmup
    x = torch.randn((S, Bt, H, R, P), generator=g, device=dev, dtype=f32).to(bf)
    B = (torch.randn((S, Bt, H, R, N), generator=g, device=dev, dtype=f32) / math.sqrt(N)).to(bf)
    C = (torch.randn((S, Bt, H, R, N), generator=g, device=dev, dtype=f32) / math.sqrt(N)).to(bf)
    dt = torch.nn.functional.softplus(torch.randn((S, Bt, H), generator=g, device=dev) - 4.0).contiguous()
    lam = torch.sigmoid(torch.randn((S, Bt, H), generator=g, device=dev)).contiguous()
    A = (-torch.exp(torch.rand((H,), generator=g, device=dev) * math.log(16.0))).contiguous()
    om = torch.randn((S, Bt, N // 2), generator=g, device=dev)
    theta = (dt[:, :, :, None] * om[:, :, None, :]).contiguous()
    h = (torch.randn((Bt, H, N, P), generator=g, device=dev) * 0.1).contiguous()
    phi = torch.zeros((Bt, H, N // 2), device=dev)
    Bp = torch.zeros((Bt, H, R, N), device=dev)
    xp = torch.zeros((Bt, H, R, P), device=dev, dtype=bf)
    y = torch.empty((Bt, H, R, P), device=dev, dtype=bf)

    def step(t):
        ops.m3_ssm_decode_step(h, phi, Bp, xp, x[t], B[t], C[t], dt[t], lam[t], A, theta[t], y=y)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    # the whole sequence of steps (each with its own token's inputs) is one graph
    per_step = replay_ms(torch, [(lambda t=t: step(t)) for t in range(warmup, warmup + steps)])
    ok = bool(torch.isfinite(h).all())
    return per_step, per_step, ok


def cpu_baseline(batch_items=6):
    """The fp64 oracle, as it stands, on a bounded sample of the headline
    prefill workload: `batch_items` sequences x all 32 heads x L 4096."""
    import dataclasses

    import numpy as np

    from oracle import m3_oracle as orc
    from synth.inputs import CONFIGS, SEED_BASE, make_inputs
    s = dataclasses.replace(CONFIGS[1], Bt=batch_items)
    d = make_inputs(s, SEED_BASE + 1)
    t0 = time.perf_counter()
    orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"])
    dt = time.perf_counter() - t0
    threads = 1
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([1] + [i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"])
    except Exception:
        pass
    return dict(value=s.Bt * s.L / dt, unit="tokens/s", cores=1,
                kind="oracle",
                sample=f"{s.Bt} sequences x L={s.L} x H={s.H} of the SISO real prefill (P=64, N=128), "
                       f"fp64 numpy token loop, {dt:.1f} s wall, single process (BLAS pool {threads})",
                seconds=dt)


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
    units = {(k, g): u for u, k, g in unit_kernels()}
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


def report_pmc(fetch_prefix, write_prefix):
    """HBM bytes per launch of each timed kernel: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled by what the same counter reads for the plain
    copy of COPY_BYTES in the counter workload."""
    def per_kernel(prefix, counter):
        acc = {}
        for r in _csv_rows(prefix + "_counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
            acc.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    fetch = per_kernel(fetch_prefix, "FETCH_SIZE")
    write = per_kernel(write_prefix, "WRITE_SIZE")

    def copy_value(acc):
        cands = [(k, v) for k, v in acc.items() if "neg_kernel" in k[0]]
        k, v = max(cands, key=lambda kv: max(kv[1]))
        return k[0], sum(v) / len(v)

    cname, cf = copy_value(fetch)
    _, cw = copy_value(write)
    sf, sw = COPY_BYTES / cf, COPY_BYTES / cw
    units = {}
    lines = [f"Scale: a plain elementwise copy (negation) of {COPY_BYTES} B (`{cname}`) reads FETCH_SIZE = {cf:.4g} B and "
             f"WRITE_SIZE = {cw:.4g} B, so the factors are {sf:.4f} (fetch) and {sw:.4f} (write).", "",
             "| unit | kernel | dispatches | FETCH_SIZE B | WRITE_SIZE B | scaled HBM B per launch "
             "| algorithmic B per launch | ratio |", "|---|---|---|---|---|---|---|---|"]
    algo = {}
    for name, shp in prefill_shapes().items():
        algo["prefill_" + name] = prefill_algo(*shp)[0]
    Bt, H, P, N, R = DECODE_SHAPE
    algo["decode"] = decode_algo(Bt, H, P, N, R, True)[0]
    Bt, L, H, P, N, R, _ = prefill_shapes()["siso_rope"]
    algo["angles"] = 2 * Bt * L * H * (N // 2) * 4 + Bt * H * (N // 2) * 4
    def find(acc, k, g):  # the counter file gives the total grid: 2-D launches match by name
        if (k, g) in acc:
            return acc[(k, g)]
        hits = [v for (kk, _), v in acc.items() if kk == k]
        return hits[0] if len(hits) == 1 else None

    for unit, k, g in unit_kernels():
        fv, wv = find(fetch, k, g), find(write, k, g)
        if not fv or not wv:
            continue
        f_avg, w_avg = sum(fv) / len(fv), sum(wv) / len(wv)
        tot = f_avg * sf + w_avg * sw
        e = units.setdefault(unit, {"bytes_per_launch": 0, "fetch_bytes": 0, "write_bytes": 0})
        e["bytes_per_launch"] += round(tot)  # per call of the entry point (all its launches)
        e["fetch_bytes"] += round(f_avg * sf)
        e["write_bytes"] += round(w_avg * sw)
        lines.append(f"| {unit} | `{k}` | {len(fv)} | {f_avg:.4g} | {w_avg:.4g} | {tot:.4g} | {algo[unit]:.4g} "
                     f"| {tot / algo[unit]:.3f} |")
    lines += ["", "Per call of the entry point (a split prefill is several launches):", "",
              "| unit | HBM bytes per call | algorithmic bytes | ratio |", "|---|---|---|---|"]
    for unit, e in units.items():
        lines.append(f"| {unit} | {e['bytes_per_launch']:.4g} | {algo[unit]:.4g} | {e['bytes_per_launch'] / algo[unit]:.3f} |")
    lines += ["", "traffic-json: " + json.dumps({"source_hash": kernel_source_hash(), "units": units,
                                                 "fetch_scale": sf, "write_scale": sw})]
    print("\n".join(lines))


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
    lines = ["| unit | kernel | dispatches | bf16 MFMA flops per launch (counter) | algorithmic flops per call "
             "| MFMA busy (% of SIMD cycles) |", "|---|---|---|---|---|---|"]
    for unit, k, g in unit_kernels():
        if not unit.startswith("prefill"):
            continue
        hits = acc.get((k, g)) or next((v for (kk, _), v in acc.items() if kk == k), None)
        if not hits or "SQ_VALU_MFMA_BUSY_CYCLES" not in hits:
            continue
        n = len(hits["SQ_VALU_MFMA_BUSY_CYCLES"])
        mops = sum(hits.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])) / n * 512
        busy = sum(hits["SQ_VALU_MFMA_BUSY_CYCLES"]) / n
        gui = sum(hits["GRBM_GUI_ACTIVE"]) / n / XCDS
        lines.append(f"| {unit} | `{k}` | {n} | {mops:.4g} | {algo[unit]:.4g} | {100 * busy / (gui * SIMDS):.1f} |")
    print("\n".join(lines))


def pmc_workload(torch, ops):
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
    for i, (name, shp) in enumerate(prefill_shapes().items()):
        inp = gen_prefill(torch, *shp, seed=20260100 + i)
        time_prefill(torch, ops, inp, 2, 0)
        del inp
        torch.cuda.empty_cache()
    Bt, L, H, P, N, R, _ = prefill_shapes()["siso_rope"]
    time_angles(torch, ops, Bt, L, H, N // 2, 2, 0, seed=20260110)
    Bt, H, P, N, R = DECODE_SHAPE
    time_decode(torch, ops, Bt, H, P, N, R, 3, 1, seed=20260104)
    torch.cuda.synchronize()
    print("# counter workload done", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=("all", "prefill", "decode", "pmc"), default="all")
    ap.add_argument("--report-trace", metavar="PREFIX")
    ap.add_argument("--report-pmc", nargs=2, metavar=("FETCH_PREFIX", "WRITE_PREFIX"))
    ap.add_argument("--report-mfma", metavar="PREFIX")
    args = ap.parse_args()
    if args.report_trace:
        report_trace(args.report_trace)
        return
    if args.report_pmc:
        report_pmc(*args.report_pmc)
        return
    if args.report_mfma:
        report_mfma(args.report_mfma)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU path is "
              "not built: (batch, head) units shard with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    import torch

    from state_space_sequence_ssm_amd import ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.only == "pmc":
        pmc_workload(torch, ops)
        return

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded, device-generated, resident in HBM)"}
    results = {}
    if args.only in ("all", "prefill"):
        # the RoPE workloads also with their angles given as rates (theta = dt * omega on
        # chip), and the headline workload with A given per token
        runs = [(name, shp, "") for name, shp in prefill_shapes().items()]
        runs += [(name + "_omega", shp, "omega") for name, shp in prefill_shapes().items() if shp[-1]]
        runs += [("siso_real_atok", prefill_shapes()["siso_real"], "atok")]
        # and the SISO workloads with x, B, C, y head-major ([Bt, H, L, R, .])
        runs += [(name + "_headmajor", prefill_shapes()[name], "hm") for name in ("siso_real", "siso_rope")]
        for i, (name, shp, mode) in enumerate(runs):
            Bt, L, H, P, N, R, rope = shp
            inp = gen_prefill(torch, Bt, L, H, P, N, R, rope, seed=20260100 + i)
            torch.cuda.synchronize()
            ms, launch_ms, flushed = time_prefill(torch, ops, inp, args.steps, args.warmup, mode)
            byts, flops = prefill_algo(*shp, omega=mode == "omega", a_tok=mode == "atok")
            angles = "RoPE, angles from rates" if mode == "omega" else ("RoPE" if rope else "real")
            if mode == "atok":
                angles += ", A per token"
            if mode == "hm":
                angles += ", head-major x/B/C/y"
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
        Bt, H, P, N, R = DECODE_SHAPE
        per_step, kern, ok = time_decode(torch, ops, Bt, H, P, N, R, args.decode_steps, 20, seed=20260104)
        byts, flops = decode_algo(Bt, H, P, N, R, True)
        results["decode"] = dict(
            workload=f"decode MIMO RoPE: Bt={Bt} H={H} P={P} N={N} R={R} bf16 inputs, fp32 state, "
                     f"{args.decode_steps} sequential steps",
            us_per_step=per_step * 1e3, kernel_us=kern * 1e3, gbs=byts / (kern * 1e-3) / 1e9,
            hbm_frac=byts / (kern * 1e-3) / 1e9 / HBM_PEAK_GBS, bytes=byts, flops=flops, finite=ok,
            traffic=traffic_for("decode"))
        print(f"# decode: {per_step * 1e3:.1f} us/step, {results['decode']['gbs']:.0f} GB/s "
              f"({100 * results['decode']['hbm_frac']:.1f}% HBM)", file=sys.stderr, flush=True)

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
        out["decode_roofline"] = {"bound": "hbm", "achieved": dres["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": dres["hbm_frac"], "traffic": traffic_for("decode"),
                                  "kernel": decode_kernel_name(*DECODE_SHAPE)}
    for k in ("siso_rope", "mimo_rope", "siso_rope_omega", "mimo_rope_omega", "siso_real_atok",
              "siso_real_headmajor", "siso_rope_headmajor"):
        if k in results:
            out["prefill_" + k] = results[k]
    if "angles" in results:
        out["angles"] = results["angles"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
