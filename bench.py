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
                       [--no-cpu-baseline] [--only prefill|decode|all]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
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


def prefill_algo(Bt, L, H, P, N, R, rope):
    """Algorithmic bytes (each input read once, each output written once) and
    MFMA flops (chunked-scan count 2L[Q R^2 (N+P) + 2 R N P] per (b,h), Q = 64/R)."""
    bf, f4 = 2, 4
    tok = Bt * L * H
    byts = tok * R * (P + 2 * N) * bf + tok * 2 * f4 + H * f4   # x, B, C, dt, lam, A
    if rope:
        byts += tok * (N // 2) * f4                               # theta
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
    theta = None
    if rope:
        om = torch.randn((Bt, L, N // 2), generator=g, device=dev)
        theta = (dt[:, :, :, None] * om[:, :, None, :]).contiguous()
    return dict(x=x, B=B, C=C, dt=dt, lam=lam, A=A, theta=theta)


def time_prefill(torch, ops, inp, steps, warmup):
    y = torch.empty_like(inp["x"])
    Bt, L, H, R, P = inp["x"].shape
    N = inp["B"].shape[-1]
    hf = torch.empty((Bt, H, N, P), device="cuda", dtype=torch.float32)

    def run():
        ops.m3_ssm_prefill(inp["x"], inp["B"], inp["C"], inp["dt"], inp["lam"], inp["A"], inp["theta"],
                           y=y, h_final=hf)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    # per-launch HIP events on the launch stream (torch's current stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    return total_ms / steps, sum(launch_ms) / len(launch_ms), wall


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
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # a few individually bracketed launches give the kernel-only duration
    nk = min(50, steps)
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nk)]
    start.record()
    for i in range(steps):
        if i < nk:
            kev[i][0].record()
        step(warmup + i)
        if i < nk:
            kev[i][1].record()
    end.record()
    torch.cuda.synchronize()
    per_step = start.elapsed_time(end) / steps
    kern = sum(a.elapsed_time(b) for a, b in kev) / nk
    ok = bool(torch.isfinite(h).all())
    return per_step, kern, ok


def cpu_baseline(batch_items=2):
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
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "state_space_sequence_ssm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key, launch_units):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counters, if they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=("all", "prefill", "decode"), default="all")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU path is "
              "not built: (batch, head) units shard with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    import torch

    from state_space_sequence_ssm_amd import ops
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded, device-generated, resident in HBM)"}
    results = {}
    if args.only in ("all", "prefill"):
        for i, (name, shp) in enumerate(prefill_shapes().items()):
            Bt, L, H, P, N, R, rope = shp
            inp = gen_prefill(torch, Bt, L, H, P, N, R, rope, seed=20260100 + i)
            torch.cuda.synchronize()
            ms, launch_ms, wall = time_prefill(torch, ops, inp, args.steps, args.warmup)
            byts, flops = prefill_algo(*shp)
            res = dict(workload=f"prefill {name}: Bt={Bt} L={L} H={H} P={P} N={N} R={R} "
                                f"{'RoPE' if rope else 'real'} bf16 chunk {Q_ROWS // R}",
                       tokens_per_s=Bt * L / (ms * 1e-3), ms_per_step=ms, kernel_ms=launch_ms,
                       gbs=byts / (launch_ms * 1e-3) / 1e9, tflops=flops / (launch_ms * 1e-3) / 1e12,
                       bytes=byts, flops=flops)
            res["hbm_frac"] = res["gbs"] / HBM_PEAK_GBS
            res["mfma_frac"] = res["tflops"] / MFMA_BF16_PEAK_TFS
            res["roofline_frac"] = max(byts / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFS * 1e12)) / (
                launch_ms * 1e-3)
            results[name] = res
            print(f"# {res['workload']}: {ms:.3f} ms/step, {res['tokens_per_s']:.3e} tok/s, "
                  f"{res['gbs']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% HBM), "
                  f"{res['tflops']:.1f} TFLOP/s ({100 * res['mfma_frac']:.2f}% MFMA)", file=sys.stderr, flush=True)
            del inp
            torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        Bt, H, P, N, R = 256, 32, 64, 64, 4
        per_step, kern, ok = time_decode(torch, ops, Bt, H, P, N, R, args.decode_steps, 20, seed=20260104)
        byts, flops = decode_algo(Bt, H, P, N, R, True)
        results["decode"] = dict(
            workload=f"decode MIMO RoPE: Bt={Bt} H={H} P={P} N={N} R={R} bf16 inputs, fp32 state, "
                     f"{args.decode_steps} sequential steps",
            us_per_step=per_step * 1e3, kernel_us=kern * 1e3, gbs=byts / (kern * 1e-3) / 1e9,
            hbm_frac=byts / (kern * 1e-3) / 1e9 / HBM_PEAK_GBS, bytes=byts, flops=flops, finite=ok)
        print(f"# decode: {per_step * 1e3:.1f} us/step ({kern * 1e3:.1f} us kernel), "
              f"{results['decode']['gbs']:.0f} GB/s", file=sys.stderr, flush=True)

    head = results.get("siso_real")
    if head is not None:
        out["value"] = head["tokens_per_s"]
        out["unit"] = "tokens/s"
        out["ms_per_step"] = head["ms_per_step"]
        out["config"] = {"workload": head["workload"], "global_batch": 8, "seq_len": 4096}
        tr = traffic_for("prefill_siso_real", 1)
        out["roofline"] = {"bound": "hbm", "achieved": head["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": head["hbm_frac"], "traffic": tr,
                           "kernel": "m3::pc::prefill_pc_kernel<128,64>",
                           "algorithmic_bytes_per_launch": head["bytes"],
                           "mfma_tflops": head["tflops"], "mfma_frac": head["mfma_frac"]}
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
                                  "frac": dres["hbm_frac"], "traffic": traffic_for("decode", 1),
                                  "kernel": "m3::decode_step_kernel<bf16_t,64,64,4>"}
    for k in ("siso_rope", "mimo_rope"):
        if k in results:
            out["prefill_" + k] = results[k]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
