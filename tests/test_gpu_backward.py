"""GPU parity of the backward pass (NEXT-4): the HIP kernel's gradients
against the fp64 oracle's adjoint (oracle.ssm_backward) on the same seeded
bf16 inputs and upstream gradients.  Every gradient buffer is NaN-filled
before the call."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import m3_oracle as orc  # noqa: E402
from synth.inputs import bf16_round  # noqa: E402
from tests.fixtures import Shape, make_inputs  # noqa: E402
from tests.gpu_util import NAN, dev, host, to_device  # noqa: E402

pytestmark = pytest.mark.gpu

# Relative-L2 bar of the bf16 path (gradients stored in bf16 or accumulated
# from bf16 operands), as for the forward outputs.
TOL = 2e-2


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from state_space_sequence_ssm_amd import ops as o
    return o


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _nan_out(dd, Bt, L, H, P, N, R, rope, a_tok, carry):
    f32 = torch.float32
    nanf = lambda *shape: torch.full(shape, NAN, device="cuda", dtype=f32)  # noqa: E731
    o = dict(dx=torch.full_like(dd["x"], NAN), dB=torch.full_like(dd["B"], NAN), dC=torch.full_like(dd["C"], NAN),
             ddt=nanf(Bt, L, H), dlam=nanf(Bt, L, H), dA=nanf(Bt, L, H) if a_tok else nanf(H),
             dh0=nanf(Bt, H, N, P))
    if rope:
        o["dtheta"] = nanf(Bt, L, H, N // 2)
        o["dphi0"] = nanf(Bt, H, N // 2)
    if carry:
        o["dBprev_rot"] = nanf(Bt, H, R, N)
        o["dxprev"] = torch.full((Bt, H, R, P), NAN, device="cuda", dtype=torch.bfloat16)
    return o


CASES = [
    # Bt, L, H, P, N, R, rope, carry, A per token
    (2, 131, 3, 64, 64, 1, True, True, False),
    (1, 150, 2, 64, 128, 1, False, True, False),
    (1, 100, 2, 64, 64, 4, True, True, False),
    (1, 45, 2, 16, 32, 8, True, False, False),
    (1, 77, 2, 32, 16, 2, True, True, True),
    (2, 64, 2, 32, 32, 1, False, False, True),
    (1, 1, 2, 64, 64, 1, True, True, False),
    (1, 200, 2, 128, 64, 1, True, True, False),
    (1, 96, 3, 16, 128, 2, True, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_vs_oracle(ops, case):
    Bt, L, H, P, N, R, rope, carry, a_tok = case
    s = Shape(Bt, L, H, P, N, R, "bf16", rope)
    _say("backward", case)
    d = make_inputs(s, 15000 + L + N + R, h0=carry, carry=carry)
    rng = np.random.default_rng(15001 + L)
    dy = bf16_round(rng.standard_normal((Bt, L, H, R, P)).astype(np.float32))
    dhf = rng.standard_normal((Bt, H, N, P)).astype(np.float32)
    A_tok = None
    if a_tok:
        A_tok = (-np.exp(rng.random((Bt, L, H), dtype=np.float32) * np.float32(np.log(16.0)))).astype(np.float32)
    dd = to_device(d, s)
    out = _nan_out(dd, Bt, L, H, P, N, R, rope, a_tok, carry)
    got = ops.m3_ssm_prefill_backward(dd["x"], dd["B"], dd["C"], dd["dt"], dd["lam"], None if a_tok else dd["A"],
                                      dd["theta"], dd.get("h0"), dd.get("Bprev_rot"), dd.get("xprev"),
                                      dd.get("phi0"), dy=dev(dy, torch.bfloat16), dh_final=dev(dhf),
                                      A_tok=dev(A_tok) if a_tok else None, want_carry_grads=True, out=out)
    torch.cuda.synchronize()
    ref = orc.ssm_backward(d["x"], d["B"], d["C"], d["dt"], d["lam"], A_tok if a_tok else d["A"], d["theta"],
                           d.get("h0"), d.get("Bprev_rot"), d.get("xprev"), d.get("phi0"), dy=dy, dh_final=dhf)
    keys = ["dx", "dB", "dC", "ddt", "dlam", "dA", "dh0"] + (["dtheta", "dphi0"] if rope else []) + (
        ["dBprev_rot", "dxprev"] if carry else [])
    errs = {}
    for k in keys:
        g = host(got[k])
        assert np.all(np.isfinite(g)), k
        errs[k] = orc.rel_l2(g, ref[k])
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL, (k, e)


def test_backward_deterministic(ops):
    s = Shape(2, 150, 2, 64, 64, 4, "bf16", True)
    d = make_inputs(s, 15500, h0=True, carry=True)
    dd = to_device(d, s)
    dy = dev(bf16_round(np.random.default_rng(7).standard_normal((2, 150, 2, 4, 64)).astype(np.float32)),
             torch.bfloat16)
    run = lambda: ops.m3_ssm_prefill_backward(dd["x"], dd["B"], dd["C"], dd["dt"], dd["lam"], dd["A"],  # noqa: E731
                                              dd["theta"], dd["h0"], dd["Bprev_rot"], dd["xprev"], dd["phi0"], dy=dy,
                                              want_carry_grads=True)
    a, b = run(), run()
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
