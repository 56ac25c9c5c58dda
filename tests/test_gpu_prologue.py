"""GPU parity of the prologue fused in front of the core: RMS normalisation of
the B and C rows, head-specific biases added after it, and Delta = softplus
of the raw step plus a head bias.  The library gets the raw B, C and step; the
reference is the oracle's ``prologue`` followed by the oracle core, on the
same seeded bits.  Outputs are NaN-filled before every call."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import m3_oracle as orc  # noqa: E402
from tests.fixtures import Shape, make_inputs  # noqa: E402
from tests.gpu_util import TOL, angle_diff, decode, dev, host, prefill, storage_dtype, to_device  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from state_space_sequence_ssm_amd import ops as o
    return o


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _params(H, R, N, seed, norm=True, gains=True, bias=True, softplus=True, dtb=True, eps=1e-6):
    """Prologue parameters drawn for a test: gains U(0.5, 1.5), biases N(0, 0.3^2),
    step biases N(0, 0.5^2)."""
    rng = np.random.default_rng(seed)
    f = np.float32
    q = dict(bc_norm=norm, bc_eps=eps, dt_softplus=softplus)
    q["B_norm_w"] = (rng.random(N) + 0.5).astype(f) if (norm and gains) else None
    q["C_norm_w"] = (rng.random(N) + 0.5).astype(f) if (norm and gains) else None
    q["B_bias"] = (rng.standard_normal((H, R, N)) * 0.3).astype(f) if bias else None
    q["C_bias"] = (rng.standard_normal((H, R, N)) * 0.3).astype(f) if bias else None
    q["dt_bias"] = (rng.standard_normal(H) * 0.5).astype(f) if (softplus and dtb) else None
    return q


def _dev_params(q):
    return {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in q.items()}


def _ref_inputs(d, q):
    """The oracle's prologue on the raw inputs: (B, C, Delta) for the core."""
    return orc.prologue(d["B"], d["C"], d["dt_raw"] if q["dt_softplus"] else d["dt"], bc_norm=q["bc_norm"],
                        B_norm_w=q["B_norm_w"], C_norm_w=q["C_norm_w"], eps=q["bc_eps"], B_bias=q["B_bias"],
                        C_bias=q["C_bias"], dt_softplus=q["dt_softplus"], dt_bias=q["dt_bias"])


CASES = [
    # name, Bt, L, H, P, N, R, dtype, rope, carry, options
    ("n64_r1_all", 2, 131, 3, 64, 64, 1, "bf16", True, True, {}),
    ("n128_r1_real_rows_by_kind", 1, 150, 2, 64, 128, 1, "bf16", False, True, {}),
    ("n128_r1_rope_gains", 1, 100, 2, 64, 128, 1, "bf16", True, False, {}),
    ("n128_p128_r1_real", 1, 70, 2, 128, 128, 1, "bf16", False, True, {}),
    ("n64_r1_real", 1, 130, 2, 64, 64, 1, "bf16", False, True, {}),
    ("n64_p128_r1", 1, 100, 2, 128, 64, 1, "bf16", True, True, {}),
    ("n128_r1_rope", 1, 90, 2, 64, 128, 1, "bf16", True, True, dict(gains=False)),
    ("n64_r4_by_kind", 1, 100, 2, 64, 64, 4, "bf16", True, True, {}),
    ("n32_r8", 1, 45, 2, 16, 32, 8, "bf16", True, False, dict(gains=False)),
    ("n16_r2_padded", 1, 77, 2, 32, 16, 2, "bf16", True, True, {}),
    ("n128_r4_real", 1, 90, 2, 64, 128, 4, "bf16", False, True, {}),
    ("split_two_part", 1, 1500, 2, 64, 64, 1, "bf16", True, True, {}),
    ("split_mimo", 2, 600, 2, 64, 64, 4, "bf16", True, True, {}),
    ("softplus_only", 2, 131, 3, 64, 64, 1, "bf16", True, True, dict(norm=False, bias=False)),
    ("bias_only", 1, 100, 2, 64, 64, 4, "bf16", True, True, dict(norm=False, softplus=False)),
    ("norm_eps0", 1, 70, 2, 64, 64, 1, "bf16", True, False, dict(eps=0.0, bias=False, softplus=False)),
    ("f32_rope", 2, 150, 2, 32, 32, 2, "f32", True, True, {}),
    ("f32_n128_real", 1, 200, 3, 16, 128, 1, "f32", False, True, {}),
    ("f32_n16_r4", 1, 90, 2, 32, 16, 4, "f32", True, True, {}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_prefill_prologue(ops, case):
    name, Bt, L, H, P, N, R, dt_, rope, carry, opts = case
    s = Shape(Bt, L, H, P, N, R, dt_, rope)
    _say("prefill prologue", case)
    d = make_inputs(s, 11000 + L + N + R, h0=carry, carry=carry)
    q = _params(H, R, N, 12000 + L, **opts)
    dd = to_device(d, s)
    raw_dt = dev(d["dt_raw"]) if q["dt_softplus"] else dd["dt"]
    out = prefill(ops, dd["x"], dd["B"], dd["C"], raw_dt, dd["lam"], dd["A"], dd["theta"], dd.get("h0"),
                  dd.get("Bprev_rot"), dd.get("xprev"), dd.get("phi0"), **_dev_params(q))
    torch.cuda.synchronize()
    B2, C2, dt2 = _ref_inputs(d, q)
    ref = orc.ssm_reference(d["x"], B2, C2, dt2, d["lam"], d["A"], d["theta"], d.get("h0"), d.get("Bprev_rot"),
                            d.get("xprev"), d.get("phi0"))
    ey = orc.rel_l2(host(out["y"]), ref["y"])
    eh = orc.rel_l2(host(out["h"]), ref["h"])
    _say(f"  rel_l2 y={ey:.2e} h={eh:.2e}")
    assert ey <= TOL[dt_] and eh <= TOL[dt_]
    assert orc.rel_l2(host(out["Bprev_rot"]), ref["Bprev_rot"]) <= 1e-5
    assert np.array_equal(host(out["xprev"]), ref["xprev"])
    if rope:
        assert np.max(angle_diff(host(out["phi"]), ref["phi"])) <= 1e-4


def test_prefill_prologue_with_rates_head_major_and_A_tok(ops):
    """The prologue together with the other options: angles as rates (the
    angle then uses the softplus step), head-major x/B/C/y, A per token."""
    Bt, L, H, P, N, R = 1, 140, 3, 64, 64, 2
    s = Shape(Bt, L, H, P, N, R, "bf16", True)
    _say("prefill prologue + omega + head-major + A_tok")
    d = make_inputs(s, 13000, h0=True, carry=True)
    q = _params(H, R, N, 13001)
    a_tok = (-np.exp(np.random.default_rng(13002).random((Bt, L, H), dtype=np.float32)
                     * np.float32(np.log(16.0)))).astype(np.float32)
    dd = to_device(d, s)
    swap = lambda t: t.permute(0, 2, 1, 3, 4).contiguous()  # noqa: E731
    out = prefill(ops, swap(dd["x"]), swap(dd["B"]), swap(dd["C"]), dev(d["dt_raw"]), dd["lam"], None, None,
                  dd["h0"], dd["Bprev_rot"], dd["xprev"], dd["phi0"], head_major=True, omega=dd["omega"],
                  A_tok=dev(a_tok), **_dev_params(q))
    torch.cuda.synchronize()
    B2, C2, dt2 = _ref_inputs(d, q)
    ref = orc.ssm_reference(d["x"], B2, C2, dt2, d["lam"], a_tok, None, d["h0"], d["Bprev_rot"], d["xprev"],
                            d["phi0"], omega=d["omega"])
    ey = orc.rel_l2(host(swap(out["y"])), ref["y"])
    eh = orc.rel_l2(host(out["h"]), ref["h"])
    _say(f"  rel_l2 y={ey:.2e} h={eh:.2e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    assert np.max(angle_diff(host(out["phi"]), ref["phi"])) <= 1e-3


def test_prologue_zero_bias_is_the_plain_call(ops):
    """A prologue that adds zero biases changes no bit of the result."""
    s = Shape(1, 100, 2, 64, 64, 4, "bf16", True)
    d = make_inputs(s, 13100, h0=True, carry=True)
    dd = to_device(d, s)
    z = torch.zeros((2, 4, 64), device="cuda")
    a = prefill(ops, dd["x"], dd["B"], dd["C"], dd["dt"], dd["lam"], dd["A"], dd["theta"], dd["h0"],
                dd["Bprev_rot"], dd["xprev"], dd["phi0"])
    b = prefill(ops, dd["x"], dd["B"], dd["C"], dd["dt"], dd["lam"], dd["A"], dd["theta"], dd["h0"],
                dd["Bprev_rot"], dd["xprev"], dd["phi0"], B_bias=z, C_bias=z)
    torch.cuda.synchronize()
    for k in ("y", "h", "Bprev_rot", "phi"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("case", [(3, 2, 64, 64, 4, "bf16", True, 30), (2, 3, 32, 128, 1, "f32", False, 12),
                                  (2, 2, 16, 16, 3, "bf16", True, 10), (2, 2, 64, 64, 16, "bf16", True, 10),
                                  (1, 2, 64, 128, 8, "bf16", True, 8), (2, 2, 128, 32, 2, "bf16", False, 8),
                                  (2, 2, 32, 64, 4, "bf16", True, 8)],
                         ids=lambda c: "-".join(map(str, c)))
def test_decode_prologue_chain(ops, case):
    """Decode steps with the prologue: the oracle's prologue on every token."""
    Bt, H, P, N, R, dt_, rope, steps = case
    _say("decode prologue chain", case)
    s = Shape(Bt, steps, H, P, N, R, dt_, rope)
    d = make_inputs(s, 14000 + steps, h0=True)
    q = _params(H, R, N, 14001 + steps)
    st = storage_dtype(s)
    mv = lambda a, t=torch.float32: dev(np.moveaxis(a, 1, 0), t)  # noqa: E731
    dec = dict(x=mv(d["x"], st), B=mv(d["B"], st), C=mv(d["C"], st), dt=mv(d["dt_raw"]), lam=mv(d["lam"]),
               theta=mv(d["theta"]) if rope else None)
    state = dict(h=dev(d["h0"]), phi=dev(np.zeros((Bt, H, N // 2))) if rope else None,
                 Bprev_rot=dev(np.zeros((Bt, H, R, N))), xprev=dev(np.zeros((Bt, H, R, P)), st))
    A = dev(d["A"])
    qd = _dev_params(q)
    ys = []
    for t in range(steps):
        ys.append(host(decode(ops, state, dec["x"][t], dec["B"][t], dec["C"][t], dec["dt"][t], dec["lam"][t], A,
                              dec["theta"][t] if rope else None, **qd)))
    torch.cuda.synchronize()
    B2, C2, dt2 = _ref_inputs(d, q)
    ref = orc.ssm_reference(d["x"], B2, C2, dt2, d["lam"], d["A"], d["theta"], d["h0"])
    ey = orc.rel_l2(np.stack(ys, axis=1), ref["y"])
    eh = orc.rel_l2(host(state["h"]), ref["h"])
    _say(f"  rel_l2 y={ey:.2e} h={eh:.2e}")
    assert ey <= TOL[dt_] and eh <= TOL[dt_]
    assert orc.rel_l2(host(state["Bprev_rot"]), ref["Bprev_rot"]) <= 1e-5


def test_prefill_then_decode_with_prologue(ops):
    """Prefill [0, k) then decode [k, L), both with the prologue, equals the
    oracle on the whole sequence."""
    Bt, L, H, P, N, R, k = 2, 90, 2, 64, 64, 4, 70
    s = Shape(Bt, L, H, P, N, R, "bf16", True)
    d = make_inputs(s, 14500, h0=True, carry=True)
    q = _params(H, R, N, 14501)
    qd = _dev_params(q)
    dd = to_device(d, s)
    raw = dev(d["dt_raw"])
    cut = lambda t: t[:, :k].contiguous()  # noqa: E731
    a = prefill(ops, cut(dd["x"]), cut(dd["B"]), cut(dd["C"]), cut(raw), cut(dd["lam"]), dd["A"],
                cut(dd["theta"]), dd["h0"], dd["Bprev_rot"], dd["xprev"], dd["phi0"], **qd)
    state = dict(h=a["h"], phi=a["phi"], Bprev_rot=a["Bprev_rot"], xprev=a["xprev"])
    ys = []
    for t in range(k, L):
        ys.append(host(decode(ops, state, dd["x"][:, t].contiguous(), dd["B"][:, t].contiguous(),
                              dd["C"][:, t].contiguous(), raw[:, t].contiguous(), dd["lam"][:, t].contiguous(),
                              dd["A"], dd["theta"][:, t].contiguous(), **qd)))
    torch.cuda.synchronize()
    B2, C2, dt2 = _ref_inputs(d, q)
    ref = orc.ssm_reference(d["x"], B2, C2, dt2, d["lam"], d["A"], d["theta"], d["h0"], d["Bprev_rot"],
                            d["xprev"], d["phi0"])
    y = np.concatenate([host(a["y"]), np.stack(ys, axis=1)], axis=1)
    assert orc.rel_l2(y, ref["y"]) <= TOL["bf16"]
    assert orc.rel_l2(host(state["h"]), ref["h"]) <= TOL["bf16"]
