"""HIP-graph capture of the library's launches (the benchmark times its
kernels this way).  Every replay is checked against the eager result, with
eager work and synchronisations between the replays, because graph replays
after the first are where wrong results would show."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.fixtures import Shape, make_inputs  # noqa: E402
from tests.gpu_util import to_device  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from state_space_sequence_ssm_amd import ops as o
    return o


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("R,rope", [(1, False), (4, True)])
def test_prefill_graph_replays(ops, R, rope):
    s = Shape(2, 300, 4, 64, 64, R, "bf16", rope)
    dd = to_device(make_inputs(s, 900 + R, h0=True, carry=True), s)
    args = (dd["x"], dd["B"], dd["C"], dd["dt"], dd["lam"], dd["A"], dd["theta"], dd["h0"], dd["Bprev_rot"],
            dd["xprev"], dd["phi0"])
    ref = ops.m3_ssm_prefill(*args, want_carry=True)
    torch.cuda.synchronize()
    out = {k: torch.empty_like(v) for k, v in ref.items() if v is not None}
    g = _capture(lambda: ops.m3_ssm_prefill(*args, y=out["y"], h_final=out["h"], Bprev_rot_out=out["Bprev_rot"],
                                           xprev_out=out["xprev"], phi_out=out.get("phi"), want_carry=True))
    for rep in range(3):
        for v in out.values():
            v.fill_(float("nan") if v.dtype.is_floating_point else 0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, ref[k]), (rep, k)


def test_decode_graph_replays(ops):
    Bt, H, P, N, R, steps = 4, 3, 64, 64, 4, 5
    s = Shape(Bt, steps, H, P, N, R, "bf16", True)
    d = make_inputs(s, 77, h0=True)
    st = torch.bfloat16
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dt)
    xs = [dev(d["x"][:, t], st) for t in range(steps)]
    Bs = [dev(d["B"][:, t], st) for t in range(steps)]
    Cs = [dev(d["C"][:, t], st) for t in range(steps)]
    dts = [dev(d["dt"][:, t]) for t in range(steps)]
    lams = [dev(d["lam"][:, t]) for t in range(steps)]
    ths = [dev(d["theta"][:, t]) for t in range(steps)]
    A = dev(d["A"])
    h_init = dev(d["h0"])
    zeros = dict(phi=torch.zeros((Bt, H, N // 2), device="cuda"), Bp=torch.zeros((Bt, H, R, N), device="cuda"),
                 xp=torch.zeros((Bt, H, R, P), device="cuda", dtype=st))
    state = dict(h=h_init.clone(), phi=zeros["phi"].clone(), Bp=zeros["Bp"].clone(), xp=zeros["xp"].clone())
    ys = [torch.empty((Bt, H, R, P), device="cuda", dtype=st) for _ in range(steps)]

    def run():
        for t in range(steps):
            ops.m3_ssm_decode_step(state["h"], state["phi"], state["Bp"], state["xp"], xs[t], Bs[t], Cs[t], dts[t],
                                   lams[t], A, ths[t], y=ys[t])

    def reset():
        state["h"].copy_(h_init)
        state["phi"].copy_(zeros["phi"])
        state["Bp"].copy_(zeros["Bp"])
        state["xp"].copy_(zeros["xp"])

    run()
    torch.cuda.synchronize()
    ref_y = [y.clone() for y in ys]
    ref_s = {k: v.clone() for k, v in state.items()}
    reset()
    torch.cuda.synchronize()
    g = _capture(run)  # capture does not execute the steps
    for rep in range(3):
        reset()
        for y in ys:
            y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(steps):
            assert torch.equal(ys[t], ref_y[t]), (rep, t)
        for k in state:
            assert torch.equal(state[k], ref_s[k]), (rep, k)
