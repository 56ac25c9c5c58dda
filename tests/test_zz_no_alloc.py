"""m3_ssm_prefill_noalloc (the static-scratch prefill for callers that cannot
allocate) against m3_ssm_prefill with a caller workspace: two calls in a row,
the second with a smaller input, both taking the sequence split (the path
that uses scratch).  Same kernels, so the results must be bit-identical; both
are also checked against the oracle."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import m3_oracle as orc  # noqa: E402
from tests.fixtures import Shape, make_inputs  # noqa: E402
from tests.gpu_util import TOL, angle_diff, host, oracle_prefill, prefill_d, to_device  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from state_space_sequence_ssm_amd import ops as o
    return o


CASES = [
    # Bt, L, H, P, N, R, rope  (first larger, then smaller; both split)
    (2, 1500, 4, 64, 64, 1, True),
    (1, 600, 2, 64, 64, 4, True),
]


def test_noalloc_matches_workspace_call_twice(ops):
    for i, (Bt, L, H, P, N, R, rope) in enumerate(CASES):
        print("noalloc case", i, (Bt, L, H, P, N, R, rope), flush=True)
        sys.stdout.flush()
        assert 0 < ops.prefill_workspace_bytes(Bt, L, H, P, N, R, rope=rope) <= 16 << 20
        s = Shape(Bt, L, H, P, N, R, "bf16", rope)
        d = make_inputs(s, 9100 + i, h0=True, carry=True)
        dd = to_device(d, s)
        ref_gpu = prefill_d(ops, dd)               # caller workspace (allocated by the binding)
        got = prefill_d(ops, dd, noalloc=True)      # static scratch
        torch.cuda.synchronize()
        for k in ("y", "h", "Bprev_rot", "xprev", "phi"):
            assert torch.equal(got[k], ref_gpu[k]), (i, k)
        ref = oracle_prefill(d)
        ey = orc.rel_l2(host(got["y"]), ref["y"])
        eh = orc.rel_l2(host(got["h"]), ref["h"])
        print(f"  rel_l2 y={ey:.2e} h={eh:.2e}", flush=True)
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
        assert np.max(angle_diff(host(got["phi"]), ref["phi"])) <= 1e-4
