"""Write tests/golden/oracle_tiny.json: the first outputs of the fp64 oracle on a
tiny seeded RoPE MIMO case with a carry-in.  Calls only the oracle and the
seeded input generator; rerun only when the oracle's arithmetic changes for a
reason stated in the commit message."""
import dataclasses
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import m3_oracle as orc  # noqa: E402
from tests.fixtures import Shape, make_inputs  # noqa: E402

shape = Shape(Bt=1, L=20, H=2, P=4, N=6, R=2, dtype="bf16", rope=True)
seed = 424242
d = make_inputs(shape, seed, h0=True, carry=True)
out = orc.ssm_reference(d["x"], d["B"], d["C"], d["dt"], d["lam"], d["A"], d["theta"],
                        d["h0"], d["Bprev_rot"], d["xprev"], d["phi0"])
g = dict(shape=dataclasses.asdict(shape), seed=seed,
         y_head=out["y"].ravel()[:64].tolist(), h_head=out["h"].ravel()[:48].tolist())
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json"), "w") as f:
    json.dump(g, f, indent=1)
print("wrote oracle_tiny.json")
