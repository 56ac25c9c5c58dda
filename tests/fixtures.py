"""Seeded test inputs: the shared generator's draws (synth.inputs) plus the
angles theta = Delta * omega, formed from the drawn rates by the oracle's
``angles_from_rates`` and rounded to fp32 for the device (the product of two
fp32 values rounded once, the same bits an fp32 multiply gives).  Test
infrastructure only."""
from __future__ import annotations

import numpy as np

from oracle import m3_oracle as orc
from synth import inputs as _syn
from synth.inputs import CONFIGS, SEED_BASE, Shape  # noqa: F401  (re-exported)


def with_theta(d: dict) -> dict:
    """Copy of ``d`` with ``theta`` [.., H, N/2] fp32 from dt and omega (None
    without omega)."""
    d = dict(d)
    om = d.get("omega")
    d["theta"] = None if om is None else orc.angles_from_rates(d["dt"], om).astype(np.float32)
    return d


def make_inputs(s: Shape, seed: int, **kw) -> dict:
    return with_theta(_syn.make_inputs(s, seed, **kw))


def make_decode_inputs(s: Shape, steps: int, seed: int) -> dict:
    return with_theta(_syn.make_decode_inputs(s, steps, seed))


def config_inputs(cfg: int, **kw) -> dict:
    return make_inputs(CONFIGS[cfg], SEED_BASE + cfg, **kw)
