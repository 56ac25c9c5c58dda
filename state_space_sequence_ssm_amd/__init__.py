"""Mamba-3 SSM core on AMD MI355X (gfx950): hand-written HIP kernels behind a
C ABI (libm3ssm.so, include/m3ssm.h) with a thin torch binding.

Entry points (same names as the C ABI):
  m3_ssm_prefill        chunked prefill over whole sequences
  m3_ssm_decode_step    one token against a resident fp32 state
  m3_rope_angles_cumsum cumulative rotation angles
"""
from ._lib import LIB_PATH, load  # noqa: F401

__version__ = "0.1.0"


def __getattr__(name):
    # the torch binding is imported lazily so that the ctypes layer can be
    # used (and tested) without initialising a GPU runtime
    if name in ("m3_ssm_prefill", "m3_ssm_decode_step", "m3_rope_angles_cumsum", "M3Error"):
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
