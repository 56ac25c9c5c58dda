"""ctypes view of libm3ssm.so (the C ABI declared in include/m3ssm.h).

Only argument structures and function prototypes live here; no arithmetic.
Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libm3ssm.so")

M3_OK = 0
M3_ERR_INVALID_ARG = -1
M3_ERR_UNSUPPORTED = -2
M3_ERR_HIP = -3
M3_ERR_SCRATCH = -4
NOALLOC_SCRATCH_BYTES = 16 << 20  # M3_NOALLOC_SCRATCH_BYTES
M3_F32 = 0
M3_BF16 = 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class Prologue(ctypes.Structure):
    _fields_ = [("bc_norm", _i32), ("dt_softplus", _i32), ("bc_eps", ctypes.c_float),
                ("B_norm_w", _vp), ("C_norm_w", _vp), ("B_bias", _vp), ("C_bias", _vp), ("dt_bias", _vp)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("Bt", _i32), ("L", _i32), ("H", _i32), ("P", _i32), ("N", _i32), ("R", _i32), ("chunk", _i32),
        ("in_dtype", _i32),
        ("x", _vp), ("B", _vp), ("C", _vp), ("dt", _vp), ("lam", _vp), ("A", _vp), ("theta", _vp),
        ("h0", _vp), ("Bprev_rot", _vp), ("xprev", _vp), ("phi0", _vp),
        ("y", _vp), ("h_final", _vp), ("Bprev_rot_out", _vp), ("xprev_out", _vp), ("phi_out", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t), ("omega", _vp), ("A_tok", _vp),
        ("layout", ctypes.c_int32), ("pro", Prologue),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("Bt", _i32), ("H", _i32), ("P", _i32), ("N", _i32), ("R", _i32), ("in_dtype", _i32),
        ("h", _vp), ("phi", _vp), ("Bprev_rot", _vp), ("xprev", _vp),
        ("x", _vp), ("B", _vp), ("C", _vp), ("dt", _vp), ("lam", _vp), ("A", _vp), ("theta", _vp),
        ("y", _vp), ("A_tok", _vp), ("omega", _vp), ("pro", Prologue),
    ]


class BackwardArgs(ctypes.Structure):
    _fields_ = [
        ("Bt", _i32), ("L", _i32), ("H", _i32), ("P", _i32), ("N", _i32), ("R", _i32), ("in_dtype", _i32),
        ("x", _vp), ("B", _vp), ("C", _vp), ("dt", _vp), ("lam", _vp), ("A", _vp), ("A_tok", _vp), ("theta", _vp),
        ("h0", _vp), ("Bprev_rot", _vp), ("xprev", _vp), ("phi0", _vp), ("dy", _vp), ("dh_final", _vp),
        ("dx", _vp), ("dB", _vp), ("dC", _vp), ("ddt", _vp), ("dlam", _vp), ("dA", _vp), ("dtheta", _vp),
        ("dh0", _vp), ("dBprev_rot", _vp), ("dxprev", _vp), ("dphi0", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


EXPORTS = ("m3_ssm_prefill", "m3_ssm_prefill_workspace_size", "m3_ssm_prefill_noalloc", "m3_ssm_decode_step",
           "m3_ssm_prefill_backward", "m3_ssm_prefill_backward_workspace_size",
           "m3_rope_angles_cumsum", "m3_status_string", "m3_version")

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and declare its prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libm3ssm.so not found at {path}: build it first "
            "(python -m state_space_sequence_ssm_amd.build); there is no fallback")
    lib = ctypes.CDLL(path)
    lib.m3_ssm_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
    lib.m3_ssm_prefill.restype = ctypes.c_int
    lib.m3_ssm_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
    lib.m3_ssm_prefill_noalloc.restype = ctypes.c_int
    lib.m3_ssm_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs)]
    lib.m3_ssm_prefill_workspace_size.restype = ctypes.c_size_t
    lib.m3_ssm_prefill_backward.argtypes = [ctypes.POINTER(BackwardArgs), _vp]
    lib.m3_ssm_prefill_backward.restype = ctypes.c_int
    lib.m3_ssm_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(BackwardArgs)]
    lib.m3_ssm_prefill_backward_workspace_size.restype = ctypes.c_size_t
    lib.m3_ssm_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
    lib.m3_ssm_decode_step.restype = ctypes.c_int
    lib.m3_rope_angles_cumsum.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
    lib.m3_rope_angles_cumsum.restype = ctypes.c_int
    lib.m3_status_string.argtypes = [ctypes.c_int]
    lib.m3_status_string.restype = ctypes.c_char_p
    lib.m3_version.argtypes = []
    lib.m3_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().m3_status_string(code).decode()
