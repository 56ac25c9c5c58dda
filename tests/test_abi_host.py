"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function the header declares, and rejects invalid arguments before any launch."""
import ctypes
import os
import re

import pytest

from state_space_sequence_ssm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3ssm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libm3ssm.so not built (run __graft_entry__.build())")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(m3_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function():
    lib = _lib.load()
    decl = _declared_functions()
    assert set(decl) == set(_lib.EXPORTS), decl
    for name in decl:
        assert hasattr(lib, name), name
    assert _lib.status_string(0) == "ok"
    assert lib.m3_version().decode().count(".") == 2


def _good_prefill():
    a = _lib.PrefillArgs()
    a.Bt, a.L, a.H, a.P, a.N, a.R, a.chunk, a.in_dtype = 2, 100, 3, 64, 64, 1, 0, _lib.M3_BF16
    base = 0x10000000
    for i, f in enumerate(("x", "B", "C", "dt", "lam", "A", "y")):
        setattr(a, f, base + 0x100000 * i)
    return a


def _rc_prefill(a):
    return _lib.load().m3_ssm_prefill(ctypes.byref(a), None)


def test_prefill_validation():
    lib = _lib.load()
    assert lib.m3_ssm_prefill(None, None) == _lib.M3_ERR_INVALID_ARG
    cases = [
        (lambda a: setattr(a, "x", None), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "A", None), _lib.M3_ERR_INVALID_ARG),  # neither A nor A_tok
        (lambda a: (setattr(a, "A", None), setattr(a, "A_tok", 0x30200002)), _lib.M3_ERR_INVALID_ARG),  # misaligned
        (lambda a: setattr(a, "y", None), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "L", 0), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "R", 0), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "R", 3), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "N", 48), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "P", 8), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "in_dtype", 7), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "chunk", 32), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "x", 0x10000008), _lib.M3_ERR_INVALID_ARG),  # misaligned
        (lambda a: setattr(a, "Bprev_rot", 0x20000000), _lib.M3_ERR_INVALID_ARG),  # without xprev
        (lambda a: setattr(a, "phi0", 0x20000000), _lib.M3_ERR_INVALID_ARG),  # angle without theta
        (lambda a: setattr(a, "phi_out", 0x20000000), _lib.M3_ERR_INVALID_ARG),
        (lambda a: (setattr(a, "theta", 0x30000000), setattr(a, "omega", 0x30100000)),
         _lib.M3_ERR_INVALID_ARG),  # two angle sources
        (lambda a: setattr(a, "omega", 0x30100008), _lib.M3_ERR_INVALID_ARG),  # misaligned
        (lambda a: (setattr(a, "in_dtype", _lib.M3_F32), setattr(a, "N", 128), setattr(a, "P", 128),
                    setattr(a, "theta", 0x30000000)), _lib.M3_ERR_UNSUPPORTED),  # LDS too large
        (lambda a: setattr(a, "layout", 2), _lib.M3_ERR_INVALID_ARG),  # no such layout
        (lambda a: setattr(a, "layout", -1), _lib.M3_ERR_INVALID_ARG),
    ]
    for mutate, code in cases:
        a = _good_prefill()
        mutate(a)
        assert _rc_prefill(a) == code
    assert lib.m3_ssm_prefill_workspace_size(ctypes.byref(_good_prefill())) == 0


def _up256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("Bt,H,L,N,P,R,rope,split", [
    (1, 32, 4096, 64, 64, 4, True, True),     # 32 units: the sequences are split in two
    (4, 32, 8192, 64, 64, 4, True, True),     # 128 units fill 256 compute units when split
    (8, 32, 4096, 128, 64, 1, False, False),  # 256 units already fill the device
    (1, 2, 511, 64, 64, 1, False, False),     # shorter than 8 chunks
    (1, 2, 512, 64, 64, 1, False, True),
    (1, 2, 128, 32, 16, 4, False, True),      # chunks of 16 tokens at R = 4
])
def test_prefill_workspace_size(Bt, H, L, N, P, R, rope, split):
    """The split needs the state and carry in the middle of each sequence; the
    size rule assumes the 256 compute units of MI355X (the host here has no GPU)."""
    lib = _lib.load()
    a = _good_prefill()
    a.Bt, a.H, a.L, a.N, a.P, a.R = Bt, H, L, N, P, R
    a.theta = 0x30000000 if rope else None
    got = lib.m3_ssm_prefill_workspace_size(ctypes.byref(a))
    u = Bt * H
    # state and carry of two segments
    want = (_up256(2 * u * N * P * 4) + _up256(2 * u * R * N * 4) + _up256(2 * u * R * P * 2)
            + _up256(2 * u * (N // 2) * 4 if rope else 0))
    assert got == (want if split else 0)
    a.in_dtype = _lib.M3_F32
    assert lib.m3_ssm_prefill_workspace_size(ctypes.byref(a)) == 0  # fp32 runs unsplit
    assert lib.m3_ssm_prefill_workspace_size(None) == 0


def test_prefill_workspace_validation():
    a = _good_prefill()
    a.Bt, a.H, a.L, a.R = 1, 2, 1024, 1
    need = _lib.load().m3_ssm_prefill_workspace_size(ctypes.byref(a))
    assert need > 0
    a.workspace, a.workspace_bytes = 0x40000000, need - 1  # too small
    assert _rc_prefill(a) == _lib.M3_ERR_INVALID_ARG
    a.workspace, a.workspace_bytes = 0x40000010, need  # not 256-byte aligned
    assert _rc_prefill(a) == _lib.M3_ERR_INVALID_ARG


def test_decode_validation():
    lib = _lib.load()
    assert lib.m3_ssm_decode_step(None, None) == _lib.M3_ERR_INVALID_ARG

    def good():
        a = _lib.DecodeArgs()
        a.Bt, a.H, a.P, a.N, a.R, a.in_dtype = 4, 2, 64, 64, 4, _lib.M3_BF16
        for i, f in enumerate(("h", "Bprev_rot", "xprev", "x", "B", "C", "dt", "lam", "A", "y")):
            setattr(a, f, 0x10000000 + 0x100000 * i)
        return a

    cases = [
        (lambda a: setattr(a, "h", None), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "theta", 0x30000000), _lib.M3_ERR_INVALID_ARG),  # theta without phi
        (lambda a: setattr(a, "phi", 0x30000000), _lib.M3_ERR_INVALID_ARG),  # phi without theta
        (lambda a: setattr(a, "omega", 0x30000000), _lib.M3_ERR_INVALID_ARG),  # omega without phi
        (lambda a: (setattr(a, "omega", 0x30000000), setattr(a, "theta", 0x30100000), setattr(a, "phi", 0x30200000)),
         _lib.M3_ERR_INVALID_ARG),  # two angle sources
        (lambda a: setattr(a, "A", None), _lib.M3_ERR_INVALID_ARG),  # neither A nor A_tok
        (lambda a: setattr(a, "R", 17), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "N", 24), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "Bt", 0), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "y", 0x10000004), _lib.M3_ERR_INVALID_ARG),
    ]
    for mutate, code in cases:
        a = good()
        mutate(a)
        assert lib.m3_ssm_decode_step(ctypes.byref(a), None) == code


def test_angles_validation():
    f = _lib.load().m3_rope_angles_cumsum
    assert f(None, None, 0x1000, 1, 1, 1, 4, None) == _lib.M3_ERR_INVALID_ARG
    assert f(0x1000, None, 0x1000, 1, 1, 1, 4, None) == _lib.M3_ERR_INVALID_ARG  # aliasing
    assert f(0x1000, None, 0x2000, 1, 0, 1, 4, None) == _lib.M3_ERR_INVALID_ARG
    assert f(0x1000, None, 0x2000, 1, 5, 1, 3, None) == _lib.M3_ERR_UNSUPPORTED
    assert f(0x1004, None, 0x2000, 1, 5, 1, 4, None) == _lib.M3_ERR_INVALID_ARG
