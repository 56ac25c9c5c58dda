"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function the header declares, and rejects invalid arguments before any launch.
The same checks also run against a build of the host-side layer with
AddressSanitizer and UBSan (test_validation_under_host_sanitizers)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from state_space_sequence_ssm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3ssm.h")
# set by test_validation_under_host_sanitizers for the run in its subprocess
_SAN_LIB = os.environ.get("M3SSM_HOSTSAN_LIB")
if _SAN_LIB:
    _lib.load(_SAN_LIB)  # every test below then calls the sanitized build

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
        (lambda a: setattr(a, "chunk", 32), _lib.M3_ERR_UNSUPPORTED),  # bf16: chunks of 64 / R only
        (lambda a: (setattr(a, "in_dtype", _lib.M3_F32), setattr(a, "chunk", 24)), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: (setattr(a, "in_dtype", _lib.M3_F32), setattr(a, "chunk", 128)), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: (setattr(a, "in_dtype", _lib.M3_F32), setattr(a, "R", 4), setattr(a, "chunk", 32)),
         _lib.M3_ERR_UNSUPPORTED),  # 32 tokens x rank 4 > 64 rows
        (lambda a: (setattr(a, "in_dtype", _lib.M3_F32), setattr(a, "chunk", -16)), _lib.M3_ERR_UNSUPPORTED),
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


def _pro_cases():
    """Invalid prologues (each a mutation of m3_prologue) -> M3_ERR_INVALID_ARG."""
    return [
        lambda q: setattr(q, "bc_norm", 2),
        lambda q: setattr(q, "dt_softplus", -1),
        lambda q: (setattr(q, "bc_norm", 1), setattr(q, "bc_eps", -1e-3)),
        lambda q: (setattr(q, "bc_norm", 1), setattr(q, "bc_eps", float("nan"))),
        lambda q: (setattr(q, "bc_norm", 1), setattr(q, "bc_eps", float("inf"))),
        lambda q: setattr(q, "B_norm_w", 0x50000000),            # gain without the normalisation
        lambda q: setattr(q, "dt_bias", 0x50000000),             # step bias without the softplus
        lambda q: setattr(q, "C_bias", 0x50000002),              # misaligned
        lambda q: (setattr(q, "bc_norm", 1), setattr(q, "C_norm_w", 0x50000001)),
    ]


def test_prologue_validation():
    lib = _lib.load()
    for mutate in _pro_cases():
        a = _good_prefill()
        mutate(a.pro)
        assert _rc_prefill(a) == _lib.M3_ERR_INVALID_ARG


def test_prefill_workspace_validation():
    a = _good_prefill()
    a.Bt, a.H, a.L, a.R = 1, 2, 1024, 1
    need = _lib.load().m3_ssm_prefill_workspace_size(ctypes.byref(a))
    assert need > 0
    a.workspace, a.workspace_bytes = 0x40000000, need - 1  # too small
    assert _rc_prefill(a) == _lib.M3_ERR_INVALID_ARG
    a.workspace, a.workspace_bytes = 0x40000010, need  # not 256-byte aligned
    assert _rc_prefill(a) == _lib.M3_ERR_INVALID_ARG


def test_prefill_noalloc_validation():
    """The no-allocation entry point validates like m3_ssm_prefill, refuses a
    workspace, and refuses (before any GPU call) a call whose split needs more
    than its static scratch."""
    lib = _lib.load()
    f = lambda a: lib.m3_ssm_prefill_noalloc(ctypes.byref(a), None)  # noqa: E731
    assert lib.m3_ssm_prefill_noalloc(None, None) == _lib.M3_ERR_INVALID_ARG
    a = _good_prefill()
    a.x = None
    assert f(a) == _lib.M3_ERR_INVALID_ARG
    a = _good_prefill()
    a.R = 3
    assert f(a) == _lib.M3_ERR_UNSUPPORTED
    a = _good_prefill()
    a.Bt, a.H, a.L = 1, 2, 1024  # takes the split
    a.workspace, a.workspace_bytes = 0x40000000, 1 << 20
    assert f(a) == _lib.M3_ERR_INVALID_ARG
    # 128 units at N = P = 128 split, and need more than the 16 MiB scratch
    a = _good_prefill()
    a.Bt, a.H, a.L, a.N, a.P, a.R = 4, 32, 4096, 128, 128, 1
    need = lib.m3_ssm_prefill_workspace_size(ctypes.byref(a))
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert f(a) == _lib.M3_ERR_SCRATCH
    assert "scratch" in _lib.status_string(_lib.M3_ERR_SCRATCH)
    a.P = 64  # the headline shape's state fits
    assert 0 < lib.m3_ssm_prefill_workspace_size(ctypes.byref(a)) <= _lib.NOALLOC_SCRATCH_BYTES


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
    for mutate in _pro_cases():
        a = good()
        mutate(a.pro)
        assert lib.m3_ssm_decode_step(ctypes.byref(a), None) == _lib.M3_ERR_INVALID_ARG


def test_angles_validation():
    f = _lib.load().m3_rope_angles_cumsum
    assert f(None, None, 0x1000, 1, 1, 1, 4, None) == _lib.M3_ERR_INVALID_ARG
    assert f(0x1000, None, 0x1000, 1, 1, 1, 4, None) == _lib.M3_ERR_INVALID_ARG  # aliasing
    assert f(0x1000, None, 0x2000, 1, 0, 1, 4, None) == _lib.M3_ERR_INVALID_ARG
    assert f(0x1000, None, 0x2000, 1, 5, 1, 3, None) == _lib.M3_ERR_UNSUPPORTED
    assert f(0x1004, None, 0x2000, 1, 5, 1, 4, None) == _lib.M3_ERR_INVALID_ARG


@pytest.mark.skipif(_SAN_LIB is not None, reason="this is the sanitized run itself")
def test_validation_under_host_sanitizers():
    """Every host check above, again in a fresh process whose library has its
    C-ABI layer built with AddressSanitizer and UBSan (no recovery: any
    report fails the run)."""
    from state_space_sequence_ssm_amd import build as b
    try:
        lib = b.build_hostsan()
        rt = b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"host sanitizer build unavailable: {e}")
    env = dict(os.environ, M3SSM_HOSTSAN_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.abspath(__file__)],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


def _good_backward():
    a = _lib.BackwardArgs()
    a.Bt, a.L, a.H, a.P, a.N, a.R, a.in_dtype = 2, 100, 3, 64, 64, 1, _lib.M3_BF16
    for i, f in enumerate(("x", "B", "C", "dt", "lam", "A", "dy", "dx", "dB", "dC", "ddt", "dlam", "dA")):
        setattr(a, f, 0x10000000 + 0x100000 * i)
    a.workspace = 0x40000000
    a.workspace_bytes = _lib.load().m3_ssm_prefill_backward_workspace_size(ctypes.byref(a))
    return a


def test_backward_validation_and_workspace():
    lib = _lib.load()
    f = lambda a: lib.m3_ssm_prefill_backward(ctypes.byref(a), None)  # noqa: E731
    assert lib.m3_ssm_prefill_backward(None, None) == _lib.M3_ERR_INVALID_ARG
    a = _good_backward()
    # states of every chunk (2 x 3 units, 2 chunks of 64, 64 x 64 bf16) and per-unit dA sums
    assert a.workspace_bytes == _up256(6 * 2 * 64 * 64 * 2) + _up256(6 * 4)
    cases = [
        (lambda a: setattr(a, "dy", None), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "dA", None), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "workspace", None), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "workspace_bytes", a.workspace_bytes - 1), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "workspace", 0x40000010), _lib.M3_ERR_INVALID_ARG),  # not 256-aligned
        (lambda a: setattr(a, "in_dtype", _lib.M3_F32), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: setattr(a, "theta", 0x30000000), _lib.M3_ERR_INVALID_ARG),   # theta without dtheta
        (lambda a: setattr(a, "dtheta", 0x30000000), _lib.M3_ERR_INVALID_ARG),  # dtheta without theta
        (lambda a: setattr(a, "A_tok", 0x30000000), _lib.M3_ERR_INVALID_ARG),   # both A and A_tok
        (lambda a: setattr(a, "Bprev_rot", 0x30000000), _lib.M3_ERR_INVALID_ARG),
        (lambda a: setattr(a, "R", 16), _lib.M3_ERR_UNSUPPORTED),
        (lambda a: (setattr(a, "N", 128), setattr(a, "P", 128)), _lib.M3_ERR_UNSUPPORTED),  # LDS
        (lambda a: setattr(a, "dx", 0x10000008), _lib.M3_ERR_INVALID_ARG),
    ]
    for mutate, code in cases:
        a = _good_backward()
        mutate(a)
        if code == _lib.M3_ERR_UNSUPPORTED and a.N == 128:
            a.workspace_bytes = lib.m3_ssm_prefill_backward_workspace_size(ctypes.byref(a))
        assert f(a) == code
    # with RoPE the angle entering every chunk is kept too
    a = _good_backward()
    a.theta, a.dtheta = 0x30000000, 0x30100000
    assert lib.m3_ssm_prefill_backward_workspace_size(ctypes.byref(a)) == (
        _up256(6 * 2 * 64 * 64 * 2) + _up256(6 * 2 * 32 * 4) + _up256(6 * 4))


def test_backward_split_workspace():
    """With few (batch, head) units and enough chunks the backward splits the
    sequence (two workgroups per unit; 256 compute units are assumed when no
    device can be queried): its workspace adds the values joined at the split
    chunk and a second set of dA sums."""
    lib = _lib.load()
    a = _good_backward()
    a.L = 600  # 10 chunks of 64 tokens, 6 units
    a.theta, a.dtheta = 0x30000000, 0x30100000
    u, nch, NP, J = 6, 10, 64 * 64, 32
    want = (_up256(u * nch * NP * 2) + _up256(u * nch * J * 4) + _up256(2 * u * 4)  # states, angles, dA sums
            + 2 * _up256(u * NP * 4)                                                # state and gradient sum
            + _up256(u * J * 4) + _up256(u * 4) + _up256(u * J * 4) + _up256(2 * u * 2 * 4))
    assert lib.m3_ssm_prefill_backward_workspace_size(ctypes.byref(a)) == want
    # 7 chunks: too short to split
    a.L = 7 * 64
    assert lib.m3_ssm_prefill_backward_workspace_size(ctypes.byref(a)) == (
        _up256(u * 7 * NP * 2) + _up256(u * 7 * J * 4) + _up256(u * 4))
    # more units than half the compute units: no split
    a.L, a.Bt, a.H = 600, 1, 129
    assert lib.m3_ssm_prefill_backward_workspace_size(ctypes.byref(a)) == (
        _up256(129 * nch * NP * 2) + _up256(129 * nch * J * 4) + _up256(129 * 4))
