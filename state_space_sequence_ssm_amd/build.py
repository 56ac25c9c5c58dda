"""Build libm3ssm.so (the HIP kernels + C ABI) in-tree for gfx950.

Usage: python -m state_space_sequence_ssm_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libm3ssm.so")
# the largest units first, so the parallel build ends sooner
SOURCES = ["prefill_bf16_n128.hip", "prefill_bf16_n128_pro.hip", "prefill_bf16_n64.hip", "prefill_bf16_n64_pro.hip",
           "prefill_bf16_n32.hip", "prefill_bf16_n32_pro.hip", "prefill_bf16_n16.hip", "prefill_bf16_n16_pro.hip",
           "backward_main.hip", "backward.hip", "backward_pre.hip", "prefill_f32.hip", "decode.hip", "decode_mma.hip",
           "api.hip", "angles.hip", "split.hip", "prefill_bf16.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libm3ssm.so")


def cflags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *cflags(), "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libm3ssm.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


SAN_DIR = os.path.join(OBJ, "hostsan")
SAN_LIB = os.path.join(SAN_DIR, "libm3ssm_hostsan.so")
# host-side sanitizers only: each flag goes to the host compilation of api.hip
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that a host process must preload to
    load the sanitized library."""
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm")
    r = subprocess.run([os.path.join(llvm, "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return path


def build_hostsan(verbose: bool = False) -> str:
    """libm3ssm_hostsan.so: the host-side C-ABI layer (api.hip: argument
    validation and dispatch) built with AddressSanitizer and UBSan, linked
    with the regular kernel objects of the last build().  For host-only
    tests of the validation paths (no kernel is launched)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(x)[0] + ".o") for x in SOURCES if x != "api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: missing {missing}")
    api_o = os.path.join(SAN_DIR, "api_hostsan.o")
    cmd = [hipcc(), *cflags(), *SAN_FLAGS, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc (host sanitizers) failed:\n" + r.stdout + r.stderr)
    # a plain host link: the objects already embed their device code
    llvm = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm")
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    tmp = SAN_LIB + ".tmp"
    cmd = [os.path.join(llvm, "bin", "clang++"), "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined",
           "-o", tmp, api_o, *objs, "-L" + rocm_lib, "-Wl,-rpath," + rocm_lib, "-lamdhip64"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("host-sanitizer link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--hostsan" in sys.argv:
        print(build_hostsan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
