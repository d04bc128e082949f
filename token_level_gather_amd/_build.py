"""Build step of the HIP library: ``python -m token_level_gather_amd._build``.

Compiles the gfx950 kernels and the C-ABI host runtime into
``token_level_gather_amd/libkvs.so`` with hipcc.  Every HIP translation unit
gets ``-Xclang -target-feature -Xclang -packed-fp32-ops`` (no packed fp32 VALU
instructions are emitted).

``--device-checks`` builds ``token_level_gather_amd/libkvs_checked.so``: the
same library with ``KVS_DEVICE_CHECKS=1``, device-side bounds checks on every
index the kernels take from the Top-K, the maps, the LRU order and the step's
lists (a debugging aid; ``kvs.load_library(kvs.CHECKED_LIB_PATH)`` or
``KVS_LIB`` selects it).

``--host-sanitizers`` builds ``_build/hostsan/libkvs.so`` instead, with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (each
``-fsanitize`` behind ``-Xarch_host``; device code is built as usual), for
running the CPU tests of the host runtime::

    python -m token_level_gather_amd._build --host-sanitizers
    LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) \
        ASAN_OPTIONS=detect_leaks=0 KVS_LIB=_build/hostsan/libkvs.so \
        python -m pytest tests/test_abi.py
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvs.so")
CHECKED_LIB = os.path.join(HERE, "libkvs_checked.so")
SOURCES = ["kvs_kernels.hip", "kvs_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def build(verbose: bool = False, out: str = LIB, host_sanitizers: bool = False,
          device_checks: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    sub = "hostsan" if host_sanitizers else "checked" if device_checks else ""
    build_dir = os.path.join(ROOT, "_build", sub)
    os.makedirs(build_dir, exist_ok=True)
    if host_sanitizers and out == LIB:
        out = os.path.join(build_dir, "libkvs.so")
    if device_checks and out == LIB:
        out = CHECKED_LIB
    extra = HOST_SANITIZE + ["-Xarch_host", "-fno-omit-frame-pointer", "-g"] \
        if host_sanitizers else []
    if device_checks:
        extra = extra + ["-DKVS_DEVICE_CHECKS=1"]
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + compile_flags() + extra + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                     "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    link = HOST_SANITIZE if host_sanitizers else []
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + link + ["-o", tmp] + objs
         + ["-lrocprofiler-sdk-roctx"], verbose)
    os.replace(tmp, out)
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; drop that line
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, host_sanitizers="--host-sanitizers" in sys.argv,
                device_checks="--device-checks" in sys.argv))
