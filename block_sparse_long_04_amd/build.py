"""Build the HIP library libflashprefill.so in-tree for gfx950.

Usage: python -m block_sparse_long_04_amd.build  (or build_library() from Python).
hipcc compiles every csrc/*.hip file (the kernels and the C ABI), one
process per file, and links them into one shared library next to this file.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libflashprefill.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        "-Wno-unused-function",
        # no packed-fp32 VALU instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(os.path.dirname(PKG_DIR), "include"),
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        # keep warnings visible (the host pass warns about the GPU-only feature flag)
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


def build_library(verbose: bool = True, extra: list = None) -> str:
    """Compile every csrc/*.hip to an object in parallel, then link them into
    the shared library (each object carries its own gfx950 code object)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = [f for f in compile_flags() if f != "-shared"] + (extra or [])
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="fpbuild_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda so: _run([hipcc()] + flags + ["-c", so[0], "-o", so[1]], verbose),
                        zip(srcs, objs)))
        tmp = LIB_PATH + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library())
