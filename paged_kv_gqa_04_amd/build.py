"""Build the HIP library ``libpkv.so`` in-tree for gfx950.

``python -m paged_kv_gqa_04_amd.build`` (or ``build()``) compiles the host
planner and the HIP kernels with hipcc into the package directory. No GPU is
needed to build.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HOST_SOURCES = ["plan.cpp", "pool.cpp"]  # plain C++, built by the host compiler
HIP_SOURCES = ["decode.hip", "append.hip", "stream.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
              "-I", os.path.join(ROCM, "include")]

# -packed-fp32-ops off: hipcc must not emit packed fp32 arithmetic
# (v_pk_fma_f32 and friends) for these kernels.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Preload the leading kernel arguments into SGPRs at wave launch (the
    # partial kernel passes its prologue's arguments first for this).
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"{cmd[0]} failed with exit code {res.returncode}")
    noise = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = True, extra_flags=None) -> str:
    """Compile libpkv.so; returns its path. Always recompiles."""
    cxx = shutil.which("g++") or "g++"
    build_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        _run([cxx, *HOST_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        objs.append(obj)
    out_tmp = LIB_PATH + ".tmp"
    _run([hipcc(), *HIP_FLAGS, *(extra_flags or []), "-shared", "-I", INCLUDE,
          "-o", out_tmp, *[os.path.join(CSRC, s) for s in HIP_SOURCES], "-x", "none", *objs],
         verbose)
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
