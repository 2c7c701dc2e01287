"""Build the HIP library in-tree: ``python -m projection_residual_rmsnorm_amd.build``.

Compiles every source under csrc/ for gfx950 with hipcc and links
``projection_residual_rmsnorm_amd/libprojaddnorm.so``, and the diagnostic variant
``libprojaddnorm_stamps.so``: the same sources and ABI with pr_kernels.hip compiled with
PR_PHASE_STAMPS (in-kernel phase and clock stamps of the single launch, read by
``python -m projection_residual_rmsnorm_amd.phases``).  Works without a GPU (hipcc
cross-compiles).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libprojaddnorm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
STAMPS_LIB_PATH = os.path.join(PKG_DIR, "libprojaddnorm_stamps.so")

SOURCES = ["pr_kernels.hip", "pr_silu.hip", "pr_fp8.hip", "pr_noalloc.hip", "pr_host.cpp", "pr_runtime.cpp",
           "pr_tune.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # code object v5 loads on every ROCm 6.x/7.x runtime, including the one bundled with torch
    "-mcode-object-version=5",
    "-Wno-unused-command-line-argument",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(hipcc: str, src: str, defines: tuple = ()) -> str:
    suffix = "".join("_" + d.lower() for d in defines)
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *("-D" + d for d in defines), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    return obj


def _link(hipcc: str, objs: list, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-mcode-object-version=5", "-shared", "-fPIC", "-o",
           tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, path)


def build_library(verbose: bool = False) -> str:
    """Compile and link the library and its phase-stamp variant; always rebuilds.  Returns the
    default library's path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    assert SOURCES[0] == "pr_kernels.hip"  # the one source the variant compiles differently
    jobs = [(src, ()) for src in SOURCES] + [("pr_kernels.hip", ("PR_PHASE_STAMPS",))]
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(hipcc, *j), jobs))
    _link(hipcc, objs[:len(SOURCES)], LIB_PATH)
    _link(hipcc, [objs[-1]] + objs[1:len(SOURCES)], STAMPS_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
        print(f"built {STAMPS_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
