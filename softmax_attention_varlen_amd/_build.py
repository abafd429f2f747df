"""Build the in-tree HIP library ``libattn_mi355x.so`` for gfx950 with hipcc.

Every source compiles to its own object in parallel, then one shared library
is linked next to this file. All GPU code is built with packed-fp32 VALU
instructions disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["attn_api.cpp", "varlen_fwd.hip", "prefill_pipe.hip", "paged_decode_stream.hip", "decode_scratch.hip", "paged_cache.hip", "padding.hip", "block_sparse.hip", "block_sparse_pipe.hip", "vsa_prep.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False, jobs: int | None = None, extra_flags=()) -> str:
    """Compile every source and link the shared library. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *COMMON_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        _run(cmd, verbose)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    build_calib(verbose=verbose, extra_flags=extra_flags)
    return LIB_PATH


# The MFMA calibration kernel that bench.py times beside the attention
# roofline; a library of its own, not part of the attention C ABI.
CALIB_SOURCE = os.path.join(HERE, "calib", "mfma_stream.hip")
CALIB_LIB_PATH = os.path.join(HERE, "libattn_calib.so")


def build_calib(verbose: bool = False, extra_flags=()) -> str:
    tmp = CALIB_LIB_PATH + ".tmp"
    _run([_hipcc(), "-x", "hip", *COMMON_FLAGS, *extra_flags, "-shared", CALIB_SOURCE, "-o", tmp], verbose)
    os.replace(tmp, CALIB_LIB_PATH)
    return CALIB_LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
