"""Build liblcsa.so (the C-ABI library) for gfx950 in-tree.

Usage: python -m block_sparse_attention_03_amd.build_lib
Every call recompiles every source.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblcsa.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_SOURCES = ["lcsa_api.hip", "partition_pool.hip", "draft_mask.hip", "sparse_attn.hip",
               "fixed_lists.hip", "attn_bwd.hip"]
CXX_SOURCES = ["lcsa_host.cpp"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall",
             # keep hand-written float code off the packed-fp32 instructions
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # register arrays stay in registers (not silently moved to LDS)
             "-mllvm", "-disable-promote-alloca-to-lds"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


# per-source extras for the attention kernel:
# - its max reductions need no NaN propagation (a NaN input yields NaN output
#   either way), which lets the compiler use v_max3 without canonicalising
#   every operand;
# - the scheduler that favours instruction-level parallelism over register
#   pressure orders its main loop about 1 % faster at the same 225 registers
EXTRA = {"sparse_attn.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _clear_stale_objects() -> None:
    """Remove build objects whose source is no longer part of the library."""
    keep = {s + ".o" for s in HIP_SOURCES + CXX_SOURCES}
    for name in os.listdir(BUILD):
        if name.endswith(".o") and name not in keep:
            os.remove(os.path.join(BUILD, name))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _clear_stale_objects()
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", obj])
    for s in CXX_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj])
    workers = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        logs = list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
