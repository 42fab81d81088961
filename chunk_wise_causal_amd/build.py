"""Build libwf.so in-tree for gfx950 with hipcc.

    python -m chunk_wise_causal_amd.build          # or __graft_entry__.build()

Always recompiles (the sources in parallel).  Flags: -O3, C++17, position-independent shared library,
and packed FP32 instructions disabled on the device (hipcc's host pass warns
that it does not know that target feature; the warning is harmless).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libwf.so")
SOURCES = ["api.cpp", "status.hip", "publish.hip", "attn_bf16.hip", "attn_fp32.hip",
           "rotate.hip", "attn_mx.hip", "qkv_gemm.hip"]
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}"]


# per-source options: the 8-bit attention kernel's grouping hints name only the
# vector work and the reads and leave its block-scaled products to the machine
# scheduler, which places them better with the maximum-ILP strategy
SOURCE_FLAGS = {"attn_mx.hip": ["-mllvm", "--amdgpu-sched-strategy=max-ilp"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel, `jobs` at a time; 0: one per CPU,
    at most 8) and link libwf.so."""
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(build_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        return obj

    workers = jobs or max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
