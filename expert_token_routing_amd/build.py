"""Build libocc.so (the HIP library) in-tree for gfx950.

Each .hip source is compiled to an object with hipcc in parallel, then linked
into ``expert_token_routing_amd/libocc.so``.  Packed-fp32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libocc.so")
ARCH = os.environ.get("OCC_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "route.hip", "brim.hip", "rows.hip", "gemm_bf16.hip", "gemm_f32.hip",
           "coact.hip", "similarity.hip", "gate.hip", "gemm_bf16_m128.hip", "gemm_bf16_dense.hip",
           "gemm_bwd.hip", "backward.hip"]

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep small per-thread arrays (GEMM staging registers) out of LDS: the
    # promotion runs before unrolling and would add a conflicting LDS copy
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CXXFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in r.stderr.splitlines() if ln.strip() and noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(extra: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every source and link libocc.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra or [])
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
