"""Build libcsa.so for gfx950 with hipcc (in-tree; objects under _build/).

Usage: python -m sparse_long_context_csa_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")

ARCH = "gfx950"
# No fast-math; packed fp32 instructions are disabled (hipcc otherwise emits v_pk_* ops).
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["compress.hip", "index_scan.hip", "index_prefill.hip", "topk.hip", "attention.hip", "norm_rope.hip",
           "mxfp4.hip", "kv_fp8.hip", "kv_fp4.hip", "api.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libcsa needs ROCm's hipcc to build")


def _run(cmd: list[str]) -> None:
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libcsa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []

    def one(src: str) -> str:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
