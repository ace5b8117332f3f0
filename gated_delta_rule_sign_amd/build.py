"""Build libckda.so (HIP kernels + C ABI) for gfx950, in-tree.

Usage: python -m gated_delta_rule_sign_amd.build  (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libckda.so")
SOURCES = ["api.cpp", "decode.hip", "chunk.hip", "chunk_rev.hip", "chunk_grad.hip", "state.hip", "bwd.hip",
           "rev.hip", "grad.hip", "conv.hip"]
ARCH = os.environ.get("CKDA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, obj: str, extra=()) -> None:
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libckda.so next to this file."""
    from concurrent.futures import ThreadPoolExecutor

    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    extra = ["-Rpass-analysis=kernel-resource-usage"] if verbose else []
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(os.path.join(CSRC, so[0]), so[1], extra), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
