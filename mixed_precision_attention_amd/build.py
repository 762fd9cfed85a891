"""Build libtilemix.so in-tree with hipcc for gfx950.

Run as ``python -m mixed_precision_attention_amd.build`` (or through
``__graft_entry__.build()``).  The library is written next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libtilemix.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["tilemix_host.cpp", "tilemix_kernels.hip", "tilemix_decode.hip", "tilemix_adaptive.hip",
           "tilemix_stack.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU forms.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libtilemix)")
    return path


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source into ``libtilemix.so``; returns its path."""
    out_tmp = LIB_PATH + ".tmp"
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "c++"]
        cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
               *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
    os.replace(out_tmp, LIB_PATH)
    for obj in objs:
        os.remove(obj)
    return LIB_PATH


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
