"""Build libtilemix.so in-tree with hipcc for gfx950.

Run as ``python -m mixed_precision_attention_amd.build`` (or through
``__graft_entry__.build()``).  The library is written next to this file.

Two checking builds, written under ``_build/`` (never loaded unless the
``TILEMIX_LIB`` environment variable names them):

* ``--debug``: every device entry point also reads back the device copy of
  the plan's header and requires it to equal the host copy's (checksum
  included), which costs a synchronous copy per call;
* ``--host-sanitize``: the host code (routing, planner, argument checks of
  every entry point) instrumented with AddressSanitizer and
  UndefinedBehaviorSanitizer; the device code is unchanged.  Run the CPU
  tests against it with the sanitizer runtime preloaded, e.g.
  ``ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD=<clang asan runtime>
  TILEMIX_LIB=_build/host_sanitize/libtilemix.so python -m pytest
  tests/test_abi_cpu.py tests/test_oracle_routing.py``, the runtime being
  ``$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)``
  (``tests/test_host_sanitize.py`` does exactly this).
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

# The hardware-rate probes (timing-only kernels for the measurement record),
# a library of their own.
PROBES_NAME = "libtilemix_probes.so"
PROBES_PATH = os.path.join(HERE, PROBES_NAME)
PROBES_SOURCES = ["tilemix_probes.hip"]

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


# Host-side sanitizers: each -fsanitize= goes to the host compilation only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
DEBUG_FLAGS = ["-DTILEMIX_DEBUG_PLAN"]


def build(verbose: bool = False, extra_flags=None, out_path: str = LIB_PATH, link_flags=None,
          sources=None) -> str:
    """Compile every source into ``libtilemix.so`` (at ``out_path``); returns its path."""
    out_dir = os.path.dirname(out_path)
    os.makedirs(out_dir, exist_ok=True)
    out_tmp = out_path + ".tmp"
    objs = []
    for src in sources or SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "c++"]
        cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
               *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *(link_flags or []), *objs, "-o", out_tmp],
         verbose)
    os.replace(out_tmp, out_path)
    for obj in objs:
        os.remove(obj)
    return out_path


def build_probes(verbose: bool = False) -> str:
    """The hardware-rate probe library ``libtilemix_probes.so``, next to this file."""
    return build(verbose, out_path=PROBES_PATH, sources=PROBES_SOURCES)


def build_checking(kind: str, verbose: bool = False) -> str:
    """The ``debug`` or ``host_sanitize`` build, under ``_build/<kind>/``."""
    out = os.path.join(ROOT, "_build", kind, LIB_NAME)
    if kind == "debug":
        return build(verbose, DEBUG_FLAGS, out)
    if kind == "host_sanitize":
        return build(verbose, SANITIZE_HOST, out, link_flags=SANITIZE_HOST)
    raise ValueError(kind)


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
    if "--debug" in sys.argv[1:]:
        print(build_checking("debug", verbose=True))
    elif "--host-sanitize" in sys.argv[1:]:
        print(build_checking("host_sanitize", verbose=True))
    else:
        print(build(verbose=True))
        print(build_probes(verbose=True))
