"""The host half of libtilemix under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): build.py's host-sanitized build, then
the host-side ABI and routing tests in a child process with the sanitizer
runtime preloaded.  Any report (out-of-bounds access, use after free,
undefined behaviour such as a NULL pointer handed to memcpy) aborts the child
and fails this test."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _asan_runtime():
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime not found")
    sys.path.insert(0, ROOT)
    from mixed_precision_attention_amd import build as b
    lib = b.build_checking("host_sanitize")
    log = str(tmp_path / "san")
    env = dict(os.environ, TILEMIX_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS=f"detect_leaks=0:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:log_path={log}")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_abi_cpu.py", "tests/test_oracle_routing.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(f).read() for f in glob.glob(log + "*"))
    assert res.returncode == 0 and not reports, (res.stdout[-2000:], reports[:4000])
