"""The hardware-rate probe library (libtilemix_probes.so, the timing-only
kernels behind the cost model) runs on the GPU: every probe launches at a
tiny size and returns 0, an out-of-range argument returns -1 with nothing
launched, and the shader-clock probe reports a plausible clock."""

import ctypes
import os

import pytest

import mixed_precision_attention_amd as tm

torch = pytest.importorskip("torch")

PROBES = os.path.join(os.path.dirname(tm.LIB_PATH), "libtilemix_probes.so")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
              pytest.mark.skipif(not os.path.exists(PROBES), reason="libtilemix_probes.so not built")]


def test_probes_run():
    lib = ctypes.CDLL(PROBES)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.tilemix_probe_valu.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_coexec.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_copy.argtypes = [vp, ci, ci, ci, ci, vp, vp]
    lib.tilemix_probe_lds.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_skeleton.argtypes = [ci, ci, ci, vp, vp]
    lib.tilemix_probe_clock.argtypes = [ci, ci, vp, vp]
    lib.tilemix_probe_read.argtypes = [ci, vp, vp, vp, vp]
    out = torch.zeros(512 * 512, dtype=torch.int32, device="cuda")
    p = out.data_ptr()
    for op in (0, 1):
        assert lib.tilemix_probe_valu(op, 256, 16, p, None) == 0
        assert lib.tilemix_probe_lds(op, 256, 4, p, None) == 0
    for mode in (0, 1, 2):
        assert lib.tilemix_probe_coexec(mode, 256, 16, p, None) == 0
    for extra in (0, 64, 128):
        assert lib.tilemix_probe_skeleton(extra, 256, 8, p, None) == 0
    src = torch.zeros(1 << 20, dtype=torch.int8, device="cuda")
    assert lib.tilemix_probe_copy(src.data_ptr(), 1024, 256, 4, 4, p, None) == 0
    assert lib.tilemix_probe_copy(src.data_ptr(), 1024, 256, 4, 17, p, None) == -1  # batch out of range
    n = 32768 * 8 * 128
    kbuf = torch.zeros(n, dtype=torch.int8, device="cuda")
    vbuf = torch.zeros(n, dtype=torch.int8, device="cuda")
    for pattern in range(4):
        assert lib.tilemix_probe_read(pattern, kbuf.data_ptr(), vbuf.data_ptr(), p, None) == 0
    stamps = torch.zeros(4, dtype=torch.int64, device="cuda")
    assert lib.tilemix_probe_clock(256, 20000, stamps.data_ptr(), None) == 0
    torch.cuda.synchronize()
    t0, t1, r0, r1 = stamps.tolist()
    ghz = (t1 - t0) / max(r1 - r0, 1) * 0.1
    assert 0.5 < ghz < 3.5, ghz
