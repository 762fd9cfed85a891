"""One sequence longer than 1024 key tiles (L = 66,600: Tn = 1041, g = 17),
against the oracle on sampled query-tile rows, the last row included.  Such a
row visits key tiles 0..1040, so the fused kernels re-stage the key-tile
scales (INT8, and FP8 in the three-path kernel) at tile 1024 -- a path no
shorter sequence reaches.  Two-path prefill (Q's codes read from the
quantiser, and Q quantised inside the kernel: bit-identical) and three-path
prefill (both forms, bit-identical)."""

import numpy as np
import pytest

import oracle
import synth
import mixed_precision_attention_amd as tm

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MAX_ABS = 4e-3
MEAN_ABS = 5e-4
L = 66600
ROWS = [(0, 0, 0), (0, 1, 256), (0, 0, 519), (0, 1, 520)]


def _rows_err(out, ref):
    errs = []
    for (s, h, r) in ROWS:
        a, b = 128 * r, min(128 * r + 128, L)
        errs.append(np.abs(out[a:b, h].astype(np.float64) - ref[a:b, h]).ravel())
    e = np.concatenate(errs)
    assert np.all(np.isfinite(e))
    return e.max(), e.mean()


def test_two_path_beyond_1024_key_tiles():
    print(f"two-path prefill L={L} (Tn=1041, g=17), rowrandom 75%", flush=True)
    q, k, v, cu = synth.make_qkv([L], 2, 1, 128, outliers=True, seed=61)
    geo = oracle.seq_geometry(L)
    assert (geo.Tn, geo.g) == (1041, 17)
    tp = tm.TileMixPrefill(cu, 2, 1, 128, "rowrandom", 7500)
    assert int(tp.words[0, 520]) >> 60   # INT8 groups 60, 61: key tiles from 1020 on
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = tp(qd, kd, vd)
    out_inline = tp(qd, kd, vd, inline_q=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_inline.view(torch.int16))
    ref = oracle.run(q, k, v, cu, 2, 1, "rowrandom", 7500, rows=ROWS)
    assert np.array_equal(tp.words, ref["words"])
    assert np.array_equal(tp.k_scale.cpu().numpy()[:, :tp.tk].view(np.uint32), ref["k_scale"].view(np.uint32))
    mx, mean = _rows_err(out.cpu().numpy(), ref["out"])
    print(f"  err max/mean {mx:.3e} {mean:.3e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS


def test_three_path_beyond_1024_key_tiles():
    # N(0,1) inputs: the FP8 matrix instruction's accumulation stays far below
    # the bar there (outlier channels are covered by test_gpu_fp8.py)
    print(f"three-path prefill L={L}, rowrandom int8 50% fp8 25%", flush=True)
    q, k, v, cu = synth.make_qkv([L], 2, 1, 128, outliers=False, seed=62)
    tp = tm.TileMixPrefill3(cu, 2, 1, 128, "rowrandom", 5000, 2500)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = tp(qd, kd, vd)
    out_inline = tp(qd, kd, vd, inline_q=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_inline.view(torch.int16))
    q_i8, qs = oracle.quantize_blocks(q, cu, 128)
    k_i8, ks = oracle.quantize_blocks(k, cu, 64)
    qf, qfs = oracle.quantize_blocks_fp8(q, cu, 128)
    kf, kfs = oracle.quantize_blocks_fp8(k, cu, 64)
    assert np.array_equal(tp.k_scale_f8.cpu().numpy()[:, :tp.tk].view(np.uint32), kfs.view(np.uint32))
    ref = oracle.prefill_attention3(q, k, v, q_i8, k_i8, qs, ks, qf, kf, qfs, kfs, tp.words, tp.words_f8,
                                    cu, 2, 1, rows=ROWS)
    # past key tile 1024 (group 60 on): row 519 has an FP8 group, row 520 INT8 ones
    assert (int(tp.words_f8[0, 519]) >> 61) & 1 and int(tp.words[0, 520]) >> 60
    mx, mean = _rows_err(out.cpu().numpy(), ref)
    print(f"  err max/mean {mx:.3e} {mean:.3e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
