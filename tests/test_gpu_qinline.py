"""The prefill variant that quantises Q inside the kernel, through the C ABI:
its key-only quantiser is bit-exact with the oracle's key blocks, and its
output is bit-identical to the two-kernel path (quantiser, then prefill) on
the same inputs, and so within the oracle bar of that path."""

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


def _log(msg):
    print(msg, flush=True)


def both_paths(q, k, v, cu, hq, hkv, template, cov, seed=0):
    d = q.shape[2]
    tp = tm.TileMixPrefill(cu, hq, hkv, d, template, cov, seed)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    ref = torch.full_like(qd, float("nan"))
    tp(qd, kd, vd, ref)
    k_i8 = tp.k_i8.clone()
    k_scale = tp.k_scale.clone()
    tp.k_i8.fill_(0x55)
    tp.k_scale.fill_(float("nan"))
    out = torch.full_like(qd, float("nan"))
    tp(qd, kd, vd, out, inline_q=True)
    torch.cuda.synchronize()
    T = q.shape[0]
    assert torch.equal(tp.k_i8[:T], k_i8[:T])
    assert torch.equal(tp.k_scale[:, :tp.tk].view(torch.int32), k_scale[:, :tp.tk].view(torch.int32))
    return ref, out, tp


def assert_bit_identical(a, b):
    same = a.view(torch.int16) == b.view(torch.int16)
    assert bool(same.all()), f"{int((~same).sum())} of {same.numel()} outputs differ"


@pytest.mark.parametrize("lens,hq,hkv,d", [([256], 1, 1, 64), ([300, 77, 0, 129, 1, 64], 4, 2, 64),
                                           ([1024] * 2, 24, 8, 128), ([200, 513], 7, 1, 128)])
def test_quantize_k_bit_exact(lens, hq, hkv, d):
    _log(f"quantize_k lens={lens} hq={hq} hkv={hkv} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=23)
    tp = tm.TileMixPrefill(cu, hq, hkv, d, "band", 5000)
    kd = torch.from_numpy(k).cuda()
    tp.k_i8.fill_(0x55)
    tp.quantize_k(kd)
    torch.cuda.synchronize()
    ok, osk = oracle.quantize_blocks(k, cu, 64)
    assert np.array_equal(tp.k_i8.cpu().numpy()[:k.shape[0]], ok)
    assert np.array_equal(tp.k_scale.cpu().numpy()[:, :tp.tk].view(np.uint32), osk.view(np.uint32))


@pytest.mark.parametrize("template,cov,d", [("band", 5000, 64), ("global", 10000, 128), ("rowrandom", 2500, 128),
                                            ("sptrans", 7500, 64), ("bigbird", 0, 128)])
def test_bit_identical_and_oracle_varlen(template, cov, d):
    lens, hq, hkv = [300, 77, 0, 129, 1, 520], 6, 2
    _log(f"qinline varlen {template} cov={cov} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=29)
    ref, out, tp = both_paths(q, k, v, cu, hq, hkv, template, cov, seed=3)
    assert_bit_identical(ref, out)
    exp = oracle.run(q, k, v, cu, hq, hkv, template, cov, seed=3)["out"]
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - exp)
    assert np.all(np.isfinite(got))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


def test_zero_and_tie_q_blocks():
    # an all-zero Q block (s = 0), a block whose values sit on rounding ties,
    # and a block whose absmax is carried by one row of one wave
    _log("qinline zero/tie blocks")
    lens, hq, hkv, d = [300], 3, 1, 64
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=31)
    q[:128, 0] = 0
    q[:128, 1] = 0
    q[:128, 1, 0] = 127.0
    q[:128, 1, 1:8] = np.array([2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0], dtype=np.float16)
    q[128:256, 2] *= 0.01
    q[200, 2, 5] = 40.0
    for cov in (10000, 5000):
        ref, out, tp = both_paths(q, k, v, cu, hq, hkv, "band", cov)
        assert_bit_identical(ref, out)


@pytest.mark.parametrize("cov", [7500, 10000])
def test_headline_bit_identical(cov):
    _log(f"qinline 3B L=4096 B=8 sptrans cov={cov}")
    q, k, v, cu, spec = synth.make_workload("llama3b_l4k")
    ref, out, _ = both_paths(q, k, v, cu, spec["hq"], spec["hkv"], "sptrans", cov)
    assert_bit_identical(ref, out)


@pytest.mark.parametrize("workload,template,cov", [("llama3b_l8k", "rowrandom", 5000),
                                                   ("qwen2_7b_varlen", None, None)])
def test_other_workloads_bit_identical(workload, template, cov):
    q, k, v, cu, spec = synth.make_workload(workload)
    template = template or spec["template"]
    cov = spec["coverage_bp"] if cov is None else cov
    _log(f"qinline {workload} {template} cov={cov}")
    ref, out, _ = both_paths(q, k, v, cu, spec["hq"], spec["hkv"], template, cov)
    assert_bit_identical(ref, out)
