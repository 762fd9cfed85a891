"""Parity of the adaptive-routing statistic (HIP, through the C ABI) with the
oracle: group importances bit-exact, the words built from them bit-exact, and
the fused prefill under those words within the fp16 tolerance."""

import numpy as np
import pytest

import oracle
import synth
import mixed_precision_attention_amd as tm

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _log(msg):
    print(msg, flush=True)


def _run(q, k, v, cu, hq, hkv, cov):
    d = q.shape[2]
    tp = tm.TileMixPrefill(cu, hq, hkv, d, "band", 0)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    tp.quantize(qd, kd)
    imp = tp.set_routing_adaptive(cov)
    out = torch.full_like(qd, float("nan"))
    tp.attend(qd, kd, vd, out)
    torch.cuda.synchronize()
    T = q.shape[0]
    return tp, imp, out.cpu().numpy(), tp.q_i8.cpu().numpy()[:T], tp.k_i8.cpu().numpy()[:T], \
        tp.q_scale.cpu().numpy()[:, :tp.tq], tp.k_scale.cpu().numpy()[:, :tp.tk]


@pytest.mark.parametrize("lens,hq,hkv,d,cov", [([256], 1, 1, 64, 5000), ([300, 77, 0, 129, 1, 64], 6, 2, 64, 2500),
                                               ([1024, 513], 6, 2, 128, 7500), ([4160], 3, 1, 128, 5000)])
def test_importance_and_words_bit_exact(lens, hq, hkv, d, cov):
    _log(f"adaptive lens={lens} hq={hq} hkv={hkv} d={d} cov={cov}")
    q, k, v, cu = synth.make_qkv_local(lens, hq, hkv, d, seed=41)
    tp, imp, out, q_i8, k_i8, qs, ks = _run(q, k, v, cu, hq, hkv, cov)
    oq, oqs = oracle.quantize_blocks(q, cu, 128)
    ok, oks = oracle.quantize_blocks(k, cu, 64)
    assert np.array_equal(q_i8, oq) and np.array_equal(k_i8, ok)
    oimp = oracle.routing_importance(oq, ok, oqs, oks, cu, hq, hkv)
    assert np.array_equal(imp.view(np.uint32), oimp.view(np.uint32))
    ow, og, on8, onl = oracle.adaptive_words(lens, oimp, cov)
    assert np.array_equal(tp.words, ow)
    ref = oracle.prefill_attention(q, k, v, oq, ok, oqs, oks, ow, cu, hq, hkv)
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(np.isfinite(out)) and err.max() <= 4e-3 and err.mean() <= 5e-4


def test_headline_shape_words():
    _log("adaptive llama3b_l4k shape (locality inputs)")
    lens, hq, hkv, d = [4096] * 2, 24, 8, 128
    q, k, v, cu = synth.make_qkv_local(lens, hq, hkv, d, seed=42)
    tp, imp, out, q_i8, k_i8, qs, ks = _run(q, k, v, cu, hq, hkv, 7500)
    oimp = oracle.routing_importance(q_i8, k_i8, qs, ks, cu, hq, hkv)
    assert np.array_equal(imp.view(np.uint32), oimp.view(np.uint32))
    ow, *_ = oracle.adaptive_words(lens, oimp, 7500)
    assert np.array_equal(tp.words, ow)
    # words differ between KV heads (content-dependent), unlike a template
    assert not all(np.array_equal(tp.words[0], tp.words[h]) for h in range(hkv))
