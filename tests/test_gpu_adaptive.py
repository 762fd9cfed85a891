"""Parity of the adaptive-routing statistic (HIP, through the C ABI) with the
oracle: group importances bit-exact, the words selected from them bit-exact
(on the device and by the host ranking), and the fused prefill under those
words within the fp16 tolerance."""

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


def _run(q, k, v, cu, hq, hkv, cov, on_device=True):
    d = q.shape[2]
    tp = tm.TileMixPrefill(cu, hq, hkv, d, "band", 0)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    tp.quantize(qd, kd)
    imp = tp.set_routing_adaptive(cov, on_device=on_device)
    if on_device:
        imp = imp.cpu().numpy()[:, :tp.tq]
    tp.words_host()
    out = torch.full_like(qd, float("nan"))
    tp.attend(qd, kd, vd, out)
    torch.cuda.synchronize()
    T = q.shape[0]
    return tp, imp, out.cpu().numpy(), tp.q_i8.cpu().numpy()[:T], tp.k_i8.cpu().numpy()[:T], \
        tp.q_scale.cpu().numpy()[:, :tp.tq], tp.k_scale.cpu().numpy()[:, :tp.tk]


@pytest.mark.parametrize("on_device", [True, False])
@pytest.mark.parametrize("lens,hq,hkv,d,cov", [([256], 1, 1, 64, 5000), ([300, 77, 0, 129, 1, 64], 6, 2, 64, 2500),
                                               ([1024, 513], 6, 2, 128, 7500), ([4160], 3, 1, 128, 5000)])
def test_importance_and_words_bit_exact(lens, hq, hkv, d, cov, on_device):
    _log(f"adaptive lens={lens} hq={hq} hkv={hkv} d={d} cov={cov} on_device={on_device}")
    q, k, v, cu = synth.make_qkv_local(lens, hq, hkv, d, seed=41)
    tp, imp, out, q_i8, k_i8, qs, ks = _run(q, k, v, cu, hq, hkv, cov, on_device)
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


def _select_on_device(tp, imp, cov):
    """Words from the device selection for a given importance array."""
    words_d = torch.full((tp.hkv, max(tp.tq, 1)), -1, dtype=torch.int64, device="cuda")
    n8, nl = tm.tilemix_select_routing_adaptive(tp.plan_h, tp.plan_d, torch.from_numpy(imp).cuda(), cov, words_d)
    torch.cuda.synchronize()
    return words_d.cpu().numpy().view(np.uint64)[:, :tp.tq], n8, nl


@pytest.mark.parametrize("lens,hkv", [([300, 77, 0, 129, 1, 64], 2), ([4096, 8192], 3), ([65536, 1024], 1)])
def test_device_selection_ties_and_signed_zeros(lens, hkv):
    """Importances from a handful of values (so most groups tie and the
    (r, G) order decides), with -0.0 beside +0.0 and infinities: the device
    selection equals the host ranking and the oracle at every coverage,
    including the empty and full ones."""
    _log(f"device word selection lens={lens} hkv={hkv}")
    cu = synth.cu_seqlens_of(lens)
    tp = tm.TileMixPrefill(cu, hkv, hkv, 64, "band", 0)
    rng = np.random.default_rng(7)
    vals = np.array([-np.inf, -2.5, -1.0, -0.0, 0.0, 0.5, 3.0, np.inf], dtype=np.float32)
    for trial in range(2):
        imp = vals[rng.integers(0, vals.size, size=(hkv, tp.tq, 64))]
        if trial == 1:  # mostly distinct values, a few ties
            imp = rng.standard_normal((hkv, tp.tq, 64)).astype(np.float32)
            imp[rng.random(imp.shape) < 0.1] = np.float32(0.25)
            imp[rng.random(imp.shape) < 0.05] = np.float32(-0.0)
        for cov in (0, 1, 2500, 5000, 7777, 9999, 10000):
            wd, n8, nl = _select_on_device(tp, imp, cov)
            wh, gh, n8h, nlh = tm.tilemix_build_routing_adaptive(cu, imp, cov)
            ow, og, on8, onl = oracle.adaptive_words(lens, imp, cov)
            assert np.array_equal(wh, ow), (trial, cov)
            assert np.array_equal(wd, ow), (trial, cov)
            assert list(n8) == list(on8) and list(nl) == list(onl)
            r0 = 0
            for s_, L in enumerate(lens):
                r1 = r0 + -(-L // 128)
                assert sum(bin(int(x)).count("1") for x in wd[:, r0:r1].ravel()) == hkv * int(on8[s_])
                r0 = r1
