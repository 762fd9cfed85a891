"""Parity of the INT8-cache decode step (HIP, through the C ABI) with the CPU
oracle on identical seeded inputs.  The int8 cache and its scales must be
bit-exact; the fp16 output must satisfy max |err| <= 4e-3 and mean |err| <=
5e-4 against the oracle's float64 result."""

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


def run_decode(q_new, k, v, cu, hq, hkv, template, cov, seed=0):
    d = k.shape[2]
    td = tm.TileMixDecode(cu, hq, hkv, d, template, cov, seed)
    kd, vd = (torch.from_numpy(x).cuda() for x in (k, v))
    qd = torch.from_numpy(q_new).cuda()
    td.fill_cache(kd, vd)
    out = torch.full((len(cu) - 1, hq, d), float("nan"), dtype=torch.float16, device="cuda")
    td.step(qd, out)
    torch.cuda.synchronize()
    T = k.shape[0]
    return dict(out=out.cpu().numpy(), k_i8=td.k_i8.cpu().numpy()[:T], v_i8=td.v_i8.cpu().numpy()[:T],
                k_scale=td.k_scale.cpu().numpy()[:, :td.tk], v_scale=td.v_scale.cpu().numpy()[:, :td.tk],
                words=td.words, td=td, dev=(qd, kd, vd))


def oracle_decode(q_new, k, v, cu, hq, hkv, words):
    k_i8, ks, v_i8, vs = oracle.quantize_kv_cache(k, v, cu)
    return oracle.decode_attention(q_new, k_i8, ks, v_i8, vs, words, cu, hq, hkv)


def assert_close(got, ref):
    got = got.astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert err.max() <= MAX_ABS, f"max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean():.3e}"
    return err.max(), err.mean()


@pytest.mark.parametrize("lens,hkv,d", [([300, 77, 0, 129, 1, 64], 2, 64), ([1024, 513], 8, 128),
                                        ([4160, 65], 1, 128)])
def test_cache_quantizer_bit_exact(lens, hkv, d):
    _log(f"cache quantizer lens={lens} hkv={hkv} d={d}")
    q, k, v, cu = synth.make_qkv(lens, 2 * hkv, hkv, d, outliers=True, seed=31)
    g = run_decode(synth.decode_queries(q, cu), k, v, cu, 2 * hkv, hkv, "band", 5000)
    ok, oks, ov, ovs = oracle.quantize_kv_cache(k, v, cu)
    assert np.array_equal(g["k_i8"], ok) and np.array_equal(g["v_i8"], ov)
    assert np.array_equal(g["k_scale"].view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(g["v_scale"].view(np.uint32), ovs.view(np.uint32))


@pytest.mark.parametrize("template,cov,hq,hkv,d", [
    ("band", 0, 6, 2, 64), ("band", 5000, 6, 2, 64), ("band", 10000, 6, 2, 64),
    ("sptrans", 7500, 3, 1, 128), ("rowrandom", 5000, 7, 1, 128), ("global", 2500, 12, 1, 128),
    ("bigbird", 5000, 16, 2, 64), ("alignedsparse", 2500, 4, 4, 128)])
def test_decode_varlen(template, cov, hq, hkv, d):
    lens = [300, 1, 0, 64, 65, 513, 1100]
    _log(f"decode {template} cov={cov} hq={hq} hkv={hkv} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=32)
    q_new = synth.decode_queries(q, cu)
    g = run_decode(q_new, k, v, cu, hq, hkv, template, cov)
    ref = oracle_decode(q_new, k, v, cu, hq, hkv, g["words"])
    assert_close(g["out"], ref)
    assert not g["out"][2].any()  # empty sequence


def test_decode_long_rows_g2():
    # L = 4160: g = 2, so the bit of key tile t is t // 2
    lens, hq, hkv, d = [4160, 8192], 3, 1, 128
    _log(f"decode long rows lens={lens}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=33)
    q_new = synth.decode_queries(q, cu)
    for template, cov in (("sptrans", 5000), ("rowrandom", 2500)):
        g = run_decode(q_new, k, v, cu, hq, hkv, template, cov)
        assert_close(g["out"], oracle_decode(q_new, k, v, cu, hq, hkv, g["words"]))


@pytest.mark.parametrize("cov", [7500, 0, 10000])
def test_decode_llama3b_l4k(cov):
    _log(f"decode llama3b_l4k cov={cov}")
    q, k, v, cu, spec = synth.make_workload("llama3b_l4k")
    q_new = synth.decode_queries(q, cu)
    g = run_decode(q_new, k, v, cu, spec["hq"], spec["hkv"], "sptrans", cov)
    assert_close(g["out"], oracle_decode(q_new, k, v, cu, spec["hq"], spec["hkv"], g["words"]))


def test_decode_qwen_varlen():
    _log("decode qwen2_7b_varlen")
    q, k, v, cu, spec = synth.make_workload("qwen2_7b_varlen")
    q_new = synth.decode_queries(q, cu)
    g = run_decode(q_new, k, v, cu, spec["hq"], spec["hkv"], spec["template"], spec["coverage_bp"])
    assert_close(g["out"], oracle_decode(q_new, k, v, cu, spec["hq"], spec["hkv"], g["words"]))


def test_decode_special_cases():
    _log("decode special cases")
    lens, hq, hkv, d = [1, 190, 64], 4, 2, 64
    cu = synth.cu_seqlens_of(lens)
    q, k, _, _ = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=34)
    q_new = synth.decode_queries(q, cu)
    # constant values held exactly by the cache -> O is that constant
    v = np.full(k.shape, np.float16(127 / 128))
    v[:, 1, :] = np.float16(-127 / 32)
    g = run_decode(q_new, k, v, cu, hq, hkv, "rowrandom", 5000)
    want = np.where((np.arange(hq) // 2 == 0)[None, :, None], 127 / 128, -127 / 32)
    assert np.abs(g["out"].astype(np.float64) - want).max() <= 2e-3
    # a single cached token: O is its dequantised value
    v = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=35)
    g = run_decode(q_new, k, v, cu, hq, hkv, "band", 10000)
    assert np.array_equal(g["out"][0], v[0][[0, 0, 1, 1]])
    # zero cache values and zero queries: scale 0 everywhere, O = 0
    z = np.zeros_like(k)
    g = run_decode(np.zeros_like(q_new), z, z, cu, hq, hkv, "band", 5000)
    assert not g["out"].any()
    # deterministic across calls
    g1 = run_decode(q_new, k, v, cu, hq, hkv, "band", 5000)
    out2 = g1["td"].step(g1["dev"][0])
    assert np.array_equal(out2.cpu().numpy(), g1["out"])


def test_decode_matches_prefill_last_row_on_exact_cache():
    # K, V held exactly by the cache: the decode step of the newest token and
    # the fused prefill's row L - 1 compute the same attention at 0% (fp16
    # query against the same keys).
    lens, hq, hkv, d = [700, 128, 1], 6, 2, 128
    _log("decode vs prefill last row")
    cu = synth.cu_seqlens_of(lens)
    q, _, _, _ = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=36)
    k = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=37)
    v = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=38)
    q_new = synth.decode_queries(q, cu)
    g = run_decode(q_new, k, v, cu, hq, hkv, "band", 0)
    tp = tm.TileMixPrefill(cu, hq, hkv, d, "band", 0)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = tp(qd, kd, vd).cpu().numpy().astype(np.float64)
    last = out[cu[1:] - 1]
    assert np.abs(g["out"].astype(np.float64) - last).max() <= MAX_ABS


@pytest.mark.parametrize("lens,hq,hkv,d", [([4096, 3000, 1, 0, 2500, 4000], 6, 2, 128),
                                           ([1000, 4096, 77], 7, 1, 64)])
def test_decode_alternating_steps(lens, hq, hkv, d):
    """Steps alternate between two query sets, through the workspace and the
    allocation-free entry points (which share the chunk records' memory
    between calls): every output equals the first output of its set bit for
    bit (a record left from the step before would carry the other set's
    values), and both match the oracle."""
    _log(f"decode alternating steps lens={lens} hq={hq} hkv={hkv} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=51)
    q2 = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=52)[0]
    qa, qb = synth.decode_queries(q, cu), synth.decode_queries(q2, cu)
    g = run_decode(qa, k, v, cu, hq, hkv, "sptrans", 7500)
    td = g["td"]
    ref_a = oracle_decode(qa, k, v, cu, hq, hkv, g["words"])
    ref_b = oracle_decode(qb, k, v, cu, hq, hkv, g["words"])
    qd = [torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda()]
    first = [None, None]
    outs = []
    for step in range(48):
        s = step % 2
        out = torch.full((len(cu) - 1, hq, d), float("nan"), dtype=torch.float16, device="cuda")
        td.step(qd[s], out, noalloc=(step % 3 == 2))
        outs.append((s, out))
    torch.cuda.synchronize()
    for s, out in outs:
        o = out.cpu().numpy()
        if first[s] is None:
            first[s] = o
            assert_close(o, ref_a if s == 0 else ref_b)
        assert np.array_equal(o.view(np.uint16), first[s].view(np.uint16))
    assert not np.array_equal(first[0], first[1])
    for i, L in enumerate(lens):
        if L == 0:
            assert not first[0][i].any() and not first[1][i].any()
