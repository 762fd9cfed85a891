"""Parity of the HIP path (through the C ABI) with the CPU oracle on identical
seeded inputs.  Integer outputs (int8 Q/K, scales, int32 tiles) must be
bit-exact; the fp16 output must satisfy max |err| <= 4e-3 and mean |err| <=
5e-4 against the oracle's float64 result."""

import os

import numpy as np
import pytest

import oracle
import synth
import mixed_precision_attention_amd as tm
from independent import naive_causal_attention

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MAX_ABS = 4e-3
MEAN_ABS = 5e-4


def _log(msg):
    print(msg, flush=True)


def run_gpu(q, k, v, cu, hq, hkv, template, cov, seed=0, words=None):
    d = q.shape[2]
    tp = tm.TileMixPrefill(cu, hq, hkv, d, template, cov, seed)
    if words is not None:
        tp.words_d = torch.from_numpy(np.ascontiguousarray(words).view(np.int64)).cuda()
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    tp(qd, kd, vd, out)
    torch.cuda.synchronize()
    T = q.shape[0]
    return dict(out=out.cpu().numpy(), q_i8=tp.q_i8.cpu().numpy()[:T], k_i8=tp.k_i8.cpu().numpy()[:T],
                q_scale=tp.q_scale.cpu().numpy()[:, :tp.tq], k_scale=tp.k_scale.cpu().numpy()[:, :tp.tk],
                words=tp.words, tp=tp, dev=(qd, kd, vd))


def assert_close(got, ref, rows=None):
    got = got.astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert err.max() <= MAX_ABS, f"max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean():.3e}"
    return err.max(), err.mean()


# --------------------------------------------------------------- quantiser

@pytest.mark.parametrize("lens,hq,hkv,d", [([256], 1, 1, 64), ([300, 77, 0, 129, 1, 64], 4, 2, 64),
                                           ([1024] * 2, 24, 8, 128), ([200, 513], 7, 1, 128)])
def test_quantizer_bit_exact(lens, hq, hkv, d):
    _log(f"quantizer lens={lens} hq={hq} hkv={hkv} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=21)
    g = run_gpu(q, k, v, cu, hq, hkv, "band", 5000)
    oq, osq = oracle.quantize_blocks(q, cu, 128)
    ok, osk = oracle.quantize_blocks(k, cu, 64)
    assert np.array_equal(g["q_i8"], oq) and np.array_equal(g["k_i8"], ok)
    assert np.array_equal(g["q_scale"].view(np.uint32), osq.view(np.uint32))
    assert np.array_equal(g["k_scale"].view(np.uint32), osk.view(np.uint32))


def test_quantizer_zero_and_tie_blocks():
    _log("quantizer zero/tie blocks")
    lens, hq, hkv, d = [200], 2, 1, 64
    q = np.zeros((200, hq, d), dtype=np.float16)
    k = np.zeros((200, hkv, d), dtype=np.float16)
    q[:128, 1, 0] = 127.0
    q[:128, 1, 1:8] = np.array([2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0], dtype=np.float16)
    k[64:128, 0, 0] = 63.5
    k[64:128, 0, 1:4] = np.array([0.75, 1.25, -0.25], dtype=np.float16)
    v = np.zeros_like(k)
    g = run_gpu(q, k, v, synth.cu_seqlens_of(lens), hq, hkv, "band", 0)
    oq, osq = oracle.quantize_blocks(q, [0, 200], 128)
    ok, osk = oracle.quantize_blocks(k, [0, 200], 64)
    assert np.array_equal(g["q_i8"], oq) and np.array_equal(g["k_i8"], ok)
    assert np.array_equal(g["q_scale"], osq) and np.array_equal(g["k_scale"], osk)
    assert g["q_i8"][0, 1, :8].tolist() == [127, 2, -4, 0, 0, 2, 126, -127]


# ------------------------------------------------------------ int32 tiles

@pytest.mark.parametrize("d", [64, 128])
def test_int32_tiles_bit_exact(d):
    lens, hq, hkv = [300, 129], 4, 2
    _log(f"int32 tiles d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=22)
    g = run_gpu(q, k, v, cu, hq, hkv, "band", 10000)
    tp = g["tp"]
    qi = torch.from_numpy(g["q_i8"]).cuda()
    ki = torch.from_numpy(g["k_i8"]).cuda()
    acc = torch.empty((128, 64), dtype=torch.int32, device="cuda")
    for (s, h, r, t) in [(0, 0, 0, 0), (0, 3, 2, 4), (0, 1, 1, 3), (1, 2, 1, 2), (1, 0, 0, 1), (0, 2, 2, 0)]:
        tm.tilemix_debug_qk_i32_tile(tp.plan_h, tp.plan_d, qi, ki, s, h, r, t, acc)
        torch.cuda.synchronize()
        ref = oracle.qk_int32_tile(g["q_i8"], g["k_i8"], cu, s, h, r, t, hq, hkv)
        assert np.array_equal(acc.cpu().numpy(), ref), (s, h, r, t)


# --------------------------------------------------------------- outputs

@pytest.mark.parametrize("cov", [0, 5000, 10000])
def test_tiny_band(cov):
    spec = synth.WORKLOADS["tiny"]
    _log(f"tiny band cov={cov}")
    q, k, v, cu = synth.make_qkv(spec["seqlens"], 1, 1, 64, False, 0)
    g = run_gpu(q, k, v, cu, 1, 1, "band", cov)
    ref = oracle.run(q, k, v, cu, 1, 1, "band", cov)
    assert np.array_equal(g["words"], ref["words"])
    assert_close(g["out"], ref["out"])


@pytest.mark.parametrize("template,cov,d", [("band", 5000, 64), ("global", 2500, 128),
                                            ("rowrandom", 5000, 64), ("alignedsparse", 7500, 128),
                                            ("bigbird", 5000, 128), ("sptrans", 7500, 64),
                                            ("sptrans", 10000, 128), ("band", 0, 128)])
def test_varlen_gqa_ragged(template, cov, d):
    lens, hq, hkv = [300, 77, 0, 129, 1, 64, 640], 6, 2
    _log(f"varlen {template} cov={cov} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, True, 23)
    g = run_gpu(q, k, v, cu, hq, hkv, template, cov, seed=5)
    ref = oracle.run(q, k, v, cu, hq, hkv, template, cov, seed=5)
    assert_close(g["out"], ref["out"])


def test_long_rows_g2():
    # 8256 tokens -> 129 key tiles -> g = 3 groups of tiles per bit
    lens, hq, hkv, d = [8256], 2, 1, 64
    _log("g=3 sequence")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, True, 24)
    assert oracle.seq_geometry(8256).g == 3
    g = run_gpu(q, k, v, cu, hq, hkv, "rowrandom", 5000, seed=2)
    geo = oracle.seq_geometry(8256)
    rows = [(0, h, r) for h in range(hq) for r in (0, 1, 31, 63, geo.Tm - 1)]
    ref = oracle.run(q, k, v, cu, hq, hkv, "rowrandom", 5000, seed=2, rows=rows)["out"]
    for (_, h, r) in rows:
        sl = slice(128 * r, min(128 * r + 128, 8256))
        assert_close(g["out"][sl, h], ref[sl, h])


def test_llama3b_l1k_full():
    spec = synth.WORKLOADS["llama3b_l1k"]
    _log("llama3b L=1024 B=8 sptrans 25% (full oracle)")
    q, k, v, cu, spec = synth.make_workload("llama3b_l1k")
    g = run_gpu(q, k, v, cu, spec["hq"], spec["hkv"], spec["template"], spec["coverage_bp"])
    ref = oracle.run(q, k, v, cu, spec["hq"], spec["hkv"], spec["template"], spec["coverage_bp"])
    assert np.array_equal(g["q_i8"], ref["q_i8"]) and np.array_equal(g["k_i8"], ref["k_i8"])
    _log("  err max/mean %.3e %.3e" % assert_close(g["out"], ref["out"]))


def _sampled_rows(cu, hq, heads, seed, n_random=6):
    lens = np.diff(cu)
    rng = np.random.default_rng(seed)
    rows = set()
    for s, L in enumerate(lens):
        tm_ = oracle.seq_geometry(int(L)).Tm
        if tm_ == 0:
            continue
        for r in {0, tm_ // 2, tm_ - 1}:
            for h in heads:
                rows.add((s, h, r))
    for _ in range(n_random):
        s = int(rng.integers(len(lens)))
        tm_ = oracle.seq_geometry(int(lens[s])).Tm
        if tm_:
            rows.add((s, int(rng.integers(hq)), int(rng.integers(tm_))))
    return sorted(rows)


def _check_rows(got, ref, cu, rows):
    errs = []
    for (s, h, r) in rows:
        a = int(cu[s]) + 128 * r
        b = min(int(cu[s]) + 128 * r + 128, int(cu[s + 1]))
        errs.append(np.abs(got[a:b, h].astype(np.float64) - ref[a:b, h]))
    e = np.concatenate([x.ravel() for x in errs])
    assert np.all(np.isfinite(e))
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS, (e.max(), e.mean())
    return e.max(), e.mean()


@pytest.mark.parametrize("cov", [7500, 0, 10000])
def test_headline_sampled(cov):
    _log(f"llama3b L=4096 B=8 sptrans {cov / 100:.0f}% (sampled rows)")
    q, k, v, cu, spec = synth.make_workload("llama3b_l4k")
    g = run_gpu(q, k, v, cu, spec["hq"], spec["hkv"], "sptrans", cov)
    rows = _sampled_rows(cu, spec["hq"], [0, 13, 23], seed=1)
    ref = oracle.run(q, k, v, cu, spec["hq"], spec["hkv"], "sptrans", cov, rows=rows)
    assert np.array_equal(g["words"], ref["words"])
    assert np.array_equal(g["q_i8"], ref["q_i8"]) and np.array_equal(g["k_i8"], ref["k_i8"])
    _log("  err max/mean %.3e %.3e" % _check_rows(g["out"], ref["out"], cu, rows))


@pytest.mark.parametrize("template", oracle.TEMPLATES)
def test_sweep_l8k_sampled(template):
    # the coverage/layout sweep shape (8 x 8192 tokens, Hq 24, Hkv 8, g = 2)
    # at 50% for every template, on sampled query-tile rows
    _log(f"llama3b L=8192 B=8 {template} 50% (sampled rows)")
    q, k, v, cu, spec = synth.make_workload("llama3b_l8k")
    g = run_gpu(q, k, v, cu, spec["hq"], spec["hkv"], template, 5000)
    rows = _sampled_rows(cu, spec["hq"], [0, 11], seed=4, n_random=4)
    ref = oracle.run(q, k, v, cu, spec["hq"], spec["hkv"], template, 5000, rows=rows)
    assert np.array_equal(g["words"], ref["words"])
    _log("  err max/mean %.3e %.3e" % _check_rows(g["out"], ref["out"], cu, rows))


def test_qwen_varlen_sampled():
    _log("qwen2-7b varlen rowrandom 50% (sampled rows)")
    q, k, v, cu, spec = synth.make_workload("qwen2_7b_varlen")
    g = run_gpu(q, k, v, cu, spec["hq"], spec["hkv"], spec["template"], spec["coverage_bp"])
    rows = _sampled_rows(cu, spec["hq"], [0, 27], seed=2, n_random=4)
    ref = oracle.run(q, k, v, cu, spec["hq"], spec["hkv"], spec["template"], spec["coverage_bp"], rows=rows)
    assert np.array_equal(g["words"], ref["words"])
    _log("  err max/mean %.3e %.3e" % _check_rows(g["out"], ref["out"], cu, rows))


# --------------------------------------------------------- special cases

def test_special_cases_and_determinism():
    lens, hq, hkv, d = [300, 200], 4, 2, 128
    _log("special cases")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, True, 25)
    for cov in (0, 5000, 10000):
        g = run_gpu(q, k, np.ones_like(v), cu, hq, hkv, "sptrans", cov)
        assert np.all(g["out"] == np.float16(1.0))          # V == 1 -> O == 1
    zq = np.zeros_like(q)
    g = run_gpu(zq, k, v, cu, hq, hkv, "bigbird", 5000)
    for s in range(2):
        a, b = int(cu[s]), int(cu[s + 1])
        cm = np.cumsum(v[a:b].astype(np.float64), axis=0) / np.arange(1, b - a + 1)[:, None, None]
        for h in range(hq):
            assert np.abs(g["out"][a:b, h] - cm[:, h // 2]).max() <= MAX_ABS
    # an all-zero K block on diagonal tiles: INT8 tiles with a zero scale
    # product (factor 0) under the causal mask, against the oracle
    zk = k.copy()
    zk[64:128] = 0                       # sequence 0, key tile 1 (row 0's diagonal)
    zk[300 + 128:300 + 192] = 0          # sequence 1, key tile 2 (row 1's diagonal)
    for cov in (5000, 10000):
        g = run_gpu(q, zk, v, cu, hq, hkv, "sptrans", cov)
        assert not np.isnan(g["out"]).any()
        assert_close(g["out"], oracle.run(q, zk, v, cu, hq, hkv, "sptrans", cov)["out"])
    # 0% is plain attention
    g0 = run_gpu(q, k, v, cu, hq, hkv, "band", 0)
    assert_close(g0["out"], naive_causal_attention(q, k, v, cu, hq, hkv))
    # garbage in bits of illegal groups changes nothing; two runs are identical
    g1 = run_gpu(q, k, v, cu, hq, hkv, "rowrandom", 5000, seed=1)
    w = g1["words"].copy()
    for s, L in enumerate(lens):
        geo = oracle.seq_geometry(L)
        off = sum(oracle.seq_geometry(x).Tm for x in lens[:s])
        for r in range(geo.Tm):
            w[:, off + r] |= np.uint64(((1 << 64) - 1) ^ ((1 << (geo.D[r] + 1)) - 1))
    g2 = run_gpu(q, k, v, cu, hq, hkv, "rowrandom", 5000, seed=1, words=w)
    g3 = run_gpu(q, k, v, cu, hq, hkv, "rowrandom", 5000, seed=1)
    assert np.array_equal(g1["out"], g2["out"]) and np.array_equal(g1["out"], g3["out"])


def test_deviation_grows_with_coverage():
    lens, hq, hkv, d = [1024] * 2, 4, 2, 128
    _log("MAD vs coverage")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, True, 26)
    base = run_gpu(q, k, v, cu, hq, hkv, "band", 0)["out"].astype(np.float64)
    mads = [np.mean(np.abs(run_gpu(q, k, v, cu, hq, hkv, "band", c)["out"] - base)) for c in (2500, 5000, 10000)]
    assert 0 < mads[0] <= mads[1] <= mads[2]


@pytest.mark.parametrize("d", [64, 128])
def test_lossless_inputs_coverage_independent(d):
    # Q blocks (128 rows) and K blocks (64 rows) of values k * 2^-6 with one
    # +-127 * 2^-6 per (block, head): the scale is 2^-6 and the codes are k,
    # so both score paths give the same exact scores (products and partial
    # sums exact in fp32, the scale factors differ by powers of two) and the
    # output does not depend on the routing at all.
    lens, hq, hkv = [300, 77, 129, 1], 4, 2
    _log(f"lossless inputs d={d}")
    q = synth.lossless_blocks(lens, hq, d, 128, seed=27)
    k = synth.lossless_blocks(lens, hkv, d, 64, seed=28)
    _, _, v, cu = synth.make_qkv(lens, hq, hkv, d, False, 29)
    base = run_gpu(q, k, v, cu, hq, hkv, "band", 0)["out"]
    for template, cov in (("band", 5000), ("rowrandom", 2500), ("sptrans", 10000)):
        assert np.array_equal(run_gpu(q, k, v, cu, hq, hkv, template, cov)["out"], base), (template, cov)
    assert_close(base, naive_causal_attention(q, k, v, cu, hq, hkv))


@pytest.mark.parametrize("cov", [0, 5000, 10000])
def test_running_max_ramps(cov):
    # Scores that grow linearly along the keys at a per-row rate of 10, 20,
    # -10 or 5 log2 units per 64-key tile (rows interleaved, so one wave holds
    # every rate): the rows at 20 push the running maximum past the lazy
    # margin on every tile, the rows at 10 and 5 only every second or third
    # tile on their own (then they take their tile maximum with the wave's
    # rescale), the falling rows never after their first tile.
    _log(f"running-max ramps cov={cov}")
    lens, hq, hkv, d = [1024, 300], 2, 1, 64
    T = sum(lens)
    rng = np.random.default_rng(41)
    b = 10.0 * np.sqrt(d) / (64 * np.log2(np.e))  # 10 log2 units per tile at rate 1
    rate = np.array([1.0, 2.0, -1.0, 0.5])
    q = np.zeros((T, hq, d), dtype=np.float16)
    k = np.zeros((T, hkv, d), dtype=np.float16)
    off = 0
    for L in lens:
        j = np.arange(L)
        q[off:off + L, :, 0] = rate[j % 4][:, None]
        q[off:off + L, :, 1:] = rng.normal(0, 0.05, (L, hq, d - 1))
        k[off:off + L, 0, 0] = b * j
        k[off:off + L, 0, 1:] = rng.normal(0, 0.05, (L, d - 1))
        off += L
    v = rng.normal(0, 1, (T, hkv, d)).astype(np.float16)
    cu = synth.cu_seqlens_of(lens)
    g = run_gpu(q, k, v, cu, hq, hkv, "band", cov)
    ref = oracle.run(q, k, v, cu, hq, hkv, "band", cov)
    assert_close(g["out"], ref["out"])
