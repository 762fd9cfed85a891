"""Parity of the FP8 (E4M3) third path (HIP, through the C ABI) with the
oracle: FP8 codes and scales bit-exact, three-path prefill output within the
fp16 tolerance, and identical to the two-path kernel when no group is FP8."""

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


def run3(q, k, v, cu, hq, hkv, template, c8, cf, seed=0):
    d = q.shape[2]
    tp = tm.TileMixPrefill3(cu, hq, hkv, d, template, c8, cf, seed)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    tp(qd, kd, vd, out)
    torch.cuda.synchronize()
    T = q.shape[0]
    return tp, out.cpu().numpy(), dict(
        q_f8=tp.q_f8.cpu().numpy()[:T], k_f8=tp.k_f8.cpu().numpy()[:T],
        q_scale_f8=tp.q_scale_f8.cpu().numpy()[:, :tp.tq], k_scale_f8=tp.k_scale_f8.cpu().numpy()[:, :tp.tk],
        q_i8=tp.q_i8.cpu().numpy()[:T], k_i8=tp.k_i8.cpu().numpy()[:T],
        q_scale=tp.q_scale.cpu().numpy()[:, :tp.tq], k_scale=tp.k_scale.cpu().numpy()[:, :tp.tk])


def oracle3(q, k, v, cu, hq, hkv, tp, rows=None):
    q_i8, qs = oracle.quantize_blocks(q, cu, 128)
    k_i8, ks = oracle.quantize_blocks(k, cu, 64)
    qf, qfs = oracle.quantize_blocks_fp8(q, cu, 128)
    kf, kfs = oracle.quantize_blocks_fp8(k, cu, 64)
    return oracle.prefill_attention3(q, k, v, q_i8, k_i8, qs, ks, qf, kf, qfs, kfs, tp.words, tp.words_f8,
                                     cu, hq, hkv, rows=rows)


def assert_close(got, ref):
    got = got.astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert err.max() <= MAX_ABS, f"max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean():.3e}"


# The FP8 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4) sums each
# 64-product step with about 12 bits relative to the step's largest product,
# not to fp32: test_fp8_tile_accumulation_bound holds every sum of a score
# tile within EPS_F8 * (sum over steps of the step's largest |q8 k8|) of the
# exact one (worst seen 2^-11.12, codes spanning the whole E4M3 range).  The
# score error of an FP8 tile is then at most delta = EPS_F8 * that sum *
# s_q s_k / sqrt(d), and a row's softmax output moves by at most
# exp(2 delta) - 1 times max |V|.  On inputs whose blocks are dominated by a
# few large products (the outlier channels) this lets a few rows exceed the
# fp16 bar: those tests hold each row to 4e-3 plus that bound, all outputs
# to F8_MAX_FACTOR times the bar (worst seen 3.6 times) and the mean to the
# bar itself.
EPS_F8 = 2.0 ** -11
F8_MAX_FACTOR = 4.0


def fp8_row_bound(q, k, v, cu, hq, hkv, tp, rows_sel):
    """Per output row, the bound above: max over its FP8 tiles' scores."""
    qf, qfs = oracle.quantize_blocks_fp8(q, cu, 128)
    kf, kfs = oracle.quantize_blocks_fp8(k, cu, 64)
    qv, kv_ = oracle.fp8_e4m3_decode(qf), oracle.fp8_e4m3_decode(kf)
    d = q.shape[2]
    grp = hq // hkv
    bound = np.zeros((q.shape[0], hq))
    lens = np.diff(cu)
    qt = np.concatenate([[0], np.cumsum([-(-int(L) // 128) for L in lens])])
    kt = np.concatenate([[0], np.cumsum([-(-int(L) // 64) for L in lens])])
    for s, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        geo = oracle.seq_geometry(L)
        for h in range(hq):
            kvh = h // grp
            for i in range(L):
                if rows_sel is not None and (s, i) not in rows_sel:
                    continue
                r = i // 128
                wf = int(tp.words_f8[kvh, qt[s] + r])
                w8 = int(tp.words[kvh, qt[s] + r])
                delta = 0.0
                for t in range(i // 64 + 1):
                    G = t // geo.g
                    if not ((wf >> G) & 1) or ((w8 >> G) & 1):
                        continue
                    j0, j1 = 64 * t, min(64 * t + 64, i + 1)
                    prod = np.abs(qv[cu[s] + i, h][None, :] * kv_[cu[s] + j0:cu[s] + j1, kvh])
                    steps = prod.reshape(j1 - j0, -1, 64).max(axis=2).sum(axis=1)
                    scale = float(qfs[h, qt[s] + r]) * float(kfs[kvh, kt[s] + t]) / np.sqrt(d)
                    delta = max(delta, EPS_F8 * steps.max() * scale)
                vmax = np.abs(v[cu[s]:cu[s] + i + 1, kvh].astype(np.float64)).max()
                bound[cu[s] + i, h] = (np.exp(2 * delta) - 1) * vmax
    return bound


def assert_close_f8(got, ref, bound):
    got = got.astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    row = err.max(axis=2)
    _log(f"  err max {err.max():.3e} ({err.max() / MAX_ABS:.2f} x bar), mean {err.mean():.3e}, "
         f"rows above 4e-3 {np.mean(row > MAX_ABS):.4f}")
    excess = row - (MAX_ABS + bound)
    assert excess.max() <= 0, f"max abs err {err.max():.3e}, worst excess {excess.max():.3e}"
    assert err.max() <= F8_MAX_FACTOR * MAX_ABS, f"max abs err {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"mean abs err {err.mean():.3e}"


def _tile_sums(codes_q, codes_k, L, d):
    """(device sums, exact sums, per-sum bound base) of every legal FP8 score
    tile of one single-head sequence, through the kernel's tile routine."""
    cu = synth.cu_seqlens_of([L])
    plan = tm.tilemix_build_plan(cu, 1, 1, d)
    pd = torch.from_numpy(plan).cuda()
    qd, kd = torch.from_numpy(codes_q).cuda(), torch.from_numpy(codes_k).cuda()
    acc = torch.zeros(128 * 64, dtype=torch.float32, device="cuda")
    qv = oracle.fp8_e4m3_decode(codes_q)[:, 0].astype(np.float64)
    kv = oracle.fp8_e4m3_decode(codes_k)[:, 0].astype(np.float64)
    got, exact, base = [], [], []
    for r in range(-(-L // 128)):
        for t in range(min(2 * r + 2, -(-L // 64))):
            tm.tilemix_debug_qk_f8_tile(plan, pd, qd, kd, 0, 0, r, t, acc)
            g = acc.cpu().numpy().reshape(128, 64)
            qs, ks = np.arange(128 * r, min(128 * r + 128, L)), np.arange(64 * t, min(64 * t + 64, L))
            prod = qv[qs][:, None, :] * kv[ks][None, :, :]
            got.append(g[:len(qs), :len(ks)].ravel())
            exact.append(prod.sum(axis=2).ravel())
            base.append(np.abs(prod).reshape(len(qs), len(ks), -1, 64).max(axis=3).sum(axis=2).ravel())
            # rows and keys past the sequence end are reported as 0
            assert not g[len(qs):].any() and not g[:, len(ks):].any()
    return np.concatenate(got), np.concatenate(exact), np.concatenate(base)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_tile_accumulation_bound(d):
    """Pins EPS_F8: each sum of the FP8 score-tile routine is within EPS_F8
    times the sum over its 64-wide steps of the step's largest |product| of
    the exact sum of E4M3 products -- on codes spanning every finite E4M3
    value, on quantised N(0,1) blocks, on blocks with outlier channels, and
    on one large product among small ones; products of small exact values
    come out exactly."""
    L = 300
    rng = np.random.default_rng(71)
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[np.isfinite(oracle.fp8_e4m3_decode(codes))]
    x = rng.standard_normal((L, 1, d)).astype(np.float16)
    y = rng.standard_normal((L, 1, d)).astype(np.float16)
    cu = synth.cu_seqlens_of([L])
    xo, yo = x.copy(), y.copy()
    xo[..., :4] *= 10
    yo[..., :4] *= 10
    big_q = np.full((L, 1, d), 0x30, np.uint8)                    # 0.5
    small = finite[np.abs(oracle.fp8_e4m3_decode(finite)) < 4]
    big_k = rng.choice(small, (L, 1, d))
    big_q[..., 5] = 0x7E                                            # 448 x 448 in step 0
    big_k[..., 5] = 0x7E
    cases = {
        "every E4M3 value": (rng.choice(finite, (L, 1, d)), rng.choice(finite, (L, 1, d))),
        "N(0,1) blocks": (oracle.quantize_blocks_fp8(x, cu, 128)[0], oracle.quantize_blocks_fp8(y, cu, 64)[0]),
        "outlier channels": (oracle.quantize_blocks_fp8(xo, cu, 128)[0], oracle.quantize_blocks_fp8(yo, cu, 64)[0]),
        "one large product": (big_q, big_k),
    }
    for name, (cq, ck) in cases.items():
        got, exact, base = _tile_sums(cq, ck, L, d)
        ratio = np.abs(got - exact) / np.maximum(base, 1e-300)
        _log(f"  fp8 tile d={d} {name}: worst error / step-max sum = 2^{np.log2(max(ratio.max(), 1e-30)):.2f}")
        assert np.all(np.abs(got - exact) <= EPS_F8 * base), name
    # integers 1..4 times 2^-2 .. 2^1: every partial sum is exact in any format
    # with 12 bits below the largest product, so the sums are exact
    vals = finite[np.isin(oracle.fp8_e4m3_decode(finite), [0.25, 0.5, 1.0, 2.0, -0.5, -1.0])]
    got, exact, _ = _tile_sums(rng.choice(vals, (L, 1, d)), rng.choice(vals, (L, 1, d)), L, d)
    assert np.array_equal(got, exact)


@pytest.mark.parametrize("lens,hq,hkv,d", [([256], 1, 1, 64), ([300, 77, 0, 129, 1, 64], 4, 2, 64),
                                           ([1024, 513], 6, 2, 128)])
def test_fp8_quantizer_bit_exact(lens, hq, hkv, d):
    _log(f"fp8 quantizer lens={lens} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=51)
    tp, out, g = run3(q, k, v, cu, hq, hkv, "band", 2500, 2500)
    oq, oqs = oracle.quantize_blocks_fp8(q, cu, 128)
    ok, oks = oracle.quantize_blocks_fp8(k, cu, 64)
    assert np.array_equal(g["q_f8"], oq) and np.array_equal(g["k_f8"], ok)
    assert np.array_equal(g["q_scale_f8"].view(np.uint32), oqs.view(np.uint32))
    assert np.array_equal(g["k_scale_f8"].view(np.uint32), oks.view(np.uint32))


@pytest.mark.parametrize("template,c8,cf,d", [("band", 0, 10000, 64), ("sptrans", 2500, 5000, 128),
                                              ("rowrandom", 5000, 2500, 64), ("global", 0, 5000, 128),
                                              ("bigbird", 3000, 3000, 128)])
def test_three_path_varlen(template, c8, cf, d):
    # N(0,1) inputs: the FP8 accumulation error is far below the fp16 bar
    lens, hq, hkv = [300, 77, 0, 129, 1, 64, 700], 6, 2
    _log(f"three-path {template} c8={c8} cf={cf} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=52)
    tp, out, _ = run3(q, k, v, cu, hq, hkv, template, c8, cf)
    assert_close(out, oracle3(q, k, v, cu, hq, hkv, tp))


@pytest.mark.parametrize("cf,d", [(10000, 64), (5000, 128)])
def test_three_path_outlier_channels(cf, d):
    # outlier channels: blocks dominated by a few large products, where the
    # FP8 instruction's accumulation error is visible; held to the derived bound
    lens, hq, hkv = [300, 129], 2, 1
    _log(f"three-path outliers cf={cf} d={d}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=58)
    tp, out, _ = run3(q, k, v, cu, hq, hkv, "band", 0, cf)
    ref = oracle3(q, k, v, cu, hq, hkv, tp)
    assert_close_f8(out, ref, fp8_row_bound(q, k, v, cu, hq, hkv, tp, None))


def test_three_path_long_rows_g2():
    lens, hq, hkv, d = [4160], 2, 1, 128
    _log("three-path L=4160")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=53)
    tp, out, _ = run3(q, k, v, cu, hq, hkv, "sptrans", 2500, 5000)
    rows = [(0, h, r) for h in range(hq) for r in (0, 16, 32)]
    ref = oracle3(q, k, v, cu, hq, hkv, tp, rows=rows)
    sel = np.concatenate([np.arange(128 * r, min(128 * r + 128, 4160)) for r in (0, 16, 32)])
    assert_close(out[sel], ref[sel])


def test_three_path_without_fp8_equals_two_path():
    lens, hq, hkv, d = [1024, 300], 6, 2, 128
    _log("three-path with no FP8 groups vs two-path kernel")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=54)
    tp3, out3, _ = run3(q, k, v, cu, hq, hkv, "sptrans", 7500, 0)
    tp = tm.TileMixPrefill(cu, hq, hkv, d, "sptrans", 7500)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out2 = tp(qd, kd, vd).cpu().numpy()
    assert np.array_equal(out3, out2)


def test_fp8_lossless_inputs_give_plain_attention():
    lens, hq, hkv, d = [300, 129], 2, 1, 128
    _log("fp8 lossless inputs")
    cu = synth.cu_seqlens_of(lens)
    q = synth.lossless_blocks_fp8(lens, hq, d, 128, seed=55)
    k = synth.lossless_blocks_fp8(lens, hkv, d, 64, seed=56)
    _, _, v, _ = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=57)
    tp, out, _ = run3(q, k, v, cu, hq, hkv, "band", 0, 10000)
    from independent import naive_causal_attention
    ref = naive_causal_attention(q, k, v, cu, hq, hkv)
    assert_close_f8(out, ref, fp8_row_bound(q, k, v, cu, hq, hkv, tp, None))


@pytest.mark.parametrize("c8,cf", [(5000, 2500), (0, 7500)])
def test_three_path_headline_sampled(c8, cf):
    # the 3B shape at 8 x 4096 tokens (outlier channels), SpTrans, at the two
    # INT8 / FP8 mixes the three-path leg times; sampled work units, each
    # row held to 4e-3 plus the derived FP8 bound
    _log(f"three-path 3B L=4096 B=8 sptrans int8 {c8 / 100:.0f}% fp8 {cf / 100:.0f}% (sampled)")
    q, k, v, cu, spec = synth.make_workload("llama3b_l4k")
    hq, hkv, d = spec["hq"], spec["hkv"], spec["d"]
    tp, out, _ = run3(q, k, v, cu, hq, hkv, "sptrans", c8, cf)
    lens = [int(x) for x in np.diff(cu)]
    w8, wf, *_ = oracle.routing_words3(lens, hkv, "sptrans", c8, cf)
    assert np.array_equal(tp.words, w8) and np.array_equal(tp.words_f8, wf)
    units = [(0, 0, 0), (0, 23, 31), (3, 11, 15), (7, 5, 31), (5, 17, 6)]
    q_i8, qs = oracle.quantize_blocks(q, cu, 128)
    k_i8, ks = oracle.quantize_blocks(k, cu, 64)
    qf, qfs = oracle.quantize_blocks_fp8(q, cu, 128)
    kf, kfs = oracle.quantize_blocks_fp8(k, cu, 64)
    ref = oracle.prefill_attention3(q, k, v, q_i8, k_i8, qs, ks, qf, kf, qfs, kfs, w8, wf, cu, hq, hkv,
                                    rows=units)
    qv, kv_ = oracle.fp8_e4m3_decode(qf), oracle.fp8_e4m3_decode(kf)
    grp = hq // hkv
    all_err = []
    for (s, h, r) in units:
        L, a = lens[s], int(cu[s])
        kvh = h // grp
        geo = oracle.seq_geometry(L)
        rows = np.arange(128 * r, min(128 * r + 128, L))
        delta = np.zeros(len(rows))
        for t in range(rows[-1] // 64 + 1):
            G = t // geo.g
            word = r + sum(oracle.seq_geometry(x).Tm for x in lens[:s])
            if not ((int(wf[kvh, word]) >> G) & 1) or ((int(w8[kvh, word]) >> G) & 1):
                continue
            keys = np.arange(64 * t, min(64 * t + 64, L))
            prod = np.abs(qv[a + rows, h][:, None, :] * kv_[a + keys, kvh][None, :, :])
            steps = prod.reshape(len(rows), len(keys), -1, 64).max(axis=3).sum(axis=2)
            steps = np.where(keys[None, :] <= rows[:, None], steps, 0.0)
            scale = float(qfs[h, word]) * float(kfs[kvh, sum(oracle.seq_geometry(x).Tn for x in lens[:s]) + t])
            delta = np.maximum(delta, EPS_F8 * steps.max(axis=1) * scale / np.sqrt(d))
        vmax = np.maximum.accumulate(np.abs(v[a:a + L, kvh].astype(np.float64)).max(axis=1))[rows]
        bound = (np.exp(2 * delta) - 1) * vmax
        errs = np.abs(out[a + rows, h].astype(np.float64) - ref[a + rows, h])
        err = errs.max(axis=1)
        assert np.all(np.isfinite(out[a + rows, h]))
        assert np.all(err <= MAX_ABS + bound), (s, h, r, float((err - MAX_ABS - bound).max()))
        all_err.append(errs.ravel())
    all_err = np.concatenate(all_err)
    _log(f"  err max {all_err.max():.3e} ({all_err.max() / MAX_ABS:.2f} x bar), mean {all_err.mean():.3e}")
    assert all_err.max() <= F8_MAX_FACTOR * MAX_ABS
    assert all_err.mean() <= MEAN_ABS


# ------------------------------------- Q's INT8 and FP8 codes made in-kernel

def three_path_both(q, k, v, cu, hq, hkv, template, c8, cf, seed=0):
    """The three-path prefill after the two Q/K quantisers, and the variant
    that quantises Q inside the kernel after the key-only quantisers; the key
    codes of both quantiser pairs must agree."""
    tp, ref, _ = run3(q, k, v, cu, hq, hkv, template, c8, cf, seed)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    saved = [t.clone() for t in (tp.k_i8, tp.k_scale, tp.k_f8, tp.k_scale_f8)]
    tp.k_i8.fill_(0x55)
    tp.k_f8.fill_(0x55)
    tp.k_scale.fill_(float("nan"))
    tp.k_scale_f8.fill_(float("nan"))
    out = torch.full_like(qd, float("nan"))
    tp(qd, kd, vd, out, inline_q=True)
    torch.cuda.synchronize()
    T = q.shape[0]
    for a, b in zip((tp.k_i8, tp.k_f8), saved[0:4:2]):
        assert torch.equal(a[:T], b[:T])
    for a, b in zip((tp.k_scale, tp.k_scale_f8), saved[1:4:2]):
        assert torch.equal(a[:, :tp.tk].view(torch.int32), b[:, :tp.tk].view(torch.int32))
    return ref, out.cpu().numpy()


def assert_bits_equal(a, b):
    same = a.view(np.uint16) == b.view(np.uint16)
    assert same.all(), f"{int((~same).sum())} of {same.size} outputs differ"


@pytest.mark.parametrize("lens,hq,hkv,d,c8,cf", [([300, 77, 0, 129, 1, 520], 6, 2, 64, 5000, 2500),
                                                 ([300, 77, 0, 129, 1, 520], 6, 2, 128, 0, 10000),
                                                 ([1024, 200], 24, 8, 128, 2500, 5000)])
def test_three_path_qinline_bit_identical(lens, hq, hkv, d, c8, cf):
    _log(f"three-path inline-Q lens={lens} d={d} int8 {c8} fp8 {cf}")
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=37)
    ref, out = three_path_both(q, k, v, cu, hq, hkv, "sptrans", c8, cf)
    assert_bits_equal(ref, out)


def test_three_path_qinline_midpoints_and_zero_blocks():
    # absmax 448 makes s = 1: values on E4M3 rounding midpoints (ties to even),
    # an all-zero block (s = 0) and a block scaled far down
    _log("three-path inline-Q midpoints / zero blocks")
    lens, hq, hkv, d = [300], 3, 1, 64
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=43)
    q[:128, 0] = 0
    q[:128, 1] = 0
    q[:128, 1, 0] = 448.0
    q[:128, 1, 1:9] = np.array([1.0625, -1.1875, 17.0, -19.0, 0.015625 * 1.0625, 100.0, -232.0, 3.125],
                               dtype=np.float16)
    q[128:256, 2] *= 1e-3
    for c8, cf in [(0, 10000), (5000, 5000)]:
        ref, out = three_path_both(q, k, v, cu, hq, hkv, "band", c8, cf)
        assert_bits_equal(ref, out)


@pytest.mark.parametrize("c8,cf", [(5000, 2500), (0, 7500)])
def test_three_path_qinline_headline_bit_identical(c8, cf):
    _log(f"three-path inline-Q 3B L=4096 B=8 int8 {c8} fp8 {cf}")
    q, k, v, cu, spec = synth.make_workload("llama3b_l4k")
    ref, out = three_path_both(q, k, v, cu, spec["hq"], spec["hkv"], "sptrans", c8, cf)
    assert_bits_equal(ref, out)


@pytest.mark.parametrize("lens,hkv,d", [([300, 77, 0, 129, 1, 64], 2, 64), ([1024, 200], 8, 128)])
def test_key_quantisers_one_pass_bit_exact(lens, hkv, d):
    _log(f"key INT8+FP8 one pass lens={lens} hkv={hkv} d={d}")
    q, k, v, cu = synth.make_qkv(lens, 2 * hkv, hkv, d, outliers=True, seed=47)
    k[:64, 0] = 0  # an all-zero block: both scales 0, codes 0
    tp = tm.TileMixPrefill3(cu, 2 * hkv, hkv, d, "band", 5000, 2500)
    kd = torch.from_numpy(k).cuda()
    for t in (tp.k_i8, tp.k_f8):
        t.fill_(0x55)
    tp.quantize_k(kd)
    torch.cuda.synchronize()
    T = k.shape[0]
    ki8, ks = oracle.quantize_blocks(k, cu, 64)
    kf8, ksf = oracle.quantize_blocks_fp8(k, cu, 64)
    assert np.array_equal(tp.k_i8.cpu().numpy()[:T], ki8)
    assert np.array_equal(tp.k_f8.cpu().numpy()[:T], kf8)
    assert np.array_equal(tp.k_scale.cpu().numpy()[:, :tp.tk].view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(tp.k_scale_f8.cpu().numpy()[:, :tp.tk].view(np.uint32), ksf.view(np.uint32))
