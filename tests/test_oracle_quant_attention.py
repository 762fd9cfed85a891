"""Pins of the oracle's quantiser, int32 tiles and attention (CPU only)."""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from independent import (mixed_closed_form, naive_causal_attention, round_fraction_to_f32,
                         round_half_even)


# ----------------------------- quantiser ---------------------------------

def test_quant_closed_form_unit_scale():
    # absmax 127 -> s = 1 exactly, q = round-half-even(x)
    x = np.array([[127.0, 2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0]], dtype=np.float16)
    q, s = oracle.quantize_blocks(x[:, None, :], [0, 1], 64)
    assert s[0, 0] == np.float32(1.0)
    assert q[0, 0].tolist() == [127, 2, -4, 0, 0, 2, 126, -127]


def test_quant_closed_form_half_scale():
    # absmax 63.5 -> s = 0.5 exactly, q = rne(2x)
    x = np.array([[63.5, 0.75, 1.25, -0.25, -63.5, 0.0]], dtype=np.float16)
    q, s = oracle.quantize_blocks(x[:, None, :], [0, 1], 128)
    assert s[0, 0] == np.float32(0.5)
    assert q[0, 0].tolist() == [127, 2, 2, 0, -127, 0]


def test_quant_zero_block():
    x = np.zeros((70, 2, 64), dtype=np.float16)
    x[64:, 1, 3] = 1.0
    q, s = oracle.quantize_blocks(x, [0, 70], 64)
    assert s.shape == (2, 2)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert s[1, 1] == np.float32(np.float32(1.0) / np.float32(127.0))
    assert np.all(q[:, 0] == 0) and q[64, 1, 3] == 127


def test_quant_exact_rational():
    """Every code and scale equals the exactly-rounded IEEE result computed in
    rational arithmetic (independent of numpy's binary32 division)."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((130, 1, 64)) * rng.choice([0.01, 1.0, 30.0], size=(130, 1, 1)))
    x = x.astype(np.float16)
    q, s = oracle.quantize_blocks(x, [0, 130], 64)
    for b, (b0, b1) in enumerate([(0, 64), (64, 128), (128, 130)]):
        blk = x[b0:b1, 0].astype(np.float64)
        a = Fraction(float(np.abs(blk).max()))
        sf = round_fraction_to_f32(a / 127)
        assert Fraction(float(s[0, b])) == sf
        for i in range(b1 - b0):
            for c in range(64):
                ratio = round_fraction_to_f32(Fraction(float(blk[i, c])) / sf)
                expect = max(-127, min(127, round_half_even(ratio)))
                assert q[b0 + i, 0, c] == expect


def test_quant_invariants_and_partial_blocks():
    q16, k16, v16, cu = synth.make_qkv([300, 70, 1], 4, 2, 128, outliers=True, seed=3)
    for x, blk in [(q16, 128), (k16, 64)]:
        qi, sc = oracle.quantize_blocks(x, cu, blk)
        tile = 0
        for s in range(len(cu) - 1):
            for b0 in range(int(cu[s]), int(cu[s + 1]), blk):
                b1 = min(b0 + blk, int(cu[s + 1]))
                xb = x[b0:b1].astype(np.float64)
                for h in range(x.shape[1]):
                    a = np.abs(xb[:, h]).max()
                    sv = float(sc[h, tile])
                    assert sv == float(np.float32(np.float32(a) / np.float32(127)))
                    qb = qi[b0:b1, h].astype(np.int64)
                    assert qb.min() >= -127 and qb.max() <= 127
                    # the absmax element maps to +-127
                    i, c = np.unravel_index(np.argmax(np.abs(xb[:, h])), xb[:, h].shape)
                    assert abs(qb[i, c]) == 127
                    # half a step, plus rounding of the division
                    assert np.all(np.abs(xb[:, h] - qb * sv) <= sv * (0.5 + 2 ** -16) + 1e-30)
                tile += 1
        assert tile == sc.shape[1]
    # a block at a sequence end does not see the next sequence's rows
    k2 = k16.copy()
    k2[300:] *= 100
    _, sc1 = oracle.quantize_blocks(k16, cu, 64)
    _, sc2 = oracle.quantize_blocks(k2, cu, 64)
    n_first = -(-300 // 64)
    assert np.array_equal(sc1[:, :n_first], sc2[:, :n_first])


# ----------------------------- int32 tiles -------------------------------

def test_int32_tile_brute_force():
    q16, k16, v16, cu = synth.make_qkv([200], 2, 1, 64, outliers=True, seed=4)
    qi, _ = oracle.quantize_blocks(q16, cu, 128)
    ki, _ = oracle.quantize_blocks(k16, cu, 64)
    for (h, r, t) in [(0, 0, 0), (1, 1, 3), (1, 1, 2), (0, 0, 1)]:
        tile = oracle.qk_int32_tile(qi, ki, cu, 0, h, r, t, 2, 1)
        for i in range(0, 128, 9):
            for j in range(0, 64, 5):
                qq, kk = 128 * r + i, 64 * t + j
                if qq < 200 and kk < 200:
                    e = sum(int(qi[qq, h, c]) * int(ki[kk, 0, c]) for c in range(64))
                else:
                    e = 0
                assert tile[i, j] == e
    # |acc| <= 127^2 d < 2^24: exact in binary32
    assert 127 * 127 * 128 < 2 ** 24


# ----------------------------- attention ---------------------------------

def _prep(seqlens, hq, hkv, d, outliers, seed, template, cov, rseed=0):
    q, k, v, cu = synth.make_qkv(seqlens, hq, hkv, d, outliers, seed)
    res = oracle.run(q, k, v, cu, hq, hkv, template, cov, seed=rseed, round_p=False)
    return q, k, v, cu, res


@pytest.mark.parametrize("seqlens,hq,hkv,d", [([256], 1, 1, 64), ([300, 77, 129], 4, 2, 64),
                                              ([1], 2, 2, 128), ([200, 0, 64], 3, 1, 128)])
def test_zero_coverage_is_plain_attention(seqlens, hq, hkv, d):
    q, k, v, cu = synth.make_qkv(seqlens, hq, hkv, d, outliers=False, seed=1)
    ref = naive_causal_attention(q, k, v, cu, hq, hkv)
    exact = oracle.run(q, k, v, cu, hq, hkv, "band", 0, round_p=False)["out"]
    # the method rounds 1/sqrt(d) to binary32 (exact for d = 64): relative
    # score error <= 2^-24, i.e. ~1e-7 on O for |S| ~ 5
    assert np.max(np.abs(exact - ref)) < (1e-12 if d == 64 else 1e-6)
    rounded = oracle.run(q, k, v, cu, hq, hkv, "band", 0, round_p=True)["out"]
    assert np.max(np.abs(rounded - ref)) < 1e-3


@pytest.mark.parametrize("template,cov", [("band", 5000), ("global", 2500), ("sptrans", 7500),
                                          ("rowrandom", 5000), ("bigbird", 10000),
                                          ("alignedsparse", 1000)])
def test_mixed_closed_form(template, cov):
    seqlens, hq, hkv = [300, 129, 256], 4, 2
    q, k, v, cu, res = _prep(seqlens, hq, hkv, 64, False, 2, template, cov, rseed=9)
    ref = mixed_closed_form(q, k, v, res["q_i8"], res["k_i8"], res["q_scale"], res["k_scale"],
                            res["words"], res["g"], cu, hq, hkv)
    assert np.max(np.abs(res["out"] - ref)) < 1e-5


def test_mixed_closed_form_g2():
    # 4160 keys -> 65 key tiles -> g = 2; sample rows against the closed form
    seqlens, hq, hkv = [4160], 1, 1
    q, k, v, cu = synth.make_qkv(seqlens, hq, hkv, 64, False, 5)
    geo = oracle.seq_geometry(4160)
    assert geo.g == 2
    rows = [(0, 0, r) for r in (0, 17, geo.Tm - 1)]
    res = oracle.run(q, k, v, cu, hq, hkv, "rowrandom", 5000, seed=3, rows=rows, round_p=False)
    qh = res["q_i8"].astype(np.float64) * np.repeat(res["q_scale"][0], 128)[:4160, None, None]
    kh = res["k_i8"].astype(np.float64) * np.repeat(res["k_scale"][0], 64)[:4160, None, None]
    for (_, _, r) in rows:
        for i in range(128 * r, min(128 * r + 128, 4160), 31):
            w = int(res["words"][0, r])
            j = np.arange(i + 1)
            bits = (w >> ((j // 64) // 2)) & 1
            s = np.where(bits == 1, kh[:i + 1, 0] @ qh[i, 0], k[:i + 1, 0].astype(np.float64) @ q[i, 0].astype(np.float64))
            s = s / 8.0
            p = np.exp(s - s.max())
            o = (p / p.sum()) @ v[:i + 1, 0].astype(np.float64)
            assert np.max(np.abs(res["out"][i, 0] - o)) < 1e-5


def test_special_cases():
    seqlens, hq, hkv, d = [300, 64], 2, 1, 64
    q, k, v, cu = synth.make_qkv(seqlens, hq, hkv, d, True, 6)
    ones = np.ones_like(v)
    for cov in (0, 5000, 10000):
        o = oracle.run(q, k, ones, cu, hq, hkv, "sptrans", cov)["out"]
        assert np.max(np.abs(o - 1.0)) < 1e-12          # V == 1 -> O == 1
    zq = np.zeros_like(q)
    for cov in (0, 5000, 10000):
        o = oracle.run(zq, k, v, cu, hq, hkv, "band", cov, round_p=False)["out"]
        for s in range(2):
            a, b = int(cu[s]), int(cu[s + 1])
            cm = np.cumsum(v[a:b, 0].astype(np.float64), axis=0) / np.arange(1, b - a + 1)[:, None]
            for h in range(hq):
                assert np.max(np.abs(o[a:b, h] - cm)) < 1e-12  # Q == 0 -> prefix mean of V


def test_lossless_inputs_make_coverage_irrelevant():
    seqlens, hq, hkv, d = [256, 130], 2, 2, 64
    q = synth.lossless_blocks(seqlens, hq, d, 128, seed=1)
    k = synth.lossless_blocks(seqlens, hkv, d, 64, seed=2)
    _, _, v, cu = synth.make_qkv(seqlens, hq, hkv, d, False, 3)
    q = (q.astype(np.float32) / 4).astype(np.float16)   # keep scores moderate (still exact)
    o0 = oracle.run(q, k, v, cu, hq, hkv, "band", 0, round_p=False)
    assert np.all(o0["q_scale"] == np.float32(2.0 ** -8)) and np.all(o0["k_scale"] == np.float32(2.0 ** -6))
    for t, cov in [("band", 5000), ("global", 10000), ("rowrandom", 7500)]:
        o = oracle.run(q, k, v, cu, hq, hkv, t, cov, round_p=False)["out"]
        assert np.max(np.abs(o - o0["out"])) < 1e-9


def test_row_sums_and_illegal_bits():
    seqlens, hq, hkv, d = [300], 2, 1, 64
    q, k, v, cu = synth.make_qkv(seqlens, hq, hkv, d, True, 7)
    res = oracle.run(q, k, v, cu, hq, hkv, "sptrans", 5000)
    o, stats = oracle.prefill_attention(q, k, v, res["q_i8"], res["k_i8"], res["q_scale"],
                                        res["k_scale"], res["words"], cu, hq, hkv, return_stats=True)
    for key, rs in stats.items():
        assert np.max(np.abs(rs - 1.0)) < 1e-12
    # garbage in bits of illegal groups leaves the output bitwise unchanged
    w2 = res["words"].copy()
    geo = oracle.seq_geometry(300)
    for r in range(geo.Tm):
        w2[0, r] |= np.uint64(((1 << 64) - 1) ^ ((1 << (geo.D[r] + 1)) - 1))
    o2 = oracle.prefill_attention(q, k, v, res["q_i8"], res["k_i8"], res["q_scale"],
                                  res["k_scale"], w2, cu, hq, hkv)
    assert np.array_equal(o, o2)


def test_gqa_and_varlen_independence():
    seqlens, hq, hkv, d = [200, 150], 4, 2, 64
    q, k, v, cu = synth.make_qkv(seqlens, hq, hkv, d, True, 8)
    full = oracle.run(q, k, v, cu, hq, hkv, "bigbird", 5000, seed=4)["out"]
    # sequence 1 alone gives the same output
    a, b = int(cu[1]), int(cu[2])
    alone = oracle.run(q[a:b], k[a:b], v[a:b], [0, b - a], hq, hkv, "bigbird", 5000, seed=4)["out"]
    assert np.array_equal(full[a:b], alone)
    # GQA: a query head equals the MHA computation with its KV head replicated
    kr = np.repeat(k, hq // hkv, axis=1)
    vr = np.repeat(v, hq // hkv, axis=1)
    mha = oracle.run(q, kr, vr, cu, hq, hq, "bigbird", 5000, seed=4)["out"]
    assert np.array_equal(full, mha)


def test_int8_path_deviates_and_grows_with_coverage():
    seqlens, hq, hkv, d = [512], 2, 1, 128
    q, k, v, cu = synth.make_qkv(seqlens, hq, hkv, d, True, 9)
    base = oracle.run(q, k, v, cu, hq, hkv, "band", 0)["out"]
    mads = [np.mean(np.abs(oracle.run(q, k, v, cu, hq, hkv, "band", c)["out"] - base))
            for c in (2500, 5000, 10000)]
    assert 0 < mads[0] <= mads[1] <= mads[2]
