"""Pins of the oracle's FP8 (E4M3) third path (CPU only): published format
values, brute-force nearest rounding, quantiser invariants, three-class
routing against the two-class template words, and the FP8 attention path
against closed forms."""

import math

import numpy as np
import pytest

import oracle
import synth
from independent import naive_causal_attention


def _grid():
    """All finite E4M3 values with their codes, from the format's definition
    (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals; 0x7F and
    0xFF are NaN)."""
    vals = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        mag = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals[c] = -mag if s else mag
    return vals


def test_decode_published_values():
    dec = oracle.fp8_e4m3_decode
    assert dec([0x38])[0] == 1.0 and dec([0x7E])[0] == 448.0 and dec([0xFE])[0] == -448.0
    assert dec([0x01])[0] == 2.0 ** -9 and dec([0x08])[0] == 2.0 ** -6 and dec([0x77])[0] == 240.0
    assert np.isnan(dec([0x7F])[0]) and np.isnan(dec([0xFF])[0])
    grid = _grid()
    codes = np.array(sorted(grid), dtype=np.uint8)
    np.testing.assert_array_equal(dec(codes), [grid[c] for c in codes])
    pos = dec(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)          # monotone in the code


def _nearest(x):
    """Brute force: the finite E4M3 value nearest to x, ties to the even
    mantissa; magnitudes above 448 saturate."""
    grid = _grid()
    best = None
    for c, v in grid.items():
        if v == 0 and c == 0x80:
            continue
        dist = abs(v - x)
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    if c == 0 and math.copysign(1.0, x) < 0:
        c = 0x80
    return c


def test_encode_is_nearest_with_ties_to_even():
    grid = np.array(sorted(v for v in _grid().values() if v >= 0))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(0)
    xs = np.concatenate([grid, -grid, mids, -mids, rng.uniform(-460, 460, 3000),
                         rng.uniform(-0.03, 0.03, 3000)]).astype(np.float32)
    got = oracle.fp8_e4m3_encode(xs)
    want = np.array([_nearest(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_fp8_quantizer_invariants():
    lens = [300, 0, 77, 129]
    q, k, _, cu = synth.make_qkv(lens, 3, 1, 64, outliers=True, seed=3)
    codes, sc = oracle.quantize_blocks_fp8(q, cu, 128)
    grid = _grid()
    col = 0
    for s in range(len(lens)):
        for b0 in range(cu[s], cu[s + 1], 128):
            b1 = min(b0 + 128, cu[s + 1])
            for h in range(3):
                blk = q[b0:b1, h].astype(np.float32)
                a = np.abs(blk).max()
                assert sc[h, col] == np.float32(a / np.float32(448.0))
                c = codes[b0:b1, h]
                # the absmax element maps to +-448
                i = np.unravel_index(np.abs(blk).argmax(), blk.shape)
                assert c[i] in (0x7E, 0xFE)
                # a sample of elements is the nearest grid value of fl32(x/s)
                for (r, j) in [(0, 0), (b1 - b0 - 1, 63), ((b1 - b0) // 2, 17)]:
                    y = float(np.float32(blk[r, j] / sc[h, col]))
                    assert c[r, j] == _nearest(y)
            col += 1
    z, zs = oracle.quantize_blocks_fp8(np.zeros((70, 1, 64), dtype=np.float16), [0, 70], 64)
    assert not z.any() and not zs.any()


@pytest.mark.parametrize("template", oracle.TEMPLATES)
def test_three_class_routing_matches_two_class_words(template):
    lens = [1024, 300, 4160]
    for c8, cf in [(0, 0), (2500, 2500), (5000, 2500), (0, 10000), (7500, 2500), (1000, 0)]:
        w8, wf, g, n8, nf, nl = oracle.routing_words3(lens, 2, template, c8, cf, 3)
        a, *_ = oracle.routing_words(lens, 2, template, c8, 3)
        b, *_ = oracle.routing_words(lens, 2, template, c8 + cf, 3)
        assert np.array_equal(w8, a)                        # INT8 set of coverage c8
        assert np.array_equal(w8 | wf, b) and not (w8 & wf).any()
        assert np.array_equal(n8 + nf, [oracle.int8_group_count(c8 + cf, x) for x in nl])
    with pytest.raises(ValueError):
        oracle.routing_words3(lens, 1, template, 6000, 5000)


def test_fp8_path_lossless_equals_attention():
    # inputs on the E4M3 grid times a power of two per block: every FP8 tile
    # is exact, so all-FP8 routing gives plain causal attention
    lens, hq, hkv, d = [300, 129, 1], 4, 2, 64
    cu = synth.cu_seqlens_of(lens)
    q = synth.lossless_blocks_fp8(lens, hq, d, 128, seed=4)
    k = synth.lossless_blocks_fp8(lens, hkv, d, 64, seed=5)
    _, _, v, _ = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=6)
    q_i8, qs = oracle.quantize_blocks(q, cu, 128)
    k_i8, ks = oracle.quantize_blocks(k, cu, 64)
    qf, qfs = oracle.quantize_blocks_fp8(q, cu, 128)
    kf, kfs = oracle.quantize_blocks_fp8(k, cu, 64)
    w8, wf, *_ = oracle.routing_words3(lens, hkv, "band", 0, 10000)
    out = oracle.prefill_attention3(q, k, v, q_i8, k_i8, qs, ks, qf, kf, qfs, kfs, w8, wf, cu, hq, hkv,
                                    round_p=False)
    ref = naive_causal_attention(q, k, v, cu, hq, hkv)
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-12)


def test_three_class_reduces_to_two_class():
    lens, hq, hkv, d = [300, 64], 2, 1, 64
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=8)
    q_i8, qs = oracle.quantize_blocks(q, cu, 128)
    k_i8, ks = oracle.quantize_blocks(k, cu, 64)
    qf, qfs = oracle.quantize_blocks_fp8(q, cu, 128)
    kf, kfs = oracle.quantize_blocks_fp8(k, cu, 64)
    w8, wf, *_ = oracle.routing_words3(lens, hkv, "sptrans", 5000, 0)
    a = oracle.prefill_attention3(q, k, v, q_i8, k_i8, qs, ks, qf, kf, qfs, kfs, w8, wf, cu, hq, hkv)
    b = oracle.prefill_attention(q, k, v, q_i8, k_i8, qs, ks, w8, cu, hq, hkv)
    np.testing.assert_array_equal(a, b)
    # and FP8 changes the result on lossy inputs
    w8, wf, *_ = oracle.routing_words3(lens, hkv, "sptrans", 0, 10000)
    c = oracle.prefill_attention3(q, k, v, q_i8, k_i8, qs, ks, qf, kf, qfs, kfs, w8, wf, cu, hq, hkv)
    assert np.abs(c - b).max() > 1e-4
