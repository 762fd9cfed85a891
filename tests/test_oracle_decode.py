"""Pins of the oracle's INT8-cache decode step (CPU only).

The decode oracle is checked against things it does not restate: naive fp64
softmax attention on inputs the blockwise quantiser reproduces exactly, the
(separately pinned) prefill oracle's last row, and closed forms (constant V,
a single cached token)."""

import math

import numpy as np
import pytest

import oracle
import synth


def _naive_last_row(qrow, kseq, vseq):
    """Plain softmax attention of one query over a whole sequence (fp64)."""
    s = kseq.astype(np.float64) @ qrow.astype(np.float64) / math.sqrt(qrow.shape[-1])
    p = np.exp(s - s.max())
    return (p @ vseq.astype(np.float64)) / p.sum()


def _decode(q_new, k, v, cu, hq, hkv, template, cov, seed=0, round_p=True):
    seqlens = list(np.diff(cu))
    words, g, n8, nl = oracle.routing_words(seqlens, hkv, template, cov, seed)
    k_i8, ks, v_i8, vs = oracle.quantize_kv_cache(k, v, cu)
    return oracle.decode_attention(q_new, k_i8, ks, v_i8, vs, words, cu, hq, hkv, round_p=round_p)


@pytest.mark.parametrize("cov", [0, 5000, 10000])
def test_lossless_cache_equals_naive_attention(cov):
    # per-block power-of-two scales: dequantisation is exact, so both score
    # paths equal the exact scores and the step is plain attention; the
    # distinct scales catch a wrong scale index, GQA catches a wrong head map
    lens, hq, hkv, d = [300, 1, 64, 65, 129], 6, 2, 64
    cu = synth.cu_seqlens_of(lens)
    k = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=1)
    v = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=2)
    q_new = synth.lossless_blocks_pow2([1] * len(lens), hq, d, 1, seed=3)
    out = _decode(q_new, k, v, cu, hq, hkv, "sptrans", cov, round_p=False)
    for s, L in enumerate(lens):
        for h in range(hq):
            kv = h // (hq // hkv)
            ref = _naive_last_row(q_new[s, h], k[cu[s]:cu[s + 1], kv], v[cu[s]:cu[s + 1], kv])
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-9, atol=1e-12)


def test_rounded_p_stays_within_binary16_of_exact():
    lens, hq, hkv, d = [200, 77], 2, 1, 64
    cu = synth.cu_seqlens_of(lens)
    k = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=4)
    v = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=5)
    q_new = synth.lossless_blocks_pow2([1, 1], hq, d, 1, seed=6)
    a = _decode(q_new, k, v, cu, hq, hkv, "band", 5000, round_p=True)
    b = _decode(q_new, k, v, cu, hq, hkv, "band", 5000, round_p=False)
    assert np.abs(a - b).max() < 2e-3 * np.abs(v.astype(np.float64)).max()


@pytest.mark.parametrize("template", oracle.TEMPLATES)
@pytest.mark.parametrize("cov", [0, 2500, 7500, 10000])
def test_matches_prefill_oracle_last_row(template, cov):
    # K, V reproduced exactly by the cache; Q lossy, with the largest value of
    # every (128-row block, head) in the block's last row, so the prefill
    # block scale equals the decode row scale.  Then the decode step of the
    # newest token equals the prefill oracle's row L-1 on both paths.  L=4160
    # gives g=2, so the group index t // g is exercised.
    lens, hq, hkv, d = [4160, 128, 300], 3, 1, 64
    cu = synth.cu_seqlens_of(lens)
    q, _, _, _ = synth.make_qkv(lens, hq, hkv, d, outliers=False, seed=7)
    q = q.astype(np.float32)
    for s, L in enumerate(lens):
        last = cu[s + 1] - 1
        b0 = cu[s] + ((L - 1) // 128) * 128
        blk = np.abs(q[b0:last + 1]).max(axis=(0, 2))
        q[last, :, 5] = np.float32(2.0) * blk + 1.0
    q = q.astype(np.float16)
    k = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=8)
    v = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=9)
    words, g, n8, nl = oracle.routing_words(lens, hkv, template, cov, 0)
    assert g[0] == 2
    q_i8, q_s = oracle.quantize_blocks(q, cu, 128)
    k_i8, k_s = oracle.quantize_blocks(k, cu, 64)
    rows = [(s, h, (L - 1) // 128) for s, L in enumerate(lens) for h in range(hq)]
    pre = oracle.prefill_attention(q, k, v, q_i8, k_i8, q_s, k_s, words, cu, hq, hkv, rows=rows)
    q_new = synth.decode_queries(q, cu)
    dec = _decode(q_new, k, v, cu, hq, hkv, template, cov)
    for s in range(len(lens)):
        np.testing.assert_allclose(dec[s], pre[cu[s + 1] - 1], rtol=1e-9, atol=1e-12)


def test_routing_changes_the_result_on_lossy_inputs():
    lens, hq, hkv, d = [512], 2, 1, 64
    q, k, v, cu = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=10)
    q_new = synth.decode_queries(q, cu)
    a = _decode(q_new, k, v, cu, hq, hkv, "band", 0)
    b = _decode(q_new, k, v, cu, hq, hkv, "band", 10000)
    assert np.abs(a - b).max() > 1e-4


def test_constant_values_and_single_token():
    lens, hq, hkv, d = [1, 190, 0, 64], 4, 2, 64
    cu = synth.cu_seqlens_of(lens)
    q, k, _, _ = synth.make_qkv(lens, hq, hkv, d, outliers=True, seed=11)
    # constants whose block scale is a power of two (c = +-127 * 2^-e), so
    # the cache holds them exactly
    v = np.full(k.shape, np.float16(127 / 128))
    v[:, 1, :] = np.float16(-127 / 32)
    q_new = synth.decode_queries(q, cu)
    out = _decode(q_new, k, v, cu, hq, hkv, "rowrandom", 5000, seed=3)
    for s, L in enumerate(lens):
        for h in range(hq):
            want = 0.0 if L == 0 else (127 / 128 if h // 2 == 0 else -127 / 32)
            assert abs(out[s, h] - want).max() < 1e-12
    # one cached token: the output is that token's dequantised value
    v = synth.lossless_blocks_pow2(lens, hkv, d, 64, seed=12)
    out = _decode(q_new, k, v, cu, hq, hkv, "band", 10000)
    np.testing.assert_array_equal(out[0], v[0].astype(np.float64)[[0, 0, 1, 1]])


def test_query_rows_quantised_one_row_per_block():
    q = synth.lossless_blocks_pow2([1, 1, 1], 5, 64, 1, seed=13)
    q_i8, s = oracle.quantize_query_rows(q)
    assert s.shape == (5, 3)
    np.testing.assert_array_equal(q_i8.astype(np.float32) * s.T[:, :, None], q.astype(np.float32))
