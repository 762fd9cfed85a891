"""Pins of the oracle's geometry and routing-word builder (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "routing_worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: f"{c['template']}-L{c['L']}-{c['coverage_bp']}")
def test_worked_examples(case):
    words, g, n8, nl = oracle.routing_words([case["L"]], 1, case["template"], case["coverage_bp"],
                                            seed=case.get("seed", 0))
    assert [hex(int(w)) for w in words[0]] == case["words"]


def test_splitmix64_published_outputs():
    gold = _golden()["splitmix64"]
    for i, o in zip(gold["inputs"], gold["outputs"]):
        assert oracle.splitmix64_mix(int(i, 16)) == int(o, 16)
    # the generator's state advances by the golden-gamma constant
    assert (2 * 0x9E3779B97F4A7C15) % (1 << 64) == int(gold["inputs"][1], 16)


# Closed forms of the tile geometry.
@pytest.mark.parametrize("L,Tm,Tn,g,n_legal", [
    (256, 2, 4, 1, 6),
    (1024, 8, 16, 1, 72),
    (4096, 32, 64, 1, 32 * 33),          # g=1, L multiple of 128: Tm(Tm+1)
    (8192, 64, 128, 2, 64 * 65 // 2),    # g=2: row r has r+1 groups
    (16384, 128, 256, 4, 4160),
    (65536, 512, 1024, 16, 16640),
    (1, 1, 1, 1, 1),
    (0, 0, 0, 1, 0),
    (130, 2, 3, 1, 2 + 3),               # row 1 holds queries 128..129 -> tiles 0..2
])
def test_geometry_closed_forms(L, Tm, Tn, g, n_legal):
    geo = oracle.seq_geometry(L)
    assert (geo.Tm, geo.Tn, geo.g, geo.n_legal) == (Tm, Tn, g, n_legal)
    assert all(d <= 63 for d in geo.D)


def test_geometry_g_general():
    # g is the smallest integer with at most 64 groups in the longest row
    for L in [64 * 64, 64 * 64 + 1, 64 * 128, 64 * 128 + 64, 100000]:
        geo = oracle.seq_geometry(L)
        assert max(geo.D) <= 63
        if geo.g > 1:
            # one less would overflow the word
            assert (geo.Tn - 1) // (geo.g - 1) > 63


def test_int8_count_rounding():
    assert oracle.int8_group_count(5000, 6) == 3
    assert oracle.int8_group_count(7500, 1056) == 792
    assert oracle.int8_group_count(2500, 72) == 18
    assert oracle.int8_group_count(2500, 2) == 1      # 0.5 rounds half up
    assert oracle.int8_group_count(2499, 2) == 0
    assert oracle.int8_group_count(10000, 7) == 7
    with pytest.raises(ValueError):
        oracle.int8_group_count(10001, 7)


def _popcounts(words):
    return [bin(int(w)).count("1") for w in words]


LENGTHS = [1, 64, 127, 128, 129, 256, 300, 1000, 1024, 4096, 8192, 8200]
COVS = [0, 1000, 2500, 5000, 7500, 10000]


@pytest.mark.parametrize("template", oracle.TEMPLATES)
def test_routing_invariants(template):
    for L in LENGTHS:
        geo = oracle.seq_geometry(L)
        prev = None
        for cov in COVS:
            words, g, n8, nl = oracle.routing_words([L], 2, template, cov, seed=7)
            assert words.shape == (2, geo.Tm)                    # O(Hk x Tm) metadata
            assert np.array_equal(words[0], words[1])            # reused across KV heads
            assert g[0] == geo.g and nl[0] == geo.n_legal
            assert sum(_popcounts(words[0])) == n8[0] == oracle.int8_group_count(cov, geo.n_legal)
            sets = set()
            for r, w in enumerate(words[0]):
                w = int(w)
                assert w >> (geo.D[r] + 1) == 0                  # illegal bits are 0
                sets |= {(r, G) for G in range(64) if (w >> G) & 1}
            if prev is not None:
                assert prev <= sets                               # nested in coverage
            prev = sets
            if cov == 0:
                assert not sets
            if cov == 10000:
                assert sets == set(geo.legal_groups())


def test_orders_are_permutations():
    for L in [256, 1000, 4096, 8192]:
        geo = oracle.seq_geometry(L)
        legal = set(geo.legal_groups())
        for t in oracle.TEMPLATES:
            o = oracle.template_order(geo, t, seed=3)
            assert len(o) == len(legal) and set(o) == legal


def test_rowrandom_seed_and_row_balance():
    geo = oracle.seq_geometry(8192)
    a = oracle.routing_words([8192], 1, "rowrandom", 5000, seed=1)[0]
    b = oracle.routing_words([8192], 1, "rowrandom", 5000, seed=1)[0]
    c = oracle.routing_words([8192], 1, "rowrandom", 5000, seed=2)[0]
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # one common threshold: each row keeps about tau * n_r groups in FP16
    for cov in [1000, 5000, 7500]:
        w = oracle.routing_words([8192], 1, "rowrandom", cov, seed=5)[0][0]
        keep = [geo.n[r] - bin(int(w[r])).count("1") for r in range(geo.Tm)]
        tau = sum(keep) / geo.n_legal
        assert all(abs(k - tau * n) <= 1.0 + 1e-9 for k, n in zip(keep, geo.n))


def test_band_constant_width_and_global_leading_columns():
    geo = oracle.seq_geometry(4096)
    w = oracle.routing_words([4096], 1, "band", 5000)[0][0]
    # band: FP16 groups are the ones nearest the diagonal, a prefix in distance
    for r in range(geo.Tm):
        fp16 = [geo.D[r] - G for G in range(geo.D[r] + 1) if not (int(w[r]) >> G) & 1]
        assert sorted(fp16) == list(range(len(fp16)))
    w = oracle.routing_words([4096], 1, "global", 5000)[0][0]
    for r in range(geo.Tm):
        fp16 = [G for G in range(geo.D[r] + 1) if not (int(w[r]) >> G) & 1]
        assert fp16 == list(range(len(fp16)))


def test_sptrans_stride():
    assert oracle.sptrans_stride(oracle.seq_geometry(4096)) == 8
    assert oracle.sptrans_stride(oracle.seq_geometry(8192)) == 8
    assert oracle.sptrans_stride(oracle.seq_geometry(1024)) == 4
    assert oracle.sptrans_stride(oracle.seq_geometry(256)) == 2
    # at 4096 / 75%: the FP16 set is a distance prefix of the stride lattice
    # (d = 0 mod 8) plus a distance prefix of the remaining tail groups
    geo = oracle.seq_geometry(4096)
    w = oracle.routing_words([4096], 1, "sptrans", 7500)[0][0]
    fp16 = {(r, G) for r in range(geo.Tm) for G in range(geo.D[r] + 1) if not (int(w[r]) >> G) & 1}
    lat = [geo.D[r] - G for (r, G) in fp16 if (geo.D[r] - G) % 8 == 0]
    off = [geo.D[r] - G for (r, G) in fp16 if (geo.D[r] - G) % 8 != 0]
    assert lat and off
    for r in range(geo.Tm):
        for G in range(geo.D[r] + 1):
            d = geo.D[r] - G
            if d % 8 == 0 and d < max(lat):
                assert (r, G) in fp16
            if d % 8 != 0 and d < max(off):
                assert (r, G) in fp16


def test_union_round_robin():
    a = [1, 2, 3, 4]
    b = [4, 3, 2, 1]
    assert oracle.union_orders(a, b) == [1, 4, 2, 3]
    assert oracle.union_orders(a) == a


def test_varlen_words_concatenate():
    lens = [256, 0, 1000, 130]
    words, g, n8, nl = oracle.routing_words(lens, 3, "sptrans", 5000)
    off = 0
    for L in lens:
        single = oracle.routing_words([L], 1, "sptrans", 5000)[0][0]
        tm = oracle.seq_geometry(L).Tm
        assert np.array_equal(words[0, off:off + tm], single)
        off += tm
    assert off == words.shape[1]


def test_headline_counts():
    words, g, n8, nl = oracle.routing_words([4096] * 8, 8, "sptrans", 7500)
    assert words.shape == (8, 256) and list(n8) == [792] * 8 and list(nl) == [1056] * 8
    words, g, n8, nl = oracle.routing_words([65536, 16384, 8192, 4096, 1024, 1024], 4,
                                            "rowrandom", 5000)
    assert list(g) == [16, 4, 2, 1, 1, 1]
    assert list(nl) == [16640, 4160, 2080, 1056, 72, 72]
    assert list(n8) == [8320, 2080, 1040, 528, 36, 36]
    assert words.shape == (4, 752)
