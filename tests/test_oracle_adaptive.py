"""Pins of the oracle's adaptive routing (a per-tile statistic) and of the
importance-exposure probe (CPU only): direct block sums, inputs whose pooled
scores are known in closed form, routing invariants, and probe identities."""

import numpy as np
import pytest

import oracle
import synth


def test_block_column_sums_match_direct_sums():
    lens = [300, 0, 77, 129]
    x = np.random.default_rng(0).integers(-127, 128, size=(sum(lens), 3, 16)).astype(np.int8)
    cu = synth.cu_seqlens_of(lens)
    sums, rows = oracle.block_column_sums(x, cu, 64)
    blocks = [(s, b0) for s in range(len(lens)) for b0 in range(cu[s], cu[s + 1], 64)]
    assert sums.shape == (3, len(blocks), 16) and len(rows) == len(blocks)
    for i, (s, b0) in enumerate(blocks):
        b1 = min(b0 + 64, cu[s + 1])
        assert rows[i] == b1 - b0
        for h in range(3):
            for c in range(16):
                assert sums[h, i, c] == sum(int(x[j, h, c]) for j in range(b0, b1))


def _one_hot_blocks(L, d, q_level, k_levels):
    """Q rows all q_level * e_0; every row of key tile t equals k_levels[t] * e_0."""
    q = np.zeros((L, 1, d), dtype=np.int8)
    q[:, 0, 0] = q_level
    k = np.zeros((L, 1, d), dtype=np.int8)
    for t in range(-(-L // 64)):
        k[64 * t:64 * t + 64, 0, 0] = k_levels[t]
    return q, k


def test_importance_closed_form():
    # mean query q_level*e0, mean key of tile t k_t*e0, unit scales: the
    # pooled score is q_level*k_t exactly, so a group's importance is
    # q_level*(max k in group - max k in the row's legal tiles)
    L, d = 256, 16
    k_levels = [5, 40, -3, 17]
    q_i8, k_i8 = _one_hot_blocks(L, d, 2, k_levels)
    cu = [0, L]
    qs = np.ones((1, 2), dtype=np.float32)
    ks = np.ones((1, 4), dtype=np.float32)
    imp = oracle.routing_importance(q_i8, k_i8, qs, ks, cu, 1, 1)
    assert imp.shape == (1, 2, 64)
    # row 0: legal tiles 0, 1 -> max 40; row 1: tiles 0..3 -> max 40
    np.testing.assert_array_equal(imp[0, 0, :2], np.float32([2 * (5 - 40), 0]))
    np.testing.assert_array_equal(imp[0, 1, :4], np.float32([2 * (5 - 40), 0, 2 * (-3 - 40), 2 * (17 - 40)]))
    assert np.isinf(imp[0, 0, 2:]).all() and np.isinf(imp[0, 1, 4:]).all()
    # scales enter as fl32(fl32(s_q s_k) / (n_q n_k)) times the integer dot:
    # with 128 x 64 rows the dot is 128*64*q_level*k_t
    qs2 = np.full((1, 2), 0.5, dtype=np.float32)
    ks2 = np.full((1, 4), 0.25, dtype=np.float32)
    imp2 = oracle.routing_importance(q_i8, k_i8, qs2, ks2, cu, 1, 1)
    np.testing.assert_array_equal(imp2[0, 1, :4], imp[0, 1, :4] * np.float32(0.125))


def test_importance_takes_max_over_heads_and_groups():
    # two query heads of one KV head: the pooled score is the larger of the two;
    # L = 4160 gives g = 2, so a group's score is the max of its two tiles
    L, d = 4160, 16
    tn = -(-L // 64)
    lv = (np.arange(tn) * 7) % 23 - 11
    q0, k = _one_hot_blocks(L, d, 1, lv)
    q = np.concatenate([q0, -q0], axis=1)      # head 1 sees the negated scores
    cu = [0, L]
    qs = np.ones((2, -(-L // 128)), dtype=np.float32)
    ks = np.ones((1, tn), dtype=np.float32)
    imp = oracle.routing_importance(q, k, qs, ks, cu, 2, 1)
    geo = oracle.seq_geometry(L)
    assert geo.g == 2
    for r in (0, 17, geo.Tm - 1):
        nt = geo.last_tile[r] + 1
        # pooled score of head 0 is +lv[t], of head 1 -lv[t]: the max is |lv[t]|
        Z = np.abs(lv[:nt]).astype(np.float64)
        zrow = Z.max()
        for G in range(geo.D[r] + 1):
            assert imp[0, r, G] == np.float32(Z[2 * G:2 * G + 2].max() - zrow)


def _imp_random(lens, hkv, seed):
    geos = [oracle.seq_geometry(L) for L in lens]
    rng = np.random.default_rng(seed)
    imp = np.full((hkv, sum(g.Tm for g in geos), 64), np.inf, dtype=np.float32)
    off = 0
    for geo in geos:
        for r in range(geo.Tm):
            imp[:, off + r, :geo.D[r] + 1] = -rng.integers(0, 5, size=(hkv, geo.D[r] + 1)).astype(np.float32)
        off += geo.Tm
    return imp, geos


@pytest.mark.parametrize("lens", [[256], [1024, 300, 1, 0], [4160]])
def test_adaptive_words_invariants(lens):
    imp, geos = _imp_random(lens, 3, 1)
    prev = None
    for cov in (0, 1000, 2500, 5000, 7500, 10000):
        w, g, n8, nl = oracle.adaptive_words(lens, imp, cov)
        off = 0
        for s, geo in enumerate(geos):
            assert n8[s] == oracle.int8_group_count(cov, geo.n_legal) and nl[s] == geo.n_legal
            for kv in range(3):
                rows = w[kv, off:off + geo.Tm]
                assert sum(bin(int(x)).count("1") for x in rows) == n8[s]
                for r in range(geo.Tm):
                    assert int(rows[r]) >> (geo.D[r] + 1) == 0          # illegal bits clear
                    if cov == 10000:
                        assert int(rows[r]) == (1 << (geo.D[r] + 1)) - 1
                    # every INT8 group is at least as unimportant as every FP16 one
                chosen = [imp[kv, off + r, G] for r in range(geo.Tm) for G in range(geo.D[r] + 1)
                          if (int(rows[r]) >> G) & 1]
                kept = [imp[kv, off + r, G] for r in range(geo.Tm) for G in range(geo.D[r] + 1)
                        if not (int(rows[r]) >> G) & 1]
                if chosen and kept:
                    assert max(chosen) <= min(kept)
            off += geo.Tm
        if prev is not None:
            assert np.all((prev & w) == prev)                               # nested
        prev = w


def test_adaptive_words_worked_example():
    # one sequence of 256 (rows 0 and 1; 2 and 4 legal groups), one KV head;
    # importances by hand: row 0 [-3, 0], row 1 [-1, 0, -3, -2]
    imp = np.full((1, 2, 64), np.inf, dtype=np.float32)
    imp[0, 0, :2] = [-3, 0]
    imp[0, 1, :4] = [-1, 0, -3, -2]
    # order: (-3,0,0) (-3,1,2) (-2,1,3) (-1,1,0) (0,0,1) (0,1,1)
    want = {0: [0x0, 0x0], 1700: [0x1, 0x0], 3400: [0x1, 0x4], 5000: [0x1, 0xC],
            6700: [0x1, 0xD], 8400: [0x3, 0xD], 10000: [0x3, 0xF]}
    for cov, words in want.items():
        w, _, n8, _ = oracle.adaptive_words([256], imp, cov)
        assert [int(x) for x in w[0]] == words, (cov, [hex(int(x)) for x in w[0]])


def test_exposure_identities():
    # (L = 4160 has g = 2: the probe must map key tiles to groups)
    lens, hq, hkv, d = [300, 4160], 1, 1, 64
    q, k, _, cu = synth.make_qkv_local(lens, hq, hkv, d, seed=2)
    none, *_ = oracle.routing_words(lens, hkv, "band", 0)
    full, *_ = oracle.routing_words(lens, hkv, "band", 10000)
    assert oracle.importance_exposure(q, k, cu, hq, hkv, none) == 0.0
    assert abs(oracle.importance_exposure(q, k, cu, hq, hkv, full) - 1.0) < 1e-12
    # a layout and its complement within the legal groups split the mass
    w, *_ = oracle.routing_words(lens, hkv, "rowrandom", 4000, 5)
    comp = full ^ w
    a = oracle.importance_exposure(q, k, cu, hq, hkv, w)
    b = oracle.importance_exposure(q, k, cu, hq, hkv, comp)
    assert abs(a + b - 1.0) < 1e-12


def test_exposure_of_one_hot_attention_counts_rows():
    # keys are huge multiples of e_j so each query's attention sits on one key
    # (the query's own position): the probe is the share of rows whose own
    # key's group is INT8
    L, d = 200, 256
    q = np.zeros((L, 1, d), dtype=np.float16)
    k = np.zeros((L, 1, d), dtype=np.float16)
    for i in range(L):
        q[i, 0, i] = 30.0
        k[i, 0, i] = 30.0
    cu = [0, L]
    w, *_ = oracle.routing_words([L], 1, "band", 5000)
    geo = oracle.seq_geometry(L)
    rows_int8 = sum((int(w[0, i // 128]) >> ((i // 64) // geo.g)) & 1 for i in range(L))
    got = oracle.importance_exposure(q, k, cu, 1, 1, w, tau=0.5)
    assert abs(got - rows_int8 / L) < 1e-9
