"""The importance-exposure probe on synthetic inputs with locality and a sink
(CPU oracle): the share of high-importance attention mass (per row, the
fewest keys holding half of it) that each layout routes to INT8.  The
numbers are printed for the record; the test only checks the probe's range
and that the content-dependent layout exposes less than the SpTrans template
once coverage is large."""

import numpy as np

import oracle
import synth


def test_exposure_sptrans_vs_adaptive(capsys):
    lens, hq, hkv, d = [2048], 2, 1, 128
    q, k, _, cu = synth.make_qkv_local(lens, hq, hkv, d, seed=7)
    q_i8, qs = oracle.quantize_blocks(q, cu, 128)
    k_i8, ks = oracle.quantize_blocks(k, cu, 64)
    imp = oracle.routing_importance(q_i8, k_i8, qs, ks, cu, hq, hkv)
    rows = []
    for cov in (2500, 5000, 7500):
        sw, *_ = oracle.routing_words(lens, hkv, "sptrans", cov)
        aw, *_ = oracle.adaptive_words(lens, imp, cov)
        es = oracle.importance_exposure(q, k, cu, hq, hkv, sw)
        ea = oracle.importance_exposure(q, k, cu, hq, hkv, aw)
        rows.append((cov, es, ea))
        assert 0.0 <= ea <= 1.0 and 0.0 <= es <= 1.0
    with capsys.disabled():
        for cov, es, ea in rows:
            print(f"\nexposure at {cov / 100:.0f}% INT8 groups: sptrans {es:.4f}, adaptive {ea:.4f}")
    assert rows[-1][2] < rows[-1][1]
