"""Pins of the oracle's synthetic multi-layer stack (CPU only).

Each check rests on something other than the oracle's own formula: closed
forms of the RMS norm, one-hot weights whose products are exact and whose
expected outputs are found by indexing, brute-force loops on tiny inputs,
and attention special cases with closed forms (uniform attention when the
queries vanish, one key per sequence)."""

import numpy as np
import pytest

import oracle
import synth

F16 = np.float16


def _ulp16(x):
    return np.spacing(np.abs(np.asarray(x, dtype=F16))).astype(np.float64)


# --------------------------------------------------------------- RMS norm

def test_rms_norm_closed_forms():
    hq, hkv, d = 4, 2, 64
    W = oracle.stack_width(hq, hkv, d)
    assert W == 128
    x = np.zeros((4, hq * d), dtype=np.float32)
    # token 0: stream 0 all +-1 -> u = +-1 exactly (1/sqrt(1 + 1e-6) rounds to 1)
    signs = np.where(np.arange(W) % 3 == 0, -1.0, 1.0)
    x[0, :W] = signs
    # token 0, stream 1: a single nonzero entry c normalises to sign(c) sqrt(W)
    # (sqrt(128) = 11.3137..., nearest binary16 11.3125)
    x[0, W + 17] = -3.0
    # token 1: the same single-entry pattern at a very different scale in
    # each stream (each stream normalises on its own)
    x[1, 5] = 0.5
    x[1, W + 100] = 1e3
    # token 2: stream 0 zero -> u = 0 (eps keeps it finite); stream 1 all 2
    x[2, W:] = 2.0
    u = oracle.stack_rms_norm(x, hkv).astype(np.float64)
    assert u.dtype == np.float64
    assert np.array_equal(u[0, :W], signs)
    want = np.zeros(W)
    want[17] = -11.3125
    assert np.array_equal(u[0, W:], want)
    assert u[1, 5] == 11.3125 and u[1, W + 100] == 11.3125
    assert np.count_nonzero(u[1]) == 2
    assert not u[2, :W].any() and np.all(u[2, W:] == 1.0)
    assert not u[3].any()
    # where mean(x^2) is comparable to eps, eps shows: c = 0.01, W = 128 ->
    # 0.01 / sqrt(1e-4/128 + 1e-6) = 7.4927..., binary16 7.4921875 (step 2^-8)
    x1 = np.zeros((1, hq * d), dtype=np.float32)
    x1[0, 3] = 0.01
    assert float(oracle.stack_rms_norm(x1, hkv)[0, 3]) == 7.4921875


def test_rms_norm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(5)
    hq, hkv, d = 6, 3, 64
    x = rng.standard_normal((40, hq * d)).astype(np.float32)
    x[:, : hq * d // hkv] *= 50.0    # stream 0 at another scale
    u = oracle.stack_rms_norm(x, hkv).astype(np.float64).reshape(40, hkv, -1)
    ms = (u * u).mean(axis=2)
    assert np.all(np.abs(ms - 1.0) < 2e-3)
    u4 = oracle.stack_rms_norm(x * np.float32(4.0), hkv).astype(np.float64).reshape(40, hkv, -1)
    assert np.all(np.abs(u4 - u) <= _ulp16(u))


# ------------------------------------------------------------- projections

def _one_hot(rows, cols, rng, scales=True):
    """Weights with one entry per row: w[n, src[n]] = 2^e[n] (exact products)."""
    src = rng.integers(0, cols, size=rows)
    e = rng.integers(-2, 3, size=rows) if scales else np.zeros(rows, dtype=np.int64)
    w = np.zeros((rows, cols), dtype=F16)
    w[np.arange(rows), src] = np.ldexp(1.0, e).astype(F16)
    return w, src, np.ldexp(1.0, e)


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (6, 2, 64), (3, 1, 128)])
def test_qkv_one_hot_weights(hq, hkv, d):
    rng = np.random.default_rng(hq * 100 + d)
    W = oracle.stack_width(hq, hkv, d)
    r = hq // hkv
    T = 7
    u = rng.standard_normal((T, hq * d)).astype(F16)
    wqkv = np.zeros((hkv, W + 2 * d, W), dtype=F16)
    src = np.zeros((hkv, W + 2 * d), dtype=np.int64)
    sc = np.zeros((hkv, W + 2 * d))
    for g in range(hkv):
        wqkv[g], src[g], sc[g] = _one_hot(W + 2 * d, W, rng)
    q, k, v = oracle.stack_qkv(u, wqkv, hq, hkv, d)
    assert q.dtype == F16 and q.shape == (T, hq, d) and k.shape == (T, hkv, d) and v.shape == (T, hkv, d)
    uf = u.astype(np.float64)
    for t in range(T):
        for g in range(hkv):
            for n in range(W + 2 * d):
                val = uf[t, g * W + src[g, n]] * sc[g, n]
                if n < W:
                    got = q[t, g * r + n // d, n % d]
                elif n < W + d:
                    got = k[t, g, n - W]
                else:
                    got = v[t, g, n - W - d]
                assert float(got) == val


def test_qkv_brute_force_random_weights():
    rng = np.random.default_rng(9)
    hq, hkv, d = 2, 1, 64
    W = oracle.stack_width(hq, hkv, d)
    T = 3
    u = rng.standard_normal((T, hq * d)).astype(F16)
    wqkv = (rng.standard_normal((hkv, W + 2 * d, W)) / np.sqrt(W)).astype(F16)
    q, k, v = oracle.stack_qkv(u, wqkv, hq, hkv, d)
    for t in range(T):
        for n in range(W + 2 * d):
            s = 0.0
            for j in range(W):
                s += float(u[t, j]) * float(wqkv[0, n, j])
            want = F16(s)
            got = (q[t, n // d, n % d] if n < W else k[t, 0, n - W] if n < W + d else v[t, 0, n - W - d])
            # the exact sum and this float64 loop differ far below binary16 resolution
            assert abs(float(got) - float(want)) <= float(_ulp16(want))


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (3, 1, 128)])
def test_out_residual_one_hot_weights(hq, hkv, d):
    rng = np.random.default_rng(hq + d)
    W = oracle.stack_width(hq, hkv, d)
    r = hq // hkv
    T = 5
    x = rng.standard_normal((T, hq * d))
    o = rng.standard_normal((T, hq, d)).astype(F16)
    wo = np.zeros((hkv, W, W), dtype=F16)
    src = np.zeros((hkv, W), dtype=np.int64)
    sc = np.zeros((hkv, W))
    for g in range(hkv):
        wo[g], src[g], sc[g] = _one_hot(W, W, rng)
    y = oracle.stack_out_residual(x, o, wo, hq, hkv, d)
    for t in range(T):
        for g in range(hkv):
            for n in range(W):
                j = src[g, n]
                want = x[t, g * W + n] + float(o[t, g * r + j // d, j % d]) * sc[g, n]
                assert y[t, g * W + n] == want


# ------------------------------------------------------------- whole layer

def _layer_setup(lens, hq, hkv, d, seed):
    cu = synth.cu_seqlens_of(lens)
    T = int(cu[-1])
    wqkv, wo = synth.stack_weights(2, hq, hkv, d, seed=seed)
    x = synth.stack_input(T, hq, d, seed=seed + 1).astype(np.float64)
    return cu, T, wqkv, wo, x


@pytest.mark.parametrize("cov", [0, 5000, 10000])
def test_layer_uniform_attention_when_queries_vanish(cov):
    # Wq = 0 -> q = 0 -> every score is 0 on both paths (INT8: codes and
    # scale 0) -> P = 1 and O is the running mean of v over the sequence.
    lens, hq, hkv, d = [150, 1, 70, 129], 6, 2, 64
    cu, T, wqkv, wo, x = _layer_setup(lens, hq, hkv, d, seed=11)
    W = oracle.stack_width(hq, hkv, d)
    r = hq // hkv
    wq0 = wqkv[0].copy()
    wq0[:, :W] = 0
    words = oracle.routing_words(lens, hkv, "rowrandom", cov)[0]
    y = oracle.stack_layer(x, wq0, wo[0], words, cu, hq, hkv, d)
    _, _, v = oracle.stack_qkv(oracle.stack_rms_norm(x, hkv), wq0, hq, hkv, d)
    o = np.zeros((T, hq, d))
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        vs = v[a:b].astype(np.float64)
        run = np.cumsum(vs, axis=0) / np.arange(1, b - a + 1)[:, None, None]
        for h in range(hq):
            o[a:b, h] = run[:, h // r]
    want = oracle.stack_out_residual(x, o.astype(F16), wo[0], hq, hkv, d)
    # one binary16 step of O (a tie decided by the last float64 bit of the
    # mean) pushed through Wo
    tol = 2.0 ** -10 * np.abs(v.astype(np.float64)).max() * np.abs(wo[0].astype(np.float64)).sum(axis=2).max()
    assert np.abs(y - want).max() <= tol
    assert np.mean(y != want) < 1e-3


def test_layer_one_key_per_sequence():
    # sequences of one token: the softmax has one entry, O = v of that token
    # for every query head of its KV head (at any routing)
    lens, hq, hkv, d = [1] * 6, 4, 2, 128
    cu, T, wqkv, wo, x = _layer_setup(lens, hq, hkv, d, seed=12)
    r = hq // hkv
    _, _, v = oracle.stack_qkv(oracle.stack_rms_norm(x, hkv), wqkv[0], hq, hkv, d)
    want = oracle.stack_out_residual(x, np.repeat(v, r, axis=1), wo[0], hq, hkv, d)
    for cov in (0, 10000):
        words = oracle.routing_words(lens, hkv, "band", cov)[0]
        y = oracle.stack_layer(x, wqkv[0], wo[0], words, cu, hq, hkv, d)
        assert np.array_equal(y, want)


def test_layer_zero_output_weights_keep_the_state():
    lens, hq, hkv, d = [200, 33], 4, 2, 64
    cu, T, wqkv, wo, x = _layer_setup(lens, hq, hkv, d, seed=13)
    words = oracle.routing_words(lens, hkv, "sptrans", 7500)[0]
    y = oracle.stack_layer(x, wqkv[0], np.zeros_like(wo[0]), words, cu, hq, hkv, d)
    assert np.array_equal(y, x)


def test_forward_applies_each_layers_weights_in_order():
    lens, hq, hkv, d = [130, 20], 4, 2, 64
    cu, T, wqkv, wo, x = _layer_setup(lens, hq, hkv, d, seed=14)
    words = oracle.routing_words(lens, hkv, "band", 5000)[0]
    wo2 = wo.copy()
    wo2[1] = 0
    xs = oracle.stack_forward(x, wqkv, wo2, words, cu, hq, hkv, d)
    assert len(xs) == 2 and np.array_equal(xs[1], xs[0])
    xs = oracle.stack_forward(x, wqkv, wo, words, cu, hq, hkv, d)
    assert not np.array_equal(xs[1], xs[0])
    # layer 0 alone, then layer 1 on its output
    y0 = oracle.stack_layer(x, wqkv[0], wo[0], words, cu, hq, hkv, d)
    y1 = oracle.stack_layer(y0, wqkv[1], wo[1], words, cu, hq, hkv, d)
    assert np.array_equal(xs[0], y0) and np.array_equal(xs[1], y1)
    # swapping the two layers' weights changes the result
    xs_sw = oracle.stack_forward(x, wqkv[::-1], wo[::-1], words, cu, hq, hkv, d)
    assert not np.array_equal(xs_sw[1], xs[1])


def test_depth_deviation():
    lens, hq, hkv, d = [300, 77], 4, 2, 64
    cu, T, wqkv, wo, x = _layer_setup(lens, hq, hkv, d, seed=15)
    w0 = oracle.routing_words(lens, hkv, "sptrans", 0)[0]
    w1 = oracle.routing_words(lens, hkv, "sptrans", 7500)[0]
    xa = oracle.stack_forward(x, wqkv, wo, w0, cu, hq, hkv, d)
    xb = oracle.stack_forward(x, wqkv, wo, w1, cu, hq, hkv, d)
    assert np.array_equal(oracle.depth_deviation(xa, xa), [0.0, 0.0])
    dev = oracle.depth_deviation(xa, xb)
    assert dev.shape == (2,) and np.all(dev > 0)
    assert dev[0] == np.abs(xa[0] - xb[0]).mean()
