"""Parity of the synthetic multi-layer stack (HIP, through the C ABI) with
the CPU oracle on identical seeded inputs.

Tolerances, each derived from the arithmetic:
  * RMS norm and Q/K/V: the oracle rounds the exact value once to binary16;
    the kernels round an fp32 value whose error is at most
    gamma_n * sum|terms| (gamma_n = n 2^-24 / (1 - n 2^-24), n terms), so
    |got - exact| <= half a binary16 step + that bound;
  * output projection + residual: fp32 accumulation and one fp32 add,
    |got - exact| <= gamma_(W+1) * (|x| + sum |o w|);
  * one layer: the attention output obeys the prefill bars (max 4e-3, mean
    5e-4 against the oracle); pushed through Wo that is
    |dx_n| <= 4e-3 * sum_k |Wo[n, k]| per element and, on average,
    5e-4 * W * mean|Wo| over all elements;
  * several layers: each layer's attention output moved by the bar (random
    signs, seeded) and carried through the oracle's own stack gives the
    deviation a kernel within the bars can produce; the test allows twice
    that."""

import numpy as np
import pytest

import oracle
import synth
import mixed_precision_attention_amd as tm

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ATTN_MAX = 4e-3
ATTN_MEAN = 5e-4


def _log(msg):
    print(msg, flush=True)


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def _half_step(x):
    return 0.5 * np.spacing(np.abs(np.asarray(x, dtype=np.float16))).astype(np.float64)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


SHAPES = [([300, 77, 0, 129, 1, 64], 6, 2, 64), ([513, 200], 3, 1, 128), ([260, 131], 24, 8, 128),
          ([190, 5], 28, 4, 128)]


def _stream_scaled_input(T, hq, hkv, d, seed):
    x = synth.stack_input(T, hq, d, seed=seed)
    # streams at different scales (each normalises on its own)
    scale = np.repeat(np.float32(2.0) ** np.arange(-3, hkv - 3, dtype=np.float32), hq * d // hkv)
    return np.ascontiguousarray(x * scale[None, :])


@pytest.mark.parametrize("lens,hq,hkv,d", SHAPES)
def test_rms_norm(lens, hq, hkv, d):
    _log(f"stack rms norm lens={lens} hq={hq} hkv={hkv} d={d}")
    T = int(sum(lens))
    x = _stream_scaled_input(T, hq, hkv, d, seed=40)
    u = torch.empty((T, hq * d), dtype=torch.float16, device="cuda")
    tm.tilemix_stack_rms_norm(_dev(x), u, hq, hkv, d, 1e-6)
    torch.cuda.synchronize()
    got = u.cpu().numpy().astype(np.float64)
    xg = x.astype(np.float64).reshape(T, hkv, -1)
    W = xg.shape[2]
    exact = (xg / np.sqrt((xg * xg).mean(axis=2, keepdims=True) + 1e-6)).reshape(T, -1)
    # fp32: sum of squares, one division, sqrt, reciprocal, product: a few
    # units of 2^-24 relative on top of gamma_W on the sum
    rel = 0.5 * _gamma(W) + 8 * 2.0 ** -24
    assert np.all(np.abs(got - exact) <= _half_step(got) + rel * np.abs(exact))
    ref = oracle.stack_rms_norm(x, hkv).astype(np.float64)
    assert np.mean(got != ref) < 1e-2


@pytest.mark.parametrize("lens,hq,hkv,d", SHAPES)
def test_qkv_projection(lens, hq, hkv, d):
    _log(f"stack qkv lens={lens} hq={hq} hkv={hkv} d={d}")
    T = int(sum(lens))
    W = oracle.stack_width(hq, hkv, d)
    rng = np.random.default_rng(41)
    u = rng.standard_normal((T, hq * d)).astype(np.float16)
    wqkv, _ = synth.stack_weights(1, hq, hkv, d, seed=42)
    q = torch.empty((T, hq, d), dtype=torch.float16, device="cuda")
    k = torch.empty((T, hkv, d), dtype=torch.float16, device="cuda")
    v = torch.empty((T, hkv, d), dtype=torch.float16, device="cuda")
    tm.tilemix_stack_qkv(_dev(u), _dev(wqkv[0]), q, k, v, hq, hkv, d)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.stack_qkv(u, wqkv[0], hq, hkv, d)
    ug = u.astype(np.float64).reshape(T, hkv, W)
    w = wqkv[0].astype(np.float64)
    for got, ref, sl in ((q, rq, slice(0, W)), (k, rk, slice(W, W + d)), (v, rv, slice(W + d, W + 2 * d))):
        got = got.cpu().numpy().astype(np.float64).reshape(T, hkv, -1)
        exact = np.stack([ug[:, g] @ w[g, sl].T for g in range(hkv)], axis=1)
        absum = np.stack([np.abs(ug[:, g]) @ np.abs(w[g, sl]).T for g in range(hkv)], axis=1)
        assert np.all(np.abs(got - exact) <= _half_step(got) + _gamma(W) * absum)
        assert np.mean(got != ref.astype(np.float64).reshape(T, hkv, -1)) < 1e-2


@pytest.mark.parametrize("lens,hq,hkv,d", SHAPES)
def test_out_projection_residual(lens, hq, hkv, d):
    _log(f"stack out+residual lens={lens} hq={hq} hkv={hkv} d={d}")
    T = int(sum(lens))
    W = oracle.stack_width(hq, hkv, d)
    rng = np.random.default_rng(43)
    x = synth.stack_input(T, hq, d, seed=44)
    o = rng.standard_normal((T, hq, d)).astype(np.float16)
    _, wo = synth.stack_weights(1, hq, hkv, d, seed=45)
    xd = _dev(x)
    tm.tilemix_stack_out_residual(_dev(o), _dev(wo[0]), xd, hq, hkv, d)
    torch.cuda.synchronize()
    got = xd.cpu().numpy().astype(np.float64)
    ref = oracle.stack_out_residual(x, o, wo[0], hq, hkv, d)
    og = np.abs(o.astype(np.float64)).reshape(T, hkv, W)
    absum = np.stack([og[:, g] @ np.abs(wo[0, g].astype(np.float64)).T for g in range(hkv)], axis=1)
    bound = _gamma(W + 1) * (np.abs(x.astype(np.float64)) + absum.reshape(T, -1))
    assert np.all(np.abs(got - ref) <= bound)


def _run_stack(lens, hq, hkv, d, template, cov, n_layers, seed, gain_qk=1.0):
    cu = synth.cu_seqlens_of(lens)
    T = int(cu[-1])
    wqkv, wo = synth.stack_weights(n_layers, hq, hkv, d, seed=seed, gain_qk=gain_qk)
    x0 = synth.stack_input(T, hq, d, seed=seed + 1)
    st = tm.TileMixStack(cu, hq, hkv, d, template, cov)
    st.set_weights(_dev(wqkv), _dev(wo))
    x = _dev(x0)
    snaps = st.forward(x, record=set(range(1, n_layers + 1)))
    torch.cuda.synchronize()
    # the oracle takes its own routing words (the library's are bit-exact with them)
    words = oracle.routing_words(list(lens), hkv, template, cov)[0]
    assert np.array_equal(st.words, words)
    return cu, x0, wqkv, wo, words, {l: s.cpu().numpy().astype(np.float64) for l, s in snaps.items()}


def _wo_bounds(wo, hq, hkv, d):
    """Per-channel max bound and mean bound of Wo applied to an attention
    error within the prefill bars."""
    a = np.abs(wo.astype(np.float64))          # [Hkv, W, W]
    per_n = ATTN_MAX * a.sum(axis=2).reshape(-1)
    mean = ATTN_MEAN * a.shape[2] * a.mean()
    return per_n, mean


@pytest.mark.parametrize("lens,hq,hkv,d,template,cov", [
    ([300, 77, 0, 129, 1, 64], 6, 2, 64, "sptrans", 7500),
    ([300, 77, 0, 129, 1, 64], 6, 2, 64, "band", 0),
    ([513, 200], 3, 1, 128, "rowrandom", 5000),
    ([260, 131], 24, 8, 128, "sptrans", 10000),
    ([190, 5], 28, 4, 128, "bigbird", 2500)])
def test_one_layer(lens, hq, hkv, d, template, cov):
    _log(f"stack one layer lens={lens} hq={hq} hkv={hkv} d={d} {template} {cov}")
    cu, x0, wqkv, wo, words, snaps = _run_stack(lens, hq, hkv, d, template, cov, 1, seed=46)
    ref = oracle.stack_layer(x0, wqkv[0], wo[0], words, cu, hq, hkv, d)
    err = np.abs(snaps[1] - ref)
    per_n, mean = _wo_bounds(wo[0], hq, hkv, d)
    assert np.all(err <= per_n[None, :] + _gamma(64) * np.abs(ref)), err.max()
    assert err.mean() <= mean


@pytest.mark.parametrize("template,cov", [("sptrans", 7500), ("band", 0), ("rowrandom", 10000)])
def test_three_layers(template, cov):
    lens, hq, hkv, d, n = [300, 77, 129, 1], 6, 2, 64, 3
    _log(f"stack three layers {template} {cov}")
    cu, x0, wqkv, wo, words, snaps = _run_stack(lens, hq, hkv, d, template, cov, n, seed=47)
    clean = oracle.stack_forward(x0, wqkv, wo, words, cu, hq, hkv, d)
    T = x0.shape[0]
    rng = np.random.default_rng(48)
    offs_max = [ATTN_MAX * rng.choice([-1.0, 1.0], size=(T, hq, d)) for _ in range(n)]
    offs_mean = [ATTN_MEAN * rng.choice([-1.0, 1.0], size=(T, hq, d)) for _ in range(n)]
    pmax = oracle.stack_forward(x0, wqkv, wo, words, cu, hq, hkv, d, attn_offsets=offs_max)
    pmean = oracle.stack_forward(x0, wqkv, wo, words, cu, hq, hkv, d, attn_offsets=offs_mean)
    for l in range(n):
        err = np.abs(snaps[l + 1] - clean[l])
        assert err.max() <= 2 * np.abs(pmax[l] - clean[l]).max(), (l, err.max())
        assert err.mean() <= 2 * np.abs(pmean[l] - clean[l]).mean(), (l, err.mean())


def test_layer_llama3b_l4k_sampled():
    # one layer at the 3B shape (8 x 4096 tokens, Hq 24, Hkv 8, d 128):
    # compared on sampled query tiles of sampled streams, each computed by
    # the oracle from its own sequence and stream
    spec = synth.WORKLOADS["llama3b_l4k"]
    lens, hq, hkv, d = spec["seqlens"], spec["hq"], spec["hkv"], spec["d"]
    _log("stack one layer llama3b_l4k sampled")
    cu, x0, wqkv, wo, words, snaps = _run_stack(lens, hq, hkv, d, "sptrans", 7500, 1, seed=49)
    W = oracle.stack_width(hq, hkv, d)
    r = hq // hkv
    per_n, _ = _wo_bounds(wo[0], hq, hkv, d)
    qt_off = np.concatenate([[0], np.cumsum([-(-L // 128) for L in lens])])
    for s, g, rows in ((0, 0, [0, 13, 31]), (3, 5, [1, 30]), (7, 7, [31])):
        a, b = int(cu[s]), int(cu[s + 1])
        xs = x0[a:b, g * W:(g + 1) * W]
        ws = words[g:g + 1, qt_off[s]:qt_off[s + 1]]
        u = oracle.stack_rms_norm(xs, 1)
        q, k, v = oracle.stack_qkv(u, wqkv[0, g:g + 1], r, 1, d)
        scu = [0, b - a]
        q_i8, q_s = oracle.quantize_blocks(q, scu, 128)
        k_i8, k_s = oracle.quantize_blocks(k, scu, 64)
        o = oracle.prefill_attention(q, k, v, q_i8, k_i8, q_s, k_s, ws, scu, r, 1,
                                     rows=[(0, h, rr) for h in range(r) for rr in rows])
        ref = oracle.stack_out_residual(xs, o.astype(np.float16), wo[0, g:g + 1], r, 1, d)
        for rr in rows:
            t0, t1 = 128 * rr, min(128 * rr + 128, b - a)
            got = snaps[1][a + t0:a + t1, g * W:(g + 1) * W]
            err = np.abs(got - ref[t0:t1])
            assert np.all(err <= per_n[None, g * W:(g + 1) * W] + _gamma(64) * np.abs(ref[t0:t1])), \
                (s, g, rr, err.max())
