"""Seeded synthetic workloads for TileMix prefill attention.

This module only draws inputs (shapes, value distributions, packing); it holds
none of the attention, routing or quantisation arithmetic.  Both the HIP path
and the CPU oracle consume exactly the bytes produced here.

Workloads stand in for the attention layers the TileMix pages measure
(LLaMA 3.2 3B: Hq=24, Hkv=8, d=128; Qwen-2-7B: Hq=28, Hkv=4, d=128) with
synthetic N(0,1) activations; the pages' own tasks (LongEval, LV-Eval) are not
used.  Recipe:

* ``rng = numpy.random.default_rng(seed)`` (PCG64);
* Q, K, V drawn as float32 standard normal, in that order, with shapes
  [T, Hq, d], [T, Hkv, d], [T, Hkv, d] (T = total packed tokens);
* when ``outliers`` is set, ``chan = rng.choice(d, 4, replace=False)`` and the
  same four channels of Q and K are multiplied by 10 (in float32);
* everything is then rounded to float16 (round-to-nearest-even).
"""

from __future__ import annotations

import numpy as np

# Template ids shared by every layer of the stack (C-ABI, binding, oracle).
TEMPLATE_IDS = {
    "band": 0,
    "global": 1,
    "rowrandom": 2,
    "alignedsparse": 3,
    "bigbird": 4,
    "sptrans": 5,
}
TEMPLATE_NAMES = {v: k for k, v in TEMPLATE_IDS.items()}

# Named workloads.  ``template``/``coverage_bp`` are the routing settings the
# workload is quoted with; sweeps override them.
WORKLOADS = {
    "tiny": dict(seqlens=[256], hq=1, hkv=1, d=64, outliers=False,
                 template="band", coverage_bp=5000),
    "llama3b_l1k": dict(seqlens=[1024] * 8, hq=24, hkv=8, d=128, outliers=True,
                        template="sptrans", coverage_bp=2500),
    "llama3b_l4k": dict(seqlens=[4096] * 8, hq=24, hkv=8, d=128, outliers=True,
                        template="sptrans", coverage_bp=7500),
    "llama3b_l8k": dict(seqlens=[8192] * 8, hq=24, hkv=8, d=128, outliers=True,
                        template="sptrans", coverage_bp=7500),
    "qwen2_7b_varlen": dict(seqlens=[65536, 16384, 8192, 4096, 1024, 1024], hq=28,
                            hkv=4, d=128, outliers=True, template="rowrandom",
                            coverage_bp=5000),
}


def cu_seqlens_of(seqlens) -> np.ndarray:
    """Prefix sums [0, L0, L0+L1, ...] as int32."""
    cu = np.zeros(len(seqlens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(seqlens, dtype=np.int64))
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("total token count does not fit int32")
    return cu.astype(np.int32)


def make_qkv(seqlens, hq: int, hkv: int, d: int, outliers: bool, seed: int = 0):
    """Draw packed fp16 Q, K, V ([T, H, d], token-major) and cu_seqlens."""
    cu = cu_seqlens_of(seqlens)
    t = int(cu[-1])
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((t, hq, d), dtype=np.float32)
    k = rng.standard_normal((t, hkv, d), dtype=np.float32)
    v = rng.standard_normal((t, hkv, d), dtype=np.float32)
    if outliers:
        chan = rng.choice(d, 4, replace=False)
        q[..., chan] *= np.float32(10.0)
        k[..., chan] *= np.float32(10.0)
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16), cu


def make_workload(name: str, seed: int = 0):
    """Inputs of a named workload: (q, k, v, cu_seqlens, spec dict)."""
    spec = dict(WORKLOADS[name])
    q, k, v, cu = make_qkv(spec["seqlens"], spec["hq"], spec["hkv"], spec["d"],
                           spec["outliers"], seed)
    return q, k, v, cu, spec


def lossless_blocks(seqlens, heads: int, d: int, block: int, seed: int = 0):
    """Values k * 2^-6 with integer k in [-127, 127] and one entry of +-127 per
    (block, head): blockwise absmax/127 quantisation reproduces them exactly."""
    cu = cu_seqlens_of(seqlens)
    rng = np.random.default_rng(seed)
    ints = rng.integers(-127, 128, size=(int(cu[-1]), heads, d))
    for s in range(len(seqlens)):
        start, end = int(cu[s]), int(cu[s + 1])
        for b0 in range(start, end, block):
            ints[b0, :, 0] = 127 * np.where(rng.random(heads) < 0.5, -1, 1)
    return (ints.astype(np.float32) * np.float32(2.0 ** -6)).astype(np.float16)


def lossless_blocks_pow2(seqlens, heads: int, d: int, block: int, seed: int = 0):
    """Like ``lossless_blocks`` but every (block, head) has its own
    power-of-two step 2^-e, e in [3, 9]: values k * 2^-e with one entry of
    +-127 * 2^-e, so each block's scale differs and is still reproduced
    exactly."""
    cu = cu_seqlens_of(seqlens)
    rng = np.random.default_rng(seed)
    ints = rng.integers(-127, 128, size=(int(cu[-1]), heads, d)).astype(np.float32)
    for s in range(len(seqlens)):
        start, end = int(cu[s]), int(cu[s + 1])
        for b0 in range(start, end, block):
            b1 = min(b0 + block, end)
            ints[b0, :, 0] = 127 * np.where(rng.random(heads) < 0.5, -1, 1)
            e = rng.integers(3, 10, size=heads).astype(np.float32)
            ints[b0:b1] *= np.exp2(-e)[None, :, None]
    return ints.astype(np.float16)


def decode_queries(q, cu_seqlens):
    """The decode query of each sequence: the row of ``q`` at position L - 1
    (the newest token), [B, H, d]; zeros for an empty sequence."""
    cu = [int(c) for c in cu_seqlens]
    out = np.zeros((len(cu) - 1,) + q.shape[1:], dtype=q.dtype)
    for s in range(len(cu) - 1):
        if cu[s + 1] > cu[s]:
            out[s] = q[cu[s + 1] - 1]
    return out


def make_qkv_local(seqlens, hq: int, hkv: int, d: int, seed: int = 0, amp: float = 1.5,
                   sink: float = 8.0):
    """Inputs whose attention has the structure real layers show: locality
    and a sink.  Q, K, V are drawn as in ``make_qkv`` (no outlier channels);
    then, per sequence-local position i, channels 2c, 2c+1 (c < 16) of Q and K
    gain amp * (cos, sin)(w_c i) with periods 32 * 2^(c/2) tokens, so q_i . k_j
    grows as |i - j| shrinks, and channel 32 gains 2 in every query and
    ``sink`` in each sequence's first key.  Rounded to float16."""
    cu = cu_seqlens_of(seqlens)
    rng = np.random.default_rng(seed)
    t = int(cu[-1])
    q = rng.standard_normal((t, hq, d), dtype=np.float32)
    k = rng.standard_normal((t, hkv, d), dtype=np.float32)
    v = rng.standard_normal((t, hkv, d), dtype=np.float32)
    pos = np.concatenate([np.arange(int(cu[s + 1] - cu[s])) for s in range(len(seqlens))]
                         + [np.zeros(0)]).astype(np.float64)
    for c in range(16):
        w = 2.0 * np.pi / (32.0 * 2.0 ** (c / 2.0))
        cs = (amp * np.cos(w * pos)).astype(np.float32)[:, None]
        sn = (amp * np.sin(w * pos)).astype(np.float32)[:, None]
        q[:, :, 2 * c] += cs
        q[:, :, 2 * c + 1] += sn
        k[:, :, 2 * c] += cs
        k[:, :, 2 * c + 1] += sn
    q[:, :, 32] += np.float32(2.0)
    for s in range(len(seqlens)):
        if cu[s + 1] > cu[s]:
            k[int(cu[s]), :, 32] += np.float32(sink)
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16), cu


def lossless_blocks_fp8(seqlens, heads: int, d: int, block: int, seed: int = 0):
    """Values that blockwise E4M3 quantisation reproduces exactly: every
    (block, head) holds E4M3 grid values (|v| >= 1) times 2^-e, e in
    [4, 9], with one entry of +-448 * 2^-e, so the scale is exactly 2^-e."""
    grid = np.array([(1.0 + m / 8.0) * 2.0 ** x for x in range(0, 9) for m in range(8)
                     if (1.0 + m / 8.0) * 2.0 ** x <= 448.0])
    cu = cu_seqlens_of(seqlens)
    rng = np.random.default_rng(seed)
    t = int(cu[-1])
    vals = grid[rng.integers(0, len(grid), size=(t, heads, d))] * np.where(rng.random((t, heads, d)) < 0.5, -1, 1)
    for s in range(len(seqlens)):
        start, end = int(cu[s]), int(cu[s + 1])
        for b0 in range(start, end, block):
            b1 = min(b0 + block, end)
            vals[b0, :, 0] = 448.0 * np.where(rng.random(heads) < 0.5, -1, 1)
            e = rng.integers(4, 10, size=heads).astype(np.float64)
            vals[b0:b1] *= np.exp2(-e)[None, :, None]
    return vals.astype(np.float16)


def stack_weights(n_layers: int, hq: int, hkv: int, d: int, seed: int = 0, gain_qk: float = 1.0):
    """Random weights of a synthetic attention stack: wqkv float16
    [n_layers, Hkv, W+2d, W] and wo float16 [n_layers, Hkv, W, W], W =
    (Hq/Hkv)*d.  Entries are N(0, 1/W) in float32 (the q and k rows times
    ``gain_qk``), drawn layer by layer (wqkv then wo), rounded to float16."""
    W = (hq // hkv) * d
    rng = np.random.default_rng(seed)
    wqkv = np.empty((n_layers, hkv, W + 2 * d, W), dtype=np.float16)
    wo = np.empty((n_layers, hkv, W, W), dtype=np.float16)
    sd = np.float32(1.0 / np.sqrt(W))
    for l in range(n_layers):
        a = rng.standard_normal((hkv, W + 2 * d, W), dtype=np.float32) * sd
        a[:, :W + d] *= np.float32(gain_qk)
        wqkv[l] = a.astype(np.float16)
        wo[l] = (rng.standard_normal((hkv, W, W), dtype=np.float32) * sd).astype(np.float16)
    return wqkv, wo


def stack_input(tokens: int, hq: int, d: int, seed: int = 0):
    """Initial hidden state of the stack: float32 N(0, 1), [tokens, Hq*d]."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((tokens, hq * d), dtype=np.float32)
