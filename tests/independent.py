"""Independent formulations used to pin the oracle (not the oracle itself).

Each helper states the same quantity as the oracle by a different route:
textbook softmax attention, attention on block-dequantised operands, exact
rational IEEE rounding.  None of them imports the oracle's arithmetic.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax with -inf entries excluded (fp64)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def naive_causal_attention(q, k, v, cu_seqlens, hq, hkv):
    """Textbook causal attention per sequence and head, fp64, scale 1/sqrt(d)."""
    cu = [int(c) for c in cu_seqlens]
    T, _, d = q.shape
    out = np.zeros((T, hq, d))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        n = b - a
        mask = np.tril(np.ones((n, n), dtype=bool))
        for h in range(hq):
            kv = h * hkv // hq
            qq = q[a:b, h].astype(np.float64)
            kk = k[a:b, kv].astype(np.float64)
            vv = v[a:b, kv].astype(np.float64)
            s_ = (qq @ kk.T) / math.sqrt(d)
            s_ = np.where(mask, s_, -np.inf)
            out[a:b, h] = softmax_rows(s_) @ vv
    return out


def dequantized(x_i8, scales, cu_seqlens, block):
    """Block-dequantised operand x_i8 * s (fp64), tiles numbered per sequence."""
    cu = [int(c) for c in cu_seqlens]
    out = np.zeros(x_i8.shape)
    tile = 0
    for s in range(len(cu) - 1):
        for b0 in range(cu[s], cu[s + 1], block):
            b1 = min(b0 + block, cu[s + 1])
            out[b0:b1] = x_i8[b0:b1].astype(np.float64) * scales[:, tile][None, :, None].astype(np.float64)
            tile += 1
    return out


def element_route_bits(words, cu_seqlens, g, seq, kv, n):
    """n x n matrix of routing bits for one sequence, looked up per element."""
    cu = [int(c) for c in cu_seqlens]
    row_off = sum(-(-(cu[i + 1] - cu[i]) // 128) for i in range(seq))
    bits = np.zeros((n, n), dtype=bool)
    for i in range(n):
        w = int(words[kv, row_off + i // 128])
        for j in range(n):
            bits[i, j] = (w >> ((j // 64) // int(g[seq]))) & 1
    return bits


def mixed_closed_form(q, k, v, q_i8, k_i8, q_scale, k_scale, words, g, cu_seqlens, hq, hkv):
    """Attention on the per-element mixed score matrix
    S_ij = (bit ? qhat_i . khat_j : q_i . k_j) / sqrt(d), where qhat/khat are the
    block-dequantised operands -- algebraically the INT8 path (acc * s_q * s_k)."""
    cu = [int(c) for c in cu_seqlens]
    T, _, d = q.shape
    qh = dequantized(q_i8, q_scale, cu, 128)
    kh = dequantized(k_i8, k_scale, cu, 64)
    out = np.zeros((T, hq, d))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        n = b - a
        if n == 0:
            continue
        mask = np.tril(np.ones((n, n), dtype=bool))
        for h in range(hq):
            kv = h * hkv // hq
            bits = element_route_bits(words, cu, g, s, kv, n)
            s16 = q[a:b, h].astype(np.float64) @ k[a:b, kv].astype(np.float64).T
            s8 = qh[a:b, h] @ kh[a:b, kv].T
            sc = np.where(bits, s8, s16) / math.sqrt(d)
            sc = np.where(mask, sc, -np.inf)
            out[a:b, h] = softmax_rows(sc) @ v[a:b, kv].astype(np.float64)
    return out


def round_fraction_to_f32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest IEEE binary32 value, ties to even
    (normal range only; enough for quantiser quotients and scales)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    ax = abs(x)
    e = math.floor(math.log2(ax))
    # fix e so that 2^e <= ax < 2^(e+1)
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = ax / ulp                       # in [2^23, 2^24)
    fl = math.floor(m)
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def round_half_even(x: Fraction) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl
