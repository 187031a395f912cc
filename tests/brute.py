"""Scalar brute-force attention shared by the CPU pin tests.

It shares nothing with the oracle (no NumPy matrix products, no vectorised
softmax): RoPE by complex multiplication, scores and sums with math.fsum.
"""
import cmath
import math

import numpy as np

ALIBI_GEOMETRIC = 1
ALIBI_PAGE1 = 2


def brute_attention(q, k, v, pos0, base, causal, alibi, q_offset=0, window=0):
    """Scalar loops. RoPE as multiplication of (x0 + i x1) by e^{i p theta}
    (the complex form of the RoPE equation on the transformer-from-scratch page);
    the softmax as exp / fsum without max subtraction; heads grouped by repetition.
    Query row i is token q_offset + i of the key sequence; with a window of W
    tokens it sees keys q_offset + i - W + 1 .. q_offset + i."""
    B, H, Tq, hd = q.shape
    KV, T = k.shape[1], k.shape[2]
    kv_of = [g for g in range(KV) for _ in range(H // KV)]
    if alibi == ALIBI_GEOMETRIC:
        slope = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]
    elif alibi == ALIBI_PAGE1:
        slope = [1.0 / 2.0 ** (2.0 * (h + 1) / H) for h in range(H)]
    else:
        slope = [0.0] * H

    def rot(vec, p):
        if base == 0:
            return [float(x) for x in vec]
        outv = []
        for i in range(hd // 2):
            theta = base ** (-(2.0 * i) / hd)
            z = complex(vec[2 * i], vec[2 * i + 1]) * cmath.exp(1j * p * theta)
            outv += [z.real, z.imag]
        return outv

    out = np.zeros((B, H, Tq, hd))
    lse = np.zeros((B, H, Tq))
    for b in range(B):
        for h in range(H):
            g = kv_of[h]
            keys = [rot(k[b, g, j], pos0 + j) for j in range(T)]
            for r in range(Tq):
                i = q_offset + r
                qi = rot(q[b, h, r], pos0 + i)
                js = [j for j in range(T) if (j <= i or not causal) and (window == 0 or i - j < window)]
                sc = [math.fsum(a * c for a, c in zip(qi, keys[j])) / math.sqrt(hd) - slope[h] * abs(i - j)
                      for j in js]
                ex = [math.exp(s) for s in sc]
                z = math.fsum(ex)
                for d in range(hd):
                    out[b, h, r, d] = math.fsum(e * v[b, g, j, d] for e, j in zip(ex, js)) / z
                lse[b, h, r] = math.log(z)
    return out, lse
