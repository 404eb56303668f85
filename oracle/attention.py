"""Brute-force causal attention in float64, for the Theorem 3 equivalence check.

Source: the InferScale review (arXiv 2607.27090), "Core claim" and "Circularity
Check" (Theorem 3: for causal decoders, injecting precomputed KV at the
intended positions equals prompt-injecting the same tokens), and reference [1]
(grouped-query attention: several query heads share one KV head).

Readings: scores q.k * scale with scale = 1/sqrt(D); a query at position p
attends to every key at position <= p; softmax in float64; query head h reads
KV head h // (Hq / Hkv).
"""

import math

import numpy as np


def causal_gqa(q, q_pos, k, v, k_pos, scale=None):
    """q[Tq][Hq][D] (already rotated), k/v[Tk][Hkv][D]; positions are integers.

    Returns float64 out[Tq][Hq][D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((tq, hq, d), dtype=np.float64)
    k_pos = np.asarray(k_pos)
    for i in range(tq):
        seen = k_pos <= q_pos[i]
        for h in range(hq):
            g = h // group
            scores = (k[seen, g, :] @ q[i, h]) * scale
            w = np.exp(scores - scores.max())
            w /= w.sum()
            out[i, h] = w @ v[seen, g, :]
    return out
