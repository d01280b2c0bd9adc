"""Scalar pure-Python attention for tiny inputs (pin for the fp64 oracle).

Independent of ``oracle/``: nested lists, ``math.exp`` and ``math.fsum``; the
visible key set of a query is enumerated key by key from the mask rules
(bottom-right causal alignment, inclusive half-width window, consecutive GQA
grouping), and the softmax is taken over that set.
"""

from __future__ import annotations

import math


def brute_attention(q, k, v, scale, causal=False, window=-1):
    """q: [B][Hq][Sq][D], k/v: [B][Hkv][Sk][D] nested lists of floats.

    Returns (o [B][Hq][Sq][D], lse [B][Hq][Sq]).
    """
    B, Hq, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0]) if q[0][0] else 0
    Hkv, Sk = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    o_all, lse_all = [], []
    for b in range(B):
        o_b, lse_b = [], []
        for h in range(Hq):
            kv_head = h // group
            o_h, lse_h = [], []
            for i in range(Sq):
                pos = i + Sk - Sq
                keys = []
                for j in range(Sk):
                    if causal and j > pos:
                        continue
                    if window >= 0 and abs(pos - j) > window:
                        continue
                    keys.append(j)
                if not keys:
                    o_h.append([0.0] * D)
                    lse_h.append(-math.inf)
                    continue
                scores = [scale * math.fsum(q[b][h][i][d] * k[b][kv_head][j][d] for d in range(D))
                          for j in keys]
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                z = math.fsum(w)
                o_h.append([math.fsum(w[t] * v[b][kv_head][j][d] for t, j in enumerate(keys)) / z
                            for d in range(D)])
                lse_h.append(top + math.log(z))
            o_b.append(o_h)
            lse_b.append(lse_h)
        o_all.append(o_b)
        lse_all.append(lse_b)
    return o_all, lse_all
