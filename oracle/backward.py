"""fp64 reference for the gradient of exact attention (test infrastructure only).

The pages name training as a use of the fused method (FlashAttention
explainer, "Overview": long-context training and inference made faster;
FlashAttention-3 article, "Benefits of FlashAttention-3": faster training) but
print no backward algorithm.  The gradient is therefore taken as the plain
definition: the derivative of ``attention`` (``oracle/attention.py``, same
readings for scale, masks, GQA and empty rows) written out by the chain rule.

With ``s = scale * q k^T`` (visible pairs only), ``P = softmax_rows(s)`` and
``o = P v``, for an upstream gradient ``do``:

* ``dv = P^T do``
* ``dP = do v^T`` and ``delta_i = sum_d do[i, d] * o[i, d]`` (= ``sum_j P_ij dP_ij``)
* ``ds = P * (dP - delta)`` (masked pairs have ``P = 0``, so ``ds = 0`` there)
* ``dq = scale * ds k`` and ``dk = scale * ds^T q``

Under GQA a key/value head feeds ``Hq / Hkv`` query heads; its ``dk`` and
``dv`` are the sums over those heads.  A query row with no visible key has
``o = 0`` and contributes nothing.  Nothing here is fused, blocked or
reordered beyond the definition; ``tests/pins_backward.py`` pins it against
central finite differences of ``attention`` and against torch autograd.
"""

from __future__ import annotations

import numpy as np

from .attention import visibility

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_backward(q, k, v, do, scale: float, causal: bool = False, window: int = -1):
    """Gradients ``(dq, dk, dv)`` of ``sum(do * attention(q, k, v))``, fp64.

    Shapes: ``q, do [B, Hq, Sq, D]``, ``k, v [B, Hkv, Sk, D]``; the outputs
    have the shapes of ``q``, ``k`` and ``v``.  Also returns ``delta [B, Hq, Sq]``
    (the row sums ``sum_d do * o`` the gradient uses).
    """
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    assert v.shape == k.shape and do.shape == q.shape
    G = Hq // Hkv
    dq = np.zeros((B, Hq, Sq, D))
    dk = np.zeros((B, Hkv, Sk, D))
    dv = np.zeros((B, Hkv, Sk, D))
    delta = np.zeros((B, Hq, Sq))
    vis = visibility(np.arange(Sq), Sq, Sk, causal, window)
    live = vis.any(axis=1)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qq, kk, vv, dd = _f64(q[b, h]), _f64(k[b, g]), _f64(v[b, g]), _f64(do[b, h])
            s = np.where(vis, scale * (qq @ kk.T), NEG_INF)
            m = np.where(live, s.max(axis=1) if Sk else 0.0, 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            l = e.sum(axis=1)
            p = e / np.where(live, l, 1.0)[:, None]          # rows with no key: all zero
            o = p @ vv
            dv[b, g] += p.T @ dd
            dp = dd @ vv.T
            dl = (dd * o).sum(axis=1)
            delta[b, h] = dl
            ds = p * (dp - dl[:, None])
            dq[b, h] = scale * (ds @ kk)
            dk[b, g] += scale * (ds.T @ qq)
    return dq, dk, dv, delta
