"""fp64 reference for exact scaled-dot-product attention (test infrastructure only).

Layout: ``q [B, Hq, Sq, D]``, ``k, v [B, Hkv, Sk, D]``; outputs ``o [B, Hq, Sq, D]``
and ``lse [B, Hq, Sq]``.  Inputs may be any real numpy dtype; every value is
upcast to float64 before use, so bf16/fp32 inputs enter exactly.

Readings of the pages that this file takes (the pages print no formula):

* Score: ``s_ij = scale * <q_i, k_j>``, scale applied before the softmax.
* Log-sum-exp: natural log, scale included: ``lse_i = ln sum_{visible j} exp(s_ij)``.
* GQA: query head ``h`` reads key/value head ``h // (Hq // Hkv)`` (consecutive
  grouping).  GQA is not on the pages; it is part of the hot-path scope.
* Causal alignment when ``Sq != Sk``: bottom-right, i.e. query ``i`` sits at key
  position ``c = i + (Sk - Sq)`` and sees keys ``j <= c``.
* Sliding window: ``window = w >= 0`` is a half width, key ``j`` visible iff
  ``|c - j| <= w`` (inclusive, ``2w + 1`` keys for interior rows); with causal
  as well, ``0 <= c - j <= w``.  ``window < 0`` means no window.  Local
  attention -- each token attends only to its neighbours -- is point 1 of the
  thread on extending LLM context (web3.ouzhyi.biz).
* A row with no visible key has ``o = 0`` and ``lse = -inf``.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def visibility(rows, Sq: int, Sk: int, causal: bool, window: int, cols=None) -> np.ndarray:
    """Boolean mask ``vis[r, j]``: may query ``rows[r]`` attend to key ``cols[j]``?

    ``vis(i, j) = [not causal or j <= c] and [window < 0 or |c - j| <= window]``
    with ``c = i + (Sk - Sq)`` (bottom-right alignment).
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = (np.arange(Sk, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64))[None, :]
    c = i + (Sk - Sq)
    vis = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        vis &= j <= c
    if window >= 0:
        vis &= np.abs(c - j) <= window
    return vis


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(s: np.ndarray, vis: np.ndarray, vv: np.ndarray):
    """Two-pass softmax of masked score rows, then the weighted sum of value rows.

    Returns ``(o, lse)``; fully masked rows give ``o = 0``, ``lse = -inf``.
    """
    s = np.where(vis, s, NEG_INF)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[:, None])  # masked entries: exp(-inf) = 0
    l = e.sum(axis=1)
    o = e @ vv
    o = np.where(live[:, None], o / np.where(live, l, 1.0)[:, None], 0.0)
    lse = np.where(live, m_safe + np.log(np.where(live, l, 1.0)), NEG_INF)
    return o, lse


def attention(q, k, v, scale: float, causal: bool = False, window: int = -1,
              rows=None, block: int = 256):
    """Exact attention, two-pass softmax, fp64.

    ``rows`` optionally restricts the computation to some query indices
    (same for every batch and head); the result then has ``len(rows)`` rows.
    Work is blocked over query rows; each block only multiplies against the
    key range its mask can reach, found from the mask itself.  Blocking and
    range restriction do not change the definition.
    """
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    assert v.shape == k.shape and Bk == B and Dk == D
    assert Hkv > 0 and Hq % Hkv == 0
    G = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    o = np.zeros((B, Hq, R, D), dtype=np.float64)
    lse = np.full((B, Hq, R), NEG_INF, dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            kk = _f64(k[b, g])
            vv = _f64(v[b, g])
            for h in range(g * G, (g + 1) * G):
                for r0 in range(0, R, block):
                    rr = rows[r0:r0 + block]
                    vis = visibility(rr, Sq, Sk, causal, window)
                    reach = np.flatnonzero(vis.any(axis=0))
                    if reach.size == 0:
                        continue  # every row of the block is fully masked
                    lo, hi = int(reach[0]), int(reach[-1]) + 1
                    qq = _f64(q[b, h, rr])
                    s = scale * (qq @ kk[lo:hi].T)
                    ob, lb = _softmax_rows(s, vis[:, lo:hi], vv[lo:hi])
                    o[b, h, r0:r0 + block] = ob
                    lse[b, h, r0:r0 + block] = lb
    return o, lse


def attention_online(q, k, v, scale: float, causal: bool = False, window: int = -1,
                     tile: int = 64):
    """The same quantity by the online softmax: keys arrive ``tile`` at a time.

    Per query row keep the running max ``m``, running sum ``l`` and the
    unnormalised accumulator ``acc``.  On each new tile:
    ``m' = max(m, max s)``, ``alpha = exp(m - m')``, ``p = exp(s - m')``,
    ``l = alpha l + sum p``, ``acc = alpha acc + p v``.  At the end
    ``o = acc / l`` and ``lse = m + ln l``.  (FlashAttention explainer,
    "Technical insight": partial results rescaled as new blocks arrive, so the
    final normalisation is exact without seeing all scores at once.)
    """
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    G = Hq // Hkv
    o = np.zeros((B, Hq, Sq, D))
    lse = np.full((B, Hq, Sq), NEG_INF)
    rows = np.arange(Sq)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            qq = _f64(q[b, h])
            m = np.full(Sq, NEG_INF)
            l = np.zeros(Sq)
            acc = np.zeros((Sq, D))
            for t0 in range(0, Sk, tile):
                cols = np.arange(t0, min(t0 + tile, Sk))
                kk = _f64(k[b, g, t0:t0 + tile])
                vv = _f64(v[b, g, t0:t0 + tile])
                vis = visibility(rows, Sq, Sk, causal, window, cols=cols)
                s = np.where(vis, scale * (qq @ kk.T), NEG_INF)
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)
                m_ref = np.where(live, m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
                p = np.exp(s - m_ref[:, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ vv
                m = m_new
            live = l > 0
            o[b, h] = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
            lse[b, h] = np.where(live, m + np.log(np.where(live, l, 1.0)), NEG_INF)
    return o, lse


def decode(q, kcache, vcache, scale: float):
    """Single-token decode: ``q [B, Hq, D]`` against every cached key.

    The exact result, i.e. ``attention`` with ``Sq = 1``, no causal mask and
    no window (the new token sees the whole cache).
    """
    o, lse = attention(q[:, :, None, :], kcache, vcache, scale)
    return o[:, :, 0, :], lse[:, :, 0]


# ----------------------------------------------------------------------------
# Split-KV partials and their log-sum-exp merge (Tree Attention abstract: the
# reduction along the sequence axis can be computed in parallel as a tree).
# A partial is (m, l, acc): m the max scaled score of the chunk, l the sum of
# exp(s - m), acc the sum of exp(s - m) * v.  Over rows, m and l are [R] and
# acc is [R, D].
# ----------------------------------------------------------------------------

def split_bounds(Sk: int, num_splits: int):
    """Chunk ``c`` covers keys ``[c*L, min((c+1)*L, Sk))`` with ``L = ceil(Sk/ns)``.

    Chunks past the end are empty.
    """
    L = -(-Sk // num_splits)
    return [(min(c * L, Sk), min((c + 1) * L, Sk)) for c in range(num_splits)]


def split_partials(q_rows, k_rows, v_rows, scale: float, num_splits: int):
    """Partials of query rows ``q_rows [R, D]`` over ``num_splits`` key chunks.

    All keys are visible (decode).  An empty chunk yields the identity
    ``(-inf, 0, 0)``.
    """
    qq = _f64(q_rows)
    kk = _f64(k_rows)
    vv = _f64(v_rows)
    R, D = qq.shape
    parts = []
    for lo, hi in split_bounds(kk.shape[0], num_splits):
        if hi <= lo:
            parts.append((np.full(R, NEG_INF), np.zeros(R), np.zeros((R, D))))
            continue
        s = scale * (qq @ kk[lo:hi].T)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        parts.append((m, e.sum(axis=1), e @ vv[lo:hi]))
    return parts


def merge(a, b):
    """The log-sum-exp merge of two partials.

    ``(m1,l1,a1) + (m2,l2,a2) = (M, l1 e^{m1-M} + l2 e^{m2-M}, a1 e^{m1-M} + a2 e^{m2-M})``
    with ``M = max(m1, m2)``; a side with ``m = -inf`` contributes nothing.
    """
    m1, l1, a1 = a
    m2, l2, a2 = b
    M = np.maximum(m1, m2)
    live = np.isfinite(M)
    M_ref = np.where(live, M, 0.0)
    f1 = np.where(np.isfinite(m1), np.exp(m1 - M_ref), 0.0)
    f2 = np.where(np.isfinite(m2), np.exp(m2 - M_ref), 0.0)
    return M, l1 * f1 + l2 * f2, a1 * f1[:, None] + a2 * f2[:, None]


def combine(parts, tree: str = "balanced", rng=None):
    """Reduce a list of partials with ``merge``.

    ``tree``: ``"balanced"`` pairs neighbours level by level (an odd element
    passes up unmerged); ``"left"`` and ``"right"`` are the two sequential
    folds; ``"random"`` merges two randomly chosen pool members until one is
    left (needs ``rng``).  All are equal in exact arithmetic.
    """
    parts = list(parts)
    if tree == "balanced":
        while len(parts) > 1:
            nxt = [merge(parts[i], parts[i + 1]) for i in range(0, len(parts) - 1, 2)]
            if len(parts) % 2:
                nxt.append(parts[-1])
            parts = nxt
        return parts[0]
    if tree == "left":
        acc = parts[0]
        for p in parts[1:]:
            acc = merge(acc, p)
        return acc
    if tree == "right":
        acc = parts[-1]
        for p in reversed(parts[:-1]):
            acc = merge(p, acc)
        return acc
    if tree == "random":
        while len(parts) > 1:
            i, j = rng.choice(len(parts), size=2, replace=False)
            merged = merge(parts[i], parts[j])
            parts = [p for t, p in enumerate(parts) if t not in (i, j)] + [merged]
        return parts[0]
    raise ValueError(tree)


def finish(part):
    """Normalise a fully merged partial: ``o = acc / l``, ``lse = m + ln l``."""
    m, l, acc = part
    live = l > 0
    o = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
    lse = np.where(live, m + np.log(np.where(live, l, 1.0)), NEG_INF)
    return o, lse
