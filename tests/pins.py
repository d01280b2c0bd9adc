"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` takes the oracle module as its argument, so the same pins can
be run against deliberately broken copies of the oracle (see
``test_oracle_mutants.py``) to show that a plausible mistake fails one of them.

Sources of the expectations:
* FlashAttention explainer (aiunderstanding.org), "Deep dive" and FAQ: the
  tiled method computes exactly the values of standard attention.
* Same page, "Technical insight" and FAQ: the online softmax (running max and
  sum, rescaling as tiles arrive) gives the exact normalisation.
* Tree Attention abstract (express24.ir page): the reduction along the sequence
  axis can be computed as a tree -- the log-sum-exp merge is associative and
  commutative, so every split count and merge order gives the unsplit result;
  the same abstract derives attention as the gradient of a scalar energy.
* Thread on extending LLM context (web3.ouzhyi.biz), point 1: local attention
  lets a token attend to its neighbours only (window mask counts below).
* Closed forms of the softmax itself (uniform scores -> mean, one key ->
  that key, a dominant key -> its value) and an independent library (torch
  SDPA) for a cross-check.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from brute_force import brute_attention

MASKS = [(False, -1), (True, -1), (False, 0), (False, 2), (True, 2), (True, 0)]
TINY_SHAPES = [  # B, Hq, Hkv, Sq, Sk, D
    (1, 1, 1, 5, 5, 3),
    (2, 4, 2, 3, 7, 4),
    (1, 2, 1, 6, 4, 2),   # Sq > Sk: causal rows before the first key are empty
    (1, 1, 1, 1, 8, 4),
    (1, 2, 2, 8, 8, 1),
]


def _qkv(rng, B, Hq, Hkv, Sq, Sk, D):
    return (rng.standard_normal((B, Hq, Sq, D)), rng.standard_normal((B, Hkv, Sk, D)),
            rng.standard_normal((B, Hkv, Sk, D)))


def _same_lse(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.array_equal(np.isneginf(a), np.isneginf(b)), "fully-masked rows differ"
    fin = np.isfinite(a)
    assert np.all(np.isfinite(b) == fin)
    np.testing.assert_allclose(a[fin], b[fin], rtol=0, atol=tol)


def pin_brute_force(O):
    """P1: the vectorised oracle equals scalar pure-Python loops (all masks, GQA)."""
    rng = np.random.default_rng(101)
    for shape in TINY_SHAPES:
        for causal, window in MASKS:
            q, k, v = _qkv(rng, *shape)
            scale = float(rng.uniform(0.2, 1.5))
            o, lse = O.attention(q, k, v, scale, causal, window)
            ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal, window)
            np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
            _same_lse(lse, lb, 1e-12)


def pin_online_equals_two_pass(O):
    """P2: online softmax with tile sizes 1, 3, 16 and Sk equals the two-pass form."""
    rng = np.random.default_rng(202)
    for shape in [(1, 2, 1, 9, 13, 5), (2, 2, 2, 16, 16, 8), (1, 1, 1, 4, 11, 3)]:
        for causal, window in MASKS:
            q, k, v = _qkv(rng, *shape)
            o, lse = O.attention(q, k, v, 0.6, causal, window)
            for tile in (1, 3, 16, shape[4]):
                oo, lo = O.attention_online(q, k, v, 0.6, causal, window, tile=tile)
                np.testing.assert_allclose(oo, o, rtol=0, atol=1e-12)
                _same_lse(lo, lse, 1e-12)


def pin_split_tree_equals_unsplit(O):
    """P3: split partials merged by any tree, in any order, equal unsplit decode."""
    rng = np.random.default_rng(303)
    B, Hq, Hkv, Sk, D = 2, 4, 2, 37, 6
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Hkv, Sk, D))
    vc = rng.standard_normal((B, Hkv, Sk, D))
    scale = 0.45
    o_ref, lse_ref = O.decode(q, kc, vc, scale)
    G = Hq // Hkv
    for ns in (1, 2, 3, 7, 16, 36, 37):
        for b in range(B):
            for h in range(Hq):
                parts = O.split_partials(q[b, h][None], kc[b, h // G], vc[b, h // G], scale, ns)
                assert len(parts) == ns
                for tree in ("balanced", "left", "right", "random"):
                    order = rng.permutation(ns) if tree != "left" else np.arange(ns)
                    merged = O.combine([parts[i] for i in order], tree=tree, rng=rng)
                    o, lse = O.finish(merged)
                    np.testing.assert_allclose(o[0], o_ref[b, h], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(lse[0], lse_ref[b, h], rtol=0, atol=1e-12)


def pin_merge_algebra(O):
    """The merge has the empty chunk as identity and is commutative and associative."""
    rng = np.random.default_rng(404)
    R, D = 3, 4

    def rand_part():
        m = rng.normal(size=R) * 3
        return m, rng.uniform(0.5, 4.0, size=R), rng.normal(size=(R, D))

    ident = (np.full(R, -np.inf), np.zeros(R), np.zeros((R, D)))
    a, b, c = rand_part(), rand_part(), rand_part()
    for x, y in [(O.merge(a, ident), a), (O.merge(ident, a), a)]:
        for u, w in zip(x, y):
            np.testing.assert_allclose(u, w, rtol=1e-15, atol=0)
    e = O.merge(ident, ident)
    assert np.all(np.isneginf(e[0])) and np.all(e[1] == 0) and np.all(e[2] == 0)
    ab, ba = O.merge(a, b), O.merge(b, a)
    for u, w in zip(ab, ba):
        np.testing.assert_allclose(u, w, rtol=1e-14, atol=0)
    left, right = O.merge(O.merge(a, b), c), O.merge(a, O.merge(b, c))
    for u, w in zip(left, right):
        np.testing.assert_allclose(u, w, rtol=1e-13, atol=0)
    # merging a chunk with itself doubles l and acc and keeps m
    aa = O.merge(a, a)
    np.testing.assert_allclose(aa[0], a[0], rtol=0, atol=0)
    np.testing.assert_allclose(aa[1], 2 * a[1], rtol=1e-15)
    np.testing.assert_allclose(aa[2], 2 * a[2], rtol=1e-15)


def _uniform_cases():
    """(Sq, Sk, causal, window, keys visible to row i as a closed form)."""
    def causal_square(i, S, w):
        return list(range(0, i + 1))

    def window_square(i, S, w):
        return list(range(i - min(i, w), i + min(S - 1 - i, w) + 1))

    def causal_window_square(i, S, w):
        return list(range(i - min(i, w), i + 1))

    return [
        (9, 9, True, -1, lambda i: causal_square(i, 9, -1)),
        (9, 9, False, 2, lambda i: window_square(i, 9, 2)),
        (12, 12, False, 0, lambda i: window_square(i, 12, 0)),
        (12, 12, False, 64, lambda i: window_square(i, 12, 64)),
        (9, 9, True, 2, lambda i: causal_window_square(i, 9, 2)),
        (5, 9, True, -1, lambda i: list(range(0, i + 4 + 1))),   # bottom-right: row i at key i+4
        (7, 7, False, -1, lambda i: list(range(7))),
    ]


def pin_uniform_scores(O):
    """P4: with q = 0 every visible score is 0: o is the mean of the visible v rows
    and lse = ln(number visible).  Counts are the closed forms
    i+1 (causal), min(i,w)+min(S-1-i,w)+1 (window), min(i,w)+1 (both)."""
    rng = np.random.default_rng(505)
    for Sq, Sk, causal, window, keys_of in _uniform_cases():
        D = 3
        q = np.zeros((1, 1, Sq, D))
        k = rng.standard_normal((1, 1, Sk, D))
        v = rng.standard_normal((1, 1, Sk, D))
        o, lse = O.attention(q, k, v, 0.9, causal, window)
        for i in range(Sq):
            keys = keys_of(i)
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, keys].mean(axis=0), rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[0, 0, i], math.log(len(keys)), rtol=0, atol=1e-14)


def pin_window_count_at_64(O):
    """The configured encoder window (half width 64) gives 129 keys to interior rows."""
    Sq = Sk = 300
    q = np.zeros((1, 1, Sq, 2))
    k = np.ones((1, 1, Sk, 2))
    v = np.ones((1, 1, Sk, 2))
    _, lse = O.attention(q, k, v, 1.0, False, 64)
    counts = np.rint(np.exp(lse[0, 0])).astype(int)
    assert counts[150] == 129 and counts[0] == 65 and counts[-1] == 65 and counts[64] == 129


def pin_kv_permutation(O):
    """P5: without causal mask or window, permuting (k, v) rows jointly changes nothing."""
    rng = np.random.default_rng(606)
    q, k, v = _qkv(rng, 2, 4, 2, 6, 19, 5)
    o, lse = O.attention(q, k, v, 0.7)
    perm = rng.permutation(19)
    o2, lse2 = O.attention(q, k[:, :, perm], v[:, :, perm], 0.7)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def pin_special_cases(O):
    """P6: one key -> that value, lse = its score; causal row 0 sees only key 0;
    a dominant key (k = c q, c large) takes all the weight."""
    rng = np.random.default_rng(707)
    q, k, v = _qkv(rng, 1, 2, 1, 4, 1, 5)
    o, lse = O.attention(q, k, v, 0.3)
    for h in range(2):
        for i in range(4):
            np.testing.assert_allclose(o[0, h, i], v[0, 0, 0], rtol=0, atol=1e-15)
            np.testing.assert_allclose(lse[0, h, i], 0.3 * float(q[0, h, i] @ k[0, 0, 0]), atol=1e-14)
    q, k, v = _qkv(rng, 1, 1, 1, 6, 6, 4)
    o, lse = O.attention(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], 0.5 * float(q[0, 0, 0] @ k[0, 0, 0]), atol=1e-14)
    q, k, v = _qkv(rng, 1, 1, 1, 1, 10, 8)
    star = 6
    k[0, 0, star] = 60.0 * q[0, 0, 0] / float(q[0, 0, 0] @ q[0, 0, 0])  # score 60 at scale 1
    o, lse = O.attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, star], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 0], 60.0, rtol=0, atol=1e-12)


def pin_overflow_safety(O):
    """P7: huge scores (scale 100) stay finite and match the scalar brute force;
    ln(max weight) <= lse - max score <= ln(n) for every row."""
    rng = np.random.default_rng(808)
    q, k, v = _qkv(rng, 1, 2, 2, 5, 7, 4)
    for causal, window in MASKS[:3]:
        o, lse = O.attention(q, k, v, 100.0, causal, window)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), 100.0, causal, window)
        np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-9)
        np.testing.assert_allclose(lse, np.array(lb), rtol=1e-13, atol=0)
    o, lse = O.attention(q, k, v, 100.0)
    s = 100.0 * np.einsum("bhid,bhjd->bhij", q, k)
    gap = lse - s.max(axis=-1)
    assert np.all(gap >= -1e-12) and np.all(gap <= math.log(7) + 1e-12)


def pin_gqa_equals_mha(O):
    """P8: GQA equals MHA with each k/v head repeated for its consecutive query heads."""
    rng = np.random.default_rng(909)
    for causal, window in MASKS:
        q, k, v = _qkv(rng, 2, 6, 2, 5, 9, 4)
        o, lse = O.attention(q, k, v, 0.8, causal, window)
        o2, lse2 = O.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.8, causal, window)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, lse2)
        # and differs from a wrong (modulo) grouping on generic data
        wrong = np.stack([k[:, h % 2] for h in range(6)], axis=1)
        o3, _ = O.attention(q, wrong, np.stack([v[:, h % 2] for h in range(6)], axis=1), 0.8, causal, window)
        assert np.abs(o3 - o).max() > 1e-3


def pin_energy_gradient(O):
    """P9: with F(z) = ln sum_j exp(s_j + z v_j[d]) (lse of augmented scores),
    dF/dz at z = 0 is o[d] (attention as the gradient of an energy; Tree
    Attention abstract).  Central differences in fp64."""
    rng = np.random.default_rng(1010)
    scale = 0.7
    eps = 1e-5
    for causal, window in [(False, -1), (True, -1), (False, 1)]:
        q, k, v = _qkv(rng, 1, 2, 1, 4, 6, 3)
        o, _ = O.attention(q, k, v, scale, causal, window)
        for d in range(3):
            def F(z):
                qa = np.concatenate([q, np.full(q.shape[:-1] + (1,), z / scale)], axis=-1)
                ka = np.concatenate([k, v[..., d:d + 1]], axis=-1)
                va = np.concatenate([v, v[..., :1]], axis=-1)
                return O.attention(qa, ka, va, scale, causal, window)[1]
            grad = (F(eps) - F(-eps)) / (2 * eps)
            np.testing.assert_allclose(grad, o[..., d], rtol=0, atol=1e-7)


def pin_torch_sdpa(O):
    """P10: torch's CPU scaled_dot_product_attention in fp64 with an explicit band mask,
    and torch.logsumexp for lse (library routines the oracle does not use)."""
    rng = np.random.default_rng(1111)
    for (B, Hq, Hkv, Sq, Sk, D) in [(2, 4, 2, 7, 7, 8), (1, 3, 1, 5, 9, 4)]:
        for causal, window in [(False, -1), (True, -1), (False, 2), (True, 3)]:
            q, k, v = _qkv(rng, B, Hq, Hkv, Sq, Sk, D)
            G = Hq // Hkv
            tq = torch.from_numpy(q)
            tk = torch.from_numpy(k).repeat_interleave(G, dim=1)
            tv = torch.from_numpy(v).repeat_interleave(G, dim=1)
            ones = torch.ones(Sq, Sk, dtype=torch.bool)
            mask = ones.clone()
            if causal:
                mask &= torch.tril(ones, diagonal=Sk - Sq)
            if window >= 0:
                mask &= torch.tril(ones, diagonal=Sk - Sq + window) & torch.triu(ones, diagonal=Sk - Sq - window)
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.55)
            s = 0.55 * tq @ tk.transpose(-1, -2)
            ref_lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
            o, lse = O.attention(q, k, v, 0.55, causal, window)
            np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)


ALL_PINS = [
    pin_brute_force,
    pin_online_equals_two_pass,
    pin_split_tree_equals_unsplit,
    pin_merge_algebra,
    pin_uniform_scores,
    pin_window_count_at_64,
    pin_kv_permutation,
    pin_special_cases,
    pin_overflow_safety,
    pin_gqa_equals_mha,
    pin_energy_gradient,
    pin_torch_sdpa,
]
