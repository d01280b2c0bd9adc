"""Pins for the fp64 gradient oracle (``oracle.attention_backward``).

Each ``pinb_*`` takes a module providing ``attention`` and
``attention_backward`` so the same pins can run against planted mistakes
(``test_oracle_backward.py``).  Expectations come from outside the formula
being checked:

* central finite differences of the forward oracle ``attention`` (itself
  pinned in ``pins.py``): the gradient of ``L = sum(do * o)`` along random
  directions;
* torch autograd through torch's CPU scaled_dot_product_attention in fp64
  with an explicit band mask (a library the oracle does not use);
* closed forms of the softmax derivative: with one key per row the output is
  that key's value whatever q and k are (so dq = dk = 0, dv = sum of do);
  with q = 0 the weights are uniform over the visible keys (dk = 0 because
  dk is a combination of query rows, dv_j = sum_i do_i / n_i); keys no query
  sees get dk = dv = 0.
"""

from __future__ import annotations

import numpy as np
import torch

MASKS = [(False, -1), (True, -1), (False, 1), (True, 2)]
SHAPES = [(1, 2, 1, 5, 6, 3), (2, 4, 2, 4, 4, 2), (1, 2, 2, 6, 3, 4)]   # B, Hq, Hkv, Sq, Sk, D


def _rand(rng, B, Hq, Hkv, Sq, Sk, D):
    return (rng.standard_normal((B, Hq, Sq, D)), rng.standard_normal((B, Hkv, Sk, D)),
            rng.standard_normal((B, Hkv, Sk, D)), rng.standard_normal((B, Hq, Sq, D)))


def pinb_finite_differences(O):
    """dL/dx . delta == (L(x + e delta) - L(x - e delta)) / 2e for L = sum(do * o)."""
    rng = np.random.default_rng(2024)
    scale, eps = 0.6, 1e-6
    for shape in SHAPES:
        for causal, window in MASKS:
            q, k, v, do = _rand(rng, *shape)
            dq, dk, dv, _ = O.attention_backward(q, k, v, do, scale, causal, window)

            def L(qq, kk, vv):
                return float((do * O.attention(qq, kk, vv, scale, causal, window)[0]).sum())

            for which, grad in (("q", dq), ("k", dk), ("v", dv)):
                for _ in range(2):
                    d = rng.standard_normal(grad.shape)
                    args_p = dict(qq=q, kk=k, vv=v)
                    args_m = dict(qq=q, kk=k, vv=v)
                    args_p[which * 2] = args_p[which * 2] + eps * d
                    args_m[which * 2] = args_m[which * 2] - eps * d
                    fd = (L(**args_p) - L(**args_m)) / (2 * eps)
                    an = float((grad * d).sum())
                    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (shape, causal, window, which, fd, an)


def _torch_mask(Sq, Sk, causal, window):
    ones = torch.ones(Sq, Sk, dtype=torch.bool)
    mask = ones.clone()
    if causal:
        mask &= torch.tril(ones, diagonal=Sk - Sq)
    if window >= 0:
        mask &= torch.tril(ones, diagonal=Sk - Sq + window) & torch.triu(ones, diagonal=Sk - Sq - window)
    return mask


def pinb_torch_autograd(O):
    """Agreement with torch autograd through SDPA (fp64, CPU) to 1e-11."""
    rng = np.random.default_rng(2025)
    for (B, Hq, Hkv, Sq, Sk, D) in [(2, 4, 2, 7, 7, 8), (1, 3, 1, 5, 9, 4), (1, 2, 1, 9, 5, 3)]:
        for causal, window in [(False, -1), (True, -1), (False, 2), (True, 3)]:
            mask = _torch_mask(Sq, Sk, causal, window)
            if not bool(mask.any(dim=1).all()):
                continue   # torch's SDPA returns NaN for rows with no key; the oracle's reading is o = 0
            q, k, v, do = _rand(rng, B, Hq, Hkv, Sq, Sk, D)
            G = Hq // Hkv
            tq = torch.from_numpy(q).requires_grad_(True)
            tk = torch.from_numpy(k).requires_grad_(True)
            tv = torch.from_numpy(v).requires_grad_(True)
            out = torch.nn.functional.scaled_dot_product_attention(
                tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), attn_mask=mask, scale=0.45)
            (out * torch.from_numpy(do)).sum().backward()
            dq, dk, dv, _ = O.attention_backward(q, k, v, do, 0.45, causal, window)
            np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
            np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
            np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


def pinb_closed_forms(O):
    """One key per row; q = 0 (uniform weights); keys nobody sees."""
    rng = np.random.default_rng(2026)
    # one key: o = v_0 regardless of q, k
    q, k, v, do = _rand(rng, 1, 4, 2, 5, 1, 3)
    dq, dk, dv, _ = O.attention_backward(q, k, v, do, 0.8)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13   # zero up to rounding of dP - delta
    np.testing.assert_allclose(dv[0, 0, 0], do[0, 0:2].sum(axis=(0, 1)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv[0, 1, 0], do[0, 2:4].sum(axis=(0, 1)), rtol=0, atol=1e-13)
    # q = 0: uniform weights over the n_i visible keys
    for causal, window in [(False, -1), (True, -1), (False, 1)]:
        Sq, Sk = 6, 6
        q, k, v, do = _rand(rng, 1, 1, 1, Sq, Sk, 2)
        q[:] = 0.0
        dq, dk, dv, _ = O.attention_backward(q, k, v, do, 0.9, causal, window)
        assert np.abs(dk).max() == 0.0   # dk is a combination of query rows, all zero
        vis = O.visibility(np.arange(Sq), Sq, Sk, causal, window)
        n = vis.sum(axis=1)
        ref = (vis / n[:, None]).T @ do[0, 0]
        np.testing.assert_allclose(dv[0, 0], ref, rtol=0, atol=1e-13)
    # keys outside every window get nothing
    q, k, v, do = _rand(rng, 1, 2, 1, 2, 10, 3)
    dq, dk, dv, _ = O.attention_backward(q, k, v, do, 0.7, False, 1)
    assert np.abs(dk[0, 0, :7]).max() == 0.0 and np.abs(dv[0, 0, :7]).max() == 0.0
    assert np.abs(dv[0, 0, 7:]).min() > 0.0


def pinb_gqa_equals_mha(O):
    """A shared kv head's gradient is the sum of the per-query-head gradients."""
    rng = np.random.default_rng(2027)
    q, k, v, do = _rand(rng, 2, 6, 2, 5, 7, 3)
    dq, dk, dv, _ = O.attention_backward(q, k, v, do, 0.5, True, -1)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    dq2, dk2, dv2, _ = O.attention_backward(q, kr, vr, do, 0.5, True, -1)
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(2, 2, 3, 7, 3).sum(axis=2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(2, 2, 3, 7, 3).sum(axis=2), rtol=0, atol=1e-13)


ALL_PINS_B = [pinb_finite_differences, pinb_torch_autograd, pinb_closed_forms, pinb_gqa_equals_mha]
