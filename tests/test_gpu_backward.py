"""GPU parity of the backward (attn_bwd, through the C ABI) against the fp64
gradient oracle ``oracle.attention_backward`` on the same seeded inputs.

The kernels recompute P from the forward's lse and round P and dS to bf16 for
the matrix products (fp32 accumulation), then round dq, dk, dv once to bf16.
Each gradient entry is a sum of products whose two factors each carry at most
one bf16 rounding (relative 2^-9), so with random signs the error of the sum
is ~2^-8 of the norm of its terms, plus 2^-9 for the final rounding: a
relative-L2 error around 5e-3.  The test allows 1.5e-2 (3x), and bounds the
largest entry error by 2e-2 of the largest gradient magnitude.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_attention_33_amd import ops, synth
from exact_attention_33_amd.synth import to_numpy_exact
from gpu_util import announce

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_L2 = 1.5e-2
MAX_REL = 2e-2


def _check(name, got_t, ref, what):
    got = to_numpy_exact(got_t).astype(np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what} {name}: non-finite"
    nref = np.linalg.norm(ref)
    if nref == 0:
        assert np.abs(got).max() == 0.0, f"{what} {name}: expected all zero"
        return 0.0, 0.0
    rel = np.linalg.norm(got - ref) / nref
    mx = np.abs(got - ref).max() / np.abs(ref).max()
    print(f"  {what} {name}: rel_l2 {rel:.2e} max_err/max_ref {mx:.2e}", flush=True)
    assert rel <= REL_L2, f"{what} {name}: rel_l2 {rel}"
    assert mx <= MAX_REL, f"{what} {name}: max err {mx}"
    return rel, mx


def _bwd_case(B, Hq, Hkv, Sq, Sk, D, causal, window, seed=0, scale=None):
    q, k, v = synth.draw_qkv((B, Hq, Sq, D), (B, Hkv, Sk, D), "bf16", seed, DEV)
    do = synth.draw_grad((B, Hq, Sq, D), "bf16", seed, DEV)
    scale = synth.default_scale(D) if scale is None else scale
    what = f"bwd B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D} causal{causal} w{window} seed{seed}"
    announce(what)
    o, lse = ops.attn_fwd(q, k, v, causal=causal, window=window, scale=scale)
    dq, dk, dv = ops.attn_bwd(q, k, v, o, do, lse, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv, rdel = oracle.attention_backward(to_numpy_exact(q), to_numpy_exact(k), to_numpy_exact(v),
                                                 to_numpy_exact(do), scale, bool(causal), window)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check(name, got, ref, what)
    return q, k, v, do, o, lse


SHAPES = [
    (1, 2, 2, 257, 257, 128, 1, -1),
    (2, 4, 2, 130, 300, 128, 1, -1),     # Sq < Sk, GQA
    (1, 2, 1, 300, 130, 128, 1, -1),     # Sq > Sk: rows with no visible key
    (1, 3, 1, 200, 200, 128, 0, -1),     # GQA 3:1, no mask
    (1, 2, 2, 400, 400, 64, 0, 40),      # window, D = 64
    (1, 2, 2, 333, 333, 64, 1, 50),      # causal + window
    (1, 2, 2, 96, 517, 128, 0, 100),     # window with Sq < Sk
    (2, 2, 1, 33, 33, 64, 1, -1),        # a single partial tile
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_shapes(shape):
    _bwd_case(*shape, seed=11)


def test_backward_long_causal():
    """A 2048-token causal head group (the causal-prefill sequence length)."""
    _bwd_case(1, 4, 4, 2048, 2048, 128, 1, -1, seed=12)


def test_backward_peaky():
    """scale = 1: near one-hot rows, large dS contrasts."""
    _bwd_case(1, 2, 1, 160, 160, 128, 1, -1, seed=13, scale=1.0)


def test_backward_empty():
    announce("bwd empty inputs")
    q, k, v = synth.draw_qkv((1, 2, 0, 64), (1, 2, 50, 64), "bf16", 3, DEV)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dq, dk, dv = ops.attn_bwd(q, k, v, o, torch.empty_like(q), lse, causal=True)
    torch.cuda.synchronize()
    assert dk.abs().max().item() == 0.0 and dv.abs().max().item() == 0.0
    q, k, v = synth.draw_qkv((1, 2, 40, 64), (1, 2, 0, 64), "bf16", 3, DEV)
    o, lse = ops.attn_fwd(q, k, v)
    dq, dk, dv = ops.attn_bwd(q, k, v, o, synth.draw_grad(q.shape, "bf16", 3, DEV), lse)
    torch.cuda.synchronize()
    assert dq.abs().max().item() == 0.0


def test_backward_deterministic_and_delta():
    """Two runs give identical bits; delta holds rowsum(dout * o) of the bf16 o."""
    q, k, v, do, o, lse = _bwd_case(1, 4, 2, 190, 190, 128, 1, -1, seed=14)
    delta = torch.empty((1, 4, 190), dtype=torch.float32, device=DEV)
    a = ops.attn_bwd(q, k, v, o, do, lse, causal=True, delta=delta)
    b = ops.attn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ref = (to_numpy_exact(do).astype(np.float64) * to_numpy_exact(o)).sum(axis=-1)
    np.testing.assert_allclose(to_numpy_exact(delta), ref, rtol=0, atol=1e-4)


def test_backward_full_size_sampled_heads():
    """The causal-prefill shape the bench times (B4 H16 S2048 D128, one launch
    pair over all 64 heads); heads are independent (no GQA), so the fp64
    gradient oracle of a head's own q, k, v, dout slice is exact for it."""
    w = synth.WORKLOADS["causal_prefill"]
    B, H, S, D = w["B"], w["Hq"], w["Sq"], w["D"]
    q, k, v = synth.draw_qkv((B, H, S, D), (B, H, S, D), "bf16", synth.SEEDS["causal_prefill"], DEV)
    do = synth.draw_grad((B, H, S, D), "bf16", synth.SEEDS["causal_prefill"], DEV)
    scale = synth.default_scale(D)
    announce(f"bwd full size B{B} H{H} S{S} D{D} causal, sampled heads")
    o, lse = ops.attn_fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = ops.attn_bwd(q, k, v, o, do, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv, _ = oracle.attention_backward(to_numpy_exact(q[sl]), to_numpy_exact(k[sl]),
                                                  to_numpy_exact(v[sl]), to_numpy_exact(do[sl]), scale, True, -1)
        for name, got, ref in (("dq", dq[sl], rq), ("dk", dk[sl], rk), ("dv", dv[sl], rv)):
            _check(name, got, ref, f"full size b{b} h{h}")
