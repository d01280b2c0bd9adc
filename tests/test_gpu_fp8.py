"""GPU parity of the fp8 (e4m3) prefill against the fp64 oracle of the
dequantized inputs (through the C ABI).

Tolerance, derived from the arithmetic: the kernel's scores are exact
products of fp8 values summed in fp32, its lse comes from the unrounded fp32
probabilities, and its only coarse rounding is the e4m3 rounding of the
probabilities before the p.v product (relative error at most 2^-4 for
p >= 2^-6, absolute at most 2^-10 below) plus the final bf16 rounding of o.
So o - o_ref = sum_j (p~_j - p_j) v_j / l: at most 2^-4 * max|v| where one
key dominates, and about 2.6 % of |o| (the RMS of the rounding) for spread
rows with random signs.  The tests allow relative L2 <= 5e-2 and max-abs <=
2^-4 * max|v| + 2e-2.  The lse is exact up to the score accumulation: one
fp8 matrix instruction returns each 64-product dot product within
2^-14 * |a_m| * |b_n| of the exact value (Euclidean norms of the two code
rows).  That figure is checked on the instruction alone, against exact fp64
sums of constructed operands (large-plus-tiny, cancellation, gaussian, every
finite code; worst seen 2^-14.6), by test_fp8_mfma_accumulation_precision in
tests/test_gpu_calib.py, not inferred from this kernel's own error.  D = 128
takes two instructions whose errors add, and the descales multiply both
sides, so the lse bound is 1e-3 + 2^-14 * scale * max|q_i| * max|k_j|
(dequantized rows; Cauchy-Schwarz splits the norms over the two halves).
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
REL_L2 = 5e-2
LSE_TOL = 1e-3


def _case(B, Hq, Hkv, Sq, Sk, causal, window, seed=0, scale=None, D=128):
    q8, k8, v8, qd, kd, vd = synth.draw_qkv_fp8((B, Hq, Sq, D), (B, Hkv, Sk, D), seed, DEV)
    scale = synth.default_scale(D) if scale is None else scale
    announce(f"fp8 prefill B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D} causal{causal} w{window} "
             f"scale{scale:.4g} seed{seed}")
    o, lse = ops.attn_fwd_fp8(q8, k8, v8, qd, kd, vd, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    host = [t.cpu().numpy() for t in (q8, k8, v8)]
    return o, lse, host, (qd, kd, vd), scale


def _check(o, lse, host, desc, scale, causal, window, rows=None):
    q8, k8, v8 = host
    qd, kd, vd = desc
    og = to_numpy_exact(o).astype(np.float64)
    lg = to_numpy_exact(lse).astype(np.float64)
    if rows is None:
        o_ref, l_ref = oracle.attention_fp8(q8, k8, v8, qd, kd, vd, scale, bool(causal), window)
    else:
        o_ref, l_ref = _rows_ref(host, desc, scale, causal, window, rows)
        og, lg = og[:, :, rows], lg[:, :, rows]
    vmax = float(np.abs(oracle.e4m3_decode(v8) * vd).max())
    d = np.abs(og - o_ref)
    rel = np.linalg.norm(og - o_ref) / np.linalg.norm(o_ref)
    fin = np.isfinite(l_ref)
    lerr = float(np.abs(lg[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    qn = np.linalg.norm(oracle.e4m3_decode(q8) * qd, axis=-1).max()
    kn = np.linalg.norm(oracle.e4m3_decode(k8) * kd, axis=-1).max()
    lse_tol = LSE_TOL + 2.0 ** -14 * scale * qn * kn
    assert np.array_equal(np.isneginf(lg), np.isneginf(l_ref))
    announce(f"  max-abs {d.max():.3g} (bound {2 ** -4 * vmax + 2e-2:.3g}) rel-L2 {rel:.3g} "
             f"lse {lerr:.3g} (bound {lse_tol:.3g})")
    assert d.max() <= 2 ** -4 * vmax + 2e-2
    assert rel <= REL_L2
    assert lerr <= lse_tol


def _rows_ref(host, desc, scale, causal, window, rows):
    """Oracle on the sampled query rows only: the keys a row sees do not
    depend on the other rows, so each row is the unmasked attention over its
    own visible key range [lo, hi] (bottom-right causal alignment)."""
    q8, k8, v8 = host
    qd, kd, vd = desc
    B, Hq, Sq, D = q8.shape
    Sk = k8.shape[2]
    o = np.zeros((B, Hq, len(rows), D))
    lse = np.zeros((B, Hq, len(rows)))
    G = Hq // k8.shape[1]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for n, r in enumerate(rows):
                pos = r + (Sk - Sq)
                lo, hi = 0, Sk - 1
                if causal:
                    hi = min(hi, pos)
                if window >= 0:
                    lo, hi = max(lo, pos - window), min(hi, pos + window)
                qq = q8[b:b + 1, h:h + 1, r:r + 1]
                kk = k8[b:b + 1, g:g + 1, lo:hi + 1]
                vv = v8[b:b + 1, g:g + 1, lo:hi + 1]
                oo, ll = oracle.attention_fp8(qq, kk, vv, qd, kd, vd, scale, False, -1)
                o[b, h, n] = oo[0, 0, 0]
                lse[b, h, n] = ll[0, 0, 0]
    return o, lse


@pytest.mark.parametrize("shape", [
    (1, 2, 2, 300, 300, 1, -1),      # causal, ragged tail
    (1, 4, 2, 513, 513, 0, -1),      # GQA 2:1, ragged
    (2, 2, 1, 200, 600, 1, -1),      # Sq != Sk, bottom-right causal
    (1, 2, 2, 700, 700, 0, 64),      # sliding window
    (1, 2, 2, 500, 500, 1, 40),      # causal + window
    (1, 1, 1, 33, 97, 0, -1),        # tiny, Sq != Sk
    (1, 2, 2, 1024, 1024, 1, -1),    # several full tiles
    (1, 2, 1, 600, 200, 1, -1),      # Sq > Sk causal: the first 400 rows see no key
    (1, 8, 2, 256, 16384, 1, -1),    # a 256-row block against a 16384-key cache
], ids=lambda s: "B{}Hq{}Hkv{}Sq{}Sk{}c{}w{}".format(*s))
def test_fp8_parity(shape):
    B, Hq, Hkv, Sq, Sk, causal, window = shape
    o, lse, host, desc, scale = _case(B, Hq, Hkv, Sq, Sk, causal, window, seed=sum(shape))
    _check(o, lse, host, desc, scale, causal, window)


@pytest.mark.parametrize("shape", [
    (1, 2, 2, 300, 300, 1, -1),      # causal, ragged tail
    (1, 4, 2, 513, 513, 0, -1),      # GQA 2:1, ragged
    (1, 2, 2, 700, 700, 0, 64),      # the encoder's window, several tiles
    (2, 2, 1, 200, 600, 1, 40),      # Sq != Sk, causal + window
    (1, 2, 2, 300, 100, 1, 16),      # Sq > Sk, causal + window: rows without keys
], ids=lambda s: "B{}Hq{}Hkv{}Sq{}Sk{}c{}w{}".format(*s))
def test_fp8_parity_d64(shape):
    B, Hq, Hkv, Sq, Sk, causal, window = shape
    o, lse, host, desc, scale = _case(B, Hq, Hkv, Sq, Sk, causal, window, seed=sum(shape) + 64, D=64)
    _check(o, lse, host, desc, scale, causal, window)


def test_fp8_peaky():
    """scale = 1: rows dominated by a few keys, where the e4m3 rounding of p
    shows undiluted."""
    o, lse, host, desc, scale = _case(1, 2, 2, 256, 256, 0, -1, seed=11, scale=1.0)
    _check(o, lse, host, desc, scale, 0, -1)


def test_fp8_causal_prefill_full_size_sampled_rows():
    """The causal-prefill shape (B4 H16 S2048 D128) in the launch configuration
    the benchmark times, checked on sampled rows (tile edges, first and last)."""
    o, lse, host, desc, scale = _case(4, 16, 16, 2048, 2048, 1, -1, seed=1)
    rows = [0, 1, 31, 32, 255, 256, 1023, 1024, 2046, 2047]
    _check(o, lse, host, desc, scale, 1, -1, rows=rows)


def test_fp8_window_encoder_full_size_sampled_rows():
    """The window-encoder shape (B8 H12 S8192 D64, |i-j| <= 64) on fp8 inputs,
    in the launch configuration the benchmark times, on sampled rows (both
    ends, tile edges, the window's reach)."""
    o, lse, host, desc, scale = _case(8, 12, 12, 8192, 8192, 0, 64, seed=2, D=64)
    rows = [0, 1, 63, 64, 65, 255, 256, 4095, 8127, 8191]
    _check(o, lse, host, desc, scale, 0, 64, rows=rows)


def test_fp8_empty_and_errors():
    q8 = torch.zeros((1, 2, 0, 128), dtype=torch.uint8, device=DEV)
    k8 = torch.zeros((1, 2, 16, 128), dtype=torch.uint8, device=DEV)
    o, lse = ops.attn_fwd_fp8(q8, k8, k8, 1.0, 1.0, 1.0)
    assert o.shape == (1, 2, 0, 128)
    q96 = torch.zeros((1, 2, 8, 96), dtype=torch.uint8, device=DEV)
    with pytest.raises(ops.AttnError) as e:
        ops.attn_fwd_fp8(q96, q96, q96, 1.0, 1.0, 1.0)
    assert e.value.status == 4   # ATTN_ERR_HEADDIM
    q8 = torch.zeros((1, 2, 8, 128), dtype=torch.uint8, device=DEV)
    with pytest.raises(ops.AttnError) as e:
        ops.attn_fwd_fp8(q8, q8, q8, 1.0, 0.0, 1.0)
    assert e.value.status == 9   # ATTN_ERR_ARG
