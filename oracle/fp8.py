"""fp64 reference for attention on fp8 (e4m3) inputs (test infrastructure only).

The pages name low-precision FP8 as a FlashAttention-3 feature (FlashAttention
explainer, aiunderstanding.org, "The future of FlashAttention" and the FAQ
entry on what FlashAttention-3 uses; FlashAttention-3 article, ybx.com, "FA3
innovations" point 3) but define no format or scaling.  Readings taken here:

* Values are OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; the codes
  S.1111.111 are NaN; there is no infinity; the largest finite value is 448.
* Each of q, k, v comes with one per-tensor descale factor: the real input
  is ``decode(code) * descale``.
* The result is the exact attention of those real inputs -- the same
  definition as ``attention`` -- so the only deviations of a kernel are its
  own roundings (the probabilities it rounds before the p.v product, its
  accumulation, the final rounding of o).
"""

from __future__ import annotations

import numpy as np

from .attention import attention

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each e4m3fn byte (NaN for the two NaN codes)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    mag = np.where(exp == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.exp2(exp - 7.0))
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def attention_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float, scale: float,
                  causal: bool = False, window: int = -1):
    """Exact attention of the dequantized inputs: ``attention(decode(q8) * q_descale, ...)``.

    ``q8 [B, Hq, Sq, D]``, ``k8, v8 [B, Hkv, Sk, D]`` are e4m3fn byte codes
    (uint8).  Returns ``(o, lse)`` in fp64 as ``attention`` does.
    """
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    v = e4m3_decode(v8) * float(v_descale)
    return attention(q, k, v, scale, causal, window)
