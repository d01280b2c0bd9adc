"""Pins of the fp8 (e4m3) oracle (CPU only).

Each pin takes a module exposing ``e4m3_decode`` and ``attention_fp8`` (the
oracle, or a planted mutant of it) and raises if it is wrong.  They fix the
format from outside the oracle: torch's own float8_e4m3fn conversion for all
256 codes, the format's closed forms (bias 7, subnormals m * 2^-9, largest
finite 448, two NaN codes, sign symmetry, ordering), and the descale factors
through identities the exact attention obeys.
"""

import numpy as np
import torch

import oracle

CODES = np.arange(256, dtype=np.uint8)


def pin_codes_match_torch(m):
    """Every code decodes to the value torch's float8_e4m3fn gives it."""
    want = torch.from_numpy(CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = m.e4m3_decode(CODES)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def pin_closed_forms(m):
    """1.0 is 0 0111 000, 448 is the largest finite, 2^-9 the smallest
    subnormal, exactly the two S.1111.111 codes are NaN, negation is the sign
    bit, and the positive codes are ordered by value."""
    d = m.e4m3_decode(CODES)
    assert d[0x38] == 1.0 and d[0x40] == 2.0 and d[0x30] == 0.5
    assert d[0x7E] == 448.0 and d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6
    assert d[0x00] == 0.0 and d[0x80] == 0.0
    assert np.flatnonzero(np.isnan(d)).tolist() == [0x7F, 0xFF]
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(d[0x80:0xFF], -pos)


def _case(seed=0, B=1, Hq=2, Hkv=1, S=40, D=8):
    rng = np.random.default_rng(seed)
    q8 = rng.integers(0, 256, (B, Hq, S, D)).astype(np.uint8)
    k8 = rng.integers(0, 256, (B, Hkv, S, D)).astype(np.uint8)
    v8 = rng.integers(0, 256, (B, Hkv, S, D)).astype(np.uint8)
    for t in (q8, k8, v8):       # keep magnitudes modest and drop NaN codes
        t &= 0xBF
    return q8, k8, v8


def pin_descales(m):
    """q and k descales only scale the scores; the v descale scales o."""
    q8, k8, v8 = _case()
    o1, l1 = m.attention_fp8(q8, k8, v8, 0.5, 0.25, 1.0, 0.3, True, 9)
    o2, l2 = m.attention_fp8(q8, k8, v8, 1.0, 1.0, 1.0, 0.3 * 0.5 * 0.25, True, 9)
    o3, l3 = m.attention_fp8(q8, k8, v8, 0.5, 0.25, 3.0, 0.3, True, 9)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-300) and np.allclose(l1, l2, rtol=1e-12)
    assert np.allclose(o3, 3.0 * o1, rtol=1e-12, atol=1e-300) and np.allclose(l3, l1, rtol=1e-12)


def pin_matches_dequantized_torch(m):
    """Equal to the fp64 attention of the inputs torch dequantizes (explicit
    softmax with a band mask, written here from the definition)."""
    q8, k8, v8 = _case(seed=3, Hq=2, Hkv=2, S=17, D=16)
    qd, kd, vd, sc = 0.75, 1.5, 0.5, 0.2
    deq = lambda t, s: torch.from_numpy(t.copy()).view(torch.float8_e4m3fn).to(torch.float64) * s
    q, k, v = deq(q8, qd), deq(k8, kd), deq(v8, vd)
    s = sc * q @ k.transpose(-1, -2)
    i = torch.arange(17)[:, None]
    j = torch.arange(17)[None, :]
    vis = (j <= i) & ((i - j).abs() <= 5)
    s = s.masked_fill(~vis, float("-inf"))
    want_o = torch.softmax(s, dim=-1) @ v
    want_l = torch.logsumexp(s, dim=-1)
    o, l = m.attention_fp8(q8, k8, v8, qd, kd, vd, sc, True, 5)
    assert np.allclose(o, want_o.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(l, want_l.numpy(), rtol=1e-12, atol=1e-12)


ALL_PINS_F8 = [pin_codes_match_torch, pin_closed_forms, pin_descales, pin_matches_dequantized_torch]
