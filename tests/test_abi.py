"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import glob
import os
import re

import pytest

from exact_attention_33_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, NULL, SHAPE, GQA, HEADDIM, SPLITS, WINDOW, WORKSPACE, HIP, ARG = range(10)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced on the host: every call below fails validation


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        pytest.fail("libattn.so not built (run __graft_entry__.build())")
    return ops.lib()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_bound_symbols():
    assert declared_functions() == sorted(ops.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_error_strings(L):
    assert "gfx950" in ops.version()
    for code, name in ops.STATUS_NAMES.items():
        assert ops.error_string(code).startswith(name)
    assert "unknown" in ops.error_string(99)


def fwd(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=1, Sq=8, Sk=8, D=64,
        causal=0, window=-1, scale=0.125, f32=False):
    fn = L.attn_fwd_f32 if f32 else L.attn_fwd
    return fn(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, window, scale, None)


@pytest.mark.parametrize("f32", [False, True])
def test_fwd_validation(L, f32):
    assert fwd(L, q=None, f32=f32) == NULL
    assert fwd(L, o=None, f32=f32) == NULL
    assert fwd(L, k=None, f32=f32) == NULL
    assert fwd(L, v=None, Sk=8, f32=f32) == NULL
    assert fwd(L, B=-1, f32=f32) == SHAPE
    assert fwd(L, Sq=-3, f32=f32) == SHAPE
    assert fwd(L, Sk=(1 << 29) + 1, f32=f32) == SHAPE
    assert fwd(L, Hq=3, Hkv=2, f32=f32) == GQA
    assert fwd(L, Hq=2, Hkv=0, f32=f32) == GQA
    for D in (0, 32, 96, 256):
        assert fwd(L, D=D, f32=f32) == HEADDIM
    assert fwd(L, window=-2, f32=f32) == WINDOW
    assert fwd(L, causal=2, f32=f32) == ARG
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert fwd(L, scale=s, f32=f32) == ARG
    # nothing to compute: accepted without touching pointers or the GPU
    assert fwd(L, q=None, k=None, v=None, o=None, B=0, f32=f32) == OK
    assert fwd(L, q=None, k=None, v=None, o=None, Sq=0, f32=f32) == OK
    assert fwd(L, q=None, k=None, v=None, o=None, Hq=0, Hkv=0, f32=f32) == OK


def dec_ex(L, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=2, Hq=8, Hkv=2, Sk=100, D=128, ns=4,
           scale=0.088, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = L.attn_decode_workspace_bytes(B, Hq, D, ns)
    return L.attn_decode_ex(q, k, v, o, lse, B, Hq, Hkv, Sk, D, ns, scale, ws, ws_bytes, None)


def test_decode_validation(L):
    assert dec_ex(L, q=None) == NULL
    assert dec_ex(L, k=None) == NULL
    assert dec_ex(L, Sk=-1) == SHAPE
    assert dec_ex(L, Hq=6, Hkv=4) == GQA
    assert dec_ex(L, D=80) == HEADDIM
    assert dec_ex(L, ns=0) == SPLITS
    assert dec_ex(L, ns=101, Sk=100) == SPLITS
    assert dec_ex(L, ns=2, Sk=0) == SPLITS
    assert dec_ex(L, scale=0.0) == ARG
    assert dec_ex(L, ws=None) == WORKSPACE
    need = L.attn_decode_workspace_bytes(2, 8, 128, 4)
    assert dec_ex(L, ws_bytes=need - 1) == WORKSPACE
    assert dec_ex(L, q=None, k=None, v=None, o=None, B=0, ws=None) == OK
    # attn_decode shares the same host checks
    assert L.attn_decode(None, FAKE, FAKE, FAKE, 1, 4, 2, 16, 128, 2, None) == NULL
    assert L.attn_decode(FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 16, 128, 17, None) == SPLITS
    assert L.attn_decode(FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 16, 100, 2, None) == HEADDIM


def test_workspace_bytes(L):
    for B, Hq, D, ns in [(16, 32, 128, 64), (1, 32, 128, 256), (3, 5, 64, 1)]:
        assert L.attn_decode_workspace_bytes(B, Hq, D, ns) == B * Hq * ns * (D + 2) * 4
    # above 256 partials the combine adds upper tree levels: 1000 -> 4 -> root
    assert L.attn_decode_workspace_bytes(1, 1, 64, 1000) == (1000 + 4) * 66 * 4
    # 70000 -> 274 -> 2 -> root
    assert L.attn_decode_workspace_bytes(2, 1, 128, 70000) == 2 * (70000 + 274 + 2) * 130 * 4
    assert L.attn_decode_workspace_bytes(1, 1, 96, 4) == 0
    assert L.attn_decode_workspace_bytes(1, 1, 64, 0) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.attn_fwd(q, q, q)


def test_calib_validation(L):
    sz = ctypes.c_size_t
    assert L.attn_calib_stream(None, sz(0), None, sz(0), None) == OK
    assert L.attn_calib_stream(FAKE, sz(64), None, sz(64), None) == NULL
    assert L.attn_calib_stream(None, sz(64), FAKE, sz(64), None) == NULL
    assert L.attn_calib_stream(FAKE, sz(64), FAKE, sz(0), None) == ARG
    assert L.attn_calib_stream(FAKE, sz(48), FAKE, sz(32), None) == ARG      # not a multiple
    assert L.attn_calib_stream(FAKE, sz(40), FAKE, sz(40), None) == ARG      # not 16-byte chunks
    assert L.attn_calib_stream(ctypes.c_void_p(0x1008), sz(64), FAKE, sz(64), None) == ARG
    assert L.attn_calib_mfma(None, 0, 10, None) == OK
    assert L.attn_calib_mfma(None, 4, 10, None) == NULL
    assert L.attn_calib_mfma(FAKE, -1, 10, None) == ARG
    assert L.attn_calib_mfma(FAKE, 4, -1, None) == ARG
    assert L.attn_calib_mfma_flops(3, 5) == 2.0 * 32 * 32 * 16 * 4 * 4 * 5 * 3


def test_fwd_fp8_validation(L):
    f = ctypes.c_float

    def call(D=128, qd=1.0, kd=1.0, vd=1.0, q=FAKE, Sq=8):
        return L.attn_fwd_fp8(q, FAKE, FAKE, FAKE, None, 1, 2, 1, Sq, 8, D, 0, -1, f(0.125),
                              f(qd), f(kd), f(vd), None)

    assert call(D=96) == HEADDIM
    assert call(qd=0.0) == ARG
    assert call(kd=-1.0) == ARG
    assert call(vd=float("inf")) == ARG
    assert call(q=None) == NULL
    assert call(q=None, Sq=0) == OK          # nothing to compute


def test_misaligned_pointers_are_rejected(L):
    odd = ctypes.c_void_p(0x1008)      # 8-byte aligned, not 16
    odd4 = ctypes.c_void_p(0x1002)     # not 4-byte aligned
    for f32 in (False, True):
        for name in ("q", "k", "v", "o"):
            assert fwd(L, f32=f32, **{name: odd}) == ARG, name
        assert fwd(L, f32=f32, lse=odd4) == ARG
    f = ctypes.c_float
    assert L.attn_fwd_fp8(odd, FAKE, FAKE, FAKE, None, 1, 2, 1, 8, 8, 128, 0, -1, f(0.125),
                          f(1.0), f(1.0), f(1.0), None) == ARG
    for name in ("q", "k", "v", "o"):
        assert dec_ex(L, **{name: odd}) == ARG, name
    assert dec_ex(L, lse=odd4) == ARG
    assert dec_ex(L, ws=odd) == ARG

    def bwd(**kw):
        p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE)
        p.update(kw)
        return L.attn_bwd(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], p["dq"], p["dk"], p["dv"],
                          p["delta"], 1, 2, 1, 8, 8, 64, 0, -1, ctypes.c_float(0.125), None)

    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        assert bwd(**{name: odd}) == ARG, name
    for name in ("lse", "delta"):
        assert bwd(**{name: odd4}) == ARG, name


def test_noalloc_decode_validation(L):
    def call(B=2, Hq=8, Hkv=2, Sk=100, D=128, ns=4, q=FAKE, lse=None, scale=0.088):
        return L.attn_decode_noalloc(q, FAKE, FAKE, FAKE, lse, B, Hq, Hkv, Sk, D, ns, scale, None)

    assert call(q=None) == NULL
    assert call(ns=0) == SPLITS
    assert call(D=96) == HEADDIM
    assert call(scale=0.0) == ARG
    assert call(lse=ctypes.c_void_p(0x1002)) == ARG
    assert call(q=None, B=0) == OK
    # partials beyond the 32 MiB static array: refused before any HIP call
    assert L.attn_decode_workspace_bytes(64, 32, 128, 64) > ops.NOALLOC_BYTES
    assert call(B=64, Hq=32, Hkv=8, Sk=1024, ns=64) == WORKSPACE
    assert L.attn_decode_workspace_bytes(16, 32, 128, 64) <= ops.NOALLOC_BYTES


def test_launch_size_limits(L):
    """A dispatch counts its work-items (blocks x threads) in 32 bits: shapes
    whose grid would exceed that are refused on the host with ATTN_ERR_SHAPE,
    before any launch."""
    # bf16 / fp8 / fp32 prefill: 2^16 query tiles x 256 heads x 512 threads = 2^33
    for f32 in (False, True):
        assert fwd(L, B=1, Hq=256, Hkv=256, Sq=1 << 24, Sk=16, f32=f32) == SHAPE
    # the fp32 kernel's 16-row, 1024-thread workgroups: 2^17 x 64 x 1024 = 2^33
    assert fwd(L, B=1, Hq=64, Hkv=64, Sq=1 << 21, Sk=16, f32=True) == SHAPE
    # decode split kernel: 2^20 chunks x 16 kv heads x 16 rows x 256 threads = 2^36
    assert dec_ex(L, B=16, Hq=16, Hkv=16, Sk=1 << 20, D=128, ns=1 << 20) == SHAPE
    # backward dk/dv pass: 2^21 key tiles x 8 kv heads x 256 threads = 2^32
    assert L.attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                      1, 8, 8, 16, 1 << 28, 64, 0, -1, 0.125, None) == SHAPE
