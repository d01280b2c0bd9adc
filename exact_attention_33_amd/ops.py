"""ctypes binding of libattn.so: same entry points as include/attn.h.

Argument marshalling only -- tensor checks, output allocation, device pointers
and torch's current HIP stream.  Every step of the computation runs in the
HIP kernels behind the C ABI.  If the library is not built the first call
raises; there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_GQA",
    4: "ATTN_ERR_HEADDIM", 5: "ATTN_ERR_SPLITS", 6: "ATTN_ERR_WINDOW",
    7: "ATTN_ERR_WORKSPACE", 8: "ATTN_ERR_HIP", 9: "ATTN_ERR_ARG",
}
# every symbol include/attn.h and include/attn_calib.h declare
EXPORTS = ("attn_fwd", "attn_fwd_f32", "attn_fwd_fp8", "attn_bwd", "attn_decode", "attn_decode_ex",
           "attn_decode_noalloc",
           "attn_decode_workspace_bytes", "attn_error_string", "attn_version",
           "attn_calib_stream", "attn_calib_mfma", "attn_calib_mfma_flops", "attn_calib_mfma_fp8")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libattn.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_33_amd.build` "
                           "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_f32.restype = i
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, f, f, f, vp]
    L.attn_fwd_fp8.restype = i
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    L.attn_bwd.restype = i
    L.attn_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp]
    L.attn_decode.restype = i
    L.attn_decode_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.attn_decode_ex.restype = i
    L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_decode_noalloc.restype = i
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_error_string.argtypes = [i]
    L.attn_error_string.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_version.restype = ctypes.c_char_p
    L.attn_calib_stream.argtypes = [vp, sz, vp, sz, vp]
    L.attn_calib_stream.restype = i
    L.attn_calib_mfma.argtypes = [vp, i, i, vp]
    L.attn_calib_mfma.restype = i
    L.attn_calib_mfma_flops.argtypes = [i, i]
    L.attn_calib_mfma_flops.restype = ctypes.c_double
    L.attn_calib_mfma_fp8.argtypes = [vp, vp, vp, vp]
    L.attn_calib_mfma_fp8.restype = i
    _lib = L
    return L


def error_string(status: int) -> str:
    return lib().attn_error_string(int(status)).decode()


def version() -> str:
    return lib().attn_version().decode()


def decode_workspace_bytes(B: int, Hq: int, D: int, num_splits: int) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, D, num_splits))


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, error_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _want(t: torch.Tensor, name: str, dtype, ndim: int, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: need a contiguous {dtype} tensor with {ndim} dims on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _fwd(fn, dtype, q, k, v, causal, window, scale, out, lse, return_lse):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _want(t, n, dtype, 4, dev)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    o = torch.empty_like(q) if out is None else out
    _want(o, "out", dtype, 4, dev)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    if lse is not None:
        _want(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError("lse must be [B, Hq, Sq]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Sk, D,
                  int(causal), int(window), scale, _stream(q)))
    return o, lse


def attn_fwd(q, k, v, causal=False, window=-1, scale=None, out=None, lse=None, return_lse=True):
    """Prefill, bf16 ``q [B,Hq,Sq,D]``, ``k, v [B,Hkv,Sk,D]`` -> ``(o, lse)``."""
    return _fwd(lib().attn_fwd, torch.bfloat16, q, k, v, causal, window, scale, out, lse, return_lse)


def attn_fwd_f32(q, k, v, causal=False, window=-1, scale=None, out=None, lse=None, return_lse=True):
    """Prefill on fp32 tensors (no bf16 rounding anywhere) -> ``(o, lse)``."""
    return _fwd(lib().attn_fwd_f32, torch.float32, q, k, v, causal, window, scale, out, lse, return_lse)


def attn_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal=False, window=-1, scale=None,
                 out=None, lse=None, return_lse=True):
    """Prefill on fp8 (OCP E4M3) codes: ``q8 [B,Hq,Sq,D]``, ``k8, v8 [B,Hkv,Sk,D]`` as
    uint8 tensors (or torch.float8_e4m3fn), one descale per tensor -> ``(o bf16, lse)``."""
    dev = q8.device
    if dev.type != "cuda":
        raise ValueError("q8 must be on a GPU")
    codes = []
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        _want(t, n, torch.uint8, 4, dev)
        codes.append(t)
    q8, k8, v8 = codes
    B, Hq, Sq, D = q8.shape
    Bk, Hkv, Sk, Dk = k8.shape
    if v8.shape != k8.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q8.shape)} k{tuple(k8.shape)} v{tuple(v8.shape)}")
    o = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=dev) if out is None else out
    _want(o, "out", torch.bfloat16, 4, dev)
    if tuple(o.shape) != (B, Hq, Sq, D):
        raise ValueError("out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    if lse is not None:
        _want(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, Sq):
            raise ValueError("lse must be [B, Hq, Sq]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with torch.cuda.device(q8.device):  # kernels launch on the current device
        _check(lib().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Sk, D,
                                  int(causal), int(window), scale, float(q_descale), float(k_descale),
                                  float(v_descale), _stream(q8)))
    return o, lse


def attn_bwd(q, k, v, o, dout, lse, causal=False, window=-1, scale=None, dq=None, dk=None, dv=None,
             delta=None):
    """Gradients of ``sum(dout * o)`` for the bf16 prefill -> ``(dq, dk, dv)``.

    ``o`` and ``lse`` are the forward's outputs for the same inputs and mask;
    ``delta`` (fp32 ``[B, Hq, Sq]``) is scratch, allocated here if not given.
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _want(t, n, torch.bfloat16, 4, dev)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, o, dout")
    _want(lse, "lse", torch.float32, 3, dev)
    if tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be [B, Hq, Sq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev) if delta is None else delta
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _want(t, n, torch.bfloat16, 4, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must have the shape of its input")
    _want(delta, "delta", torch.float32, 3, dev)
    if tuple(delta.shape) != (B, Hq, Sq):
        raise ValueError("delta must be [B, Hq, Sq]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _check(lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(delta), B, Hq, Hkv, Sq, Sk, D, int(causal), int(window), scale,
                              _stream(q)))
    return dq, dk, dv


def _decode_shapes(q, kcache, vcache, out):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be on a GPU")
    _want(q, "q", torch.bfloat16, 3, dev)
    _want(kcache, "kcache", torch.bfloat16, 4, dev)
    _want(vcache, "vcache", torch.bfloat16, 4, dev)
    B, Hq, D = q.shape
    Bk, Hkv, Sk, Dk = kcache.shape
    if vcache.shape != kcache.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(kcache.shape)} v{tuple(vcache.shape)}")
    o = torch.empty_like(q) if out is None else out
    _want(o, "out", torch.bfloat16, 3, dev)
    if o.shape != q.shape:
        raise ValueError("out must have q's shape")
    return B, Hq, Hkv, Sk, D, o


def attn_decode(q, kcache, vcache, num_splits, out=None):
    """Split-KV decode with the library workspace, scale 1/sqrt(D) -> ``o [B,Hq,D]``."""
    B, Hq, Hkv, Sk, D, o = _decode_shapes(q, kcache, vcache, out)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _check(lib().attn_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(o), B, Hq, Hkv, Sk, D,
                                 int(num_splits), _stream(q)))
    return o


def attn_decode_ex(q, kcache, vcache, num_splits, scale=None, out=None, lse=None,
                   return_lse=True, workspace=None):
    """Split-KV decode with explicit scale and caller workspace -> ``(o, lse)``.

    ``workspace`` (a uint8 device tensor) is allocated here when not given.
    """
    B, Hq, Hkv, Sk, D, o = _decode_shapes(q, kcache, vcache, out)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _want(lse, "lse", torch.float32, 2, q.device)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    need = decode_workspace_bytes(B, Hq, D, int(num_splits)) if num_splits >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _want(workspace, "workspace", torch.uint8, 1, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _check(lib().attn_decode_ex(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                    Sk, D, int(num_splits), scale, _ptr(workspace), workspace.numel(),
                                    _stream(q)))
    return o, lse


NOALLOC_BYTES = 32 << 20   # ATTN_DECODE_NOALLOC_BYTES


def attn_decode_noalloc(q, kcache, vcache, num_splits, out, lse=None, scale=None):
    """Split-KV decode whose partials live in the library's static device array
    (no device allocation by the library; ``out`` and the optional ``lse`` are
    the caller's) -> ``(o, lse)``."""
    B, Hq, Hkv, Sk, D, o = _decode_shapes(q, kcache, vcache, out)
    if lse is not None:
        _want(lse, "lse", torch.float32, 2, q.device)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _check(lib().attn_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(o), _ptr(lse), B, Hq,
                                         Hkv, Sk, D, int(num_splits), scale, _stream(q)))
    return o, lse


# ---- measurement reference kernels (include/attn_calib.h) -------------------

def calib_stream(src: torch.Tensor, dst: torch.Tensor):
    """dst chunk j (16 bytes) = XOR of src chunks j, j+n, j+2n, ... (n = dst chunks):
    a plain HBM stream of src.nbytes read and dst.nbytes written."""
    for t, n in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous GPU tensor")
    _check(lib().attn_calib_stream(_ptr(src), src.numel() * src.element_size(), _ptr(dst),
                                   dst.numel() * dst.element_size(), _stream(dst)))
    return dst


def calib_mfma_fp8(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """One fp8 (E4M3) matrix instruction: ``c[m, n] = sum_k a[m, k] * b[n, k]`` as the
    matrix core sums it; ``a, b`` are 32 x 64 uint8 codes on the GPU."""
    for t, n in ((a, "a"), (b, "b")):
        _want(t, n, torch.uint8, 2, a.device)
        if tuple(t.shape) != (32, 64):
            raise ValueError(f"{n} must be 32 x 64 codes")
    c = torch.empty(32, 32, dtype=torch.float32, device=a.device)
    _check(lib().attn_calib_mfma_fp8(_ptr(a), _ptr(b), _ptr(c), _stream(c)))
    return c


def calib_mfma(out: torch.Tensor, workgroups: int, iters: int) -> float:
    """A loop of bf16 MFMA instructions with no memory traffic; returns its flop count."""
    _want(out, "out", torch.float32, 1, out.device)
    if out.numel() < 4 * workgroups:
        raise ValueError("out needs 4 floats per workgroup")
    _check(lib().attn_calib_mfma(_ptr(out), int(workgroups), int(iters), _stream(out)))
    return float(lib().attn_calib_mfma_flops(int(workgroups), int(iters)))
