"""Seeded synthetic workloads for the attention hot path.

Shared by the tests and the benchmark; it holds shapes, seeds and random draws
only -- none of the attention arithmetic -- so neither the oracle nor the HIP
library depends on the other through it.

Recipe: per workload, one ``torch.Generator`` on the target device seeded with
the workload's seed (0..4 in the order listed below); ``q``, then ``k``, then
``v`` are drawn i.i.d. N(0, 1) in fp32 and rounded to the workload dtype
(round-to-nearest-even, torch's ``.to``).  ``scale = 1/sqrt(D)``.
"""

from __future__ import annotations

import math

import torch

# name -> shape and mask of each workload; the seed is its position.
WORKLOADS = {
    "tiny_f32": dict(kind="prefill", B=1, Hq=1, Hkv=1, Sq=128, Sk=128, D=64,
                     dtype="f32", causal=0, window=-1),
    "causal_prefill": dict(kind="prefill", B=4, Hq=16, Hkv=16, Sq=2048, Sk=2048, D=128,
                           dtype="bf16", causal=1, window=-1),
    "window_encoder": dict(kind="prefill", B=8, Hq=12, Hkv=12, Sq=8192, Sk=8192, D=64,
                           dtype="bf16", causal=0, window=64),
    "gqa_decode": dict(kind="decode", B=16, Hq=32, Hkv=8, Sk=32768, D=128,
                       dtype="bf16", num_splits=64),
    "long_decode": dict(kind="decode", B=1, Hq=32, Hkv=8, Sk=1048576, D=128,
                        dtype="bf16", num_splits=256),
}
SEEDS = {name: i for i, name in enumerate(WORKLOADS)}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def draw_qkv(q_shape, kv_shape, dtype: str, seed: int, device="cpu"):
    """Draw q, k, v ~ N(0,1) in fp32 from one seeded generator, then round to ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    td = TORCH_DTYPES[dtype]
    q = torch.randn(q_shape, generator=gen, device=device, dtype=torch.float32).to(td)
    k = torch.randn(kv_shape, generator=gen, device=device, dtype=torch.float32).to(td)
    v = torch.randn(kv_shape, generator=gen, device=device, dtype=torch.float32).to(td)
    return q, k, v


def draw_grad(shape, dtype: str, seed: int, device="cpu"):
    """An upstream gradient ~ N(0,1) from its own seeded generator (seed + 7919),
    rounded to ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7919)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(TORCH_DTYPES[dtype])


E4M3_MAX = 448.0


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor fp8 (OCP E4M3) codes of ``x`` for synthetic fp8 inputs: ``x`` is
    divided by ``descale = amax / 448`` (so its largest magnitude maps to the
    largest finite code), clamped to +-448 and rounded by torch's
    float8_e4m3fn conversion.  Returns ``(codes as uint8, descale)``; the real
    input is ``decode(code) * descale``."""
    amax = float(x.abs().max())
    descale = amax / E4M3_MAX if amax > 0 else 1.0
    y = (x.float() / descale).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), descale


def draw_qkv_fp8(q_shape, kv_shape, seed: int, device="cpu"):
    """q, k, v drawn as in ``draw_qkv`` (fp32 N(0, 1), one generator) and each
    quantized to e4m3 with its own per-tensor descale: returns
    ``(q8, k8, v8, q_descale, k_descale, v_descale)``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = [quantize_e4m3(torch.randn(sh, generator=gen, device=device, dtype=torch.float32))
           for sh in (q_shape, kv_shape, kv_shape)]
    return out[0][0], out[1][0], out[2][0], out[0][1], out[1][1], out[2][1]


def workload_inputs(name: str, device="cpu", seed: int | None = None):
    """Inputs of a named workload: dict with q, k, v and the call parameters."""
    w = dict(WORKLOADS[name])
    s = SEEDS[name] if seed is None else seed
    if w["kind"] == "prefill":
        qs = (w["B"], w["Hq"], w["Sq"], w["D"])
    else:
        qs = (w["B"], w["Hq"], w["D"])
    kvs = (w["B"], w["Hkv"], w["Sk"], w["D"])
    q, k, v = draw_qkv(qs, kvs, w["dtype"], s, device)
    w.update(q=q, k=k, v=v, scale=default_scale(w["D"]), seed=s, name=name)
    return w


def to_numpy_exact(t: torch.Tensor):
    """Host copy whose values equal the tensor's bit-exactly (bf16 widens to fp32)."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.numpy()
