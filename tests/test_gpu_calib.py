"""The measurement reference kernels on the GPU: the stream kernel's output is
the XOR it documents, and the MFMA loop runs and writes finite values."""

import pytest
import torch

from exact_attention_33_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("reps,chunks", [(1, 1000), (3, 4096 + 7), (256, 512)])
def test_stream_xor(reps, chunks):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(reps)
    src = torch.randint(-2**31, 2**31 - 1, (reps, chunks, 4), generator=g, device=dev, dtype=torch.int32)
    dst = torch.full((chunks, 4), 7, dtype=torch.int32, device=dev)
    ops.calib_stream(src, dst)
    want = src[0].clone()
    for r in range(1, reps):
        want ^= src[r]
    torch.cuda.synchronize()
    assert torch.equal(dst, want)


def test_stream_write_only():
    dev = torch.device("cuda:0")
    dst = torch.full((333, 4), 7, dtype=torch.int32, device=dev)
    ops.calib_stream(torch.empty(0, dtype=torch.int32, device=dev), dst)
    torch.cuda.synchronize()
    assert int(dst.abs().sum()) == 0


def test_mfma_loop():
    dev = torch.device("cuda:0")
    out = torch.zeros(4 * 8, dtype=torch.float32, device=dev)
    flops = ops.calib_mfma(out, 8, 100)
    torch.cuda.synchronize()
    assert flops == 2.0 * 32 * 32 * 16 * 16 * 100 * 8
    assert bool(torch.isfinite(out).all()) and float(out.abs().min()) > 0


# --------------------------------------------------------------------------
# The fp8 matrix instruction's accumulation precision.  The fp8 prefill's lse
# tolerance (tests/test_gpu_fp8.py) assumes that one
# v_mfma_scale_f32_32x32x64_f8f6f4 returns each of its 64-product dot products
# within 2^-14 * |a_m| * |b_n| (Euclidean norms of the row and column) of the
# exact value, plus the final fp32 rounding.  These constructed operands
# check that assumption on the instruction itself, including sums where the
# partial sums need far more than 24 bits.
# --------------------------------------------------------------------------

def _codes_of(values):
    """e4m3 codes of values that are exactly representable."""
    t = torch.tensor(values, dtype=torch.float32).to(torch.float8_e4m3fn)
    assert torch.equal(t.float(), torch.tensor(values, dtype=torch.float32)), "not representable"
    return t.view(torch.uint8)


def _fp8_cases():
    g = torch.Generator()
    g.manual_seed(1234)
    cases = {}
    # small values whose every partial sum is exact: checks the lane layout
    vals = torch.tensor([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0])
    cases["layout"] = (_codes_of(vals[torch.randint(0, 7, (32, 64), generator=g)].tolist()),
                       _codes_of(vals[torch.randint(0, 7, (32, 64), generator=g)].tolist()))
    # one large product and 63 tiny ones (b = 1): the tiny ones need 17+ bits
    # below the large one
    a = torch.full((32, 64), 2.0 ** -9)
    for m in range(32):
        a[m, m % 64] = 448.0
        a[m, (m + 32) % 64] = 2.0 ** -(m % 8)
    cases["big_plus_tiny"] = (_codes_of(a.tolist()), _codes_of(torch.ones(32, 64).tolist()))
    # exact cancellation of the two largest products, small remainder
    a = torch.full((32, 64), 2.0 ** -6)
    a[:, 0], a[:, 1] = 448.0, -448.0
    b = torch.ones(32, 64)
    b[:, 2:] = torch.where(torch.rand(32, 62, generator=g) < 0.5, 1.0, -1.0)
    cases["cancellation"] = (_codes_of(a.tolist()), _codes_of(b.tolist()))
    # attention-like operands: N(0, 1) rows quantized with a per-tensor scale
    for name, sd in (("gaussian", 1.0), ("gaussian_wide", 30.0)):
        x = (torch.randn(2, 32, 64, generator=g) * sd)
        x = (x / (x.abs().max() / 448.0)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        cases[name] = (x[0].contiguous(), x[1].contiguous())
    # every finite code equally likely (NaN codes 0x7f, 0xff excluded)
    c = torch.randint(0, 254, (2, 32, 64), generator=g, dtype=torch.int32)
    c = torch.where(c >= 0x7f, c + 1, c).to(torch.uint8)
    cases["all_codes"] = (c[0].contiguous(), c[1].contiguous())
    return cases


@pytest.mark.parametrize("name", ["layout", "big_plus_tiny", "cancellation", "gaussian", "gaussian_wide",
                                  "all_codes"])
def test_fp8_mfma_accumulation_precision(name):
    import numpy as np

    import oracle
    from gpu_util import announce

    a8, b8 = _fp8_cases()[name]
    dev = torch.device("cuda:0")
    c = ops.calib_mfma_fp8(a8.to(dev), b8.to(dev))
    torch.cuda.synchronize()
    a = oracle.e4m3_decode(a8.numpy())
    b = oracle.e4m3_decode(b8.numpy())
    exact = a @ b.T                                     # fp64: exact for 64 e4m3 products
    got = c.cpu().numpy().astype(np.float64)
    err = np.abs(got - exact)
    norms = np.linalg.norm(a, axis=1)[:, None] * np.linalg.norm(b, axis=1)[None, :]
    absum = np.abs(a) @ np.abs(b).T
    bound = 2.0 ** -14 * norms + 2.0 ** -24 * absum
    ratio = float((err / np.where(norms > 0, norms, 1)).max())
    announce(f"fp8 mfma {name}: max err {err.max():.3g}, max err/(|a||b|) {ratio:.3g} "
             f"(= 2^{np.log2(ratio) if ratio > 0 else float('-inf'):.1f}), "
             f"max err/sum|ab| {float((err / np.where(absum > 0, absum, 1)).max()):.3g}")
    if name == "layout":
        assert np.array_equal(got, exact)
    assert np.all(err <= bound), float((err - bound).max())
