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
