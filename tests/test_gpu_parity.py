"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Every test here needs an MI355X and the built library."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_33_amd import ops, synth
from exact_attention_33_amd.synth import to_numpy_exact
from gpu_util import announce, check_lse, check_o

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _prefill_case(B, Hq, Hkv, Sq, Sk, D, causal, window, dtype="bf16", seed=0, scale=None, zero_q=False):
    q, k, v = synth.draw_qkv((B, Hq, Sq, D), (B, Hkv, Sk, D), dtype, seed, DEV)
    if zero_q:
        q.zero_()
    scale = synth.default_scale(D) if scale is None else scale
    fn = ops.attn_fwd if dtype == "bf16" else ops.attn_fwd_f32
    announce(f"prefill B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} D{D} causal{causal} w{window} {dtype} "
             f"scale{scale:.4g} seed{seed}")
    o, lse = fn(q, k, v, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(to_numpy_exact(q), to_numpy_exact(k), to_numpy_exact(v),
                                      scale, bool(causal), window)
    return o, lse, o_ref, lse_ref


def _decode_case(B, Hq, Hkv, Sk, D, ns, seed=0, scale=None):
    q, k, v = synth.draw_qkv((B, Hq, D), (B, Hkv, Sk, D), "bf16", seed, DEV)
    scale = synth.default_scale(D) if scale is None else scale
    announce(f"decode B{B} Hq{Hq} Hkv{Hkv} Sk{Sk} D{D} ns{ns} scale{scale:.4g} seed{seed}")
    o, lse = ops.attn_decode_ex(q, k, v, ns, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(to_numpy_exact(q), to_numpy_exact(k), to_numpy_exact(v), scale)
    return o, lse, o_ref, lse_ref, (q, k, v)


# --------------------------------------------------------------------------
# The five named workloads at full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "causal_prefill", "window_encoder"])
def test_prefill_workload(name):
    w = synth.WORKLOADS[name]
    o, lse, o_ref, lse_ref = _prefill_case(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Sk"], w["D"],
                                           w["causal"], w["window"], w["dtype"], synth.SEEDS[name])
    e = check_o(o, o_ref, w["dtype"], name)
    le = check_lse(lse, lse_ref, w["dtype"], name)
    announce(f"{name}: {e} lse_err {le:.3g}")


@pytest.mark.parametrize("name", ["gqa_decode", "long_decode"])
def test_decode_workload(name):
    w = synth.WORKLOADS[name]
    o, lse, o_ref, lse_ref, (q, k, v) = _decode_case(w["B"], w["Hq"], w["Hkv"], w["Sk"], w["D"],
                                                     w["num_splits"], synth.SEEDS[name])
    e = check_o(o, o_ref, "bf16", name)
    le = check_lse(lse, lse_ref, "bf16", name)
    announce(f"{name}: {e} lse_err {le:.3g}")
    # attn_decode (library workspace, scale 1/sqrt(D)) gives the same bits
    o2 = ops.attn_decode(q, k, v, w["num_splits"])
    torch.cuda.synchronize()
    assert torch.equal(o2, o)


# --------------------------------------------------------------------------
# Ragged and edge shapes, all mask modes, both head dims, both dtypes
# --------------------------------------------------------------------------

PREFILL_SHAPES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, window
    (1, 1, 1, 1, 1, 64, 0, -1),
    (1, 2, 1, 37, 37, 64, 1, -1),
    (2, 4, 2, 200, 200, 128, 1, -1),
    (1, 3, 3, 129, 300, 64, 1, -1),        # Sq < Sk, bottom-right causal
    (1, 2, 2, 300, 129, 128, 1, -1),       # Sq > Sk: leading rows see no key
    (1, 2, 1, 333, 333, 128, 0, -1),
    (2, 8, 1, 257, 191, 64, 0, -1),        # GQA 8:1, ragged
    (1, 4, 4, 500, 500, 64, 0, 64),        # the encoder window on a ragged length
    (1, 2, 2, 260, 260, 128, 0, 0),        # window 0: only the diagonal
    (1, 2, 2, 260, 260, 64, 0, 1),
    (1, 2, 1, 300, 300, 128, 1, 17),       # causal + window
    (1, 2, 2, 100, 140, 64, 0, 33),        # window with Sq != Sk
    (1, 1, 1, 150, 150, 128, 0, 1000),     # window wider than the sequence
    (1, 32, 8, 64, 256, 128, 1, -1),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_shapes(shape, dtype):
    B, Hq, Hkv, Sq, Sk, D, causal, window = shape
    o, lse, o_ref, lse_ref = _prefill_case(B, Hq, Hkv, Sq, Sk, D, causal, window, dtype, seed=11)
    check_o(o, o_ref, dtype, str(shape))
    check_lse(lse, lse_ref, dtype, str(shape))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", [(1, -1), (0, -1), (1, 700)], ids=["causal", "full", "causal_w700"])
def test_chunked_prefill_long_cache(dtype, mode):
    """A block of 256 new query rows against a 16384-key cache (Sq << Sk: row
    i sees keys up to i + Sk - Sq, bottom-right causal alignment), GQA 4:1,
    every row checked against the oracle: many K/V tiles per workgroup, the
    causal diagonal at the far end of the key range."""
    causal, window = mode
    o, lse, o_ref, lse_ref = _prefill_case(1, 8, 2, 256, 16384, 128, causal, window, dtype, seed=21)
    check_o(o, o_ref, dtype, f"chunked prefill {mode}")
    check_lse(lse, lse_ref, dtype, f"chunked prefill {mode}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_peaky(dtype):
    """scale = 1 makes the softmax peaky, so |o| = O(1) and errors are not hidden."""
    for shape in [(2, 4, 2, 300, 300, 128, 1, -1), (1, 4, 4, 400, 400, 64, 0, 64)]:
        B, Hq, Hkv, Sq, Sk, D, causal, window = shape
        o, lse, o_ref, lse_ref = _prefill_case(B, Hq, Hkv, Sq, Sk, D, causal, window, dtype, seed=5,
                                               scale=1.0)
        check_o(o, o_ref, dtype, f"peaky {shape}")
        check_lse(lse, lse_ref, dtype, f"peaky {shape}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_empty_inputs(dtype):
    td = synth.TORCH_DTYPES[dtype]
    fn = ops.attn_fwd if dtype == "bf16" else ops.attn_fwd_f32
    announce(f"prefill empty inputs {dtype}")
    # B = 0 and Sq = 0: nothing to do
    for qs, ks in [((0, 2, 8, 64), (0, 2, 8, 64)), ((1, 2, 0, 64), (1, 2, 8, 64))]:
        q = torch.zeros(qs, dtype=td, device=DEV)
        k = torch.zeros(ks, dtype=td, device=DEV)
        o, lse = fn(q, k, k)
        assert o.shape == q.shape and lse.shape == qs[:3]
    # Sk = 0: every row sees nothing -> o = 0, lse = -inf
    q = torch.randn(1, 2, 5, 64, device=DEV).to(td)
    k = torch.zeros(1, 2, 0, 64, dtype=td, device=DEV)
    o = torch.full_like(q, 7.0)
    o, lse = fn(q, k, k, out=o)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", [(1, -1), (0, 64), (0, 3), (1, 5), (0, -1)])
def test_uniform_scores_window_reading(D, mode):
    """q = 0: o must be the mean of exactly the visible v rows and lse = ln(count),
    with the counts in closed form -- this pins the kernel's mask reading
    (bottom-right causal, inclusive half-width window)."""
    causal, window = mode
    Sq = Sk = 300
    o, lse, _, _ = _prefill_case(1, 2, 2, Sq, Sk, D, causal, window, "bf16", seed=3, zero_q=True)
    q, k, v = synth.draw_qkv((1, 2, Sq, D), (1, 2, Sk, D), "bf16", 3, DEV)
    vn = to_numpy_exact(v).astype(np.float64)
    lse_h = to_numpy_exact(lse)
    o_h = to_numpy_exact(o).astype(np.float64)
    for i in range(Sq):
        if window < 0:
            lo, hi = 0, (i if causal else Sk - 1)
        elif causal:
            lo, hi = i - min(i, window), i
        else:
            lo, hi = i - min(i, window), i + min(Sk - 1 - i, window)
        n = hi - lo + 1
        assert abs(lse_h[0, 0, i] - math.log(n)) < 1e-3, (i, lse_h[0, 0, i], n)
        np.testing.assert_allclose(o_h[0, :, i], vn[0, :, lo:hi + 1].mean(axis=1), atol=2e-2)


# --------------------------------------------------------------------------
# Decode: split counts (non-divisors, empty chunks, = Sk, > 256 partials)
# --------------------------------------------------------------------------

DECODE_SHAPES = [
    # B, Hq, Hkv, Sk, D, num_splits
    (1, 1, 1, 1, 64, 1),
    (2, 4, 4, 7, 128, 7),                 # one key per chunk
    (1, 8, 2, 1000, 128, 3),              # non-divisor
    (2, 8, 2, 1000, 64, 6),               # L = 167: last chunk short
    (1, 4, 1, 10, 128, 6),                # L = 2: chunk 5 empty
    (3, 32, 8, 4097, 128, 64),
    (1, 32, 1, 3000, 128, 16),            # 32 query heads per kv head: two head groups
    (2, 40, 2, 3000, 128, 16),            # 20 per kv head: a full group of 16 and one of 4
    (1, 6, 2, 999, 64, 5),                # 3 per kv head (odd), ragged chunks
    (1, 16, 16, 2048, 64, 1),
    (2, 8, 2, 3000, 128, 65),             # 65 partials: one wavefront's 64 leaves plus one
    (1, 8, 2, 5000, 64, 200),             # four combine wavefronts, the last with 8 leaves
    (832, 1, 1, 8, 64, 2),                # many (b, h) rows, two keys each
    (1, 8, 2, 2000, 128, 300),            # > 256 partials: two combine levels
    (1, 4, 2, 70000, 64, 70000),          # one key per chunk, three combine levels
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_shapes(shape):
    B, Hq, Hkv, Sk, D, ns = shape
    o, lse, o_ref, lse_ref, _ = _decode_case(B, Hq, Hkv, Sk, D, ns, seed=21)
    check_o(o, o_ref, "bf16", str(shape))
    check_lse(lse, lse_ref, "bf16", str(shape))


def test_decode_peaky_and_planted():
    o, lse, o_ref, lse_ref, _ = _decode_case(2, 8, 2, 5000, 128, 13, seed=9, scale=1.0)
    check_o(o, o_ref, "bf16", "peaky decode")
    check_lse(lse, lse_ref, "bf16", "peaky decode")
    # planted key: k_j = 4 q / |q| * sqrt(D) makes key j dominate for its head group
    B, Hq, Hkv, Sk, D = 1, 4, 1, 20000, 128
    q, k, v = synth.draw_qkv((B, Hq, D), (B, Hkv, Sk, D), "bf16", 13, DEV)
    qf = q.float()
    j = 12345
    k[0, 0, j] = (4.0 * qf[0, 0] / qf[0, 0].norm() * math.sqrt(D)).to(torch.bfloat16)
    announce("decode planted key")
    o, lse = ops.attn_decode_ex(q, k, v, 32)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode(to_numpy_exact(q), to_numpy_exact(k), to_numpy_exact(v), 1 / math.sqrt(D))
    check_o(o, o_ref, "bf16", "planted")
    check_lse(lse, lse_ref, "bf16", "planted")


def test_binding_rejects_bad_workspace_and_lse():
    """The binding refuses, before any launch, a workspace of the wrong dtype
    or in host memory and an lse of the wrong shape."""
    announce("binding checks")
    q, k, v = synth.draw_qkv((2, 4, 128), (2, 2, 100, 128), "bf16", 3, DEV)
    with pytest.raises(ValueError):
        ops.attn_decode_ex(q, k, v, 4, workspace=torch.zeros(1 << 20, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        ops.attn_decode_ex(q, k, v, 4, workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        ops.attn_decode_ex(q, k, v, 4, lse=torch.empty(2, 5, device=DEV))
    o, _ = ops.attn_decode_ex(q, k, v, 4, workspace=torch.zeros(1 << 20, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_decode_library_workspace_grows():
    """attn_decode's own workspace grows on demand: a small call, a call that
    needs more, then a small one again each give attn_decode_ex's bits."""
    for i, (B, Hq, Hkv, Sk, ns) in enumerate([(1, 4, 1, 500, 3), (8, 32, 8, 4000, 200), (2, 8, 2, 900, 5)]):
        q, k, v = synth.draw_qkv((B, Hq, 128), (B, Hkv, Sk, 128), "bf16", 40 + i, DEV)
        announce(f"attn_decode library workspace B{B} Hq{Hq} Hkv{Hkv} Sk{Sk} ns{ns}")
        o1 = ops.attn_decode(q, k, v, ns)
        o2, _ = ops.attn_decode_ex(q, k, v, ns)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


def test_decode_empty_cache():
    announce("decode Sk = 0")
    q = torch.randn(2, 4, 128, device=DEV).to(torch.bfloat16)
    kc = torch.zeros(2, 2, 0, 128, dtype=torch.bfloat16, device=DEV)
    o = torch.full_like(q, 3.0)
    o, lse = ops.attn_decode_ex(q, kc, kc, 1, out=o)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


# --------------------------------------------------------------------------
# Run-to-run determinism, output bounds, streams
# --------------------------------------------------------------------------

def test_deterministic_bits():
    announce("determinism")
    q, k, v = synth.draw_qkv((2, 8, 777, 128), (2, 4, 777, 128), "bf16", 4, DEV)
    o1, l1 = ops.attn_fwd(q, k, v, causal=True)
    o2, l2 = ops.attn_fwd(q, k, v, causal=True)
    qd, kd, vd = synth.draw_qkv((4, 16, 128), (4, 4, 9000, 128), "bf16", 4, DEV)
    d1, dl1 = ops.attn_decode_ex(qd, kd, vd, 37)
    d2, dl2 = ops.attn_decode_ex(qd, kd, vd, 37)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(d1, d2) and torch.equal(dl1, dl2)


def test_writes_stay_in_bounds():
    """Outputs are views into larger buffers filled with a sentinel; the
    sentinel outside the view must survive."""
    announce("guard bands")
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 201, 201, 128
    q, k, v = synth.draw_qkv((B, Hq, Sq, D), (B, Hkv, Sk, D), "bf16", 8, DEV)
    n = B * Hq * Sq * D
    buf = torch.full((n + 4096,), -123.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((B * Hq * Sq + 512,), -77.0, dtype=torch.float32, device=DEV)
    o = buf[:n].view(B, Hq, Sq, D)
    lse = lbuf[:B * Hq * Sq].view(B, Hq, Sq)
    ops.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    qd, kd, vd = synth.draw_qkv((3, 8, D), (3, 2, 999, D), "bf16", 8, DEV)
    nd = 3 * 8 * D
    dbuf = torch.full((nd + 2048,), -55.0, dtype=torch.bfloat16, device=DEV)
    ops.attn_decode_ex(qd, kd, vd, 7, out=dbuf[:nd].view(3, 8, D))
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == -123.0) and torch.all(lbuf[B * Hq * Sq:] == -77.0)
    assert torch.all(dbuf[nd:] == -55.0)
    assert not torch.any(buf[:n] == -123.0)


def test_runs_on_the_callers_stream():
    announce("non-default stream")
    q, k, v = synth.draw_qkv((1, 4, 300, 64), (1, 4, 300, 64), "bf16", 2, DEV)
    ref, _ = ops.attn_fwd(q, k, v)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, _ = ops.attn_fwd(q, k, v)
    s.synchronize()
    assert torch.equal(o, ref)


def test_graph_replay():
    """The prefill (bf16 and fp32), the fp8 prefill, the backward, the decode
    (caller workspace) and the allocation-free decode captured in one HIP
    graph: every replay, with eager work and synchronisations between
    replays, gives the eager results bit for bit."""
    announce("graph capture and replay")
    q, k, v = synth.draw_qkv((2, 4, 333, 128), (2, 2, 333, 128), "bf16", 5, DEV)
    qf, kf, vf = synth.draw_qkv((1, 2, 150, 64), (1, 1, 150, 64), "f32", 9, DEV)
    q8, k8, v8, qd, kd, vd = synth.draw_qkv_fp8((1, 4, 200, 64), (1, 4, 200, 64), 6, DEV)
    qd1, kd1, vd1 = synth.draw_qkv((4, 8, 128), (4, 2, 3000, 128), "bf16", 7, DEV)
    do = synth.draw_grad(q.shape, "bf16", 8, DEV)
    ns = 37
    ws = torch.zeros(ops.decode_workspace_bytes(4, 8, 128, ns), dtype=torch.uint8, device=DEV)
    bufs = dict(o=torch.empty_like(q), lse=torch.empty(2, 4, 333, device=DEV),
                o8=torch.empty(1, 4, 200, 64, dtype=torch.bfloat16, device=DEV),
                lse8=torch.empty(1, 4, 200, device=DEV),
                od=torch.empty_like(qd1), lsed=torch.empty(4, 8, device=DEV),
                dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                delta=torch.empty(2, 4, 333, device=DEV),
                of=torch.empty_like(qf), lsef=torch.empty(1, 2, 150, device=DEV),
                on=torch.empty_like(qd1), lsen=torch.empty(4, 8, device=DEV))

    def work():
        ops.attn_fwd(q, k, v, causal=True, out=bufs["o"], lse=bufs["lse"])
        ops.attn_fwd_fp8(q8, k8, v8, qd, kd, vd, window=17, out=bufs["o8"], lse=bufs["lse8"])
        ops.attn_bwd(q, k, v, bufs["o"], do, bufs["lse"], causal=True, dq=bufs["dq"], dk=bufs["dk"],
                     dv=bufs["dv"], delta=bufs["delta"])
        ops.attn_decode_ex(qd1, kd1, vd1, ns, out=bufs["od"], lse=bufs["lsed"], workspace=ws)
        ops.attn_fwd_f32(qf, kf, vf, causal=True, out=bufs["of"], lse=bufs["lsef"])
        ops.attn_decode_noalloc(qd1, kd1, vd1, 21, bufs["on"], lse=bufs["lsen"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # eager, on the capture stream
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in bufs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        work()
    for rep in range(3):
        for t in bufs.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in bufs.items():
            assert torch.equal(t, ref[n]), (rep, n)
        work()  # eager work between replays
        torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Encoder stack pattern: the global layer of the window-encoder shape
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [1, 0])
def test_long_prefill_sampled_rows(causal):
    """One long sequence, B1 H16 S8192 D128 (the benchmark's long-prefill
    line), checked on sampled rows including tile edges and both ends."""
    B, H, S, D = 1, 16, 8192, 128
    q, k, v = synth.draw_qkv((B, H, S, D), (B, H, S, D), "bf16", 9, DEV)
    scale = synth.default_scale(D)
    announce(f"long prefill B1 H16 S8192 D128 causal{causal}, sampled rows")
    o, lse = ops.attn_fwd(q, k, v, causal=bool(causal), scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 255, 256, 4095, 4096, 8190, 8191])
    o_ref, lse_ref = oracle.attention(to_numpy_exact(q), to_numpy_exact(k), to_numpy_exact(v), scale,
                                      bool(causal), -1, rows=rows)
    e = check_o(o[:, :, rows], o_ref, "bf16", "long prefill")
    le = check_lse(lse[:, :, rows], lse_ref, "bf16", "long prefill")
    announce(f"long prefill: {e} lse_err {le:.3g}")


def test_encoder_global_layer_sampled_rows():
    """Full attention (no mask) at the window-encoder shape B8 H12 S8192 D64,
    the global layer that the local/global encoder pattern interleaves with
    the windowed one; checked on sampled rows (the oracle computes them one
    by one), including the first and last rows."""
    w = synth.WORKLOADS["window_encoder"]
    q, k, v = synth.draw_qkv((w["B"], w["Hq"], w["Sq"], w["D"]), (w["B"], w["Hkv"], w["Sk"], w["D"]), "bf16",
                             synth.SEEDS["window_encoder"], DEV)
    scale = synth.default_scale(w["D"])
    announce("encoder global layer B8 H12 S8192 D64 (no mask), sampled rows")
    o, lse = ops.attn_fwd(q, k, v, causal=False, window=-1, scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 127, 128, 4095, 4096, 8190, 8191])
    o_ref, lse_ref = oracle.attention(to_numpy_exact(q), to_numpy_exact(k), to_numpy_exact(v), scale, False, -1,
                                      rows=rows)
    e = check_o(o[:, :, rows], o_ref, "bf16", "global layer")
    le = check_lse(lse[:, :, rows], lse_ref, "bf16", "global layer")
    announce(f"global layer: {e} lse_err {le:.3g}")
