"""Benchmark of the exact-attention hot path on one MI355X.

One step = one causal prefill (B=4, H=16, S=2048, D=128, bf16) plus one
split-KV GQA decode (B=16, Hq=32, Hkv=8, Sk=32768, D=128, 64 splits, bf16):
the prefill kernel plus the decode split and tree-combine kernels.  The timed
region runs the K steps' prefills back to back, then their decodes, so each
kernel is measured in its steady state; the same steps run interleaved are
reported alongside ("interleaved").

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --only WORKLOAD [--steps K] [--warmup W]   (one workload, for profilers)

Prints ONE JSON line.  `value` is the mean of the two roofline fractions, in
percent: prefill TFLOP/s over the dense bf16 MFMA peak and decode KV GB/s over
the HBM peak.  Per-call durations come from HIP events recorded on the stream
the kernels are launched on, inside the timed region; each series is reported
with its mean, median and 10th/90th percentiles.  Two plain reference kernels
built into the library (an HBM stream and an MFMA loop) give the achievable
rates, and every rate is also stated as a fraction of those.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
WARM_MS = 50.0               # minimum untimed busy time before a timed series

PREFILL = "causal_prefill"
DECODE = "gqa_decode"
KERNEL_SOURCES = ["fwd_bf16.hip", "fwd_fp8.hip", "decode.hip", "bwd.hip", "common.h"]


def progress(msg: str):
    """One line per finished phase on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs_causal(Sq: int, Sk: int) -> int:
    """Number of (query, key) pairs a bottom-right causal mask keeps."""
    off = Sk - Sq
    return sum(max(0, min(Sk, i + off + 1)) for i in range(Sq))


def prefill_flops(w) -> float:
    pairs = visible_pairs_causal(w["Sq"], w["Sk"])
    return 4.0 * w["D"] * pairs * w["B"] * w["Hq"]


def decode_kv_bytes(w) -> float:
    return 2.0 * w["B"] * w["Hkv"] * w["Sk"] * w["D"] * 2


def launch_stats(ms):
    """Mean, median and 10th/90th percentiles of per-launch durations (ms)."""
    v = sorted(ms)
    n = len(v)

    def pct(p):
        return v[min(n - 1, int(round(p * (n - 1))))]

    return {"n": n, "avg_ms": round(sum(v) / n, 5), "median_ms": round(pct(0.5), 5),
            "p10_ms": round(pct(0.1), 5), "p90_ms": round(pct(0.9), 5)}


def time_launches(fn, iters: int, stream, warm: int = 10, warm_ms: float = WARM_MS):
    """Per-launch durations (ms) of fn(i), HIP events recorded on `stream`.

    Untimed warm-up: `warm` launches, then more until `warm_ms` of wall time
    has passed with the GPU busy, so the timed launches run at the clock a
    sustained load settles at (after short warm-ups the same kernel measured
    up to 18 % slower)."""
    import time

    import torch

    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def scores_bytes_avoided(B: int, Hq: int, Sq: int, Sk: int) -> float:
    """HBM bytes of the Sq x Sk score matrix that standard attention moves and the
    fused kernels never do: S written and read back, P written and read back (bf16)."""
    return 4.0 * 2 * B * Hq * Sq * Sk


def achievable(dev):
    """Rates of the library's plain reference kernels on this GPU: an HBM read
    stream, a 3-read/1-write stream (the prefill's q, k, v -> o mix) and a bf16
    MFMA loop.  Each is the median of several launches after a warm-up."""
    import torch

    from exact_attention_33_amd import ops

    stream = torch.cuda.current_stream(dev)
    out = {}
    mib = 1 << 20
    src = torch.empty(2048 * mib, dtype=torch.uint8, device=dev)
    dst = torch.empty(8 * mib, dtype=torch.uint8, device=dev)
    ms = launch_stats(time_launches(lambda i: ops.calib_stream(src, dst), 10, stream, warm=5))["median_ms"]
    out["hbm_read_gbs"] = round((src.numel() + dst.numel()) / (ms * 1e-3) / 1e9, 1)
    del src, dst
    src = torch.empty(3 * 256 * mib, dtype=torch.uint8, device=dev)
    dst = torch.empty(256 * mib, dtype=torch.uint8, device=dev)
    ms = launch_stats(time_launches(lambda i: ops.calib_stream(src, dst), 10, stream, warm=5))["median_ms"]
    out["hbm_3read_1write_gbs"] = round((src.numel() + dst.numel()) / (ms * 1e-3) / 1e9, 1)
    del src, dst
    wg, iters = 2048, 4000
    o = torch.empty(4 * wg, dtype=torch.float32, device=dev)
    flops = [0.0]

    def run(i):
        flops[0] = ops.calib_mfma(o, wg, iters)

    ms = launch_stats(time_launches(run, 10, stream, warm=5))["median_ms"]
    out["mfma_bf16_tflops"] = round(flops[0] / (ms * 1e-3) / 1e12, 1)
    out["note"] = ("attn_calib_stream over 2 GiB (read) and 3 x 256 MiB -> 256 MiB (3:1); attn_calib_mfma: "
                   f"{wg} workgroups x 4 wavefronts x {iters} x 4 v_mfma_f32_32x32x16_bf16")
    torch.cuda.empty_cache()
    return out


def source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_33_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(kind)
    if not entry or entry.get("source_digest") != source_digest():
        return None
    return entry.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("version"), i.get("num_threads")) for i in threadpool_info()]
        threads = max([n for _, _, n in blas if n] or [1])
    except Exception:  # noqa: BLE001
        blas, threads = [], 1
    return blas, threads


def _oracle_slabs(name: str, w):
    """Slabs of a workload the fp64 oracle runs one at a time, each a tuple
    (q, k, v, call-args) of device tensors: one batch row per slab for the
    prefills and the batched decode, one kv head (with its query heads) for the
    long decode, so host memory stays near one slab (about 2 GiB in fp64)."""
    if w["kind"] == "prefill":
        for b in range(w["B"]):
            yield w["q"][b:b + 1], w["k"][b:b + 1], w["v"][b:b + 1]
    elif w["B"] > 1:
        for b in range(w["B"]):
            yield w["q"][b:b + 1], w["k"][b:b + 1], w["v"][b:b + 1]
    else:
        G = w["Hq"] // w["Hkv"]
        for g in range(w["Hkv"]):
            yield (w["q"][:, g * G:(g + 1) * G], w["k"][:, g:g + 1], w["v"][:, g:g + 1])


def cpu_baseline(dev):
    """The fp64 oracle, untuned, on every workload in full: each workload's
    own seeded inputs (the ones the GPU computes on), copied to the host one
    slab at a time; only the oracle calls are timed (time.perf_counter)."""
    import torch

    import oracle
    from exact_attention_33_amd import synth

    blas, threads = _blas_info()
    per = {}
    for name in synth.WORKLOADS:
        w = synth.workload_inputs(name, dev)
        secs = 0.0
        for q, k, v in _oracle_slabs(name, w):
            qn, kn, vn = (synth.to_numpy_exact(t) for t in (q, k, v))
            t0 = time.perf_counter()
            if w["kind"] == "prefill":
                oracle.attention(qn, kn, vn, w["scale"], bool(w["causal"]), w["window"])
            else:
                oracle.decode(qn, kn, vn, w["scale"])
            secs += time.perf_counter() - t0
            del qn, kn, vn
        progress(f"cpu oracle {name}: {secs:.2f} s")
        if w["kind"] == "prefill":
            fl = (window_flops(w) if w["window"] >= 0 else
                  prefill_flops(w) if w["causal"] else 4.0 * w["D"] * w["Sq"] * w["Sk"] * w["B"] * w["Hq"])
            per[name] = {"seconds": round(secs, 3), "gflops": round(fl / secs / 1e9, 3),
                         "algorithmic_flops": fl}
        else:
            kv = decode_kv_bytes(w)
            per[name] = {"seconds": round(secs, 3), "kv_gbs": round(kv / secs / 1e9, 3),
                         "algorithmic_bytes": kv}
        del w
        torch.cuda.empty_cache()
    p_tflops = per[PREFILL]["gflops"] / 1e3
    d_gbs = per[DECODE]["kv_gbs"]
    value = 100.0 * 0.5 * (p_tflops / PEAK_BF16_TFLOPS + d_gbs / PEAK_HBM_GBS)
    total = sum(e["seconds"] for e in per.values())
    return {
        "value": value, "unit": "% of MI355X peak (mean of prefill MFMA and decode HBM fractions)",
        "cores": threads, "kind": "oracle",
        "sample": (f"fp64 numpy oracle, one full wall-clock run of each of the five workloads on their own "
                   f"seeded inputs ({total:.1f} s of oracle time in all; slabs of one batch row, or one kv "
                   f"head for the long decode, copied to the host one at a time); value from the causal "
                   f"prefill ({per[PREFILL]['gflops']:.1f} GFLOP/s) and the GQA decode "
                   f"({d_gbs:.2f} GB/s of bf16 KV)"),
        "per_config": per,
        "affinity_cores": len(os.sched_getaffinity(0)), "blas": blas, "cpu_model": cpu_model(),
    }


def window_bytes(w) -> float:
    """q, k, v read once and o written once (bf16) plus lse (fp32)."""
    n = w["B"] * w["Hq"] * w["Sq"] * w["D"]
    return 4.0 * n * 2 + w["B"] * w["Hq"] * w["Sq"] * 4


def window_flops(w) -> float:
    S, wd = w["Sq"], w["window"]
    pairs = sum(min(S - 1, i + wd) - max(0, i - wd) + 1 for i in range(S))
    return 4.0 * w["D"] * pairs * w["B"] * w["Hq"]


def other_configs(dev, ach, iters: int = 50):
    """The sliding-window encoder, the long-context decode, the encoder-stack
    pattern and the causal-prefill backward at full size, timed with HIP events
    (reported beside the headline, not in it).  The window encoder's inputs
    and outputs (402 MB) would otherwise sit in the 256 MB last-level cache
    between launches, so launches rotate over three copies of them."""
    import torch

    from exact_attention_33_amd import ops, synth

    out = {}
    stream = torch.cuda.current_stream(dev)
    # the tiny fp32 workload is launch-latency bound: per-launch GPU time by
    # events, and the host's round trip (enqueue, then wait for completion)
    wt = synth.workload_inputs("tiny_f32", dev)
    ot = torch.empty_like(wt["q"])
    lt = torch.empty(wt["B"], wt["Hq"], wt["Sq"], dtype=torch.float32, device=dev)

    def run_t(i):
        ops.attn_fwd_f32(wt["q"], wt["k"], wt["v"], causal=False, scale=wt["scale"], out=ot, lse=lt)

    st_ev = launch_stats(time_launches(run_t, 200, stream))
    rt = []
    for _ in range(200):
        t0 = time.perf_counter()
        run_t(0)
        torch.cuda.synchronize()
        rt.append((time.perf_counter() - t0) * 1e3)
    out["tiny_f32"] = {
        "shape": {k: wt[k] for k in ("B", "Hq", "Sq", "Sk", "D")}, "dtype": "f32", "bound": "latency",
        "gpu_launch_ms": st_ev, "host_roundtrip_ms": launch_stats(rt),
        "algorithmic_flops": 4.0 * wt["D"] * wt["Sq"] * wt["Sk"],
        "note": "gpu_launch_ms: HIP events around each launch; host_roundtrip_ms: the call plus "
                "torch.cuda.synchronize(), wall clock",
    }
    del wt, ot, lt
    ww = synth.workload_inputs("window_encoder", dev)
    copies = []
    for c in range(3):
        q, k, v = (ww[n] if c == 0 else ww[n].clone() for n in ("q", "k", "v"))
        copies.append((q, k, v, torch.empty_like(q),
                       torch.empty(ww["B"], ww["Hq"], ww["Sq"], dtype=torch.float32, device=dev)))

    def run_w(i, window=ww["window"]):
        q, k, v, o, lse = copies[i % 3]
        ops.attn_fwd(q, k, v, causal=False, window=window, scale=ww["scale"], out=o, lse=lse)

    st = launch_stats(time_launches(run_w, iters, stream))
    ms = st["avg_ms"]
    nbytes = window_bytes(ww)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out["window_encoder"] = {
        "shape": {k: ww[k] for k in ("B", "Hq", "Sq", "D", "window")},
        "avg_launch_ms": ms, "launch_ms": st,
        "bound": "hbm", "achieved_gbs": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "frac_of_achievable": round(gbs / ach["hbm_3read_1write_gbs"], 4),
        "algorithmic_bytes": nbytes, "traffic": measured_traffic("window_encoder"),
        "tflops": round(window_flops(ww) / (ms * 1e-3) / 1e12, 1),
        "scores_bytes_avoided": scores_bytes_avoided(ww["B"], ww["Hq"], ww["Sq"], ww["Sq"]),
        "inputs": "three copies of q, k, v, o, lse, rotated per launch",
    }

    # encoder stack pattern at the window-encoder shape: a global (unmasked)
    # layer every third layer, windowed layers otherwise (no new kernel)
    stg = launch_stats(time_launches(lambda i: run_w(i, window=-1), 10, stream, warm=3))
    g_ms = stg["avg_ms"]
    S, D_ = ww["Sq"], ww["D"]
    g_fl = 4.0 * D_ * S * S * ww["B"] * ww["Hq"]
    out["encoder_stack"] = {
        "pattern": "one global layer (window -1) then two local layers (window 64), ModernBERT-style",
        "shape": {k: ww[k] for k in ("B", "Hq", "Sq", "D")},
        "global_layer_ms": g_ms, "global_launch_ms": stg,
        "global_layer_tflops": round(g_fl / (g_ms * 1e-3) / 1e12, 1),
        "global_frac_of_achievable_mfma": round(g_fl / (g_ms * 1e-3) / 1e12 / ach["mfma_bf16_tflops"], 4),
        "local_layer_ms": ms, "three_layer_attention_ms": round(g_ms + 2 * ms, 4),
        "global_traffic": measured_traffic("global_layer"),
    }
    # the window encoder on fp8 (e4m3) q, k, v: a third fewer bytes to read
    copies8 = []
    for c in range(3):
        q8, k8, v8, qd, kd, vd = synth.draw_qkv_fp8(ww["q"].shape, ww["k"].shape, ww["seed"] + c, dev)
        copies8.append((q8, k8, v8, qd, kd, vd, torch.empty_like(ww["q"]),
                        torch.empty(ww["B"], ww["Hq"], ww["Sq"], dtype=torch.float32, device=dev)))

    def run_w8(i):
        q8, k8, v8, qd, kd, vd, o, lse = copies8[i % 3]
        ops.attn_fwd_fp8(q8, k8, v8, qd, kd, vd, causal=False, window=ww["window"], scale=ww["scale"], out=o,
                         lse=lse)

    st8 = launch_stats(time_launches(run_w8, iters, stream))
    n = ww["B"] * ww["Hq"] * ww["Sq"] * ww["D"]
    nbytes8 = 3.0 * n + 2.0 * n + ww["B"] * ww["Hq"] * ww["Sq"] * 4
    gbs8 = nbytes8 / (st8["avg_ms"] * 1e-3) / 1e9
    out["fp8_window_encoder"] = {
        "shape": {k: ww[k] for k in ("B", "Hq", "Sq", "D", "window")},
        "avg_launch_ms": st8["avg_ms"], "launch_ms": st8,
        "bound": "hbm", "achieved_gbs": round(gbs8, 1),
        "frac_of_hbm_peak": round(gbs8 / PEAK_HBM_GBS, 4),
        "frac_of_achievable": round(gbs8 / ach["hbm_3read_1write_gbs"], 4),
        "algorithmic_bytes": nbytes8, "traffic": measured_traffic("fp8_window_encoder"),
        "inputs": "three copies of the e4m3 q, k, v and of o, lse, rotated per launch",
    }
    del copies, copies8, ww

    wl = synth.workload_inputs("long_decode", dev)
    od = torch.empty_like(wl["q"])
    lsed = torch.empty(wl["B"], wl["Hq"], dtype=torch.float32, device=dev)
    ws = torch.empty(ops.decode_workspace_bytes(wl["B"], wl["Hq"], wl["D"], wl["num_splits"]),
                     dtype=torch.uint8, device=dev)

    def run_l(i):
        ops.attn_decode_ex(wl["q"], wl["k"], wl["v"], wl["num_splits"], scale=wl["scale"], out=od,
                           lse=lsed, workspace=ws)

    st = launch_stats(time_launches(run_l, 20, stream))
    ms = st["avg_ms"]
    kv = decode_kv_bytes(wl)
    gbs = kv / (ms * 1e-3) / 1e9
    out["long_decode"] = {
        "shape": {k: wl[k] for k in ("B", "Hq", "Hkv", "Sk", "D", "num_splits")},
        "avg_launch_ms": ms, "launch_ms": st,
        "bound": "hbm", "achieved_gbs": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "frac_of_achievable": round(gbs / ach["hbm_read_gbs"], 4),
        "algorithmic_bytes": kv, "traffic": measured_traffic("long_decode"),
        "scores_bytes_avoided": scores_bytes_avoided(wl["B"], wl["Hq"], 1, wl["Sk"]),
    }
    del wl, od, lsed, ws

    # backward of the causal prefill (dq, dk, dv from the forward's o and lse)
    wp = synth.workload_inputs(PREFILL, dev)
    do = synth.draw_grad(wp["q"].shape, "bf16", wp["seed"], dev)
    op, lp = ops.attn_fwd(wp["q"], wp["k"], wp["v"], causal=True, scale=wp["scale"])
    dq, dk, dv = torch.empty_like(wp["q"]), torch.empty_like(wp["k"]), torch.empty_like(wp["v"])
    delta = torch.empty_like(lp)

    def run_b(i):
        ops.attn_bwd(wp["q"], wp["k"], wp["v"], op, do, lp, causal=True, scale=wp["scale"], dq=dq, dk=dk,
                     dv=dv, delta=delta)

    st = launch_stats(time_launches(run_b, iters, stream))
    ms = st["avg_ms"]
    fl = 2.5 * prefill_flops(wp)   # five products of the forward's size: S, dP, dV, dK, dQ
    tf = fl / (ms * 1e-3) / 1e12
    out["causal_prefill_backward"] = {
        "shape": {k: wp[k] for k in ("B", "Hq", "Hkv", "Sq", "D")}, "avg_launch_ms": ms, "launch_ms": st,
        "bound": "mfma", "tflops": round(tf, 1),
        "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "frac_of_achievable": round(tf / ach["mfma_bf16_tflops"], 4), "algorithmic_flops": fl,
        "traffic": measured_traffic("backward"),
        "note": "dq kernel + dk/dv kernel; algorithmic work counts S, dP, dV, dK, dQ once (the kernels "
                "recompute S and dP in both passes)",
    }
    # one long sequence through the same prefill kernel (B1 H16 S8192 D128),
    # where the per-workgroup start and end weigh less than at S = 2048
    ql, kl, vl = synth.draw_qkv((1, 16, 8192, 128), (1, 16, 8192, 128), "bf16", 9, dev)
    ol = torch.empty_like(ql)
    ll = torch.empty(1, 16, 8192, dtype=torch.float32, device=dev)
    for causal in (1, 0):
        stl = launch_stats(time_launches(
            lambda i: ops.attn_fwd(ql, kl, vl, causal=bool(causal), scale=wp["scale"], out=ol, lse=ll), 20, stream))
        wl_ = dict(B=1, Hq=16, Sq=8192, Sk=8192, D=128)
        fl = prefill_flops(wl_) if causal else 4.0 * 128 * 8192 * 8192 * 16
        tf = fl / (stl["avg_ms"] * 1e-3) / 1e12
        out["long_prefill_causal" if causal else "long_prefill"] = {
            "shape": {**wl_, "causal": causal}, "avg_launch_ms": stl["avg_ms"], "launch_ms": stl,
            "bound": "mfma", "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "frac_of_achievable": round(tf / ach["mfma_bf16_tflops"], 4), "algorithmic_flops": fl,
        }
    del ql, kl, vl, ol, ll
    # the causal prefill on fp8 (e4m3) inputs, one descale per tensor
    q8, k8, v8, qd, kd, vd = synth.draw_qkv_fp8(wp["q"].shape, wp["k"].shape, wp["seed"], dev)
    o8 = torch.empty_like(wp["q"])

    def run_f(i):
        ops.attn_fwd_fp8(q8, k8, v8, qd, kd, vd, causal=True, scale=wp["scale"], out=o8, lse=lp)

    st = launch_stats(time_launches(run_f, iters, stream))
    ms = st["avg_ms"]
    fl = prefill_flops(wp)
    tf = fl / (ms * 1e-3) / 1e12
    out["fp8_causal_prefill"] = {
        "shape": {k: wp[k] for k in ("B", "Hq", "Hkv", "Sq", "D")}, "avg_launch_ms": ms, "launch_ms": st,
        "bound": "mfma", "tflops": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
        "frac_of_mfma_peak": round(tf / PEAK_FP8_TFLOPS, 4), "algorithmic_flops": fl,
        "traffic": measured_traffic("fp8_prefill"),
        "note": "q, k, v as e4m3 codes with per-tensor descales; p rounded to e4m3 for the p.v product",
    }
    del wp, do, op, lp, dq, dk, dv, delta, q8, k8, v8, o8
    torch.cuda.empty_cache()
    return out


def run_only(name: str, steps: int, warmup: int, dev):
    """Run one workload alone (warm-up, then `steps` timed launches) and print
    its launch statistics: the command profilers wrap."""
    import torch

    from exact_attention_33_amd import ops, synth

    stream = torch.cuda.current_stream(dev)
    if name == "fp8_window_encoder":
        w = synth.workload_inputs("window_encoder", dev)
        cps = []
        for c in range(3):
            q8, k8, v8, qd, kd, vd = synth.draw_qkv_fp8(w["q"].shape, w["k"].shape, w["seed"] + c, dev)
            cps.append((q8, k8, v8, qd, kd, vd, torch.empty_like(w["q"]),
                        torch.empty(w["B"], w["Hq"], w["Sq"], dtype=torch.float32, device=dev)))

        def fn(i):
            q8, k8, v8, qd, kd, vd, o, lse = cps[i % 3]
            ops.attn_fwd_fp8(q8, k8, v8, qd, kd, vd, causal=False, window=w["window"], scale=w["scale"], out=o,
                             lse=lse)
    elif name == "fp8_prefill":
        w = synth.workload_inputs("causal_prefill", dev)
        q8, k8, v8, qd, kd, vd = synth.draw_qkv_fp8(w["q"].shape, w["k"].shape, w["seed"], dev)
        o = torch.empty_like(w["q"])
        lse = torch.empty(w["B"], w["Hq"], w["Sq"], dtype=torch.float32, device=dev)

        def fn(i):
            ops.attn_fwd_fp8(q8, k8, v8, qd, kd, vd, causal=True, scale=w["scale"], out=o, lse=lse)
    elif name in ("causal_prefill", "window_encoder", "global_layer", "backward"):
        w = synth.workload_inputs("window_encoder" if name == "global_layer" else
                                  ("causal_prefill" if name == "backward" else name), dev)
        window = -1 if name == "global_layer" else w["window"]
        o = torch.empty_like(w["q"])
        lse = torch.empty(w["B"], w["Hq"], w["Sq"], dtype=torch.float32, device=dev)
        if name == "backward":
            do = synth.draw_grad(w["q"].shape, "bf16", w["seed"], dev)
            ops.attn_fwd(w["q"], w["k"], w["v"], causal=True, scale=w["scale"], out=o, lse=lse)
            dq, dk, dv = torch.empty_like(w["q"]), torch.empty_like(w["k"]), torch.empty_like(w["v"])
            delta = torch.empty_like(lse)

            def fn(i):
                ops.attn_bwd(w["q"], w["k"], w["v"], o, do, lse, causal=True, scale=w["scale"], dq=dq, dk=dk,
                             dv=dv, delta=delta)
        else:
            # three rotated copies of the inputs and outputs, as in the full run
            cp = [(w["q"], w["k"], w["v"], o, lse)] + [
                (w["q"].clone(), w["k"].clone(), w["v"].clone(), torch.empty_like(o), torch.empty_like(lse))
                for _ in range(2)]

            def fn(i):
                q, k, v, oo, ll = cp[i % 3]
                ops.attn_fwd(q, k, v, causal=bool(w["causal"]), window=window, scale=w["scale"], out=oo, lse=ll)
    elif name == "tiny_f32":
        w = synth.workload_inputs(name, dev)
        o = torch.empty_like(w["q"])
        lse = torch.empty(w["B"], w["Hq"], w["Sq"], dtype=torch.float32, device=dev)

        def fn(i):
            ops.attn_fwd_f32(w["q"], w["k"], w["v"], causal=False, scale=w["scale"], out=o, lse=lse)
    elif name in ("gqa_decode", "long_decode"):
        w = synth.workload_inputs(name, dev)
        o = torch.empty_like(w["q"])
        lse = torch.empty(w["B"], w["Hq"], dtype=torch.float32, device=dev)
        ws = torch.empty(ops.decode_workspace_bytes(w["B"], w["Hq"], w["D"], w["num_splits"]),
                         dtype=torch.uint8, device=dev)

        def fn(i):
            ops.attn_decode_ex(w["q"], w["k"], w["v"], w["num_splits"], scale=w["scale"], out=o, lse=lse,
                               workspace=ws)
    else:
        raise SystemExit(f"unknown workload {name!r}")
    st = launch_stats(time_launches(fn, steps, stream, warm=warmup))
    print(json.dumps({"only": name, "launch_ms": st}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the GPU needs tens of milliseconds of work to reach its steady clock")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (three times), the known-size "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--only", default=None,
                    help="time one workload alone and print its launch statistics (for profilers): "
                         "tiny_f32, causal_prefill, fp8_prefill, window_encoder, fp8_window_encoder, "
                         "global_layer, backward, gqa_decode, long_decode")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    from exact_attention_33_amd import ops, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}), flush=True)
        return
    if args.only:
        run_only(args.only, args.steps, args.warmup, dev)
        return
    wp = synth.workload_inputs(PREFILL, dev)
    wd = synth.workload_inputs(DECODE, dev)
    o_p = torch.empty_like(wp["q"])
    lse_p = torch.empty(wp["B"], wp["Hq"], wp["Sq"], dtype=torch.float32, device=dev)
    o_d = torch.empty_like(wd["q"])
    lse_d = torch.empty(wd["B"], wd["Hq"], dtype=torch.float32, device=dev)
    ws = torch.empty(ops.decode_workspace_bytes(wd["B"], wd["Hq"], wd["D"], wd["num_splits"]),
                     dtype=torch.uint8, device=dev)

    def prefill():
        ops.attn_fwd(wp["q"], wp["k"], wp["v"], causal=True, scale=wp["scale"], out=o_p, lse=lse_p)

    def decode():
        ops.attn_decode_ex(wd["q"], wd["k"], wd["v"], wd["num_splits"], scale=wd["scale"], out=o_d,
                           lse=lse_d, workspace=ws)

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    # However few --warmup steps were asked for, the timed steps start only
    # after WARM_MS of continuous GPU work: the clock takes tens of
    # milliseconds of load to ramp (the same prefill measured 102 us cold and
    # 82 us warm).  Every other series gets the same in time_launches().
    t_w0, warm_pairs = time.perf_counter(), 0
    while (time.perf_counter() - t_w0) * 1e3 < WARM_MS:
        for _ in range(4):
            prefill()
            decode()
            warm_pairs += 1
        torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t_w0) * 1e3

    # Timed region: K steps of work (K prefills, then K decodes), each launch
    # bracketed by HIP events on the stream it runs on.  Running each kernel
    # back to back measures it in its own steady state; the interleaved order
    # (prefill right after a decode that streamed 2 GB through the caches) is
    # timed separately below and reported as "interleaved".
    stream = torch.cuda.current_stream(dev)
    evp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    evd = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(args.steps):
        evp[i][0].record(stream)
        prefill()
        evp[i][1].record(stream)
    for i in range(args.steps):
        evd[i][0].record(stream)
        decode()
        evd[i][1].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms = [e[0].elapsed_time(e[1]) for e in evp]
    d_ms = [e[0].elapsed_time(e[1]) for e in evd]
    step_ms = t_all0.elapsed_time(t_all1) / args.steps
    p_avg = sum(p_ms) / len(p_ms)
    d_avg = sum(d_ms) / len(d_ms)

    # the same work interleaved step by step (untimed for the headline value)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    ip_avg = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    id_avg = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps

    progress(f"timed steps done: prefill {p_avg * 1e3:.1f} us, decode {d_avg * 1e3:.1f} us per launch")
    ach = achievable(dev)
    progress("achievable rates done")
    flops = prefill_flops(wp)
    kv = decode_kv_bytes(wd)
    p_tflops = flops / (p_avg * 1e-3) / 1e12
    d_gbs = kv / (d_avg * 1e-3) / 1e9
    p_frac = p_tflops / PEAK_BF16_TFLOPS
    d_frac = d_gbs / PEAK_HBM_GBS
    value = 100.0 * 0.5 * (p_frac + d_frac)

    line = {
        "metric": "prefill attn TFLOP/s + decode KV GB/s, as % of MI355X MFMA/HBM peak",
        "value": round(value, 3),
        "unit": "% of MI355X peak (mean of prefill MFMA and decode HBM fractions)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warm_ms": round(warm_ms, 1), "warm_steps_busy": warm_pairs,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": ("causal prefill B4 H16 S2048 D128 bf16 + GQA decode B16 Hq32 Hkv8 "
                         "Sk32768 D128 bf16, 64 KV splits"),
            "prefill": {k: wp[k] for k in ("B", "Hq", "Hkv", "Sq", "Sk", "D", "causal", "window")},
            "decode": {k: wd[k] for k in ("B", "Hq", "Hkv", "Sk", "D", "num_splits")},
        },
        "roofline": {
            "kernel": "decode (split kernel + tree combine), the larger share of the step",
            "bound": "hbm", "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(d_frac, 4), "traffic": measured_traffic("decode"),
            "algorithmic_bytes": kv, "avg_launch_ms": round(d_avg, 5), "launch_ms": launch_stats(d_ms),
            "frac_of_achievable": round(d_gbs / ach["hbm_read_gbs"], 4),
            "scores_bytes_avoided": scores_bytes_avoided(wd["B"], wd["Hq"], 1, wd["Sk"]),
        },
        "roofline_prefill": {
            "kernel": "fwd_bf16 causal prefill",
            "bound": "mfma", "achieved": round(p_tflops, 1), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(p_frac, 4), "traffic": measured_traffic("prefill"),
            "algorithmic_flops": flops, "avg_launch_ms": round(p_avg, 5), "launch_ms": launch_stats(p_ms),
            "frac_of_achievable": round(p_tflops / ach["mfma_bf16_tflops"], 4),
            "scores_bytes_avoided": scores_bytes_avoided(wp["B"], wp["Hq"], wp["Sq"], wp["Sk"]),
        },
        "achievable": ach,
        "interleaved": {
            "note": "same steps with prefill and decode alternating: the prefill then starts with caches "
                    "flushed by the preceding decode",
            "prefill_avg_launch_ms": round(ip_avg, 5), "decode_avg_launch_ms": round(id_avg, 5),
            "prefill_tflops": round(flops / (ip_avg * 1e-3) / 1e12, 1),
            "decode_gbs": round(kv / (id_avg * 1e-3) / 1e9, 1),
        },
        "wall_s_timed": round(wall, 4),
        "kernel_source_digest": source_digest(),
    }
    line["other_configs"] = other_configs(dev, ach)
    progress("other configs done")
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
