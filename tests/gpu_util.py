"""Helpers for the GPU parity tests: host copies, oracle calls, tolerance checks.

Tolerances (max-abs, mean-abs, relative L2 of o; max-abs of lse):
  bf16 : 2e-2, 2e-3, 1e-2 ; lse 1e-3
  fp32 : 1e-4 (max-abs)   ; lse 1e-4
The relative-L2 bound keeps the check meaningful where |o| itself is small
(long decode: mean |o| ~ 1e-3, below the absolute tolerances).
"""

from __future__ import annotations

import sys

import numpy as np

from exact_attention_33_amd.synth import to_numpy_exact

TOL = {
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel_l2=1e-2, lse=1e-3),
    "f32": dict(max_abs=1e-4, mean_abs=1e-4, rel_l2=1e-4, lse=1e-4),
}


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def errors(o_gpu, o_ref):
    o = np.asarray(o_gpu, dtype=np.float64)
    d = np.abs(o - o_ref)
    ref_norm = np.linalg.norm(o_ref)
    rel = np.linalg.norm(o - o_ref) / ref_norm if ref_norm > 0 else np.linalg.norm(o)
    return dict(max_abs=float(d.max()) if d.size else 0.0, mean_abs=float(d.mean()) if d.size else 0.0,
                rel_l2=float(rel))


def check_o(o_gpu_t, o_ref, dtype, what=""):
    o = to_numpy_exact(o_gpu_t).astype(np.float64)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    e = errors(o, o_ref)
    t = TOL[dtype]
    assert e["max_abs"] <= t["max_abs"], f"{what}: {e}"
    assert e["mean_abs"] <= t["mean_abs"], f"{what}: {e}"
    assert e["rel_l2"] <= t["rel_l2"], f"{what}: {e}"
    return e


def check_lse(lse_gpu_t, lse_ref, dtype, what=""):
    lse = to_numpy_exact(lse_gpu_t).astype(np.float64)
    assert lse.shape == lse_ref.shape
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: empty rows differ"
    fin = np.isfinite(lse_ref)
    assert np.all(np.isfinite(lse[fin])), f"{what}: non-finite lse"
    err = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert err <= TOL[dtype]["lse"], f"{what}: lse max err {err}"
    return err
