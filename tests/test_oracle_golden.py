"""Hand-derived closed-form cases (tests/golden/hand_cases.json) against the oracle."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _num(x):
    return np.asarray(x, dtype=object).astype(float) if not isinstance(x, str) else float(x)


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load()["cases"], ids=lambda c: c["name"])
def test_hand_case(case):
    q, k, v = (np.array(case[n], dtype=np.float64) for n in ("q", "k", "v"))
    o, lse = oracle.attention(q, k, v, case["scale"], case["causal"], case["window"])
    np.testing.assert_allclose(o, np.array(case["o"], dtype=np.float64), rtol=0, atol=1e-13)
    want = np.array([[[float(x) for x in row] for row in h] for h in case["lse"]])
    assert np.array_equal(np.isneginf(lse), np.isneginf(want))
    fin = np.isfinite(want)
    np.testing.assert_allclose(lse[fin], want[fin], rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", _load()["split_cases"], ids=lambda c: c["name"])
def test_hand_split_case(case):
    q = np.array(case["q"], dtype=np.float64)[None]
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    parts = oracle.split_partials(q, k, v, case["scale"], case["num_splits"])
    assert len(parts) == len(case["partials"])
    for (m, l, acc), (wm, wl, wacc) in zip(parts, case["partials"]):
        assert float(m[0]) == pytest.approx(float(wm), abs=1e-13) if wm != "-inf" else np.isneginf(m[0])
        assert float(l[0]) == pytest.approx(wl, abs=1e-13)
        np.testing.assert_allclose(acc[0], wacc, rtol=0, atol=1e-13)
    o, lse = oracle.finish(oracle.combine(parts))
    np.testing.assert_allclose(o[0], case["o"], rtol=0, atol=1e-13)
    assert float(lse[0]) == pytest.approx(case["lse"], abs=1e-13)
    od, ld = oracle.decode(q[None], k[None, None], v[None, None], case["scale"])
    np.testing.assert_allclose(od[0, 0], case["o"], rtol=0, atol=1e-13)
    assert float(ld[0, 0]) == pytest.approx(case["lse"], abs=1e-13)
