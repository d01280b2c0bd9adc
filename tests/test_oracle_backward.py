"""The fp64 gradient oracle against its pins, and planted mistakes caught (CPU only)."""

import importlib
import os
import types

import pytest

import oracle
import pins_backward

# the submodule itself (the package re-exports a function of the same name)
oatt = importlib.import_module("oracle.attention")

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "backward.py")


@pytest.mark.parametrize("pin", pins_backward.ALL_PINS_B, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


MUTANTS = {
    "dv not summed over the group": ("dv[b, g] += p.T @ dd", "dv[b, g] = p.T @ dd"),
    "delta term dropped": ("ds = p * (dp - dl[:, None])", "ds = p * dp"),
    "delta sign": ("ds = p * (dp - dl[:, None])", "ds = p * (dp + dl[:, None])"),
    "dq misses scale": ("dq[b, h] = scale * (ds @ kk)", "dq[b, h] = (ds @ kk)"),
    "dk misses scale": ("dk[b, g] += scale * (ds.T @ qq)", "dk[b, g] += (ds.T @ qq)"),
    "dq from v": ("dq[b, h] = scale * (ds @ kk)", "dq[b, h] = scale * (ds @ vv)"),
    "dv from unnormalised weights": ("dv[b, g] += p.T @ dd", "dv[b, g] += e.T @ dd"),
    "delta as an unweighted row sum of dP": ("dl = (dd * o).sum(axis=1)", "dl = dp.sum(axis=1)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not unique/absent"
    src = src.replace("from .attention import visibility", "")
    mod = types.ModuleType("oracle_bwd_mutant")
    mod.__dict__["visibility"] = oatt.visibility
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    mod.attention = oatt.attention
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    failed = 0
    for pin in pins_backward.ALL_PINS_B:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed += 1
    assert failed > 0, f"mutant {name!r} passed every pin"
