"""The fp8 oracle against its pins, and planted mistakes caught (CPU only)."""

import importlib
import os
import types

import pytest

import oracle
import pins_fp8

oatt = importlib.import_module("oracle.attention")
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8.py")


@pytest.mark.parametrize("pin", pins_fp8.ALL_PINS_F8, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


MUTANTS = {
    "bias 8 instead of 7": ("np.exp2(exp - 7.0)", "np.exp2(exp - 8.0)"),
    "subnormals read as normals": ("np.where(exp == 0, man * 2.0 ** -9,", "np.where(exp == -1, man * 2.0 ** -9,"),
    "sign bit ignored": ("return np.where(sign == 1, -mag, mag)", "return mag"),
    "no NaN codes": ("mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)", "mag = mag"),
    "mantissa over 16": ("(1.0 + man / 8.0)", "(1.0 + man / 16.0)"),
    "q descale dropped": ("q = e4m3_decode(q8) * float(q_descale)", "q = e4m3_decode(q8)"),
    "v descale dropped": ("v = e4m3_decode(v8) * float(v_descale)", "v = e4m3_decode(v8)"),
    "v descale applied to k": ("k = e4m3_decode(k8) * float(k_descale)", "k = e4m3_decode(k8) * float(v_descale)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not unique/absent"
    src = src.replace("from .attention import attention", "")
    mod = types.ModuleType("oracle_fp8_mutant")
    mod.__dict__["attention"] = oatt.attention
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    failed = 0
    for pin in pins_fp8.ALL_PINS_F8:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed += 1
    assert failed > 0, f"mutant {name!r} passed every pin"
