"""The oracle's e4m3 code against torch's float8_e4m3fn, closed forms and
invariants; planted mistakes in copies of oracle/fp8.py must each fail a pin
(CPU only)."""
import os
import types

import pytest

import oracle.fp8 as real_fp8
from fp8_pins import ALL_FP8_PINS

SRC_PATH = real_fp8.__file__

MUTANTS = {
    "bias_8": ("_BIAS = 7", "_BIAS = 8"),
    "truncate_not_round": ("q = np.round(a / step)", "q = np.floor(a / step)"),
    "round_half_up": ("q = np.round(a / step)", "q = np.floor(a / step + 0.5)"),
    "no_saturation": ("a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)",
                      "a = np.abs(np.where(nan, 0.0, y))"),
    "scale_divides": ("y = (x32 * np.float32(inv_scale)).astype(np.float64)",
                      "y = (x32 / np.float32(inv_scale)).astype(np.float64)"),
    "nan_sign_dropped": ("code = np.where(nan, np.where(neg, 0xFF, 0x7F), code)",
                         "code = np.where(nan, 0x7F, code)"),
    "subnormal_step_wrong": ("sub = (m / 8.0) * 2.0 ** _MIN_NORMAL_EXP", "sub = (m / 8.0) * 2.0 ** (_MIN_NORMAL_EXP - 1)"),
    "no_nan_code": ("return np.where((e == 15) & (m == 7), np.nan, val)", "return val"),
    "sign_dropped": ("code = np.where(neg, 0x80, 0) | code_mag", "code = code_mag"),
}


@pytest.mark.parametrize("pin", ALL_FP8_PINS, ids=lambda f: f.__name__)
def test_fp8_pin(pin):
    pin(real_fp8)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fp8_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src.replace(old, new), "fp8_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in ALL_FP8_PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
