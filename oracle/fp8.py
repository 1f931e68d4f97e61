"""CPU oracle for an 8-bit KV cache: the e4m3 code (OCP FP8 E4M3, "fn" variant).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU library never uses it.

The pages note that an eight-bit KV cache costs little in quality and halves
the bytes a decode step reads ("The Serving Playbook", section "Quantized
serving"); they fix neither the format nor the scale granularity. Readings
used here (the plainest ones, also what MI355X converts natively):

  * format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
    field 0 encodes subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is
    NaN; there is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448;
  * one scale per layer for K and one for V: a stored code c stands for
    decode(c) * scale;
  * quantizing x: y = fp32(x) * fp32(1 / scale), rounded in fp32 (the
    product both sides compute); then y is clamped to [-448, 448] (so
    out-of-range values and infinities saturate), and rounded to the nearest
    code, ties to even mantissa. A NaN input stays NaN: code 0x7F, or 0xFF
    when the input's sign bit is set (IEEE 754 leaves the sign of a NaN
    product open, so the input's is the one used); -0 keeps its sign (0x80).

Everything below follows those definitions with plain integer and float64
arithmetic; no library FP8 type is used.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7
_MIN_NORMAL_EXP = 1 - _BIAS          # exponent of the smallest normal, -6
_SUBNORMAL_STEP = 2.0 ** (_MIN_NORMAL_EXP - 3)   # 2^-9, the smallest subnormal


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Value (float64) of each e4m3 code."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - _BIAS)
    sub = (m / 8.0) * 2.0 ** _MIN_NORMAL_EXP
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def fp8_e4m3_encode(x, inv_scale: float = 1.0) -> np.ndarray:
    """Code (uint8) of fp32(x) * fp32(inv_scale), saturated and rounded to nearest even."""
    x32 = np.asarray(x, dtype=np.float32)
    y = (x32 * np.float32(inv_scale)).astype(np.float64)           # the fp32 product
    nan = np.isnan(y)
    neg = np.signbit(x32)          # inv_scale > 0: the product's sign, and the NaN's
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)
    # Exponent of the binade holding a; zero and the subnormals share the
    # smallest normal binade's exponent and spacing (2^-9).
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), _MIN_NORMAL_EXP)
    e = np.where(a > 0, e, _MIN_NORMAL_EXP)
    step = np.exp2(e - 3)                      # spacing of codes in this binade
    q = np.round(a / step)                     # numpy rounds halves to even
    # q in [8, 16] for normals (16 carries into the next binade), [0, 8] below.
    code_mag = np.where(
        e == _MIN_NORMAL_EXP,
        q,                                     # 0..8: subnormals, and 8 = smallest normal
        (e + _BIAS) * 8 + (q - 8),             # exponent field * 8 + mantissa; q = 16 carries
    ).astype(np.int64)
    code = np.where(neg, 0x80, 0) | code_mag
    code = np.where(nan, np.where(neg, 0xFF, 0x7F), code)
    return code.astype(np.uint8)


def quantize_dequantize(x, scale: float) -> np.ndarray:
    """The value an fp8 pool holds for input x: decode(encode(x, 1/scale)) * scale."""
    inv = np.float32(1.0) / np.float32(scale)
    return fp8_e4m3_decode(fp8_e4m3_encode(x, inv)) * np.float64(np.float32(scale))
