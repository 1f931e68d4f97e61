"""Checks that pin the oracle's e4m3 code (oracle/fp8.py) to facts other than
itself. Each ``pin_*`` takes the fp8 oracle module, so the same checks run
against copies with a planted mistake (test_oracle_fp8.py).

  * torch's CPU float8_e4m3fn type, an independent implementation of the
    same format, for every code and for every bf16 input (torch converts with
    round-to-nearest-even and makes NaN of overflow, so inputs are clamped to
    +-448 first: the saturation the oracle defines);
  * closed forms from the format definition (bias 7, 3 mantissa bits,
    subnormal step 2^-9, largest value 448);
  * invariants: decode(encode(decode(c))) == c, monotonicity.
"""
from __future__ import annotations

import numpy as np
import torch


def _all_bf16_as_f32():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


def pin_decode_all_codes_match_torch(f8):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = f8.fp8_e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_encode_all_bf16_match_torch(f8):
    x = _all_bf16_as_f32()
    x = x[~np.isnan(x)]
    ref = torch.clamp(torch.from_numpy(x), -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = f8.fp8_e4m3_encode(x, 1.0)
    bad = got != ref
    assert not bad.any(), (x[bad][:5], got[bad][:5], ref[bad][:5])


def pin_encode_with_scale_matches_torch(f8):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-14, 12, 20000))).astype(np.float32)
    for scale in (3.0, 0.37, 1.0 / 48):
        inv = np.float32(1.0) / np.float32(scale)
        y = x * inv                                    # the fp32 product
        ref = torch.clamp(torch.from_numpy(y), -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(f8.fp8_e4m3_encode(x, inv), ref), scale


def pin_closed_forms(f8):
    cases = [
        (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E), (-448.0, 0xFE), (1000.0, 0x7E), (float("inf"), 0x7E),
        (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -6, 0x08),
        (0.0, 0x00), (-0.0, 0x80), (1.0625, 0x38), (1.1875, 0x3A), (240.0, 0x77), (464.0, 0x7E),
    ]
    for x, code in cases:
        got = int(f8.fp8_e4m3_encode(np.array([x], np.float32))[0])
        assert got == code, (x, hex(got), hex(code))
    vals = f8.fp8_e4m3_decode(np.array([0x01, 0x08, 0x38, 0x7E, 0x7F, 0x80, 0xB8]))
    assert vals[0] == 2.0 ** -9 and vals[1] == 2.0 ** -6 and vals[2] == 1.0 and vals[3] == 448.0
    assert np.isnan(vals[4]) and vals[5] == 0.0 and np.signbit(vals[5]) and vals[6] == -1.0
    nans = np.array([0x7FC00000, 0xFFC00000, 0x7F800001], np.uint32).view(np.float32)
    assert list(f8.fp8_e4m3_encode(nans, 0.125)) == [0x7F, 0xFF, 0x7F]     # a NaN keeps its sign


def pin_round_trip_and_order(f8):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = f8.fp8_e4m3_decode(codes)
    assert np.array_equal(f8.fp8_e4m3_encode(vals.astype(np.float32), 1.0), codes)
    pos = np.sort(f8.fp8_e4m3_decode(np.arange(0, 0x7F)))
    assert np.all(np.diff(pos) > 0)


ALL_FP8_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
