"""Pins for the oracle's format decoders/encoders (CPU only).

Pinned against: the values printed on the pages (tests/golden/e8m0_decode.json),
torch's CPU float8 / bfloat16 conversions (library routines applied to every
bit pattern), and hand-computed rounding cases.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.formats import (E4M3_TABLE, bf16_bits_to_f64, bf16_round, e4m3_to_f64, e8m0_to_f64,
                            f64_to_bf16_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e8m0_decode.json")


def _golden_value(entry):
    if entry.get("value") == "nan":
        return float("nan")
    if "value_log2" in entry:
        return math.ldexp(1.0, entry["value_log2"])
    return float(entry["value"])


def test_e8m0_decode_matches_printed_values():
    with open(GOLDEN) as f:
        g = json.load(f)
    for entry in g["scale_bytes"]:
        got = float(e8m0_to_f64(np.array([entry["byte"]]))[0])
        want = _golden_value(entry)
        if math.isnan(want):
            assert math.isnan(got), entry
        else:
            assert got == want, entry


def test_dequantize_matches_printed_value():
    with open(GOLDEN) as f:
        g = json.load(f)
    for entry in g["dequantize"]:
        code = [c for c in range(256) if E4M3_TABLE[c] == entry["e4m3_value"]]
        assert len(code) == 1
        got = float(e4m3_to_f64(np.array(code, dtype=np.uint8))[0] * e8m0_to_f64(np.array([entry["byte"]]))[0])
        assert got == _golden_value(entry), entry


def test_e4m3_table_matches_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(E4M3_TABLE))
    assert np.array_equal(ref[~nan], E4M3_TABLE[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(E4M3_TABLE[~nan]))
    # the landmarks of the format
    assert E4M3_TABLE[0x7E] == 448.0 and E4M3_TABLE[0x08] == 2.0 ** -6 and E4M3_TABLE[0x01] == 2.0 ** -9
    assert np.isnan(E4M3_TABLE[0x7F]) and np.isnan(E4M3_TABLE[0xFF])
    assert E4M3_TABLE[0x78] == 256.0 and E4M3_TABLE[0x38] == 1.0 and E4M3_TABLE[0x80] == 0.0


def test_e8m0_matches_torch_float8_e8m0fnu():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = e8m0_to_f64(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_bf16_decode_all_patterns_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_bf16_round_of_float32_inputs_matches_torch():
    # every float32 whose upper 16 bits are a finite BF16 and whose lower bits hit
    # the interesting places (exact, just below/at/above the midpoint, max)
    hi = np.arange(0, 65536, dtype=np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    f32 = ((hi[:, None] << 16) | lows[None, :]).ravel().view(np.float32)
    f32 = f32[np.isfinite(f32)]
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(f32.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_round_is_direct_not_double():
    # 1 + 2^-8 is the midpoint between BF16 1.0 and 1 + 2^-7; add 2^-40 so it is above:
    # direct RNE goes up; rounding through float32 first would land on the tie and go to 1.0.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert bf16_round(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert np.float32(x) == np.float32(1.0 + 2.0 ** -8)


@pytest.mark.parametrize("x,want", [
    (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3F80), (-2.0, 0xC000),
    (2.0 ** -133, 0x0001),                     # smallest subnormal
    (2.0 ** -134, 0x0000),                     # tie with zero -> even (zero)
    (3 * 2.0 ** -135, 0x0001),                 # 0.75 quantum -> 1 quantum
    (2.0 ** 128, 0x7F80), (-(2.0 ** 200), 0xFF80),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),    # tie between max and 2^128 -> even -> inf
])
def test_bf16_round_cases(x, want):
    assert int(f64_to_bf16_bits(np.array([x]))[0]) == want
