"""Pins for the oracle's E5M2 variant of the MX block rule (CPU only).

E5M2 is the alternative element format offered for the MXFP8 transport (afd-plugin PR #475
"quantize the A2E FFN transport to MXFP8", description of the transport; a review on the same
page places it at operator level). Pinned here, independently of the oracle's own tables:

* the E5M2 decode table against torch's float8_e5m2 decoder, all 256 codes;
* nearest-even rounding with saturation, for every BF16 pattern under several scale bytes,
  against an integer bit-level implementation written here and against torch's float8_e5m2
  cast applied after a clamp to +-57344;
* closed forms: the scale byte of a power-of-two amax, the top binade, subnormal ties, the
  clamp boundary;
* decode of every (code, scale byte) pair against torch's float8_e5m2 x float8_e8m0fnu.
"""
import numpy as np
import pytest
import torch

from oracle.formats import E5M2_TABLE, bf16_bits_to_f64, e8m0_to_f64
from oracle.mx import dequantize_groups, e5m2_rne_sat, quantize_blocks, scale_byte


def test_decode_table_against_torch():
    t = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e5m2).double().numpy()
    assert np.array_equal(np.isnan(E5M2_TABLE), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(E5M2_TABLE[ok], t[ok])
    assert E5M2_TABLE[0x7B] == 57344.0 and E5M2_TABLE[0x7C] == np.inf and E5M2_TABLE[0x01] == 2.0 ** -16


def _int_rne_e5m2(bits, byte):
    """Independent bit-level implementation: BF16 bits / 2^(byte-127) -> E5M2 code (RNE, sat)."""
    bits = bits.astype(np.int64)
    sign = bits >> 15
    ef = (bits >> 7) & 0xFF
    m = bits & 0x7F
    mant = np.where(ef == 0, m, m | 0x80)                        # integer significand
    e2 = np.where(ef == 0, -133, ef - 134) - (byte - 127)        # value = mant * 2^e2
    nb = np.where(mant > 0, np.floor(np.log2(np.maximum(mant, 1))).astype(np.int64), 0)
    fl = nb + e2                                                 # floor(log2 |y|)
    qexp = np.maximum(fl, -14) - 2                               # E5M2 quantum exponent
    sh = qexp - e2
    n = np.zeros_like(mant)
    left = sh <= 0
    n[left] = mant[left] << np.minimum(-sh[left], 40)
    r = ~left
    shr = np.minimum(sh[r], 62)
    base = mant[r] >> shr
    rem = mant[r] - (base << shr)
    half = np.where(shr > 0, np.int64(1) << np.maximum(shr - 1, 0), 0)
    up = (rem > half) | ((rem == half) & (half > 0) & ((base & 1) == 1))
    n[r] = base + up
    code = ((qexp + 16) << 2) + n
    code = np.where(mant == 0, 0, code)
    code = np.where(fl > 15, 0x7B, np.minimum(code, 0x7B))
    return (code | (sign << 7)).astype(np.uint8)


SCALE_BYTES = [0, 1, 100, 112, 113, 127, 135, 239]


@pytest.mark.parametrize("byte", SCALE_BYTES)
def test_brute_force_all_bf16(byte):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    y = v[fin] / e8m0_to_f64(np.array([byte]))[0]
    got = e5m2_rne_sat(y)
    assert np.array_equal(got, _int_rne_e5m2(bits[fin], byte))
    ref = torch.from_numpy(np.clip(y, -57344.0, 57344.0)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_scale_byte_from_bf16_exponent_field():
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    ef = (bits.astype(np.int64) >> 7) & 0xFF
    assert np.array_equal(scale_byte(bf16_bits_to_f64(bits), 15), np.maximum(ef - 15, 0).astype(np.uint8))


def _block(vals, fill=0.0):
    b = np.full(32, fill, dtype=np.float64)
    b[:len(vals)] = vals
    return b[None, :]


@pytest.mark.parametrize("k", [-100, -3, 0, 7, 60, 127])
def test_closed_forms(k):
    a = 2.0 ** k
    q, s = quantize_blocks(_block([a, 1.75 * a, 2.0 ** (k - 31)]), "e5m2")
    assert s[0] == k - 15 + 127                # amax 1.75 * 2^k: floor(log2) = k
    assert q[0, 1] == 0x7B                     # 1.75 * 2^15 = 57344: the top code
    assert q[0, 0] == 0x78                     # 2^15: exponent field 30, mantissa 0
    assert q[0, 2] == 0x01                     # 2^(k-31) / 2^(k-15) = 2^-16: smallest subnormal
    q, s = quantize_blocks(_block([a, -2.0 ** (k - 32), 3 * 2.0 ** (k - 32), 1.875 * 2.0 ** (k - 1)]), "e5m2")
    # amax = 2^k; y = 2^-17 (tie 0 / 2^-16 -> 0, sign kept), 3 * 2^-17 (tie 1 / 2 quanta -> 2),
    # 1.875 * 2^14 = 30720 (tie 28672 / 32768 -> even mantissa 0 of the next binade: 0x78)
    assert s[0] == k - 15 + 127 and q[0, 0] == 0x78
    assert q[0, 1] == 0x80 and q[0, 2] == 0x02 and q[0, 3] == 0x78


def test_clamp_boundary_and_zero():
    q, s = quantize_blocks(_block([2.0 ** -112]), "e5m2")
    assert s[0] == 0 and q[0, 0] == 0x78       # byte -112 - 15 + 127 = 0: 2^15
    q, s = quantize_blocks(_block([2.0 ** -113]), "e5m2")
    assert s[0] == 0 and q[0, 0] == 0x74       # clamped: y = 2^14, exponent field 29
    q, s = quantize_blocks(np.zeros((1, 32)), "e5m2")
    assert s[0] == 0 and np.all(q == 0)
    q, s = quantize_blocks(_block([1.0, np.nan]), "e5m2")
    assert s[0] == 255 and np.all((q & 0x7F) == 0x7F)


def test_saturation_beyond_top_binade():
    # amax 1.9375 * 2^k: y = 1.9375 * 2^15 = 63488 > 57344 -> saturates to 0x7B (not infinity)
    q, s = quantize_blocks(_block([1.9375 * 2.0 ** 4, -1.9375 * 2.0 ** 4]), "e5m2")
    assert s[0] == 4 - 15 + 127 and q[0, 0] == 0x7B and q[0, 1] == 0xFB


def test_dequantize_all_pairs_against_torch():
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None].repeat(8, axis=1)
    got = dequantize_groups(codes, scales, "e5m2")
    e5 = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e5m2).double().numpy()
    e8 = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e8m0fnu).double().numpy()
    with np.errstate(invalid="ignore"):
        want = e8[:, None] * e5[None, :]
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
