"""Pins for the oracle's MXFP8 block quantizer (CPU only).

The quantizer is an encoding, so it is pinned by what the rule fixes without any
implementation: closed-form hand-built blocks, a brute force over every BF16
pattern against two independent implementations (an integer bit-level RNE
written here, and torch's CPU float8_e4m3fn cast after clamping to +-448), the
round-trip error bound, and metamorphic relations (scaling by 2^j, sign flip,
permutation within a block).
"""
import numpy as np
import pytest
import torch

from oracle.formats import bf16_bits_to_f64, e4m3_to_f64, e8m0_to_f64
from oracle.mx import (dequantize_rowwise, e4m3_rne_sat, quantize_blocks, quantize_colwise,
                       quantize_rowwise, scale_byte)


def block(vals, fill=0.0):
    v = np.full(32, fill, dtype=np.float64)
    v[:len(vals)] = vals
    return v


def quant1(vals, fill=0.0):
    q, s = quantize_blocks(block(vals, fill)[None, :])
    return q[0], int(s[0])


# ----------------------------------------------------------------------------- closed forms

def test_all_zero_block():
    q, s = quant1([])
    assert s == 0 and np.all(q == 0)


def test_negative_zero_keeps_sign():
    q, s = quant1([-0.0, 1.0])
    assert s == 127 - 8 and q[0] == 0x80 and q[1] == 0x78


@pytest.mark.parametrize("k", [-100, -30, -5, 0, 1, 7, 60, 119])
def test_power_of_two_amax(k):
    q, s = quant1([2.0 ** k, -(2.0 ** k)])
    assert s == k - 8 + 127
    assert q[0] == 0x78 and q[1] == 0xF8           # 256 = 1.0 * 2^8


@pytest.mark.parametrize("k", [-20, 0, 9])
@pytest.mark.parametrize("mant,code", [(1.75, 0x7E), (1.8125, 0x7E), (1.9375, 0x7E), (1.5, 0x7C), (1.0625, 0x78)])
def test_saturation_and_top_binade(k, mant, code):
    # amax/X = 256 * mant: 448 exact, 464 ties between 448 and 480 -> even (448),
    # 496 clips to 448, 384 exact (0x7C), 272 ties between 256 and 288 -> even (256)
    q, s = quant1([mant * 2.0 ** k])
    assert s == k - 8 + 127 and q[0] == code


@pytest.mark.parametrize("k", [-40, 0, 12])
def test_subnormal_codes(k):
    # X = 2^(k-8); y = v / X
    vals = [2.0 ** k,                 # 256
            2.0 ** (k - 17),          # y = 2^-9: smallest subnormal, code 1
            2.0 ** (k - 18),          # y = 2^-10: tie 0 / 2^-9 -> even (0)
            3 * 2.0 ** (k - 19),      # y = 0.75 * 2^-9 -> 1
            3 * 2.0 ** (k - 18),      # y = 1.5 * 2^-9: tie 1 / 2 -> 2
            15 * 2.0 ** (k - 18),     # y = 7.5 * 2^-9: tie 0x07 / 0x08 -> 0x08
            -(2.0 ** (k - 30)),       # far below: -0
            2.0 ** (k - 14),          # y = 2^-6: smallest normal, 0x08
            ]
    q, s = quant1(vals)
    assert s == k - 8 + 127
    assert list(q[:8]) == [0x78, 0x01, 0x00, 0x01, 0x02, 0x08, 0x80, 0x08]


def test_clamp_boundary():
    q, s = quant1([2.0 ** -119])
    assert s == 0 and q[0] == 0x78
    q, s = quant1([2.0 ** -120])
    assert s == 0 and q[0] == 0x70               # 128 = 2^7
    q, s = quant1([2.0 ** -130])                 # a BF16 subnormal amax
    assert s == 0 and q[0] == 0x20               # 0.125; a denormal-flushing path gives 0 here
    q, s = quant1([2.0 ** -133])                 # the smallest BF16 subnormal
    assert s == 0 and q[0] == 0x08               # 2^-133 / 2^-127 = 2^-6, the smallest E4M3 normal


def test_largest_bf16_never_needs_nan_scale():
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    q, s = quant1([big])
    assert s == 127 + 127 - 8 == 246 and q[0] == 0x7E   # 1.9921875 * 256 = 510 -> clipped


def test_nonfinite_block_reading():
    q, s = quant1([1.0, np.nan, -2.0])
    assert s == 255 and q[0] == 0x7F and q[2] == 0xFF
    q, s = quant1([np.inf, 1.0])
    assert s == 255 and np.all((q & 0x7F) == 0x7F)


def test_scale_bytes_and_nonfinite_blocks_against_torch_e8m0():
    """The scale byte against torch's own E8M0 encoder (float8_e8m0fnu, an implementation
    independent of the oracle's): for finite blocks the byte is the encoding of the power of two
    2^(floor(log2 amax) - 8), clamped below at 2^-127 (byte 0); amax NaN or +Inf encodes as
    0xFF, the E8M0 NaN. In a non-finite block every code is an E4M3 NaN (magnitude bits 0x7F,
    which is what torch's float8_e4m3fn cast gives for an element divided by the NaN scale);
    the sign bit follows the element (a reading: IEEE division by NaN leaves it unspecified)."""
    rng = np.random.default_rng(3)
    exps = rng.integers(-140, 20, size=4000)
    v = rng.standard_normal((4000, 32)) * np.exp2(exps)[:, None]
    v[::7, 5] = 0.0
    v[::11] = 0.0  # all-zero blocks: byte 0 as well
    _, s = quantize_blocks(v)
    amax = np.max(np.abs(v), axis=1)
    e = np.frexp(amax)[1] - 1  # floor(log2 amax), exact
    # an all-zero block: torch encodes 0.0 as byte 0 as well
    pw = torch.tensor(np.where(amax > 0, np.exp2((e - 8).astype(np.float64)), 0.0), dtype=torch.float64)
    want = pw.to(torch.float32).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    assert np.array_equal(s, want)
    bad = np.array([block([1.0, np.nan, -2.0]), block([np.inf, 1.0]), block([-3.0, -np.inf]),
                    block([np.nan], fill=-1.0)])
    q, s = quantize_blocks(bad)
    amax_t = torch.tensor([np.nan, np.inf, np.inf, np.nan], dtype=torch.float32)
    assert np.array_equal(s, amax_t.to(torch.float8_e8m0fnu).view(torch.uint8).numpy())
    nan_div = (torch.tensor(bad, dtype=torch.float32) / torch.tensor(float("nan"))).to(torch.float8_e4m3fn)
    assert np.array_equal(q & 0x7F, nan_div.view(torch.uint8).numpy() & 0x7F)
    assert np.array_equal(q >> 7, np.signbit(bad).astype(np.uint8))


# ----------------------------------------------------------------------------- brute force

def _int_rne_e4m3(bits, byte):
    """Independent bit-level implementation: BF16 bits / 2^(byte-127) -> E4M3 code (RNE, sat)."""
    bits = bits.astype(np.int64)
    sign = bits >> 15
    ef = (bits >> 7) & 0xFF
    m = bits & 0x7F
    mant = np.where(ef == 0, m, m | 0x80)                        # integer significand
    e2 = np.where(ef == 0, -133, ef - 134) - (byte - 127)        # value = mant * 2^e2
    nbits = np.where(mant > 0, np.floor(np.log2(np.maximum(mant, 1))).astype(np.int64), 0)
    fl = nbits + e2                                              # floor(log2 |y|)
    qexp = np.maximum(fl, -6) - 3                                # E4M3 quantum exponent
    sh = qexp - e2                                               # right shift to the quantum
    n = np.zeros_like(mant)
    left = sh <= 0
    n[left] = mant[left] << (-sh[left])
    r = ~left
    shr = np.minimum(sh[r], 62)
    base = mant[r] >> shr
    rem = mant[r] - (base << shr)
    half = np.where(shr > 0, np.int64(1) << np.maximum(shr - 1, 0), 0)
    up = (rem > half) | ((rem == half) & (half > 0) & ((base & 1) == 1))
    n[r] = base + up
    code = ((qexp + 9) << 3) + n
    code = np.where(mant == 0, 0, code)
    code = np.minimum(code, 0x7E)
    return (code | (sign << 7)).astype(np.uint8)


SCALE_BYTES = [0, 1, 100, 119, 120, 127, 135, 246]


@pytest.mark.parametrize("byte", SCALE_BYTES)
def test_brute_force_all_bf16_against_bit_level_rne(byte):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    y = v[fin] / e8m0_to_f64(np.array([byte]))[0]
    got = e4m3_rne_sat(y)
    want = _int_rne_e4m3(bits[fin], byte)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("byte", SCALE_BYTES)
def test_brute_force_all_bf16_against_torch_cast(byte):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    y = v[fin] / e8m0_to_f64(np.array([byte]))[0]
    ref = torch.from_numpy(np.clip(y, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_rne_sat(y), ref)


def test_scale_byte_from_bf16_exponent_field():
    # for a finite nonzero BF16 amax the byte is max(exponent_field - 8, 0): an independent form
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    ef = (bits.astype(np.int64) >> 7) & 0xFF
    assert np.array_equal(scale_byte(bf16_bits_to_f64(bits)), np.maximum(ef - 8, 0).astype(np.uint8))


# ----------------------------------------------------------------------------- bounds and relations

def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((n, 32)) * np.ldexp(1.0, rng.integers(-135, 120, size=(n, 1)))
    v = bf16_bits_to_f64(np.frombuffer(np.float32(v).tobytes(), dtype=np.uint32).astype(np.uint64) >> 16)
    return v.reshape(n, 32)


def test_round_trip_bound():
    v = _random_blocks(4000, 1)
    q, s = quantize_blocks(v)
    x = e8m0_to_f64(s)[:, None]
    deq = e4m3_to_f64(q) * x
    y = np.abs(v) / x
    ulp = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.where(y > 0, y, 1.0))), -6).astype(int) - 3)
    err = np.abs(deq - v)
    inside = y <= 448
    assert np.all(err[inside] <= 0.5 * ulp[inside] * x.repeat(32, 1)[inside])
    assert np.all(err[~inside] < 64 * x.repeat(32, 1)[~inside])
    amax = np.max(np.abs(v), axis=1)
    dmax = np.max(np.abs(deq), axis=1)
    big = amax >= 2.0 ** -119                 # scale not clamped: amax/X in [256, 512)
    rel = np.abs(dmax[big] - amax[big]) / amax[big]
    assert np.all(rel <= 0.125)
    ratio = amax[big] / x[big, 0]
    assert np.all((ratio >= 256) & (ratio < 512))


def test_metamorphic_scale_sign_permutation():
    v = _random_blocks(500, 2)
    amax = np.max(np.abs(v), axis=1, keepdims=True)
    v = v[amax[:, 0] > 0] / amax[amax[:, 0] > 0]                # amax 1 per block (no clamping)
    q, s = quantize_blocks(v)
    for j in (-50, -3, 1, 17, 100):
        q2, s2 = quantize_blocks(v * 2.0 ** j)
        assert np.array_equal(q2, q) and np.array_equal(s2.astype(int), s.astype(int) + j)
    q3, s3 = quantize_blocks(-v)
    assert np.array_equal(s3, s) and np.array_equal(q3, q ^ 0x80)
    rng = np.random.default_rng(3)
    perm = rng.permutation(32)
    q4, s4 = quantize_blocks(v[:, perm])
    assert np.array_equal(s4, s) and np.array_equal(q4, q[:, perm])


def test_rowwise_and_colwise_layout():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((64, 96))
    q, s = quantize_rowwise(a)
    assert q.shape == (64, 96) and s.shape == (64, 3)
    qb, sb = quantize_blocks(a[5, 32:64][None])
    assert np.array_equal(q[5, 32:64], qb[0]) and s[5, 1] == sb[0]
    qc, sc = quantize_colwise(a)
    assert qc.shape == (96, 64) and sc.shape == (96, 2)
    qb, sb = quantize_blocks(a[32:64, 7][None])               # column 7, second 32-row group
    assert np.array_equal(qc[7, 32:64], qb[0]) and sc[7, 1] == sb[0]
    d = dequantize_rowwise(q, s)
    assert np.max(np.abs(d - a) / np.max(np.abs(a))) < 2 ** -3


# ------------------------------------------------------------------ dequantize (short groups)

def test_dequantize_all_codes_all_scales_against_torch_decoders():
    """Every (E4M3 code, E8M0 byte) pair decodes to the product of torch's own float8_e4m3fn
    and float8_e8m0fnu decoders (library routines, independent of the oracle's tables),
    including byte 0x00 = 2^-127 and 0xFF = NaN."""
    from oracle.mx import dequantize_groups
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # row b: all codes
    scales = np.arange(256, dtype=np.uint8)[:, None].repeat(8, axis=1)  # 256 columns = 8 groups
    got = dequantize_groups(codes, scales)
    e4 = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    e8 = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e8m0fnu).double().numpy()
    want = e8[:, None] * e4[None, :]
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert e8[0] == 2.0 ** -127 and np.isnan(e8[255])


@pytest.mark.parametrize("cols", [1, 31, 33, 63, 100, 129])
def test_dequantize_short_last_group_uses_its_own_scale(cols):
    """With C % 32 != 0 the last group of each row is short and has its own scale byte;
    full-width rows decode like the row-wise decoder on the padded matrix."""
    from oracle.mx import dequantize_groups
    rng = np.random.default_rng(cols)
    g = -(-cols // 32)
    q = rng.integers(0, 256, size=(5, cols), dtype=np.uint8)
    s = rng.integers(100, 150, size=(5, g), dtype=np.uint8)
    got = dequantize_groups(q, s)
    qp = np.zeros((5, g * 32), dtype=np.uint8)
    qp[:, :cols] = q
    want = dequantize_rowwise(qp, s)[:, :cols]
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    # element c of a row is scaled by byte s[r, c // 32] alone
    k = cols - 1
    v = e4m3_to_f64(q[:, k]) * e8m0_to_f64(s[:, k // 32])
    assert np.array_equal(np.nan_to_num(got[:, k], nan=-1.0), np.nan_to_num(v, nan=-1.0))


def test_dequantize_output_rounding_and_overflow():
    """BF16 / FP32 outputs are one RNE rounding of the exact product; 448 * 2^127 overflows
    both to infinity, and 2^-9 * 2^-127 = 2^-136 is an FP32 subnormal but rounds to zero in
    BF16 (below half of its smallest subnormal 2^-133)."""
    from oracle.mx import dequantize_to
    q = np.array([[0x7E, 0x01, 0x38, 0xFE]], dtype=np.uint8)   # 448, 2^-9, 1.0, -448
    for byte, bf16_want, f32_want in (
        # 448 * 2^127 -> inf; 2^118 -> exponent field 245; 2^127 -> field 254
        (254, [0x7F80, 0x7A80, 0x7F00, 0xFF80], [np.inf, 2.0 ** 118, 2.0 ** 127, -np.inf]),
        # 1.75 * 2^-119 -> field 8, mantissa 0x60; 2^-136 -> 0; 2^-127 -> subnormal 0x40
        (0, [0x0460, 0x0000, 0x0040, 0x8460], [448 * 2.0 ** -127, 2.0 ** -136, 2.0 ** -127, -448 * 2.0 ** -127]),
    ):
        s = np.array([[byte]], dtype=np.uint8)
        assert dequantize_to(q, s, "bf16").tolist() == [bf16_want]
        assert dequantize_to(q, s, "f32").astype(np.float64).tolist() == [f32_want]
