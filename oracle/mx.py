"""MXFP8 block quantization, written from its definition (oracle; test infrastructure).

The method (afd-plugin PR #475 "quantize the A2E FFN transport to MXFP8",
sections "Purpose" and "Test Plan"; torchtitan PR #12 "What it adds") quantizes
a tensor in groups of 32 consecutive elements. Each group stores one E8M0 scale
byte and 32 E4M3 codes. The rule (OCP MX v1.0, MXFP8):

  1. amax = max |v_i| over the 32 elements.
  2. e = floor(log2(amax)) - 8, clamped to [-127, 127]; 8 is the exponent of
     E4M3's largest binade (448 = 1.75 * 2^8). Scale byte = e + 127.
  3. q_i = the E4M3 value nearest to v_i / 2^e, ties to the even mantissa,
     saturated to +-448. The sign is kept (values that round to zero from the
     negative side give -0 = 0x80).

Readings for the points the pages and the rule leave open:
  * an all-zero block has no finite log2; it takes the lowest scale, byte 0x00,
    and all codes 0x00 (or 0x80 for -0);
  * a block holding a NaN or an infinity has no defined scale: byte 0xFF (the
    E8M0 NaN) and every code NaN (0x7F with the element's sign).

The E5M2 variant (afd-plugin PR #475, the description of the transport offers
E5M2 as the alternative element format to E4M3 under the same E8M0 block scale;
a review on the same page places E5M2 at operator level) follows the same rule with the
E5M2 element format: the scale exponent is floor(log2(amax)) - 15 (57344 =
1.75 * 2^15), codes round to nearest even and saturate to +-57344; NaN codes
are 0x7F with the sign (an E5M2 NaN). Selected with fmt="e5m2".

Dual (row-wise and column-wise) quantization is torchtitan PR #12 "What it
adds" ("dual MXFP8 quantization") and PR #2 "Summary": the same matrix is
quantized once in 32-element groups along its rows (for GEMMs contracting over
columns) and once along its columns (for GEMMs contracting over rows). The
column-wise codes are stored transposed, [cols, rows], so that each 32-group is
contiguous; the scales likewise [cols, rows/32].
"""
import numpy as np

from .formats import (E4M3_MAX, E4M3_TABLE, E5M2_MAX, E5M2_TABLE, bf16_bits_to_f64, e4m3_to_f64, e5m2_to_f64,
                      e8m0_to_f64, f64_to_bf16_bits)

BLOCK = 32

# Non-negative finite E4M3 magnitudes, ascending: codes 0x00 .. 0x7E.
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = E4M3_TABLE[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)
# Non-negative finite E5M2 magnitudes, ascending: codes 0x00 .. 0x7B (0x7C is infinity).
_POS_CODES_E5M2 = np.arange(0x7C, dtype=np.uint8)
_POS_VALUES_E5M2 = E5M2_TABLE[:0x7C]
assert np.all(np.diff(_POS_VALUES_E5M2) > 0)
EMAX = {"e4m3": 8, "e5m2": 15}


def scale_byte(amax, emax=8):
    """Step 2 of the rule: E8M0 byte for a block with the given amax (fp64 >= 0); emax is
    the exponent of the element format's largest binade (8 for E4M3, 15 for E5M2)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(np.isfinite(amax) & (amax > 0), amax, 1.0)
    _, p = np.frexp(safe)                 # safe = f * 2^p with f in [0.5, 1): floor(log2) = p - 1
    e = np.clip((p - 1) - emax, -127, 127)
    byte = (e + 127).astype(np.int64)
    byte = np.where(amax == 0, 0, byte)
    byte = np.where(~np.isfinite(amax), 255, byte)
    return byte.astype(np.uint8)


def e4m3_rne_sat(y):
    """Step 3 of the rule: nearest E4M3 code to fp64 y, ties to even, saturating.

    Nearest-value search over the table of representable magnitudes: locate the
    two neighbours of |y|, keep the closer one, and on an exact tie keep the one
    whose code (= whose mantissa) is even. |y| >= 448 gives 0x7E.
    NaN gives 0x7F with the sign bit of the input.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    fin = np.isfinite(a)
    ac = np.where(fin, np.minimum(a, E4M3_MAX), 0.0)
    hi = np.searchsorted(_POS_VALUES, ac, side="left")      # first value >= ac
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    dlo = ac - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - ac
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    pick_hi |= (_POS_VALUES[hi] == ac)
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(fin, code, np.uint8(0x7F)).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    return code


def e5m2_rne_sat(y):
    """Nearest E5M2 code to fp64 y, ties to even, saturating: the same search as
    e4m3_rne_sat over the finite E5M2 magnitudes (codes 0x00 .. 0x7B). |y| >= 57344 gives
    0x7B; NaN gives 0x7F with the sign bit of the input."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    fin = np.isfinite(a)
    ac = np.where(fin, np.minimum(a, E5M2_MAX), 0.0)
    hi = np.clip(np.searchsorted(_POS_VALUES_E5M2, ac, side="left"), 0, len(_POS_VALUES_E5M2) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES_E5M2) - 1)
    dlo = ac - _POS_VALUES_E5M2[lo]
    dhi = _POS_VALUES_E5M2[hi] - ac
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES_E5M2[hi] % 2 == 0))
    pick_hi |= (_POS_VALUES_E5M2[hi] == ac)
    code = np.where(pick_hi, _POS_CODES_E5M2[hi], _POS_CODES_E5M2[lo]).astype(np.uint8)
    code = np.where(fin, code, np.uint8(0x7F)).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)
    return code


def quantize_blocks(v, fmt="e4m3"):
    """Quantize fp64 values shaped [..., 32] block by block, with E4M3 (default) or E5M2
    elements.

    Returns (codes uint8 [..., 32], scale bytes uint8 [...]).
    """
    v = np.asarray(v, dtype=np.float64)
    assert v.shape[-1] == BLOCK and fmt in EMAX
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(v), axis=-1)
    amax = np.where(np.any(np.isnan(v), axis=-1), np.nan, amax)
    byte = scale_byte(amax) if fmt == "e4m3" else scale_byte(amax, EMAX[fmt])
    x = e8m0_to_f64(np.where(byte == 255, 127, byte))       # 2^e; exact
    y = v / x[..., None]                                    # exact: division by a power of two
    codes = e4m3_rne_sat(y) if fmt == "e4m3" else e5m2_rne_sat(y)
    bad = (byte == 255)[..., None]
    nan_codes = np.where(np.signbit(v), np.uint8(0xFF), np.uint8(0x7F)).astype(np.uint8)
    codes = np.where(bad, nan_codes, codes).astype(np.uint8)
    return codes, byte


def quantize_rowwise(a, fmt="e4m3"):
    """Row-wise MXFP8: 32-groups along the last axis of a [R, C] fp64 matrix.

    Returns q [R, C] uint8 and s [R, C/32] uint8.
    """
    a = np.asarray(a, dtype=np.float64)
    r, c = a.shape
    assert c % BLOCK == 0, "row-wise groups need cols % 32 == 0"
    q, s = quantize_blocks(a.reshape(r, c // BLOCK, BLOCK), fmt)
    return q.reshape(r, c), s


def quantize_colwise(a, fmt="e4m3"):
    """Column-wise MXFP8: 32-groups along the first axis of a [R, C] matrix.

    Returns q_c [C, R] uint8 (transposed: each column's codes contiguous) and
    s_c [C, R/32] uint8. By definition of the layout this is the row-wise
    quantization of the transpose.
    """
    a = np.asarray(a, dtype=np.float64)
    assert a.shape[0] % BLOCK == 0, "column-wise groups need rows % 32 == 0"
    return quantize_rowwise(a.T, fmt)


def dequantize_rowwise(q, s):
    """deq[r, c] = E4M3(q[r, c]) * E8M0(s[r, c // 32]), exact in fp64."""
    q = np.asarray(q, dtype=np.uint8)
    r, c = q.shape
    x = e8m0_to_f64(s).reshape(r, c // BLOCK, 1)
    return (e4m3_to_f64(q).reshape(r, c // BLOCK, BLOCK) * x).reshape(r, c)


def dequantize_groups(q, s, fmt="e4m3"):
    """Row-wise MXFP8 decode when the last group of a row may be short (afd-plugin PR #475
    "quantize the A2E FFN transport to MXFP8", third review: hidden sizes that are not a
    multiple of 32 leave a final group of fewer than 32 elements, which has its own scale).

    q [R, C] uint8 codes for any C >= 0; s [R, ceil(C/32)] uint8 scale bytes.
    deq[r, c] = E4M3(q[r, c]) * E8M0(s[r, c // 32]), exact in fp64 (E8M0 0x00 = 2^-127,
    0xFF = NaN; E4M3 0x7F / 0xFF = NaN).
    """
    q = np.asarray(q, dtype=np.uint8)
    r, c = q.shape
    s = np.asarray(s, dtype=np.uint8)
    assert s.shape == (r, -(-c // BLOCK))
    grp = np.arange(c) // BLOCK
    dec = e4m3_to_f64(q) if fmt == "e4m3" else e5m2_to_f64(q)   # E5M2: 0x7C/0xFC = +-Inf, 0x7D..0x7F NaN
    with np.errstate(invalid="ignore"):
        return dec * e8m0_to_f64(s)[:, grp]


def dequantize_to(q, s, dtype, fmt="e4m3"):
    """dequantize_groups rounded once to the output format: "bf16" (RNE, returned as uint16
    bit patterns) or "f32" (RNE, returned as float32). Both overflow to infinity."""
    v = dequantize_groups(q, s, fmt)
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    assert dtype == "f32"
    with np.errstate(over="ignore", invalid="ignore"):
        return v.astype(np.float32)

