"""Exact decoders and encoders for BF16, E4M3 and E8M0 (oracle; test infrastructure).

Everything decodes to fp64, in which every BF16, E4M3 and E8M0 value and every
product of an E4M3 value with an E8M0 scale is exactly representable.

E4M3 and E8M0 are the MXFP8 element and scale formats named in afd-plugin
PR #475 "quantize the A2E FFN transport to MXFP8" (section "Purpose": FP8 E4M3
activations plus an E8M0 block scale). Their bit layouts follow the OCP 8-bit
floating point and OCP MX v1.0 specifications:
  * E4M3: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0;
    exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity;
    largest finite magnitude 0x7E = 448.
  * E5M2 (the same page's description of the transport offers it as the
    alternative element format to E4M3, under the same E8M0 block scale): sign bit 7,
    exponent bits 6..2 with bias 15, mantissa bits 1..0; exponent field 0 is
    subnormal (m * 2^-16); exponent field 31 is infinity (m = 0) or NaN;
    largest finite magnitude 0x7B = 57344.
  * E8M0: an unsigned biased exponent, byte b -> 2^(b - 127); 0xFF is NaN.
    The third review on PR #475 (E8M0 decoding) pins the two endpoints: byte
    0x00 is 2^-127 (not zero) and 0xFF is NaN (not infinity).
"""
import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


def bf16_bits_to_f64(bits):
    """BF16 bit patterns (uint16) -> exact fp64 values.

    BF16 is the upper half of an IEEE binary32, so the decode is a 16-bit shift
    into a float32 followed by an exact widening to fp64 (subnormals, infinities
    and NaNs included).
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round fp64 values to BF16 with round-to-nearest-even, in one step.

    The rounding goes straight from fp64 to BF16 (no intermediate float32, so no
    double rounding). BF16 keeps 8 significant bits; its exponent range is that
    of binary32: normal down to 2^-126, subnormal quantum 2^-133, overflow to
    infinity at or above (2 - 2^-8) * 2^127. NaN maps to the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x)
    ax = np.abs(x)
    nan = np.isnan(x)
    fin = np.isfinite(x)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        _, p = np.frexp(np.where(fin & (ax > 0), ax, 1.0))
        e = np.maximum(p - 1, -126)          # exponent of the binade, subnormals share -126
        q = np.ldexp(1.0, e - 7)             # BF16 quantum in that binade
        n = np.rint(ax / q)                  # numpy rint rounds half to even
        v = n * q
    over = fin & (v >= 2.0 ** 128)
    mag = np.where(fin & ~over, v, 0.0).astype(np.float32).view(np.uint32) >> np.uint32(16)
    mag = mag.astype(np.uint16)
    mag = np.where(over | (np.isinf(x)), np.uint16(0x7F80), mag)
    out = np.where(sign, mag | np.uint16(0x8000), mag).astype(np.uint16)
    out = np.where(nan, np.uint16(0x7FC0), out).astype(np.uint16)
    return out


def bf16_round(x):
    """fp64 -> nearest BF16 value (RNE), returned as fp64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def e4m3_value(code):
    """Decode one E4M3 byte from its definition (see module docstring)."""
    code = int(code)
    s = code >> 7
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        v = m * 2.0 ** -9
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


# 256-entry decode table, built from the definition above.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes):
    """E4M3 bytes (uint8 array) -> fp64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e5m2_value(code):
    """Decode one E5M2 byte from its definition (see module docstring)."""
    code = int(code)
    s = code >> 7
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        v = float("inf") if m == 0 else float("nan")
    elif e == 0:
        v = m * 2.0 ** -16
    else:
        v = (1.0 + m / 4.0) * 2.0 ** (e - 15)
    return -v if s else v


E5M2_TABLE = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)


def e5m2_to_f64(codes):
    """E5M2 bytes (uint8 array) -> fp64 values."""
    return E5M2_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_to_f64(b):
    """E8M0 bytes -> 2^(b - 127) as fp64; 0xFF -> NaN; 0x00 -> 2^-127.

    Computed with ldexp on the integer exponent; no bit-shift into a float's
    exponent field (the trick the third review on PR #475 shows dropping 0x00
    to zero).
    """
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, (b - 127).astype(np.int32))
    return np.where(b == 255, np.nan, v)
