"""Helpers shared by the GPU parity tests."""
import numpy as np
import pytest
import torch

import workloads


def require_gpu():
    """Skip when no GPU is visible; with a GPU present, fail loudly if the HIP library is unusable."""
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    import mxfp8_mixed_precision_amd as mx
    mx.lib()  # raises if libmxfp8.so is missing
    assert mx.query_device(torch.cuda.current_device()) & mx.CAP_GFX950, "not a gfx950 device"
    return mx


def np_u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def bits(t):
    return workloads.bf16_bits(t)


def normwise(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return num / den if den > 0 else num


def e4m3_ordinal(c):
    c = np.asarray(c).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in representable BF16 steps between two arrays of BF16 bit patterns."""
    def ordv(b):
        b = np.asarray(b).astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(ordv(a_bits) - ordv(b_bits))


def check_fused_codes(gq, gs, rq, rs, max_frac=1e-3, label=""):
    """Fused-epilogue code tolerance.

    Groups lie along the last axis. Every scale byte within 1 of the reference; in a group
    with equal scale every code within one E4M3 step (sign-magnitude ordinal); a group whose
    scale differs counts all 32 codes as differing; at most max_frac of all codes differ.
    Returns the fraction of differing codes.
    """
    gq = np.asarray(gq, dtype=np.uint8)
    rq = np.asarray(rq, dtype=np.uint8)
    r, c = gq.shape
    assert rq.shape == gq.shape and gs.shape == rs.shape == (r, c // 32), label
    sdiff = gs.astype(np.int64) - rs.astype(np.int64)
    assert np.all(np.abs(sdiff) <= 1), (label, int(np.abs(sdiff).max()))
    same = (sdiff == 0)
    od = np.abs(e4m3_ordinal(gq) - e4m3_ordinal(rq)).reshape(r, c // 32, 32)
    assert np.all(od[same] <= 1), (label, int(od[same].max()))
    ndiff = int((od[same] > 0).sum()) + 32 * int((~same).sum())
    frac = ndiff / max(gq.size, 1)
    assert frac <= max_frac, (label, frac)
    return frac


def check_gemm(got, a_deq, b_deq, tol=1e-4, elem=2.0 ** -11, label=""):
    """GEMM parity: normwise relative error <= tol against fp64 A B^T, and every element within
    elem * (|A| |B|^T) of it (an error bound relative to the sum of absolute products, which
    stays meaningful where the sum cancels). The FP8 matrix core accumulates each 64-k step
    with less than fp32 precision; the worst measured ratio, 2.7e-4, is on weight gradients of
    experts with under 128 tokens (a single 128-k step pair), so elem is 2^-11 (4.9e-4).
    Returns (normwise, worst elementwise ratio)."""
    ref = a_deq @ b_deq.T
    got = np.asarray(got, dtype=np.float64)
    nw = normwise(got, ref)
    absref = np.abs(a_deq) @ np.abs(b_deq).T
    err = np.abs(got - ref)
    ratio = float(np.max(err / np.maximum(absref, 1e-300))) if err.size else 0.0
    assert nw <= tol, (label, nw)
    assert np.all(err <= elem * absref), (label, ratio)
    return nw, ratio
