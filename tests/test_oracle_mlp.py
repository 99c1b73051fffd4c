"""Pins for the oracle's routed-experts SwiGLU MLP (CPU only).

* GEMM orientation, packing and the backward formulas: with identity
  quantization and no rounding, the oracle's backward must equal central finite
  differences of its own forward (a transposed operand, a dropped term or a
  wrong sign in dSwiGLU fails this).
* dSwiGLU closed forms (silu'(0) = 1/2, the limits at +-infinity).
* The pages' test designs: zero-token experts get exact-zero weight gradients,
  a backward with zero routed tokens works, NaN-poisoned pad and tail rows
  leave every output bitwise unchanged (torchtitan PR #12, "Evidence"); the
  32-block pack round-trips (same section).
* The stage-wise helpers the GPU parity tests use agree with the full chain.
"""
import math

import numpy as np
import pytest

from oracle import mlp
from oracle.formats import bf16_bits_to_f64, f64_to_bf16_bits
from oracle.mx import quantize_colwise, quantize_rowwise


def _rand_problem(seed, counts, pad, d, f, scale_w=0.1):
    rng = np.random.default_rng(seed)
    e = len(counts)
    offs = [0]
    for c in counts:
        offs.append(offs[-1] + (c + pad - 1) // pad * pad)
    m = offs[-1]
    x = rng.standard_normal((m, d))
    dy = rng.standard_normal((m, d))
    w1 = rng.standard_normal((e, f, d)) * scale_w
    w3 = rng.standard_normal((e, f, d)) * scale_w
    w2 = rng.standard_normal((e, d, f)) * scale_w
    return x, dy, w1, w3, w2, offs


# ----------------------------------------------------------------------------- packing

def test_pack_layout_and_round_trip():
    rng = np.random.default_rng(0)
    w1 = rng.integers(0, 1 << 16, size=(3, 64, 8)).astype(np.uint16)
    w3 = rng.integers(0, 1 << 16, size=(3, 64, 8)).astype(np.uint16)
    w13 = mlp.pack_w13(w1, w3)
    assert w13.shape == (3, 128, 8)
    for e in range(3):
        for n in range(128):
            j, r = divmod(n, 64)
            src = w1 if r < 32 else w3
            assert np.array_equal(w13[e, n], src[e, 32 * j + r % 32])
    a, b = mlp.unpack_w13(w13)
    assert np.array_equal(a, w1) and np.array_equal(b, w3)


def test_pack_commutes_with_quantization():
    rng = np.random.default_rng(1)
    w1 = rng.standard_normal((1, 96, 64)) * 0.02
    w3 = rng.standard_normal((1, 96, 64)) * 3.0
    w13 = mlp.pack_w13(w1, w3)[0]
    q13, s13 = quantize_rowwise(w13)
    q1, s1 = quantize_rowwise(w1[0])
    q3, s3 = quantize_rowwise(w3[0])
    assert np.array_equal(q13, mlp.pack_w13(q1[None], q3[None])[0])
    assert np.array_equal(s13, mlp.pack_w13(s1[None], s3[None])[0])
    # along 2F: the 32-row interleave keeps every group inside one source matrix
    qc13, sc13 = quantize_colwise(w13)                 # [D, 2F]
    qc1, sc1 = quantize_colwise(w1[0])                 # [D, F]
    qc3, sc3 = quantize_colwise(w3[0])
    assert np.array_equal(qc13, mlp.join_gu(qc1, qc3))
    assert np.array_equal(sc13.reshape(64, -1, 2), np.stack([sc1, sc3], axis=-1))


# ----------------------------------------------------------------------------- dSwiGLU

def test_dswiglu_closed_forms():
    dg, du = mlp.dswiglu(np.array([1.0]), np.array([0.0]), np.array([1.0]))
    assert dg[0] == 0.5 and du[0] == 0.0                 # silu'(0) = 1/2, silu(0) = 0
    dg, du = mlp.dswiglu(np.array([2.0]), np.array([60.0]), np.array([3.0]))
    assert math.isclose(dg[0], 6.0, rel_tol=1e-12) and math.isclose(du[0], 120.0, rel_tol=1e-12)
    dg, du = mlp.dswiglu(np.array([2.0]), np.array([-60.0]), np.array([3.0]))
    assert abs(dg[0]) < 1e-20 and abs(du[0]) < 1e-20
    g = np.linspace(-8, 8, 101)
    h = 1e-6
    num = (mlp.swiglu(g + h, 1.0) - mlp.swiglu(g - h, 1.0)) / (2 * h)
    assert np.allclose(mlp.dswiglu(1.0, g, 1.0)[0], num, rtol=1e-8, atol=1e-10)


# ----------------------------------------------------------------------------- finite differences

def _loss(x, w1, w3, w2, offs, counts, dy):
    y = mlp.mlp_forward(x, w1, w3, w2, offs, counts, policy=mlp.Exact)["y"]
    return float(np.sum(y * dy[:offs[-1]]))


def test_exact_backward_matches_finite_differences():
    counts = [20, 0, 32]
    x, dy, w1, w3, w2, offs = _rand_problem(5, counts, 32, 32, 64)
    fwd = mlp.mlp_forward(x, w1, w3, w2, offs, counts, policy=mlp.Exact)
    bwd = mlp.mlp_backward(fwd, dy)
    rng = np.random.default_rng(6)
    h = 1e-5

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + h
        lp = _loss(x, w1, w3, w2, offs, counts, dy)
        arr[idx] = old - h
        lm = _loss(x, w1, w3, w2, offs, counts, dy)
        arr[idx] = old
        return (lp - lm) / (2 * h)

    for name, arr, grad in (("x", x, bwd["dx"]), ("w1", w1, bwd["dw1"]),
                            ("w3", w3, bwd["dw3"]), ("w2", w2, bwd["dw2"])):
        scale = np.max(np.abs(grad))
        assert scale > 0
        for _ in range(25):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            if name == "x" and idx[0] >= offs[-1]:
                continue
            want = fd(arr, idx)
            assert abs(grad[idx] - want) <= 1e-6 * scale + 1e-9, (name, idx, grad[idx], want)
    # pad rows are read as zero: their input gradient is zero, and so is the FD
    pad_row = offs[0] + counts[0] + 3
    assert np.all(bwd["dx"][pad_row] == 0)
    assert fd(x, (pad_row, 4)) == 0.0
    # the zero-token expert has exact-zero weight gradients
    assert np.all(bwd["dw1"][1] == 0) and np.all(bwd["dw3"][1] == 0) and np.all(bwd["dw2"][1] == 0)


# ----------------------------------------------------------------------------- quantized chain

def _bf16(a):
    return bf16_bits_to_f64(f64_to_bf16_bits(a))


@pytest.fixture(scope="module")
def small_mx():
    counts = [40, 0, 100, 7]
    x, dy, w1, w3, w2, offs = _rand_problem(11, counts, 128, 64, 96, scale_w=0.02)
    x, dy, w1, w3, w2 = (_bf16(a) for a in (x, dy, w1, w3, w2))
    fwd = mlp.mlp_forward(x, w1, w3, w2, offs, counts)
    bwd = mlp.mlp_backward(fwd, dy)
    return dict(x=x, dy=dy, w1=w1, w3=w3, w2=w2, offs=offs, counts=counts, fwd=fwd, bwd=bwd)


def test_zero_token_expert_exact_zero_grads(small_mx):
    b = small_mx["bwd"]
    assert np.all(b["dw1"][1] == 0) and np.all(b["dw3"][1] == 0) and np.all(b["dw2"][1] == 0)
    assert np.any(b["dw1"][0] != 0) and np.any(b["dw2"][2] != 0)


def test_pad_rows_produce_zero(small_mx):
    f, b, offs, counts = small_mx["fwd"], small_mx["bwd"], small_mx["offs"], small_mx["counts"]
    mask = mlp.real_rows_mask(offs, counts, offs[-1])
    assert np.all(f["y"][~mask] == 0) and np.all(b["dx"][~mask] == 0)
    assert np.all(f["hq_r"][~mask] & 0x7F == 0)


def test_nan_poisoned_pad_and_tail_leave_outputs_unchanged(small_mx):
    s = small_mx
    m = s["offs"][-1]
    mask = mlp.real_rows_mask(s["offs"], s["counts"], m)
    x = np.concatenate([s["x"], np.full((64, s["x"].shape[1]), np.nan)])
    dy = np.concatenate([s["dy"], np.full((64, s["dy"].shape[1]), np.nan)])
    x[:m][~mask] = np.nan
    dy[:m][~mask] = np.nan
    fwd = mlp.mlp_forward(x, s["w1"], s["w3"], s["w2"], s["offs"], s["counts"])
    bwd = mlp.mlp_backward(fwd, dy)
    assert np.array_equal(fwd["y"], s["fwd"]["y"])
    for k in ("dx", "dw1", "dw3", "dw2"):
        assert np.array_equal(bwd[k], s["bwd"][k]), k


def test_zero_routed_tokens_and_zero_dy():
    counts = [0, 0]
    x, dy, w1, w3, w2, offs = _rand_problem(12, counts, 128, 64, 64)
    fwd = mlp.mlp_forward(x, w1, w3, w2, offs, counts)
    bwd = mlp.mlp_backward(fwd, dy)
    assert fwd["y"].shape == (0, 64)
    assert all(np.all(bwd[k] == 0) for k in ("dw1", "dw3", "dw2"))
    counts = [50, 70]
    x, dy, w1, w3, w2, offs = _rand_problem(13, counts, 128, 64, 64)
    fwd = mlp.mlp_forward(x, w1, w3, w2, offs, counts)
    bwd = mlp.mlp_backward(fwd, np.zeros_like(dy))
    assert all(np.all(bwd[k] == 0) for k in ("dx", "dw1", "dw3", "dw2"))


def test_stagewise_helpers_agree_with_chain(small_mx):
    f, b = small_mx["fwd"], small_mx["bwd"]
    h13_bits = f64_to_bf16_bits(f["h13"])
    h_bits, hq_r, hs_r, hq_c, hs_c = mlp.swiglu_quant_from_h13(h13_bits)
    assert np.array_equal(hq_r, f["hq_r"]) and np.array_equal(hs_r, f["hs_r"])
    assert np.array_equal(hq_c, f["hq_c"]) and np.array_equal(hs_c, f["hs_c"])
    a, e = small_mx["offs"][2], small_mx["offs"][3]
    y = mlp.gemm_deq(f["hq_r"][a:e], f["hs_r"][a:e], f["w2q_r"][2], f["w2s_r"][2])
    assert np.array_equal(y, f["y"][a:e])
    dh = np.zeros_like(b["dh"])
    for i, (p, q) in enumerate(mlp.segments(small_mx["offs"])):
        if q > p:
            dh[p:q] = mlp.gemm_deq(b["dyq_r"][p:q], b["dys_r"][p:q], f["w2q_c"][i], f["w2s_c"][i])
    dh13, q_r, s_r, q_c, s_c = mlp.dswiglu_quant(dh, h13_bits)
    assert np.array_equal(q_r, b["dhq_r"]) and np.array_equal(q_c, b["dhq_c"])
    assert np.array_equal(s_r, b["dhs_r"]) and np.array_equal(s_c, b["dhs_c"])


def test_quantized_output_sqnr_band(small_mx):
    s = small_mx
    ex = mlp.mlp_forward(s["x"], s["w1"], s["w3"], s["w2"], s["offs"], s["counts"], policy=mlp.Exact)
    mask = mlp.real_rows_mask(s["offs"], s["counts"], s["offs"][-1])
    ref = ex["y"][mask]
    err = s["fwd"]["y"][mask] - ref
    sqnr = 10 * np.log10(np.sum(ref ** 2) / np.sum(err ** 2))
    # three MXFP8 roundings in series (X, W13, h; W2): ~6 dB per mantissa bit, 3 bits
    assert 20.0 < sqnr < 35.0, sqnr
