"""GPU parity of the E5M2 variant (mxfp8_quantize with MXF_E5M2, mxfp8_dequantize with
MXF_DEQ_E5M2) against the oracle (fmt="e5m2"): codes and scale bytes bit-exact for every
BF16 pattern under several scale bytes, hand blocks, ragged shapes and the quantizer
workload; decode bit-exact for every (code, scale byte) pair and on a round trip."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bits, np_u8, require_gpu
from oracle.formats import bf16_bits_to_f64
from oracle.mx import dequantize_to, quantize_colwise, quantize_rowwise

pytestmark = pytest.mark.gpu


def to_dev_bf16(bits_np):
    t = torch.from_numpy(np.ascontiguousarray(bits_np).astype(np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def run_and_compare(mx, x_bits, mode=3):
    x = to_dev_bf16(x_bits)
    q_r, s_r, q_c, s_c = mx.quantize(x, mode | mx.E5M2)
    torch.cuda.synchronize()
    v = bf16_bits_to_f64(x_bits)
    if mode & 1:
        rq, rs = quantize_rowwise(v, "e5m2")
        assert np.array_equal(np_u8(s_r), rs), "row scales"
        assert np.array_equal(np_u8(q_r), rq), "row codes"
    if mode & 2:
        cq, cs = quantize_colwise(v, "e5m2")
        assert np.array_equal(np_u8(s_c), cs), "column scales"
        assert np.array_equal(np_u8(q_c), cq), "column codes"


def exhaustive_matrix(byte, seed):
    """Every BF16 pattern whose magnitude fits under scale byte `byte` (E5M2: exponent field
    up to byte + 15), 31 per group, next to an amax element that fixes the byte."""
    amax = (((byte + 15) << 7) | 0x7F) if byte > 0 else ((15 << 7) | 0x7F)
    mags = np.arange(0, amax + 1, dtype=np.uint32)
    pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    rng = np.random.default_rng(seed)
    pats = pats[rng.permutation(len(pats))]
    ngroups = -(-len(pats) // 31)
    ngroups = -(-ngroups // (8 * 32)) * (8 * 32)
    body = np.zeros(ngroups * 31, dtype=np.uint16)
    body[:len(pats)] = pats
    body = body.reshape(ngroups, 31)
    pos = rng.integers(0, 32, size=ngroups)
    grp = np.zeros((ngroups, 32), dtype=np.uint16)
    for i in range(ngroups):
        grp[i] = np.insert(body[i], pos[i], np.uint16(amax | (0x8000 if i % 3 == 0 else 0)))
    return grp.reshape(ngroups // 8, 8 * 32)


@pytest.mark.parametrize("byte", [0, 1, 100, 112, 113, 127, 135, 239])
def test_every_bf16_pattern_bit_exact(byte):
    mx = require_gpu()
    print(f"\nE5M2 exhaustive, scale byte {byte}", flush=True)
    run_and_compare(mx, exhaustive_matrix(byte, seed=byte))


def _f2b(vals):
    return (np.asarray(vals, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_hand_blocks_bit_exact():
    mx = require_gpu()
    rows = []

    def grp(vals):
        g = np.zeros(32, dtype=np.uint16)
        b = _f2b(vals)
        g[:len(b)] = b
        return g
    rows.append(grp([]))
    rows.append(grp([-0.0, 1.0]))
    for k in (-100, -5, 0, 7, 60):
        rows.append(grp([2.0 ** k, -(2.0 ** k), 1.75 * 2.0 ** k]))
        rows.append(grp([1.875 * 2.0 ** k, 1.9375 * 2.0 ** k]))          # clipped to 57344
        rows.append(grp([2.0 ** k, 2.0 ** (k - 31), 2.0 ** (k - 32), 3 * 2.0 ** (k - 32), -(2.0 ** (k - 40))]))
    rows.append(grp([2.0 ** -112]))
    rows.append(grp([2.0 ** -113]))
    g = np.zeros(32, dtype=np.uint16)
    g[0] = 0x0004
    g[1] = 0x8001
    rows.append(g)
    rows.append(grp([3.3895314e38, -1.0]))
    nan = grp([1.0, 2.0])
    nan[2] = 0x7FC0
    rows.append(nan)
    inf = grp([1.0, -2.0])
    inf[5] = 0xFF80
    rows.append(inf)
    m = np.stack(rows)
    m = np.concatenate([m, np.zeros((32 - len(m) % 32, 32), dtype=np.uint16)])
    run_and_compare(mx, m)


@pytest.mark.parametrize("rows,cols,mode", [(96, 160, 3), (45, 96, 1), (160, 4128, 3), (0, 64, 3)])
def test_ragged_shapes(rows, cols, mode):
    mx = require_gpu()
    rng = np.random.default_rng(rows * 7 + cols)
    v = (rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-30, 30, size=(rows, 1)))).astype(np.float32)
    run_and_compare(mx, _f2b(v).reshape(rows, cols), mode)


def test_quant_workload_band_bit_exact():
    mx = require_gpu()
    cfg = workloads.QUANT_CONFIG
    x = workloads.quant_matrix(cfg["rows"], cfg["cols"], seed=42, device="cuda")
    q_r, s_r, q_c, s_c = mx.quantize(x, 3 | mx.E5M2)
    torch.cuda.synchronize()
    band = slice(4096, 4096 + 256)
    xb = bf16_bits_to_f64(bits(x[band].cpu()))
    rq, rs = quantize_rowwise(xb, "e5m2")
    assert np.array_equal(np_u8(q_r[band]), rq) and np.array_equal(np_u8(s_r[band]), rs)
    cq, cs = quantize_colwise(xb, "e5m2")
    assert np.array_equal(np_u8(q_c[:, band]), cq) and np.array_equal(np_u8(s_c[:, 128:136]), cs)


def _nan_agnostic_equal(got_bits, want_bits, bf16):
    if bf16:
        g = got_bits.astype(np.int64)
        w = want_bits.astype(np.int64)
        gn = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
        wn = ((w & 0x7F80) == 0x7F80) & ((w & 0x7F) != 0)
    else:
        gn, wn = np.isnan(got_bits), np.isnan(want_bits)
        g, w = got_bits.view(np.uint32), want_bits.view(np.uint32)
    assert np.array_equal(gn, wn)
    assert np.array_equal(g[~gn], w[~wn])


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dequantize_every_pair_bit_exact(out):
    mx = require_gpu()
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None].repeat(8, axis=1).copy()
    q = torch.from_numpy(codes).cuda()
    s = torch.from_numpy(scales).cuda()
    got = mx.dequantize(q, s, torch.bfloat16 if out == "bf16" else torch.float32, e5m2=True)
    torch.cuda.synchronize()
    want = dequantize_to(codes, scales, out, "e5m2")
    if out == "bf16":
        _nan_agnostic_equal(bits(got.cpu()), want, True)
    else:
        _nan_agnostic_equal(got.cpu().numpy(), want, False)


@pytest.mark.parametrize("cols", [1, 33, 100, 4097])
def test_dequantize_ragged_widths_and_round_trip(cols):
    mx = require_gpu()
    rng = np.random.default_rng(cols)
    codes = rng.integers(0, 256, size=(7, cols), dtype=np.uint8)
    scales = rng.integers(90, 160, size=(7, -(-cols // 32)), dtype=np.uint8)
    got = mx.dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), e5m2=True)
    torch.cuda.synchronize()
    _nan_agnostic_equal(bits(got.cpu()), dequantize_to(codes, scales, "bf16", "e5m2"), True)
    if cols % 32 == 0:
        return
    # round trip on a 32-multiple width: quantize then decode equals the oracle's decode
    x = workloads.randn_bf16((64, 256), 1.0, workloads._gen(cols, "cpu"), "cpu")
    q_r, s_r, _, _ = mx.quantize(x.cuda(), mx.ROW | mx.E5M2)
    back = mx.dequantize(q_r, s_r, e5m2=True)
    torch.cuda.synchronize()
    rq, rs = quantize_rowwise(bf16_bits_to_f64(bits(x)), "e5m2")
    _nan_agnostic_equal(bits(back.cpu()), dequantize_to(rq, rs, "bf16", "e5m2"), True)
