"""GPU parity of the standalone MXFP8 quantizer (mxfp8_quantize) against the oracle.

Codes and scale bytes must match bit for bit: every BF16 pattern under several scale
bytes, the closed-form hand blocks, ragged and empty shapes, and the 16384 x 7168
workload (a full band plus sampled groups, which the oracle computes group by group).
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bits, np_u8, require_gpu
from oracle.formats import bf16_bits_to_f64
from oracle.mx import quantize_colwise, quantize_rowwise

pytestmark = pytest.mark.gpu


def to_dev_bf16(bits_np):
    t = torch.from_numpy(np.ascontiguousarray(bits_np).astype(np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def run_and_compare(mx, x_bits, mode=3):
    x = to_dev_bf16(x_bits)
    q_r, s_r, q_c, s_c = mx.quantize(x, mode)
    torch.cuda.synchronize()
    v = bf16_bits_to_f64(x_bits)
    if mode & 1:
        rq, rs = quantize_rowwise(v)
        assert np.array_equal(np_u8(q_r), rq), "row codes"
        assert np.array_equal(np_u8(s_r), rs), "row scales"
    if mode & 2:
        cq, cs = quantize_colwise(v)
        assert np.array_equal(np_u8(q_c), cq), "column codes"
        assert np.array_equal(np_u8(s_c), cs), "column scales"


def exhaustive_matrix(byte, seed):
    """Every BF16 pattern whose magnitude fits under scale byte `byte`, 31 per group, next
    to an amax element that fixes the group's scale byte to `byte`."""
    amax = (((byte + 8) << 7) | 0x7F) if byte > 0 else ((8 << 7) | 0x7F)
    mags = np.arange(0, amax + 1, dtype=np.uint32)
    pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    rng = np.random.default_rng(seed)
    pats = pats[rng.permutation(len(pats))]
    ngroups = -(-len(pats) // 31)
    ngroups = -(-ngroups // (8 * 32)) * (8 * 32)          # rows of 8 groups, rows % 32 == 0
    body = np.zeros(ngroups * 31, dtype=np.uint16)
    body[:len(pats)] = pats
    body = body.reshape(ngroups, 31)
    pos = rng.integers(0, 32, size=ngroups)
    grp = np.zeros((ngroups, 32), dtype=np.uint16)
    for i in range(ngroups):
        grp[i] = np.insert(body[i], pos[i], np.uint16(amax | (0x8000 if i % 3 == 0 else 0)))
    return grp.reshape(ngroups // 8, 8 * 32)


@pytest.mark.parametrize("byte", [0, 1, 100, 119, 120, 127, 135, 246])
def test_every_bf16_pattern_bit_exact(byte):
    mx = require_gpu()
    m = exhaustive_matrix(byte, seed=byte)
    run_and_compare(mx, m)


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
    rows.append(grp([]))                                             # all zero
    rows.append(grp([-0.0, 1.0]))                                    # -0 keeps its sign
    for k in (-100, -5, 0, 7, 60):
        rows.append(grp([2.0 ** k, -(2.0 ** k), 1.75 * 2.0 ** k]))    # power-of-two amax
        rows.append(grp([1.8125 * 2.0 ** k, 1.9375 * 2.0 ** k]))      # tie at 464, clip at 496
        rows.append(grp([2.0 ** k, 2.0 ** (k - 17), 2.0 ** (k - 18), 3 * 2.0 ** (k - 19),
                         3 * 2.0 ** (k - 18), 15 * 2.0 ** (k - 18), -(2.0 ** (k - 30))]))
    rows.append(grp([2.0 ** -119]))
    rows.append(grp([2.0 ** -120]))
    g = np.zeros(32, dtype=np.uint16)
    g[0] = 0x0004                                                    # BF16 subnormal amax 2^-131
    g[1] = 0x8001                                                    # -2^-133
    rows.append(g)
    rows.append(grp([3.3895314e38, -1.0]))                           # largest finite BF16
    nan = grp([1.0, 2.0])
    nan[2] = 0x7FC0
    rows.append(nan)                                                 # NaN group
    inf = grp([1.0, -2.0])
    inf[5] = 0xFF80
    rows.append(inf)                                                 # Inf group
    m = np.stack(rows)
    m = np.concatenate([m, np.zeros((32 - len(m) % 32, 32), dtype=np.uint16)])
    run_and_compare(mx, m)
    # closed forms checked directly on the GPU output for two groups
    x = to_dev_bf16(m)
    q_r, s_r, _, _ = mx.quantize(x, mx.ROW)
    q, s = np_u8(q_r), np_u8(s_r)
    assert s[0, 0] == 0 and np.all(q[0] == 0)
    assert q[1, 0] == 0x80 and q[1, 1] == 0x78 and s[1, 0] == 119


@pytest.mark.parametrize("rows,cols,mode", [(96, 160, 3), (45, 96, 1), (32, 32, 2), (160, 4128, 3),
                                            (1, 32, 1), (0, 64, 3), (64, 0, 3)])
def test_ragged_and_empty_shapes(rows, cols, mode):
    mx = require_gpu()
    rng = np.random.default_rng(rows * 7 + cols)
    v = (rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-30, 30, size=(rows, 1)))).astype(np.float32)
    run_and_compare(mx, _f2b(v).reshape(rows, cols), mode)


@pytest.mark.parametrize("rows,cols,mode", [(2048, 4096, 3), (1984, 4096, 3), (2048, 4000, 1)])
def test_macro_tile_order_every_code(rows, cols, mode):
    """Shapes whose tile grid takes the 8x8 macro-tile block order (rows and column tiles in
    multiples of 8, macro-tiles in a multiple of 8), with a partial last row band or column
    tile: every code and scale byte against the oracle."""
    mx = require_gpu()
    rng = np.random.default_rng(rows + 3 * cols)
    v = (rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-8, 8, size=(rows, 1)))).astype(np.float32)
    run_and_compare(mx, _f2b(v).reshape(rows, cols), mode)


def test_quant_workload_bit_exact_band_and_samples():
    mx = require_gpu()
    cfg = workloads.QUANT_CONFIG
    a = workloads.quant_matrix(cfg["rows"], cfg["cols"], seed=42)
    ab = bits(a)
    x = a.cuda()
    q_r, s_r, q_c, s_c = mx.quantize(x, mx.ROW | mx.COL)
    torch.cuda.synchronize()
    q_r, s_r, q_c, s_c = (np_u8(t) for t in (q_r, s_r, q_c, s_c))
    # a full band of 256 rows x all columns
    band = bf16_bits_to_f64(ab[:256])
    rq, rs = quantize_rowwise(band)
    assert np.array_equal(q_r[:256], rq) and np.array_equal(s_r[:256], rs)
    cq, cs = quantize_colwise(band)
    assert np.array_equal(q_c[:, :256], cq) and np.array_equal(s_c[:, :8], cs)
    # sampled row groups and column groups over the whole matrix
    rng = np.random.default_rng(0)
    n = 20000
    ri = rng.integers(0, cfg["rows"], n)
    gj = rng.integers(0, cfg["cols"] // 32, n)
    vals = bf16_bits_to_f64(ab[ri[:, None], gj[:, None] * 32 + np.arange(32)])
    rq, rs = quantize_rowwise(vals)
    assert np.array_equal(q_r[ri[:, None], gj[:, None] * 32 + np.arange(32)], rq)
    assert np.array_equal(s_r[ri, gj], rs[:, 0])
    ci = rng.integers(0, cfg["cols"], n)
    gi = rng.integers(0, cfg["rows"] // 32, n)
    vals = bf16_bits_to_f64(ab[gi[:, None] * 32 + np.arange(32), ci[:, None]])
    cq, cs = quantize_rowwise(vals)
    assert np.array_equal(q_c[ci[:, None], gi[:, None] * 32 + np.arange(32)], cq)
    assert np.array_equal(s_c[ci, gi], cs[:, 0])
    # the recipe's special groups are present and handled: all-zero row groups give byte 0
    zero_groups = (np.abs(a.float().view(cfg["rows"], -1, 32)).amax(-1) == 0).numpy()
    assert zero_groups.any() and np.all(s_r[zero_groups] == 0)


def test_deterministic_and_stream_ordered():
    mx = require_gpu()
    a = workloads.quant_matrix(2048, 2048, seed=5).cuda()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r1 = mx.quantize(a, 3)
        r2 = mx.quantize(a, 3)
    s.synchronize()
    for t1, t2 in zip(r1, r2):
        assert torch.equal(t1, t2)


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_scale_arrays_at_any_byte_offset(offset):
    """mxfp8_quantize documents its scale arrays as any alignment: with s_row and s_col starting
    `offset` bytes past an aligned address (where whole-word scale stores would be misaligned)
    the codes and scales still equal the oracle's, and the bytes around the arrays are
    untouched."""
    mx = require_gpu()
    rows, cols = 256, 512
    g = torch.Generator(device="cpu")
    g.manual_seed(offset)
    x = torch.randn((rows, cols), generator=g).to(torch.bfloat16)
    xd = x.cuda()
    q_r = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    q_c = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    nsr, nsc = rows * cols // 32, cols * rows // 32
    sr_buf = torch.full((nsr + 16,), 0xA5, dtype=torch.uint8, device="cuda")
    sc_buf = torch.full((nsc + 16,), 0x5A, dtype=torch.uint8, device="cuda")
    s_r = sr_buf[offset:offset + nsr]
    s_c = sc_buf[offset:offset + nsc]
    print(f"\nscale arrays at byte offset {offset}", flush=True)
    mx.mxfp8_quantize(xd, rows, cols, 3, q_r, s_r, q_c, s_c)
    torch.cuda.synchronize()
    v = bf16_bits_to_f64(bits(x))
    rq, rs = quantize_rowwise(v)
    cq, cs = quantize_colwise(v)
    assert np.array_equal(np_u8(q_r), rq) and np.array_equal(np_u8(s_r).reshape(rows, cols // 32), rs)
    assert np.array_equal(np_u8(q_c), cq) and np.array_equal(np_u8(s_c).reshape(cols, rows // 32), cs)
    srb, scb = np_u8(sr_buf), np_u8(sc_buf)
    assert np.all(srb[:offset] == 0xA5) and np.all(srb[offset + nsr:] == 0xA5)
    assert np.all(scb[:offset] == 0x5A) and np.all(scb[offset + nsc:] == 0x5A)
