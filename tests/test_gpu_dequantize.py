"""MXFP8 dequantization on the GPU against the oracle (bit-exact), through the C ABI.

The oracle (oracle.mx.dequantize_to) decodes exactly in fp64 and rounds once to the output
format; the kernel's outputs must equal it bit for bit, for every (code, scale byte) pair, for
short last groups, and on the quantizer workload's own codes.
"""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu
from oracle.mx import dequantize_to

pytestmark = pytest.mark.gpu


def _run(mx, q, s, dtype):
    out = mx.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), out_dtype=dtype)
    torch.cuda.synchronize()
    return out.cpu()


def _mismatches(got, want, nan_got, nan_want):
    bad = (nan_got != nan_want) | (~nan_want & (got != want))
    idx = np.argwhere(bad)[:8]
    return int(bad.sum()), [(tuple(int(v) for v in i), hex(int(got[tuple(i)])), hex(int(want[tuple(i)]))) for i in idx]


def _check(mx, q, s):
    """Bit-exact for every non-NaN output; NaN exactly where the oracle has NaN (a NaN's
    payload and sign bit are not part of the decode)."""
    got = _run(mx, q, s, torch.bfloat16).view(torch.uint16).numpy()
    want = dequantize_to(q, s, "bf16")
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_w = (want & 0x7FFF) > 0x7F80
    n, ex = _mismatches(got, want, nan_g, nan_w)
    assert n == 0, f"bf16: {n} mismatches, e.g. (row, col), got, want: {ex}"
    got32 = _run(mx, q, s, torch.float32).numpy().view(np.uint32)
    want32 = dequantize_to(q, s, "f32").view(np.uint32)
    n, ex = _mismatches(got32, want32, (got32 & 0x7FFFFFFF) > 0x7F800000, (want32 & 0x7FFFFFFF) > 0x7F800000)
    assert n == 0, f"f32: {n} mismatches, e.g. (row, col), got, want: {ex}"


def test_every_code_under_every_scale_byte():
    mx = require_gpu()
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))                # row b: all 256 codes
    s = np.arange(256, dtype=np.uint8)[:, None].repeat(8, axis=1)        # row b: scale byte b
    _check(mx, q, s)


@pytest.mark.parametrize("rows,cols", [(7, 1), (5, 31), (9, 33), (3, 100), (64, 129), (17, 4097), (33, 4096)])
def test_short_last_groups_and_ragged_shapes(rows, cols):
    mx = require_gpu()
    rng = np.random.default_rng(rows * 10007 + cols)
    q = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    s = rng.integers(0, 256, size=(rows, -(-cols // 32)), dtype=np.uint8)
    _check(mx, q, s)


def test_round_trip_of_the_quantizer_workload():
    """Dequantizing the standalone quantizer's row-wise output of the 16384 x 7168 workload
    (sampled rows checked against the oracle; all rows checked for NaN-freedom)."""
    mx = require_gpu()
    import workloads
    x = workloads.quant_matrix(device="cuda")
    q, s, _, _ = mx.quantize(x, mx.ROW)
    out = mx.dequantize(q, s)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    rows = np.random.default_rng(3).choice(x.shape[0], size=24, replace=False)
    qs, ss = q[rows].cpu().numpy(), s[rows].cpu().numpy()
    got = out[rows].view(torch.uint16).cpu().numpy()
    want = dequantize_to(qs, ss, "bf16")
    n, ex = _mismatches(got, want, (got & 0x7FFF) > 0x7F80, (want & 0x7FFF) > 0x7F80)
    assert n == 0, f"{n} mismatches: {ex}"


@pytest.mark.parametrize("e5m2", [False, True])
def test_inputs_past_one_grid_pass(e5m2):
    """More 16-code units than one launch has threads (2^24): the kernel's grid-stride loop
    steps (row, chunk) by the stride, wrapping past the row end. 86000 x 7184 codes (449 chunks
    a row, 2.3 passes); the rows where the second and third passes start, the last rows and
    random rows are checked in full against the oracle, in BF16 and FP32."""
    mx = require_gpu()
    rows, cols = 86000, 7184
    gen = torch.Generator(device="cuda").manual_seed(11 + e5m2)
    q = torch.randint(0, 256, (rows, cols), dtype=torch.uint8, device="cuda", generator=gen)
    s = torch.randint(0, 256, (rows, cols // 32 + 1), dtype=torch.uint8, device="cuda", generator=gen)
    fmt = "e5m2" if e5m2 else "e4m3"
    pass_rows = [(k << 24) // (cols // 16) for k in (1, 2)]
    pick = sorted(set([0, 1] + [r + d for r in pass_rows for d in range(-3, 4)] + list(range(rows - 4, rows))
                      + np.random.default_rng(5).choice(rows, size=16, replace=False).tolist()))
    qs, ss = q[pick].cpu().numpy(), s[pick].cpu().numpy()
    for dtype, sign in ((torch.bfloat16, 0x7FFF), (torch.float32, 0x7FFFFFFF)):
        out = mx.dequantize(q, s, out_dtype=dtype, e5m2=e5m2)
        torch.cuda.synchronize()
        if dtype == torch.bfloat16:
            got = out[pick].view(torch.uint16).cpu().numpy()
            want, inf = dequantize_to(qs, ss, "bf16", fmt), 0x7F80
        else:
            got = out[pick].cpu().numpy().view(np.uint32)
            want, inf = dequantize_to(qs, ss, "f32", fmt).view(np.uint32), 0x7F800000
        del out
        n, ex = _mismatches(got, want, (got & sign) > inf, (want & sign) > inf)
        assert n == 0, f"{dtype}: {n} mismatches, e.g. (sampled row, col), got, want: {ex}"


def test_empty_is_a_noop():
    mx = require_gpu()
    mx.mxfp8_dequantize(0, 0, 0, 64, mx.DEQ_BF16, 0)
    mx.mxfp8_dequantize(0, 0, 64, 0, mx.DEQ_F32, 0)
