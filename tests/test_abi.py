"""The C-ABI library loads, exports what include/mxfp8.h declares, and rejects bad
arguments on the host before touching a GPU (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

import mxfp8_mixed_precision_amd as mx
from mxfp8_mixed_precision_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    L = mx.lib()
    decl = declared_functions()
    assert "mxfp8_quantize" in decl and "grouped_mlp_fwd" in decl and "grouped_mlp_bwd" in decl
    assert sorted(decl) == sorted(_abi.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name
    assert mx.abi_version() == 1


def test_header_enums_match_binding():
    text = open(HEADER).read()
    body = text[text.index("typedef enum {\n  MXF_T_STATUS"):]
    body = body[:body.index("} mxf_tensor;")]
    names = re.findall(r"MXF_T_([A-Z0-9_]+)", body)
    names = [n for n in names if n != "COUNT"]
    assert names == _abi.TENSORS
    for code, name in _abi.STATUS_NAMES.items():
        assert re.search(rf"{name} = {code}\b", text), name


def _desc(E=4, D=256, F=256, pad=128, m=1280, flags=0):
    return mx.make_desc(E, D, F, pad, m, flags)


def test_layout_is_consistent():
    d = _desc()
    saved, ws = mx.mlp_saved_bytes(d), mx.mlp_workspace_bytes(d)
    assert saved > 0 and ws > 0
    E, D, F, M = 4, 256, 256, 1280
    expect = {"XQ_C": D * M, "W13Q_C": E * D * 2 * F, "H13": M * 2 * F * 2, "HQ_C": F * M,
              "XQ_R": M * D, "DHQ_R": M * 2 * F, "STATUS": 4, "H13_F32": 0}
    spans = {0: [], 1: []}
    for name in _abi.TENSORS:
        region, off, nb = mx.mlp_tensor(d, name)
        if name in expect:
            assert nb == expect[name], name
        assert off % 256 == 0
        assert off + nb <= (saved if region == 1 else ws)
        spans[region].append((off, off + nb, name))
    # saved tensors never overlap each other
    s = sorted(spans[1])
    assert all(a[1] <= b[0] for a, b in zip(s, s[1:]))
    # forward-only and backward-only workspace tensors may share space, but each group is disjoint
    fwd = {"STATUS", "XQ_R", "XS_R", "W13Q_R", "W13S_R", "W2Q_R", "W2S_R", "HQ_R", "HS_R", "H13_F32"}
    for group in (fwd, set(_abi.TENSORS) - fwd - {n for _, _, n in spans[1]}):
        g = sorted(x for x in spans[0] if x[2] in group and x[1] > x[0])
        assert all(a[1] <= b[0] for a, b in zip(g, g[1:])), g
    # the debug flag adds the fp32 tensors
    d2 = _desc(flags=mx.DEBUG_F32)
    assert mx.mlp_tensor(d2, "H13_F32")[2] == M * 2 * F * 4
    assert mx.mlp_workspace_bytes(d2) > ws


@pytest.mark.parametrize("kw,code", [
    (dict(E=0), _abi.E_SHAPE), (dict(E=2000), _abi.E_SHAPE), (dict(D=200), _abi.E_SHAPE),
    (dict(F=96), _abi.E_SHAPE), (dict(pad=64), _abi.E_SHAPE), (dict(m=1000), _abi.E_SHAPE),
    (dict(m=-128), _abi.E_SHAPE),
    (dict(flags=mx.UNFUSED | mx.DEBUG_F32), _abi.E_ARG), (dict(flags=mx.SERIAL | mx.CONCURRENT), _abi.E_ARG),
    (dict(flags=64), _abi.E_ARG),
])
def test_descriptor_rejections(kw, code):
    d = _desc(**kw)
    assert mx.mlp_saved_bytes(d) == 0 and mx.mlp_workspace_bytes(d) == 0
    with pytest.raises(mx.MxfError) as ei:
        mx.mlp_tensor(d, "H13")
    assert ei.value.status == code
    with pytest.raises(mx.MxfError) as ei:
        mx.grouped_mlp_fwd(d, 16, 16, 16, 16, 16, 16, 16, 16, 16, stream=0)
    assert ei.value.status == code
    assert mx.last_error()


def test_mlp_pointer_rejections():
    d = _desc()
    good = 1 << 20
    with pytest.raises(mx.MxfError) as ei:
        mx.grouped_mlp_fwd(d, good, None, None, good, good, good, good, good, good, stream=0)
    assert ei.value.status == _abi.E_NULL and "x" in str(ei.value)
    with pytest.raises(mx.MxfError) as ei:
        mx.grouped_mlp_fwd(d, good, None, good + 8, good, good, good, good, good, good, stream=0)
    assert ei.value.status == _abi.E_ALIGN and "x" in str(ei.value)
    with pytest.raises(mx.MxfError) as ei:
        mx.grouped_mlp_fwd(d, None, None, good, good, good, good, good, good, good, stream=0)
    assert ei.value.status == _abi.E_NULL and "offs" in str(ei.value)
    with pytest.raises(mx.MxfError) as ei:
        mx.grouped_mlp_bwd(d, good, None, good, good, good, None, good, good, good, stream=0)
    assert ei.value.status == _abi.E_NULL and "dw1" in str(ei.value)


def test_offsets_alignment_rejections():
    """offs and counts are int32 arrays: a pointer that is not 4-byte aligned is rejected
    before anything is launched, by the forward, the backward and the fused dispatch."""
    d = _desc()
    good = 1 << 20
    for offs, counts, name in ((good + 2, None, "offs"), (good, good + 1, "counts")):
        with pytest.raises(mx.MxfError) as ei:
            mx.grouped_mlp_fwd(d, offs, counts, good, good, good, good, good, good, good, stream=0)
        assert ei.value.status == _abi.E_ALIGN and name in str(ei.value)
        with pytest.raises(mx.MxfError) as ei:
            mx.grouped_mlp_bwd(d, offs, counts, good, good, good, good, good, good, good, stream=0)
        assert ei.value.status == _abi.E_ALIGN and name in str(ei.value)
        with pytest.raises(mx.MxfError) as ei:
            mx.mxfp8_dispatch_quantize(d, offs, counts, good, good, 8, 2, good, good, stream=0)
        assert ei.value.status == _abi.E_ALIGN and name in str(ei.value)


@pytest.mark.parametrize("rows,cols,mode,code", [
    (64, 48, mx.ROW, _abi.E_SHAPE), (48, 64, mx.COL, _abi.E_SHAPE), (-1, 64, mx.ROW, _abi.E_SHAPE),
    (64, 64, 0, _abi.E_ARG), (64, 64, 4, _abi.E_ARG),
])
def test_quantize_rejections(rows, cols, mode, code):
    good = 1 << 20
    with pytest.raises(mx.MxfError) as ei:
        mx.mxfp8_quantize(good, rows, cols, mode, good, good, good, good, stream=0)
    assert ei.value.status == code


def test_quantize_null_and_alignment():
    good = 1 << 20
    with pytest.raises(mx.MxfError) as ei:
        mx.mxfp8_quantize(good, 64, 64, mx.ROW | mx.COL, good, good, None, good, stream=0)
    assert ei.value.status == _abi.E_NULL
    with pytest.raises(mx.MxfError) as ei:
        mx.mxfp8_quantize(good + 4, 64, 64, mx.ROW, good, good, None, None, stream=0)
    assert ei.value.status == _abi.E_ALIGN


def test_valid_call_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    good = 1 << 20
    with pytest.raises(mx.MxfError) as ei:
        mx.mxfp8_quantize(good, 64, 64, mx.ROW, good, good, None, None, stream=0)
    assert ei.value.status in (_abi.E_HIP, _abi.E_DEVICE)


def test_h13_untile_matches_documented_order():
    """The binding's row-major copy of the tiled h13 follows the element formula stated for
    MXF_T_H13 in include/mxfp8.h (checked index by index on a small case)."""
    import torch
    import mxfp8_mixed_precision_amd as mx
    M, F = 64, 96
    tiled = torch.empty(M * 2 * F, dtype=torch.int64)
    for R in range(M // 32):
        for J in range(F // 32):
            base = (R * (F // 32) + J) * 2048
            for s in range(2):
                for b in range(2):
                    for c in range(32):
                        for k in range(4):
                            for j in range(4):
                                row = 32 * R + 8 * k + 4 * b + j
                                col = 64 * J + 32 * s + c
                                tiled[base + ((2 * s + (k >> 1)) * 64 + c + 32 * b) * 8 + 4 * (k & 1) + j] = \
                                    row * 100000 + col
    rm = mx.h13_rowmajor(tiled, F)
    want = torch.arange(M)[:, None] * 100000 + torch.arange(2 * F)[None, :]
    assert torch.equal(rm, want)


def test_scale_planes_match_documented_order():
    """The binding's row-major copy of a plane-ordered scale tensor follows the byte formula
    stated in include/mxfp8.h, with and without a leading expert dimension."""
    import torch
    import mxfp8_mixed_precision_amd as mx
    for lead in ((), (3,)):
        R, G = 40, 12
        n = 1
        for d in lead:
            n *= d
        planes = torch.empty(n * R * G, dtype=torch.int64)
        for e in range(n):
            for r in range(R):
                for g in range(G):
                    planes[e * R * G + (g // 4) * 4 * R + 4 * r + g % 4] = (e * 1000 + r) * 100 + g
        rm = mx.scales_rowmajor(planes, (*lead, R, G))
        want = ((torch.arange(n)[:, None, None] * 1000 + torch.arange(R)[None, :, None]) * 100
                + torch.arange(G)[None, None, :]).reshape(*lead, R, G)
        assert torch.equal(rm, want)


def test_dequantize_rejections_before_any_launch():
    """Argument errors of mxfp8_dequantize are reported without touching a device."""
    from mxfp8_mixed_precision_amd import _abi
    def st(*a):
        with pytest.raises(mx.MxfError) as ei:
            mx.mxfp8_dequantize(*a, stream=0)
        return ei.value.status
    assert st(16, 16, 4, 32, 7, 16) == _abi.E_ARG              # unknown out_type
    assert st(16, 16, -1, 32, 0, 16) == _abi.E_SHAPE           # negative rows
    assert st(0, 16, 4, 32, 0, 16) == _abi.E_NULL              # q NULL with work to do
    assert st(16, 16, 4, 32, 0, 24) == _abi.E_ALIGN            # out not 16-byte aligned
    mx.mxfp8_dequantize(0, 0, 0, 5, 0, 0, stream=0)            # empty: no-op with NULLs


def test_dispatch_rejections_before_any_launch():
    """Argument errors of the dispatch entry points are reported without touching a device."""
    good = 1 << 20

    def st(fn, *a):
        with pytest.raises(mx.MxfError) as ei:
            fn(*a, stream=0)
        return ei.value.status
    # mxf_route_plan(expert_idx, tokens, topk, E, pad, m_cap, offs, counts, row_assign, assign_row, status, ws)
    rp = mx.mxf_route_plan
    assert st(rp, good, -1, 2, 4, 128, 256, good, good, good, good, None, good) == _abi.E_SHAPE      # tokens
    assert st(rp, good, 8, 0, 4, 128, 256, good, good, good, good, None, good) == _abi.E_SHAPE       # topk
    assert st(rp, good, 8, 65, 4, 128, 256, good, good, good, good, None, good) == _abi.E_SHAPE      # topk
    assert st(rp, good, 1 << 29, 4, 4, 128, 256, good, good, good, good, None, good) == _abi.E_SHAPE  # 2^31 assignments
    assert st(rp, good, 8, 2, 0, 128, 256, good, good, good, good, None, good) == _abi.E_SHAPE       # E
    assert st(rp, good, 8, 2, 1025, 128, 256, good, good, good, good, None, good) == _abi.E_SHAPE    # E
    assert st(rp, good, 8, 2, 4, 0, 256, good, good, good, good, None, good) == _abi.E_SHAPE         # pad
    assert st(rp, good, 8, 2, 4, 128, -1, good, good, good, good, None, good) == _abi.E_SHAPE        # capacity
    assert st(rp, None, 8, 2, 4, 128, 256, good, good, good, good, None, good) == _abi.E_NULL        # expert_idx
    assert st(rp, good, 8, 2, 4, 128, 256, None, good, good, good, None, good) == _abi.E_NULL        # offs
    assert st(rp, good, 8, 2, 4, 128, 256, good, good, None, good, None, good) == _abi.E_NULL        # row_assign
    assert st(rp, good + 2, 8, 2, 4, 128, 256, good, good, good, good, None, good) == _abi.E_ALIGN   # expert_idx
    assert st(rp, good, 8, 2, 4, 128, 256, good, good, good, good, None, None) == _abi.E_NULL        # workspace
    assert mx.route_plan_workspace_bytes(8, 2, 4) == 4 * 5
    assert mx.route_plan_workspace_bytes(1000, 8, 16) == 8 * 17 * 4
    assert mx.route_plan_workspace_bytes(0, 8, 16) == 17 * 4
    assert mx.route_plan_workspace_bytes(8, 2, 0) == 0 and mx.route_plan_workspace_bytes(8, 0, 4) == 0
    # mxf_dispatch_permute(x_tokens, tokens, topk, D, E, offs, row_assign, m_cap, x_out)
    dp = mx.mxf_dispatch_permute
    assert st(dp, good, 8, 2, 12, 4, good, good, 256, good) == _abi.E_SHAPE                  # D % 8
    assert st(dp, good, 8, 2, 64, 4, None, good, 256, good) == _abi.E_NULL                   # offs
    assert st(dp, good, 8, 2, 64, 4, good, good, 256, None) == _abi.E_NULL                   # x_out
    assert st(dp, good + 8, 8, 2, 64, 4, good, good, 256, good) == _abi.E_ALIGN              # x_tokens
    assert st(dp, good, 8, 2, 64, 4, good, good, 256, good + 8) == _abi.E_ALIGN              # x_out
    # mxfp8_dispatch_quantize(desc, offs, counts, row_assign, x_tokens, tokens, topk, saved, workspace)
    dq = mx.mxfp8_dispatch_quantize
    assert st(dq, _desc(D=200), good, good, good, good, 8, 2, good, good) == _abi.E_SHAPE
    assert st(dq, _desc(), good, good, good, good, 8, 0, good, good) == _abi.E_SHAPE
    assert st(dq, _desc(), good, good, None, good, 8, 2, good, good) == _abi.E_NULL
    assert st(dq, _desc(), good, good, good, None, 8, 2, good, good) == _abi.E_NULL
    assert st(dq, _desc(), good, good, good, good, 8, 2, None, good) == _abi.E_NULL
    # grouped_mlp_fwd under MXF_X_QUANTIZED accepts x = NULL (then fails only on the device check;
    # with a GPU present these bogus pointers would be launched on, so that case stops here)
    import torch
    if torch.cuda.is_available():
        return
    d = _desc(flags=mx.X_QUANTIZED)
    with pytest.raises(mx.MxfError) as ei:
        mx.grouped_mlp_fwd(d, good, None, None, good, good, good, good, good, good, stream=0)
    assert ei.value.status in (_abi.E_HIP, _abi.E_DEVICE)


def test_code_panels_match_documented_order():
    """The binding's row-major copy of a code tensor stored in 64-k panels follows the byte
    formula stated in include/mxfp8.h, with and without a leading expert dimension."""
    import torch
    for lead in ((), (3,)):
        R, K = 40, 192
        n = 1
        for d in lead:
            n *= d
        panels = torch.empty(n * R * K, dtype=torch.int64)
        for e in range(n):
            for r in range(R):
                for k in range(K):
                    panels[e * R * K + (k // 64) * 64 * R + 64 * r + k % 64] = (e * 1000 + r) * 1000 + k
        rm = mx.codes_rowmajor(panels, (*lead, R, K))
        want = ((torch.arange(n)[:, None, None] * 1000 + torch.arange(R)[None, :, None]) * 1000
                + torch.arange(K)[None, None, :]).reshape(*lead, R, K)
        assert torch.equal(rm, want)


def test_hbm_probe_rejections_before_any_launch():
    """Argument errors of mxf_hbm_probe are reported without touching a device."""
    def st(mode, src, dst, nbytes):
        with pytest.raises(mx.MxfError) as ei:
            mx.hbm_probe(mode, src, dst, nbytes, stream=0)
        return ei.value.status
    assert st(3, 16, 16, 1024) == _abi.E_ARG          # unknown mode
    assert st(-1, 16, 16, 1024) == _abi.E_ARG
    assert st(2, 16, 16, 0) == _abi.E_SHAPE           # empty
    assert st(2, 16, 16, 1000) == _abi.E_SHAPE        # not a multiple of 16
    assert st(0, 16, 16, 1 << 41) == _abi.E_SHAPE     # over 2^40 bytes
    assert st(0, None, 16, 1024) == _abi.E_NULL       # read needs src
    assert st(1, None, None, 1024) == _abi.E_NULL     # write needs dst
    assert st(2, 24, 16, 1024) == _abi.E_ALIGN        # src not 16-byte aligned
    assert st(1, None, 8, 1024) == _abi.E_ALIGN       # dst not 16-byte aligned


def test_mfma_probe_rejections_before_any_launch():
    """Argument errors of mxf_mfma_probe are reported without touching a device."""
    def st(mode, src, nbytes, stages, blocks, out):
        with pytest.raises(mx.MxfError) as ei:
            mx.mfma_probe(mode, src, nbytes, stages, blocks, out, stream=0)
        return ei.value.status
    ok = dict(mode=1, src=16, nbytes=1 << 21, stages=64, blocks=256, out=16)
    assert st(**ok | dict(mode=2)) == _abi.E_ARG                 # unknown mode
    assert st(**ok | dict(mode=-1)) == _abi.E_ARG
    assert st(**ok | dict(nbytes=65536)) == _abi.E_SHAPE         # below the 128 KB ring seed
    assert st(**ok | dict(nbytes=(1 << 21) + 16)) == _abi.E_SHAPE  # not whole 32 KB chunks
    assert st(**ok | dict(nbytes=1 << 41)) == _abi.E_SHAPE       # over 2^40 bytes
    assert st(**ok | dict(stages=0)) == _abi.E_SHAPE
    assert st(**ok | dict(stages=63)) == _abi.E_SHAPE            # odd
    assert st(**ok | dict(stages=(1 << 24) + 2)) == _abi.E_SHAPE
    assert st(**ok | dict(blocks=0)) == _abi.E_SHAPE
    assert st(**ok | dict(blocks=65536)) == _abi.E_SHAPE
    assert st(**ok | dict(src=None)) == _abi.E_NULL
    assert st(**ok | dict(out=None)) == _abi.E_NULL
    assert st(**ok | dict(src=24)) == _abi.E_ALIGN
    assert st(**ok | dict(out=8)) == _abi.E_ALIGN
