"""The allocation-free routing plan (mxf_route_plan_noalloc) against the workspace plan
(mxf_route_plan): bit-identical offsets, counts, row and assignment maps and status on the
same expert ids, for two calls in a row on one GPU, the second with a smaller input (the
static scratch then holds the first call's histograms). Size limit checked on the host."""
import os
import re

import numpy as np
import pytest
import torch

import mxfp8_mixed_precision_amd as mx
from mxfp8_mixed_precision_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SENT = -7


def _ids(seed, tokens, topk, E, zero=()):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.7))
    for e in zero:
        p[e] = 0
    p /= p.sum()
    return rng.choice(E, size=(tokens, topk), p=p).astype(np.int32)


def _plan(fn, ids, E, pad, mcap, with_ws):
    tokens, topk = ids.shape
    d = torch.from_numpy(ids).cuda()
    out = {"offs": torch.full((E + 1,), SENT, dtype=torch.int32, device="cuda"),
           "counts": torch.full((E,), SENT, dtype=torch.int32, device="cuda"),
           "row_assign": torch.full((max(mcap, 1),), SENT, dtype=torch.int32, device="cuda"),
           "assign_row": torch.full((max(tokens * topk, 1),), SENT, dtype=torch.int32, device="cuda"),
           "status": torch.full((1,), SENT, dtype=torch.int32, device="cuda")}
    args = [d, tokens, topk, E, pad, mcap, out["offs"], out["counts"], out["row_assign"], out["assign_row"],
            out["status"]]
    if with_ws:
        ws = torch.full((mx.route_plan_workspace_bytes(tokens, topk, E) // 4,), 12345, dtype=torch.int32,
                        device="cuda")
        args.append(ws)
    fn(*args)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.gpu
def test_noalloc_plan_matches_workspace_plan_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    mx.lib()
    cases = [
        # (seed, tokens, topk, E, pad, zero-token experts); the second input is smaller
        (6, 40000, 6, 64, 256, (7,)),
        (1, 833, 6, 16, 128, (3, 9)),
    ]
    for seed, tokens, topk, E, pad, zero in cases:
        ids = _ids(seed, tokens, topk, E, zero)
        counts = np.bincount(ids.ravel(), minlength=E)
        mcap = int(sum((c + pad - 1) // pad * pad for c in counts)) + pad
        print(f"noalloc plan: seed {seed} tokens {tokens} topk {topk} E {E} pad {pad} mcap {mcap}", flush=True)
        a = _plan(mx.mxf_route_plan_noalloc, ids, E, pad, mcap, with_ws=False)
        b = _plan(mx.mxf_route_plan, ids, E, pad, mcap, with_ws=True)
        assert int(a["status"][0]) == int(b["status"][0]) == mx.DEV_OK
        for k in ("offs", "counts", "row_assign", "assign_row"):
            assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a["counts"], counts)


def test_noalloc_limit_is_the_header_constant_and_is_checked_before_any_launch():
    text = open(os.path.join(ROOT, "include", "mxfp8.h")).read()
    m = re.search(r"#define MXF_ROUTE_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mx.ROUTE_NOALLOC_MAX_BYTES
    good = 1 << 20
    # E = 1024 with 2.4M assignments needs 2344 x 1025 x 4 bytes of histograms > 8 MiB
    assert mx.route_plan_workspace_bytes(300000, 8, 1024) > mx.ROUTE_NOALLOC_MAX_BYTES
    with pytest.raises(mx.MxfError) as ei:
        mx.mxf_route_plan_noalloc(good, 300000, 8, 1024, 128, 1 << 22, good, good, good, good, None, stream=0)
    assert ei.value.status == _abi.E_SHAPE and "allocation-free" in str(ei.value)
    # the same shape with E = 16 fits
    assert mx.route_plan_workspace_bytes(300000, 8, 16) <= mx.ROUTE_NOALLOC_MAX_BYTES
    with pytest.raises(mx.MxfError) as ei:
        mx.mxf_route_plan_noalloc(good, 8, 2, 0, 128, 256, good, good, good, good, None, stream=0)
    assert ei.value.status == _abi.E_SHAPE
