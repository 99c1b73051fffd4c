"""BF16 outputs of the plain-store GEMMs on 256 x 256 tiles (FC2, and FC1 dgrad in the
backward's merged launch) equal the round-to-nearest-even of the FP32 outputs bit for bit, on
shapes with several tiles per compute unit, tail sub-tiles first, four 64-k stages (K = 256),
zero-token experts and ragged counts, over two runs on one workspace."""
import pytest
import torch

import workloads
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # FC2 and FC1 dgrad: 94 row tiles x 8 column tiles (752 tiles, about three per block)
    dict(counts=[9000, 7000, 0, 8000], E=4, D=2048, F=512),
    # 36 x 8 = 288 tiles: 32 tail tiles split into quarter sub-tiles that run first
    dict(counts=[3000, 2500, 0, 3500], E=4, D=2048, F=384),
    # FC1 dgrad on four stages (K = 2F = 256); FC2 on two (K = 128)
    dict(counts=[8000, 13, 7900, 0, 6100], E=5, D=2048, F=128),
]


@pytest.mark.parametrize("case", CASES, ids=[f"E{c['E']}_D{c['D']}_F{c['F']}" for c in CASES])
def test_bf16_outputs_equal_rne_of_f32_medium_shapes(case):
    mx = require_gpu()
    pad = 256
    offs = workloads.padded_offsets(case["counts"], pad)
    prob = workloads.mlp_problem(None, seed=21, counts=case["counts"], E=case["E"], D=case["D"], F=case["F"],
                                 pad=pad, m_capacity=offs[-1] + pad)
    E, D, F, mcap = prob["E"], prob["D"], prob["F"], prob["m_capacity"]
    print(f"\nbf16 vs f32 case E={E} D={D} F={F} rows {offs[-1]}", flush=True)
    dev = "cuda"
    offs_t = torch.tensor(prob["offs"], dtype=torch.int32, device=dev)
    cnt_t = torch.tensor(prob["counts"], dtype=torch.int32, device=dev)
    x, w1, w3, w2, dy = (prob[k].to(dev) for k in ("x", "w1", "w3", "w2", "dy"))
    res = {}
    for flags, dt in ((mx.OUT_F32, torch.float32), (0, torch.bfloat16)):
        ctx = mx.MlpContext(E, D, F, pad, mcap, flags=flags)
        y = torch.empty((mcap, D), dtype=dt, device=dev)
        dx = torch.empty_like(y)
        dw1 = torch.empty((E, F, D), dtype=dt, device=dev)
        dw3 = torch.empty_like(dw1)
        dw2 = torch.empty((E, D, F), dtype=dt, device=dev)
        for _ in range(2):  # twice: the second run starts from the first run's workspace
            ctx.fwd(offs_t, cnt_t, x, w1, w3, w2, y)
            ctx.bwd(offs_t, cnt_t, dy, dx, dw1, dw3, dw2)
        torch.cuda.synchronize()
        assert ctx.status() == mx.DEV_OK
        res[flags] = (y, dx, dw1, dw3, dw2)
        del ctx
    m = prob["offs"][-1]
    for i, name in enumerate(("y", "dx", "dw1", "dw3", "dw2")):
        a, b = res[mx.OUT_F32][i], res[0][i]
        if name in ("y", "dx"):
            a, b = a[:m], b[:m]
        assert torch.equal(a.to(torch.bfloat16).view(torch.int16), b.view(torch.int16)), name
