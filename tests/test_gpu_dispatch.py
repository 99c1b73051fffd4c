"""GPU parity of the dispatch path against the oracle (oracle/dispatch.py): the routing plan
and the BF16 permute bit-exact, the fused dispatch + dual quantization bit-exact against the
oracle's quantization of the oracle's permuted matrix, and the MLP forward from the fused
dispatch equal to the forward from the permuted BF16 matrix."""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_util import bits, np_u8, require_gpu
from oracle import dispatch as od
from oracle import mlp as om
from oracle.formats import bf16_bits_to_f64
from oracle.mx import quantize_colwise, quantize_rowwise

pytestmark = pytest.mark.gpu
SENT = -7
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_plan_small.json")


def gpu_plan(mx, ids, E, pad, mcap):
    ids = np.asarray(ids, dtype=np.int32)
    ids = np.ascontiguousarray(ids if ids.ndim == 2 else ids.reshape(-1, 1))
    tokens, topk = ids.shape
    d = torch.from_numpy(ids).cuda()
    offs = torch.full((E + 1,), SENT, dtype=torch.int32, device="cuda")
    counts = torch.full((E,), SENT, dtype=torch.int32, device="cuda")
    ra = torch.full((max(mcap, 1),), SENT, dtype=torch.int32, device="cuda")
    ar = torch.full((max(tokens * topk, 1),), SENT, dtype=torch.int32, device="cuda")
    st = torch.full((1,), SENT, dtype=torch.int32, device="cuda")
    ws = torch.full((mx.route_plan_workspace_bytes(tokens, topk, E) // 4,), 12345, dtype=torch.int32, device="cuda")
    mx.mxf_route_plan(d, tokens, topk, E, pad, mcap, offs, counts, ra, ar, st, ws)
    torch.cuda.synchronize()
    return dict(offs=offs.cpu().numpy(), counts=counts.cpu().numpy(), row_assign=ra.cpu().numpy()[:mcap],
                assign_row=ar.cpu().numpy()[:tokens * topk], status=int(st.item()), dev=(offs, counts, ra))


def check_plan(g, r, mcap):
    assert g["status"] == r["status"]
    assert np.array_equal(g["offs"], r["offs"]) and np.array_equal(g["counts"], r["counts"])
    assert np.array_equal(g["assign_row"], r["assign_row"])
    m = len(r["row_assign"])
    assert np.array_equal(g["row_assign"][:m], r["row_assign"])
    assert np.all(g["row_assign"][m:] == SENT)        # rows past offs[E] are not written


def _random_ids(seed, tokens, topk, E, zero_experts=()):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.7))
    for e in zero_experts:
        p[e] = 0
    p /= p.sum()
    return rng.choice(E, size=(tokens, topk), p=p).astype(np.int32)


PLAN_CASES = [
    ("golden", None),
    ("tiny", None),
    ("dsv3_rank", None),
    ("rand_E16", dict(seed=1, tokens=833, topk=6, E=16, pad=256, zero=(3, 9))),
    ("E1_topk1", dict(seed=2, tokens=1000, topk=1, E=1, pad=128, zero=())),
    ("E64_pad128", dict(seed=3, tokens=4096, topk=8, E=64, pad=128, zero=(0, 63))),
    ("E1024", dict(seed=4, tokens=20000, topk=8, E=1024, pad=128, zero=(5,))),
    ("few_tokens", dict(seed=5, tokens=3, topk=2, E=8, pad=256, zero=())),
    ("many_blocks", dict(seed=6, tokens=40000, topk=6, E=64, pad=256, zero=(7,))),
    ("E1024_big", dict(seed=8, tokens=70000, topk=4, E=1024, pad=128, zero=(0, 1023))),
]


@pytest.mark.parametrize("name,case", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_route_plan_bit_exact(name, case):
    mx = require_gpu()
    if name == "golden":
        g = json.load(open(GOLDEN))
        ids, E, pad, mcap = np.array(g["expert_idx"]), g["E"], g["pad_multiple"], g["m_capacity"]
    elif case is None:
        _, ids = workloads.routed_tokens(name)
        cfg = workloads.MLP_CONFIGS[name]
        E, pad = cfg["E"], cfg["pad"]
        mcap = workloads.padded_offsets(workloads.expert_counts(name), pad)[-1] + pad
    else:
        ids = _random_ids(case["seed"], case["tokens"], case["topk"], case["E"], case["zero"])
        E, pad = case["E"], case["pad"]
        mcap = workloads.padded_offsets(np.bincount(ids.ravel(), minlength=E), pad)[-1] + 2 * pad
    print(f"\nroute plan case {name}: assignments {ids.size}, E {E}, pad {pad}, capacity {mcap}", flush=True)
    r = od.route_plan(ids, E, pad, mcap)
    g = gpu_plan(mx, ids, E, pad, mcap)
    check_plan(g, r, mcap)
    if case is None and name != "golden":
        assert g["counts"].tolist() == workloads.expert_counts(name)


def test_route_plan_empty_bad_ids_and_overflow():
    mx = require_gpu()
    # no assignments: all offsets zero, nothing else written
    g = gpu_plan(mx, np.zeros((0, 2), dtype=np.int32), 5, 128, 256)
    assert g["offs"].tolist() == [0] * 6 and g["counts"].tolist() == [0] * 5 and g["status"] == 0
    assert np.all(g["row_assign"] == SENT)
    # an out-of-range id is dropped and reported
    ids = np.array([[0, 5], [1, -1], [1, 0]], dtype=np.int32)
    r = od.route_plan(ids, 2, 128, 1024)
    g = gpu_plan(mx, ids, 2, 128, 1024)
    check_plan(g, r, 1024)
    assert g["status"] == mx.DEV_BAD_EXPERT
    # the padded layout exceeds the capacity: cut at the capacity, reported
    ids = np.array([0] * 130 + [1] * 5, dtype=np.int32)[:, None]
    r = od.route_plan(ids, 2, 128, 256)
    g = gpu_plan(mx, ids, 2, 128, 256)
    check_plan(g, r, 256)
    assert g["status"] == mx.DEV_OVERFLOW
    # capacity exactly the padded total
    ids = _random_ids(7, 500, 4, 8)
    cap = workloads.padded_offsets(np.bincount(ids.ravel(), minlength=8), 128)[-1]
    check_plan(gpu_plan(mx, ids, 8, 128, cap), od.route_plan(ids, 8, 128, cap), cap)


@pytest.mark.parametrize("D", [256, 200, 7168])
def test_permute_bit_exact(D):
    mx = require_gpu()
    if D == 256:
        tok, ids = workloads.routed_tokens("tiny")
        E, pad = 4, 128
    else:
        ids = _random_ids(11, 300, 3, 6, zero_experts=(2,))
        tok = workloads.randn_bf16((300, D), 1.0, workloads._gen(3, "cpu"), "cpu")
        E, pad = 6, 128
    topk = ids.shape[1]
    mcap = workloads.padded_offsets(np.bincount(ids.ravel(), minlength=E), pad)[-1] + pad
    print(f"\npermute case D={D}: tokens {tok.shape[0]}, topk {topk}, capacity {mcap}", flush=True)
    g = gpu_plan(mx, ids, E, pad, mcap)
    offs, _, ra = g["dev"]
    out = torch.full((mcap, D), 3.0, dtype=torch.bfloat16, device="cuda")
    mx.mxf_dispatch_permute(tok.cuda(), tok.shape[0], topk, D, E, offs, ra, mcap, out)
    torch.cuda.synchronize()
    r = od.route_plan(ids, E, pad, mcap)
    m = len(r["row_assign"])
    want = od.permute(bits(tok), r["row_assign"], topk, m)
    got = bits(out.cpu())
    assert np.array_equal(got[:m], want)
    assert np.all(got[m:] == bits(torch.tensor([3.0], dtype=torch.bfloat16))[0])   # tail untouched
    if D == 256:
        assert np.array_equal(got[:m], bits(workloads.mlp_problem("tiny")["x"]))


def _dispatch_quant(mx, name=None, case=None):
    if case is None:
        tok, ids = workloads.routed_tokens(name)
        cfg = workloads.MLP_CONFIGS[name]
        E, D, F, pad = cfg["E"], cfg["D"], cfg["F"], cfg["pad"]
    else:
        ids = _random_ids(case["seed"], case["tokens"], case["topk"], case["E"], case["zero"])
        E, D, F, pad = case["E"], case["D"], 128, case["pad"]
        tok = workloads.randn_bf16((case["tokens"], D), 1.0, workloads._gen(case["seed"], "cpu"), "cpu")
    topk = ids.shape[1]
    mcap = workloads.padded_offsets(np.bincount(ids.ravel(), minlength=E), pad)[-1] + pad
    g = gpu_plan(mx, ids, E, pad, mcap)
    offs, counts, ra = g["dev"]
    ctx = mx.MlpContext(E, D, F, pad, mcap)
    ctx.dispatch_quantize(offs, counts, ra, tok.cuda(), topk)
    torch.cuda.synchronize()
    assert ctx.status() == mx.DEV_OK
    out = {n: np_u8(ctx.view(n)) for n in ("XQ_R", "XS_R", "XQ_C", "XS_C")}
    r = od.route_plan(ids, E, pad, mcap)
    return tok, ids, r, out, (E, D, F, pad, mcap), g, ctx


DQ_CASES = [("tiny", None), ("rand_D512", dict(seed=21, tokens=700, topk=4, E=8, D=512, pad=256, zero=(1, 6))),
            ("rand_D384", dict(seed=22, tokens=96, topk=2, E=3, D=384, pad=128, zero=())),
            # E >= 64: the kernels' looping offsets check and binary-search expert lookup
            ("E64", dict(seed=23, tokens=1500, topk=4, E=64, D=256, pad=128, zero=(0, 17, 63))),
            ("E96_pad256", dict(seed=24, tokens=2000, topk=3, E=96, D=256, pad=256, zero=(5, 95)))]


@pytest.mark.parametrize("name,case", DQ_CASES, ids=[c[0] for c in DQ_CASES])
def test_dispatch_quantize_bit_exact(name, case):
    mx = require_gpu()
    print(f"\ndispatch quantize case {name}", flush=True)
    tok, ids, r, out, (E, D, F, pad, mcap), _, _ = _dispatch_quant(mx, name, case)
    m = len(r["row_assign"])
    xv = bf16_bits_to_f64(od.permute(bits(tok), r["row_assign"], ids.shape[1], m))
    rq, rs = quantize_rowwise(xv)
    assert np.array_equal(out["XQ_R"][:m], rq) and np.array_equal(out["XS_R"][:m], rs)
    cq, cs = quantize_colwise(xv)
    assert np.array_equal(out["XQ_C"][:, :m], cq) and np.array_equal(out["XS_C"][:, :m // 32], cs)


def test_mlp_from_fused_dispatch_equals_mlp_from_permuted_matrix():
    """dispatch_quantize + grouped_mlp_fwd(MXF_X_QUANTIZED) gives the same output and saved
    tensors as mxf_dispatch_permute + grouped_mlp_fwd, bit for bit, and the backward agrees."""
    mx = require_gpu()
    tok, ids, r, _, (E, D, F, pad, mcap), g, ctx_a = _dispatch_quant(mx, "tiny")
    offs, counts, ra = g["dev"]
    prob = workloads.mlp_problem("tiny", m_capacity=mcap)
    w1, w3, w2, dy = (prob[k].cuda() for k in ("w1", "w3", "w2", "dy"))
    ya = torch.empty((mcap, D), dtype=torch.bfloat16, device="cuda")
    ctx_a.fwd(offs, counts, None, w1, w3, w2, ya)
    xp = torch.zeros((mcap, D), dtype=torch.bfloat16, device="cuda")
    mx.mxf_dispatch_permute(tok.cuda(), tok.shape[0], ids.shape[1], D, E, offs, ra, mcap, xp)
    ctx_b = mx.MlpContext(E, D, F, pad, mcap)
    yb = torch.empty_like(ya)
    ctx_b.fwd(offs, counts, xp, w1, w3, w2, yb)
    grads = []
    for ctx in (ctx_a, ctx_b):
        dx = torch.empty_like(ya)
        dw1, dw3 = torch.empty_like(w1), torch.empty_like(w3)
        dw2 = torch.empty_like(w2)
        ctx.bwd(offs, counts, dy, dx, dw1, dw3, dw2)
        grads.append((dx, dw1, dw3, dw2))
    torch.cuda.synchronize()
    assert ctx_a.status() == mx.DEV_OK and ctx_b.status() == mx.DEV_OK
    m = len(r["row_assign"])
    assert torch.equal(ya[:m], yb[:m])
    # saved tensors over the layout's rows (columns of the transposed ones); the tail is not written
    assert torch.equal(ctx_a.view("H13")[:m], ctx_b.view("H13")[:m])
    for n in ("XQ_C", "HQ_C"):
        assert torch.equal(ctx_a.view(n)[:, :m], ctx_b.view(n)[:, :m]), n
    for n in ("XS_C", "HS_C"):
        assert torch.equal(ctx_a.view(n)[:, :m // 32], ctx_b.view(n)[:, :m // 32]), n
    (dxa, *wa), (dxb, *wb) = grads
    assert torch.equal(dxa[:m], dxb[:m])
    for a, b in zip(wa, wb):
        assert torch.equal(a, b)
