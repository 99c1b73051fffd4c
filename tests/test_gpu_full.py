"""GPU parity at the full workload sizes, on sampled outputs the oracle computes one by one.

Runs grouped_mlp_fwd + grouped_mlp_bwd (the kernels bench.py times) on the DSv3-16B
expert-parallel rank, the dense FFN and the large-expert rank, then checks, per expert,
sampled rows / columns / 32-groups of every stage against the oracle fed the same
upstream operands: quantizer codes bit-exact, every GEMM within 1e-4 normwise (and the
elementwise |A||B|^T bound), fused-epilogue codes within one E4M3 step on <= 0.1%.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bits, check_fused_codes, check_gemm, np_u8, require_gpu
from oracle import mlp as om
from oracle.formats import bf16_bits_to_f64, f64_to_bf16_bits
from oracle.mx import dequantize_rowwise as deq
from oracle.mx import quantize_colwise, quantize_rowwise

pytestmark = pytest.mark.gpu


def sample_rows(rng, a, n_real, k):
    """k sorted distinct rows among the expert's real rows [a, a + n_real)."""
    k = min(k, n_real)
    return a + np.sort(rng.choice(n_real, size=k, replace=False))


def sample_group(rng, a, n_real):
    """Start of one aligned 32-row group that holds real rows."""
    return a + 32 * int(rng.integers(0, (n_real + 31) // 32))


@pytest.mark.parametrize("name", ["dsv3_rank", "dense", "large_expert"])
def test_full_size_sampled_parity(name):
    mx = require_gpu()
    print(f"\n[{name}] generating inputs", flush=True)
    prob = workloads.mlp_problem(name, seed=42)
    E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
    offs, counts = prob["offs"], prob["counts"]
    dev = "cuda"
    ctx = mx.MlpContext(E, D, F, pad, mcap, flags=mx.OUT_F32 | mx.DEBUG_F32)
    offs_t = torch.tensor(offs, dtype=torch.int32, device=dev)
    cnt_t = torch.tensor(counts, dtype=torch.int32, device=dev)
    x, w1, w3, w2, dy = (prob[k].to(dev) for k in ("x", "w1", "w3", "w2", "dy"))
    y = torch.empty((mcap, D), dtype=torch.float32, device=dev)
    dx = torch.empty_like(y)
    dw1 = torch.empty((E, F, D), dtype=torch.float32, device=dev)
    dw3 = torch.empty_like(dw1)
    dw2 = torch.empty((E, D, F), dtype=torch.float32, device=dev)
    print(f"[{name}] forward", flush=True)
    ctx.fwd(offs_t, cnt_t, x, w1, w3, w2, y)
    torch.cuda.synchronize()
    assert ctx.status() == 0
    # forward-only workspace tensors are reused by backward: take the samples' operands now
    V = {n: ctx.view(n) for n in ("XQ_R", "XS_R", "W13Q_R", "W13S_R", "W2Q_R", "W2S_R", "HQ_R", "HS_R", "H13_F32")}
    rng = np.random.default_rng(7)
    segs = om.segments(offs)
    xb, dyb = bits(prob["x"]), bits(prob["dy"])
    w13b = om.pack_w13(bits(prob["w1"]), bits(prob["w3"]))
    w2b = bits(prob["w2"])
    fwd_samples = {}
    worst = {}

    def note(stage, res):
        nw, ratio = res
        w = worst.get(stage, (0.0, 0.0))
        worst[stage] = (max(w[0], nw), max(w[1], ratio))

    for e, (a, b) in enumerate(segs):
        # weights: sampled rows of both quantized directions, bit-exact
        wr = rng.choice(2 * F, size=8, replace=False)
        q, s = quantize_rowwise(bf16_bits_to_f64(w13b[e][wr]))
        assert np.array_equal(np_u8(V["W13Q_R"][e][wr]), q) and np.array_equal(np_u8(V["W13S_R"][e][wr]), s)
        wr = rng.choice(D, size=8, replace=False)
        q, s = quantize_rowwise(bf16_bits_to_f64(w2b[e][wr]))
        assert np.array_equal(np_u8(V["W2Q_R"][e][wr]), q) and np.array_equal(np_u8(V["W2S_R"][e][wr]), s)
        if counts[e] == 0:
            continue
        rows = sample_rows(rng, a, counts[e], 24)
        xq = np_u8(V["XQ_R"][rows]); xs = np_u8(V["XS_R"][rows])
        q, s = quantize_rowwise(bf16_bits_to_f64(xb[rows]))
        assert np.array_equal(xq, q) and np.array_equal(xs, s)
        B13 = deq(np_u8(V["W13Q_R"][e]), np_u8(V["W13S_R"][e]))
        note("fc1", check_gemm(V["H13_F32"][rows].double().cpu().numpy(), deq(xq, xs), B13, label=("fc1", e)))
        # FC1 epilogue on a full aligned 32-row group (both directions need all 32 rows)
        g0 = sample_group(rng, a, counts[e])
        h13g = bits(ctx.view("H13")[g0:g0 + 32].cpu())
        _, hq_r, hs_r, hq_c, hs_c = om.swiglu_quant_from_h13(h13g)
        check_fused_codes(np_u8(V["HQ_R"][g0:g0 + 32]), np_u8(V["HS_R"][g0:g0 + 32]), hq_r, hs_r, label="hq_r")
        check_fused_codes(np_u8(ctx.view("HQ_C")[:, g0:g0 + 32]), np_u8(ctx.view("HS_C")[:, g0 // 32:g0 // 32 + 1]),
                          hq_c, hs_c, label="hq_c")
        hq = np_u8(V["HQ_R"][rows]); hs = np_u8(V["HS_R"][rows])
        B2 = deq(np_u8(V["W2Q_R"][e]), np_u8(V["W2S_R"][e]))
        note("fc2", check_gemm(y[rows].double().cpu().numpy(), deq(hq, hs), B2, label=("fc2", e)))
        fwd_samples[e] = rows
    # pad rows of y are zero
    mask = om.real_rows_mask(offs, counts, offs[-1])
    pad_rows = np.nonzero(~mask)[0]
    if len(pad_rows):
        assert torch.all(y[torch.from_numpy(pad_rows).to(dev)] == 0)
    del V

    print(f"[{name}] backward", flush=True)
    ctx.bwd(offs_t, cnt_t, dy, dx, dw1, dw3, dw2)
    torch.cuda.synchronize()
    assert ctx.status() == 0
    W = {n: ctx.view(n) for n in ("DYQ_R", "DYS_R", "DYQ_C", "DYS_C", "DHQ_R", "DHS_R", "DHQ_C", "DHS_C",
                                  "DH_F32", "W2Q_C", "W2S_C", "W13Q_C", "W13S_C", "HQ_C", "HS_C", "XQ_C",
                                  "XS_C", "H13")}
    for e, (a, b) in enumerate(segs):
        if counts[e] == 0:
            assert torch.all(dw1[e] == 0) and torch.all(dw3[e] == 0) and torch.all(dw2[e] == 0)
            continue
        rows = fwd_samples[e]
        dq = np_u8(W["DYQ_R"][rows]); ds = np_u8(W["DYS_R"][rows])
        q, s = quantize_rowwise(bf16_bits_to_f64(dyb[rows]))
        assert np.array_equal(dq, q) and np.array_equal(ds, s)
        B = deq(np_u8(W["W2Q_C"][e]), np_u8(W["W2S_C"][e]))
        note("dgrad2", check_gemm(W["DH_F32"][rows].double().cpu().numpy(), deq(dq, ds), B, label=("dgrad2", e)))
        g0 = sample_group(rng, a, counts[e])
        dh = W["DH_F32"][g0:g0 + 32].double().cpu().numpy()
        _, q_r, s_r, q_c, s_c = om.dswiglu_quant(dh, bits(W["H13"][g0:g0 + 32].cpu()))
        check_fused_codes(np_u8(W["DHQ_R"][g0:g0 + 32]), np_u8(W["DHS_R"][g0:g0 + 32]), q_r, s_r, label="dhq_r")
        check_fused_codes(np_u8(W["DHQ_C"][:, g0:g0 + 32]), np_u8(W["DHS_C"][:, g0 // 32:g0 // 32 + 1]), q_c, s_c,
                          label="dhq_c")
        # column-wise token quantization of dY: sampled columns over the expert's segment
        cols = rng.choice(D, size=4, replace=False)
        q, s = quantize_colwise(bf16_bits_to_f64(dyb[a:b][:, cols]) * mask[a:b][:, None])
        assert np.array_equal(np_u8(W["DYQ_C"][cols][:, a:b]), q) and np.array_equal(np_u8(W["DYS_C"][cols][:, a // 32:b // 32]), s)
        # FC1 dgrad rows
        dhq = np_u8(W["DHQ_R"][rows]); dhs = np_u8(W["DHS_R"][rows])
        B = deq(np_u8(W["W13Q_C"][e]), np_u8(W["W13S_C"][e]))
        note("dgrad1", check_gemm(dx[rows].double().cpu().numpy(), deq(dhq, dhs), B, label=("dgrad1", e)))
        # wgrads: sampled output rows, contraction over the expert's segment
        sa, sb = a // 32, b // 32
        dr = np.sort(rng.choice(D, size=8, replace=False))
        A = deq(np_u8(W["DYQ_C"][dr][:, a:b]), np_u8(W["DYS_C"][dr][:, sa:sb]))
        B = deq(np_u8(W["HQ_C"][:, a:b]), np_u8(W["HS_C"][:, sa:sb]))
        note("wgrad2", check_gemm(dw2[e][dr].double().cpu().numpy(), A, B, label=("wgrad2", e)))
        nr = np.sort(rng.choice(2 * F, size=8, replace=False))
        A = deq(np_u8(W["DHQ_C"][nr][:, a:b]), np_u8(W["DHS_C"][nr][:, sa:sb]))
        B = deq(np_u8(W["XQ_C"][:, a:b]), np_u8(W["XS_C"][:, sa:sb]))
        frows = (nr // 64) * 32 + nr % 32
        got = np.where(((nr % 64) < 32)[:, None], dw1[e][frows].double().cpu().numpy(),
                       dw3[e][frows].double().cpu().numpy())
        note("wgrad1", check_gemm(got, A, B, label=("wgrad1", e)))
    for stage, (nw, ratio) in worst.items():
        print(f"[{name}] {stage}: worst normwise {nw:.2e}, worst |err|/(|A||B|^T) {ratio:.2e}")


def test_full_size_bf16_outputs_match_f32():
    """The benchmark's launch configuration (BF16 outputs) equals RNE of the FP32 outputs."""
    mx = require_gpu()
    prob = workloads.mlp_problem("dsv3_rank", seed=11)
    E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
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
        ctx.fwd(offs_t, cnt_t, x, w1, w3, w2, y)
        ctx.bwd(offs_t, cnt_t, dy, dx, dw1, dw3, dw2)
        torch.cuda.synchronize()
        res[flags] = (y, dx, dw1, dw3, dw2)
        del ctx
    m = prob["offs"][-1]
    for i, name in enumerate(("y", "dx", "dw1", "dw3", "dw2")):
        a, b = res[mx.OUT_F32][i], res[0][i]
        if name in ("y", "dx"):
            a, b = a[:m], b[:m]
        assert torch.equal(a.to(torch.bfloat16).view(torch.int16), b.view(torch.int16)), name
