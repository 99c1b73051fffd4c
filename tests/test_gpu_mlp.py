"""GPU parity of grouped_mlp_fwd / grouped_mlp_bwd against the oracle, stage by stage.

* Quantizer outputs inside the MLP (X, dY, W13, W2 in both directions): bit-exact.
* Every GEMM (FP32 outputs): normwise relative error <= 1e-4 against fp64 accumulation of
  the same dequantised operands (the GPU's own codes and scales, fed to the oracle).
* Saved BF16 FC1 output: exactly RNE of the FP32 result; within one BF16 step of RNE(fp64)
  wherever the sum does not nearly cancel.
* Fused-epilogue codes (h and dH13, both directions): the oracle run on the same upstream
  operands (the saved BF16 FC1 output; the FP32 dgrad accumulator); each code within one
  E4M3 step, <= 0.1% of codes differing.
* The pages' test designs: zero-token experts get exact-zero weight gradients, zero routed
  tokens work, NaN-poisoned pad and tail rows leave outputs unchanged, BF16 outputs equal
  RNE of the FP32 outputs, runs are deterministic, invalid offsets are reported.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import bf16_ulp_distance, bits, check_fused_codes, check_gemm, normwise, np_u8, require_gpu
from oracle import mlp as om
from oracle.formats import bf16_bits_to_f64, f64_to_bf16_bits
from oracle.mx import dequantize_rowwise as deq
from oracle.mx import quantize_colwise, quantize_rowwise

pytestmark = pytest.mark.gpu

GEMM_TOL = 1e-4
FWD_VIEWS = ["XQ_R", "XS_R", "XQ_C", "XS_C", "W13Q_R", "W13S_R", "W13Q_C", "W13S_C", "W2Q_R", "W2S_R",
             "W2Q_C", "W2S_C", "H13", "HQ_R", "HS_R", "HQ_C", "HS_C", "H13_F32"]
BWD_VIEWS = ["DYQ_R", "DYS_R", "DYQ_C", "DYS_C", "DHQ_R", "DHS_R", "DHQ_C", "DHS_C", "DH_F32"]
SENTINEL = 7.0


def run_mlp(mx, prob, flags, counts=True):
    E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
    ctx = mx.MlpContext(E, D, F, pad, mcap, flags=flags)
    dev = "cuda"
    offs = torch.tensor(prob["offs"], dtype=torch.int32, device=dev)
    cnt = torch.tensor(prob["counts"], dtype=torch.int32, device=dev) if counts else None
    x, w1, w3, w2, dy = (prob[k].to(dev) for k in ("x", "w1", "w3", "w2", "dy"))
    odt = torch.float32 if flags & mx.OUT_F32 else torch.bfloat16
    y = torch.full((mcap, D), SENTINEL, dtype=odt, device=dev)
    dx = torch.full((mcap, D), SENTINEL, dtype=odt, device=dev)
    dw1 = torch.full((E, F, D), SENTINEL, dtype=odt, device=dev)
    dw3 = torch.full((E, F, D), SENTINEL, dtype=odt, device=dev)
    dw2 = torch.full((E, D, F), SENTINEL, dtype=odt, device=dev)
    ctx.fwd(offs, cnt, x, w1, w3, w2, y)
    torch.cuda.synchronize()
    out = {"status_fwd": ctx.status()}
    if flags & mx.DEBUG_F32:
        for n in FWD_VIEWS:
            out[n] = ctx.view(n).cpu()
    ctx.bwd(offs, cnt, dy, dx, dw1, dw3, dw2)
    torch.cuda.synchronize()
    out["status_bwd"] = ctx.status()
    if flags & mx.DEBUG_F32:
        for n in BWD_VIEWS:
            out[n] = ctx.view(n).cpu()
    for k, t in (("y", y), ("dx", dx), ("dw1", dw1), ("dw3", dw3), ("dw2", dw2)):
        out[k] = t.cpu()
    return out


def u(t):
    return np_u8(t)


def f64(t):
    return t.double().numpy()


def check_stagewise(prob, r, weight_experts=None):
    """Every stage of one fwd+bwd run (flags OUT_F32 | DEBUG_F32) against the oracle.
    weight_experts: the experts whose weight quantization is compared (default: all)."""
    E, D, F = prob["E"], prob["D"], prob["F"]
    offs, counts = prob["offs"], prob["counts"]
    m = offs[-1]
    segs = om.segments(offs)
    assert r["status_fwd"] == 0 and r["status_bwd"] == 0
    mask = om.real_rows_mask(offs, counts, m)

    # --- quantizer stages: bit-exact
    xv = bf16_bits_to_f64(bits(prob["x"]))[:m].copy()
    xv[~mask] = 0.0
    rq, rs = quantize_rowwise(xv)
    assert np.array_equal(u(r["XQ_R"])[:m], rq) and np.array_equal(u(r["XS_R"])[:m], rs)
    cq, cs = quantize_colwise(xv)
    assert np.array_equal(u(r["XQ_C"])[:, :m], cq) and np.array_equal(u(r["XS_C"])[:, :m // 32], cs)
    w13 = bf16_bits_to_f64(om.pack_w13(bits(prob["w1"]), bits(prob["w3"])))
    w2 = bf16_bits_to_f64(bits(prob["w2"]))
    for e in (range(E) if weight_experts is None else weight_experts):
        q, s = quantize_rowwise(w13[e])
        assert np.array_equal(u(r["W13Q_R"])[e], q) and np.array_equal(u(r["W13S_R"])[e], s)
        q, s = quantize_colwise(w13[e])
        assert np.array_equal(u(r["W13Q_C"])[e], q) and np.array_equal(u(r["W13S_C"])[e], s)
        q, s = quantize_rowwise(w2[e])
        assert np.array_equal(u(r["W2Q_R"])[e], q) and np.array_equal(u(r["W2S_R"])[e], s)
        q, s = quantize_colwise(w2[e])
        assert np.array_equal(u(r["W2Q_C"])[e], q) and np.array_equal(u(r["W2S_C"])[e], s)
    dyv = bf16_bits_to_f64(bits(prob["dy"]))[:m].copy()
    dyv[~mask] = 0.0
    rq, rs = quantize_rowwise(dyv)
    assert np.array_equal(u(r["DYQ_R"])[:m], rq) and np.array_equal(u(r["DYS_R"])[:m], rs)
    cq, cs = quantize_colwise(dyv)
    assert np.array_equal(u(r["DYQ_C"])[:, :m], cq) and np.array_equal(u(r["DYS_C"])[:, :m // 32], cs)

    # --- FC1 GEMM (fp32 debug copy) and the saved BF16 h13
    h13_f32 = f64(r["H13_F32"])[:m]
    stats = {}
    for e, (a, b) in enumerate(segs):
        if b > a:
            stats[("fc1", e)] = check_gemm(h13_f32[a:b], deq(u(r["XQ_R"])[a:b], u(r["XS_R"])[a:b]),
                                           deq(u(r["W13Q_R"])[e], u(r["W13S_R"])[e]), label=("fc1", e))
    ref_h13 = np.zeros((m, 2 * F))
    abs_h13 = np.zeros((m, 2 * F))
    for e, (a, b) in enumerate(segs):
        if b > a:
            A = deq(u(r["XQ_R"])[a:b], u(r["XS_R"])[a:b])
            B = deq(u(r["W13Q_R"])[e], u(r["W13S_R"])[e])
            ref_h13[a:b] = A @ B.T
            abs_h13[a:b] = np.abs(A) @ np.abs(B).T
    h13_bits = bits(r["H13"])[:m]
    assert np.array_equal(h13_bits, f64_to_bf16_bits(h13_f32))
    # The FP8 matrix core accumulates with less than fp32 precision, so ~1% of the BF16 outputs
    # sit one step from RNE(fp64). Wherever the sum does not nearly cancel (|ref| >= |A||B|^T / 8)
    # the GEMM's elementwise bound 2^-12 |A||B|^T is below half a BF16 step of ref, so the saved
    # value is within one BF16 step of RNE(fp64) there; elsewhere it is within that bound plus
    # half a step of the rounded value.
    dist = bf16_ulp_distance(h13_bits, f64_to_bf16_bits(ref_h13))
    solid = np.abs(ref_h13) >= abs_h13 / 8
    print(f"\nh13 bf16 equal to RNE(fp64): {np.mean(dist == 0):.5f}; "
          f"worst step distance where not cancelling: {int(dist[solid].max()) if solid.any() else 0}")
    assert np.all(dist[solid] <= 1)
    h13_v = bf16_bits_to_f64(h13_bits)
    half_step = np.ldexp(1.0, np.frexp(np.abs(h13_v))[1] - 9)
    assert np.all(np.abs(h13_v - ref_h13) <= 2.0 ** -12 * abs_h13 + half_step)
    assert (dist == 0).mean() >= 0.97

    # --- FC1 epilogue: SwiGLU + dual quantization of h, from the GPU's own h13
    _, hq_r, hs_r, hq_c, hs_c = om.swiglu_quant_from_h13(h13_bits)
    f1 = check_fused_codes(u(r["HQ_R"])[:m], u(r["HS_R"])[:m], hq_r, hs_r, label="hq_r")
    f2 = check_fused_codes(u(r["HQ_C"])[:, :m], u(r["HS_C"])[:, :m // 32], hq_c, hs_c, label="hq_c")
    print(f"SwiGLU codes differing: row {f1:.2e} col {f2:.2e}")

    # --- FC2 GEMM
    y = f64(r["y"])
    ref_y = np.zeros((m, D))
    for e, (a, b) in enumerate(segs):
        if b > a:
            A = deq(u(r["HQ_R"])[a:b], u(r["HS_R"])[a:b])
            B = deq(u(r["W2Q_R"])[e], u(r["W2S_R"])[e])
            stats[("fc2", e)] = check_gemm(y[a:b], A, B, label=("fc2", e))
            ref_y[a:b] = A @ B.T
    assert np.all(y[:m][~mask] == 0)
    assert np.all(y[m:] == SENTINEL)

    # --- FC2 dgrad (fp32 debug copy) and the fused dSwiGLU + dual quantization
    dh_gpu = f64(r["DH_F32"])[:m]
    for e, (a, b) in enumerate(segs):
        if b > a:
            stats[("dgrad2", e)] = check_gemm(dh_gpu[a:b], deq(u(r["DYQ_R"])[a:b], u(r["DYS_R"])[a:b]),
                                              deq(u(r["W2Q_C"])[e], u(r["W2S_C"])[e]), label=("dgrad2", e))
    # the epilogue's upstream operand is the fp32 accumulator (gated just above)
    _, dq_r, ds_r, dq_c, ds_c = om.dswiglu_quant(dh_gpu, h13_bits)
    f1 = check_fused_codes(u(r["DHQ_R"])[:m], u(r["DHS_R"])[:m], dq_r, ds_r, label="dhq_r")
    f2 = check_fused_codes(u(r["DHQ_C"])[:, :m], u(r["DHS_C"])[:, :m // 32], dq_c, ds_c, label="dhq_c")
    print(f"dSwiGLU codes differing: row {f1:.2e} col {f2:.2e}")

    # --- wgrads and FC1 dgrad from the GPU's own codes
    dw2, dw1, dw3, dx = f64(r["dw2"]), f64(r["dw1"]), f64(r["dw3"]), f64(r["dx"])
    for e, (a, b) in enumerate(segs):
        if b == a:
            assert np.all(dw2[e] == 0) and np.all(dw1[e] == 0) and np.all(dw3[e] == 0)
            continue
        sa, sb = a // 32, b // 32
        stats[("wgrad2", e)] = check_gemm(dw2[e], deq(u(r["DYQ_C"])[:, a:b], u(r["DYS_C"])[:, sa:sb]),
                                          deq(u(r["HQ_C"])[:, a:b], u(r["HS_C"])[:, sa:sb]), label=("wgrad2", e))
        got13 = om.pack_w13(dw1[e][None], dw3[e][None])[0]
        stats[("wgrad1", e)] = check_gemm(got13, deq(u(r["DHQ_C"])[:, a:b], u(r["DHS_C"])[:, sa:sb]),
                                          deq(u(r["XQ_C"])[:, a:b], u(r["XS_C"])[:, sa:sb]), label=("wgrad1", e))
        stats[("dgrad1", e)] = check_gemm(dx[a:b], deq(u(r["DHQ_R"])[a:b], u(r["DHS_R"])[a:b]),
                                          deq(u(r["W13Q_C"])[e], u(r["W13S_C"])[e]), label=("dgrad1", e))
    assert np.all(dx[:m][~mask] == 0) and np.all(dx[m:] == SENTINEL)
    for stage in ("fc1", "fc2", "dgrad2", "wgrad2", "wgrad1", "dgrad1"):
        v = [s for k, s in stats.items() if k[0] == stage]
        print(f"{stage}: worst normwise {max(x[0] for x in v):.2e}, worst |err|/(|A||B|^T) {max(x[1] for x in v):.2e}")
    return ref_y


@pytest.fixture(scope="module")
def tiny():
    mx = require_gpu()
    prob = workloads.mlp_problem("tiny", m_capacity=1536)
    r = run_mlp(mx, prob, mx.OUT_F32 | mx.DEBUG_F32)
    return mx, prob, r


def test_tiny_stagewise_parity(tiny):
    mx, prob, r = tiny
    check_stagewise(prob, r)


def test_tiny_end_to_end_against_oracle_chain(tiny):
    mx, prob, r = tiny
    x, w1, w3, w2, dy = (bf16_bits_to_f64(bits(prob[k])) for k in ("x", "w1", "w3", "w2", "dy"))
    fwd = om.mlp_forward(x, w1, w3, w2, prob["offs"], prob["counts"])
    bwd = om.mlp_backward(fwd, dy)
    m = prob["offs"][-1]
    assert normwise(r["y"].double().numpy()[:m], fwd["y"]) <= 2e-3
    for k in ("dx", "dw1", "dw3", "dw2"):
        got = r[k].double().numpy()
        got = got[:m] if k == "dx" else got
        assert normwise(got, bwd[k]) <= 5e-3, k


def test_bf16_outputs_are_rne_of_f32_outputs(tiny):
    mx, prob, r32 = tiny
    rb = run_mlp(mx, prob, 0)
    for k in ("y", "dx", "dw1", "dw3", "dw2"):
        want = f64_to_bf16_bits(r32[k].double().numpy())
        got = bits(rb[k])
        if k in ("y", "dx"):
            m = prob["offs"][-1]
            want, got = want[:m], got[:m]
        assert np.array_equal(got, want), k


def test_deterministic(tiny):
    mx, prob, r = tiny
    r2 = run_mlp(mx, prob, mx.OUT_F32 | mx.DEBUG_F32)
    m = prob["offs"][-1]
    for k in ("y", "dx", "dw1", "dw3", "dw2"):
        assert torch.equal(r[k], r2[k]), k
    # workspace/saved tensors: only rows before offs[E] are written
    for k in ("HQ_R", "DHQ_R", "H13", "XQ_R"):
        assert torch.equal(r[k][:m].view(torch.uint8), r2[k][:m].view(torch.uint8)), k
    for k in ("HQ_C", "DHQ_C", "XQ_C", "HS_C", "DHS_C"):
        w = m if k.endswith("Q_C") else m // 32
        assert torch.equal(r[k][:, :w], r2[k][:, :w]), k


# A shape on 256-row tiles (pad 256, D and 2F multiples of 256): the backward's FC1 wgrad,
# FC2 wgrad and FC1 dgrad share one launch there.
MERGED_BWD = dict(counts=[0, 200, 0, 57], E=4, D=256, F=384, pad=256)


def _merged_problem(case, seed=5):
    return workloads.mlp_problem(None, seed=seed, counts=case["counts"], E=case["E"], D=case["D"], F=case["F"],
                                 pad=case["pad"],
                                 m_capacity=workloads.padded_offsets(case["counts"], case["pad"])[-1] + case["pad"])


@pytest.mark.parametrize("case", [
    MERGED_BWD,                                                       # FC2 wgrad on 256 x 128
    dict(counts=[2300, 2250], E=2, D=256, F=2048, pad=256),          # 256 x 256; FC1 dgrad tail tiles
    dict(counts=[512], E=1, D=512, F=640, pad=256),                  # dense (E = 1)
])
def test_merged_backward_gemms_match_separate_launches(case):
    """On 256-row tiles the serial backward runs FC1 wgrad, FC2 wgrad and FC1 dgrad in one
    launch; MXF_CONCURRENT launches them separately on helper streams. Outputs and weight
    gradients are bit-identical (each output element is the same reduction in the same order
    either way)."""
    mx = require_gpu()
    print(f"\nmerged backward case E={case['E']} D={case['D']} F={case['F']} pad={case['pad']}", flush=True)
    prob = _merged_problem(case, seed=21)
    r1 = run_mlp(mx, prob, mx.OUT_F32)
    r2 = run_mlp(mx, prob, mx.OUT_F32 | mx.CONCURRENT)
    m = prob["offs"][-1]
    for k in ("dw1", "dw3", "dw2"):
        assert torch.equal(r1[k], r2[k]), k
    for k in ("y", "dx"):
        assert torch.equal(r1[k][:m], r2[k][:m]), k


def test_serial_launches_match_concurrent(tiny):
    """The default serial launches and MXF_CONCURRENT's helper-stream fork/join give
    bit-identical outputs and saved tensors."""
    mx, prob, r = tiny
    r2 = run_mlp(mx, prob, mx.OUT_F32 | mx.DEBUG_F32 | mx.CONCURRENT)
    m = prob["offs"][-1]
    for k in ("y", "dx", "dw1", "dw3", "dw2"):
        assert torch.equal(r[k], r2[k]), k
    for k in ("HQ_R", "DHQ_R"):  # rows at or past offs[E] are never written
        assert torch.equal(r[k][:m], r2[k][:m]), k
    for k in ("W2Q_R", "W2S_R", "W2Q_C"):
        assert torch.equal(r[k], r2[k]), k


@pytest.mark.parametrize("case", [
    None,                                                             # tiny, pad 128
    dict(counts=[0, 200, 0, 57], E=4, D=256, F=384, pad=256),        # zero-token experts, pad 256
    dict(counts=[300, 77, 515], E=3, D=384, F=256, pad=128),         # ragged
])
def test_unfused_plan_matches_fused(case):
    """The unfused plan (plain GEMMs writing BF16, standalone SwiGLU / dSwiGLU + dual
    quantization kernels) computes the same rounding points as the fused epilogues: outputs
    and every saved or intermediate tensor are bit-identical."""
    mx = require_gpu()
    if case is None:
        prob = workloads.mlp_problem("tiny", m_capacity=1536)
    else:
        prob = workloads.mlp_problem(None, seed=5, counts=case["counts"], E=case["E"], D=case["D"], F=case["F"],
                                     pad=case["pad"], m_capacity=workloads.padded_offsets(case["counts"], case["pad"])[-1])
    ra = run_mlp(mx, prob, mx.OUT_F32)
    rb = run_mlp(mx, prob, mx.OUT_F32 | mx.UNFUSED)
    m = prob["offs"][-1]
    for k in ("dw1", "dw3", "dw2"):
        assert torch.equal(ra[k], rb[k]), k
    for k in ("y", "dx"):
        assert torch.equal(ra[k][:m], rb[k][:m]), k


def test_unfused_plan_intermediates_match_fused():
    """Saved h13 and the dual-quantized h and dH13 (codes and scales) of both plans agree."""
    mx = require_gpu()
    prob = workloads.mlp_problem("tiny", m_capacity=1536)
    out = {}
    for plan, flags in (("fused", 0), ("unfused", mx.UNFUSED)):
        E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
        ctx = mx.MlpContext(E, D, F, pad, mcap, flags=flags)
        offs = torch.tensor(prob["offs"], dtype=torch.int32, device="cuda")
        cnt = torch.tensor(prob["counts"], dtype=torch.int32, device="cuda")
        x, w1, w3, w2, dy = (prob[k].cuda() for k in ("x", "w1", "w3", "w2", "dy"))
        y = torch.empty((mcap, D), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty_like(y)
        dw1 = torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda")
        dw3, dw2 = torch.empty_like(dw1), torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")
        ctx.fwd(offs, cnt, x, w1, w3, w2, y)
        ctx.bwd(offs, cnt, dy, dx, dw1, dw3, dw2)
        torch.cuda.synchronize()
        out[plan] = {n: ctx.view(n).cpu() for n in ("H13", "HQ_R", "HS_R", "HQ_C", "HS_C", "DHQ_R", "DHS_R",
                                                     "DHQ_C", "DHS_C")}
    m = prob["offs"][-1]
    a, b = out["fused"], out["unfused"]
    for n in ("H13", "HQ_R", "HS_R", "DHQ_R", "DHS_R"):
        assert torch.equal(a[n][:m].view(torch.uint8), b[n][:m].view(torch.uint8)), n
    for n in ("HQ_C", "DHQ_C"):
        assert torch.equal(a[n][:, :m], b[n][:, :m]), n
    for n in ("HS_C", "DHS_C"):
        assert torch.equal(a[n][:, :m // 32], b[n][:, :m // 32]), n


def test_nan_poisoned_pad_and_tail(tiny):
    mx, prob, r = tiny
    poisoned = workloads.mlp_problem("tiny", m_capacity=1536, pad_fill=float("nan"), tail_fill=float("nan"))
    rp = run_mlp(mx, poisoned, mx.OUT_F32)
    m = prob["offs"][-1]
    for k in ("dw1", "dw3", "dw2"):
        assert torch.equal(rp[k], r[k]), k
    for k in ("y", "dx"):
        assert torch.equal(rp[k][:m], r[k][:m]), k
        assert torch.all(rp[k][m:] == SENTINEL), k


@pytest.mark.parametrize("case", [
    dict(counts=[0, 200, 0, 57], E=4, D=256, F=384, pad=256),        # zero-token experts, pad 256
    dict(counts=[300, 1, 129], E=3, D=384, F=256, pad=128),          # ragged counts, pad 128
    dict(counts=[512], E=1, D=512, F=640, pad=256),                  # dense (E = 1)
    # more tiles than compute units, with a remainder: FC1 (288 tiles of 256 x 256) and FC2
    # dgrad (288 of 256 x 128) run whole tiles plus split tail tiles; FC2 and FC1 dgrad are all
    # tail
    dict(counts=[2300, 2250], E=2, D=256, F=2048, pad=256),
    dict(counts=[300, 77, 515], E=3, D=384, F=256, pad=128),        # ragged, fused plan
])
def test_small_shapes_stagewise(case):
    mx = require_gpu()
    print(f"\nstagewise case E={case['E']} D={case['D']} F={case['F']} pad={case['pad']}", flush=True)
    prob = workloads.mlp_problem(None, seed=3, counts=case["counts"], E=case["E"], D=case["D"],
                                 F=case["F"], pad=case["pad"],
                                 m_capacity=workloads.padded_offsets(case["counts"], case["pad"])[-1] + case["pad"])
    r = run_mlp(mx, prob, mx.OUT_F32 | mx.DEBUG_F32)
    check_stagewise(prob, r)


def _many_expert_counts(E, seed, zero, total, nonzero=None):
    """Ragged per-expert counts for E experts: `zero` of them get no token; with `nonzero`,
    only that many experts (chosen at random) get tokens at all."""
    rng = np.random.default_rng(seed)
    live = rng.permutation(E)[: (nonzero if nonzero is not None else E - zero)]
    w = rng.dirichlet(np.full(len(live), 0.8))
    c = workloads.largest_remainder(w, total)
    counts = np.zeros(E, dtype=np.int64)
    counts[live] = c
    return [int(x) for x in counts]


# E >= 64 takes other code paths in every kernel: a looping offsets check instead of one lane
# per expert, a binary search for the expert of a row, and the K-grouped scheduler's longest-K
# order over more experts than a wavefront has lanes. E = 63 is the last single-wavefront case.
MANY_EXPERTS = [
    dict(E=63, D=256, F=256, pad=128, seed=11, zero=9, total=5000),
    dict(E=64, D=256, F=256, pad=128, seed=12, zero=12, total=6000),
    dict(E=72, D=256, F=256, pad=128, seed=13, zero=12, total=6000),
    dict(E=72, D=256, F=384, pad=256, seed=14, zero=12, total=9000),
    dict(E=1024, D=128, F=128, pad=128, seed=15, zero=None, total=3000, nonzero=20),
]


@pytest.mark.parametrize("case", MANY_EXPERTS, ids=[f"E{c['E']}_pad{c['pad']}_F{c['F']}" for c in MANY_EXPERTS])
def test_many_experts_stagewise(case):
    mx = require_gpu()
    counts = _many_expert_counts(case["E"], case["seed"], case["zero"] or 0, case["total"], case.get("nonzero"))
    print(f"\nmany-experts case E={case['E']} pad={case['pad']}: {sum(c == 0 for c in counts)} zero-token experts, "
          f"{sum(counts)} rows", flush=True)
    prob = workloads.mlp_problem(None, seed=case["seed"], counts=counts, E=case["E"], D=case["D"], F=case["F"],
                                 pad=case["pad"],
                                 m_capacity=workloads.padded_offsets(counts, case["pad"])[-1] + case["pad"])
    r = run_mlp(mx, prob, mx.OUT_F32 | mx.DEBUG_F32)
    E = case["E"]
    live = [e for e in range(E) if counts[e]]
    experts = None if E <= 128 else sorted(set(live + [0, 1, E // 2, E - 2, E - 1]))
    check_stagewise(prob, r, weight_experts=experts)


def test_many_experts_counts_null_means_all_rows_real():
    """E = 72 with counts NULL (every row of a segment real) equals counts = segment lengths."""
    mx = require_gpu()
    counts = _many_expert_counts(72, 16, 10, 3000)
    seg = [(c + 127) // 128 * 128 for c in counts]
    prob = workloads.mlp_problem(None, seed=16, counts=seg, E=72, D=256, F=256, pad=128,
                                 m_capacity=sum(seg))
    r1 = run_mlp(mx, prob, mx.OUT_F32, counts=True)
    r2 = run_mlp(mx, prob, mx.OUT_F32, counts=False)
    for k in ("y", "dx", "dw1", "dw3", "dw2"):
        assert torch.equal(r1[k], r2[k]), k


def test_zero_routed_tokens():
    mx = require_gpu()
    prob = workloads.mlp_problem(None, counts=[0, 0], E=2, D=256, F=256, pad=128, m_capacity=256)
    r = run_mlp(mx, prob, mx.OUT_F32)
    assert r["status_fwd"] == 0 and r["status_bwd"] == 0
    for k in ("dw1", "dw3", "dw2"):
        assert torch.all(r[k] == 0), k
    assert torch.all(r["y"] == SENTINEL) and torch.all(r["dx"] == SENTINEL)


def test_counts_null_means_all_rows_real():
    mx = require_gpu()
    counts = [256, 128]
    prob = workloads.mlp_problem(None, seed=9, counts=counts, E=2, D=256, F=256, pad=128, m_capacity=512)
    r1 = run_mlp(mx, prob, mx.OUT_F32, counts=True)
    r2 = run_mlp(mx, prob, mx.OUT_F32, counts=False)
    for k in ("y", "dx", "dw1", "dw3", "dw2"):
        assert torch.equal(r1[k], r2[k]), k


@pytest.mark.parametrize("bad", ["unaligned", "decreasing", "capacity", "count"])
def test_invalid_offsets_reported_and_nothing_written(bad):
    mx = require_gpu()
    counts = [100, 100]
    prob = workloads.mlp_problem(None, seed=1, counts=counts, E=2, D=256, F=256, pad=128, m_capacity=256)
    offs = {"unaligned": [0, 64, 256], "decreasing": [0, 256, 128], "capacity": [0, 128, 384],
            "count": [0, 128, 256]}[bad]
    if bad == "count":
        prob["counts"] = [129, 100]
    prob["offs"] = offs
    r = run_mlp(mx, prob, mx.OUT_F32)
    assert r["status_fwd"] == mx.DEV_BAD_OFFSETS and r["status_bwd"] == mx.DEV_BAD_OFFSETS
    for k in ("y", "dx", "dw1", "dw3", "dw2"):
        assert torch.all(r[k] == SENTINEL), k


def test_pack_unpack_round_trip():
    mx = require_gpu()
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    E, F, D = 3, 192, 128
    w1 = torch.randn((E, F, D), generator=g, device="cuda").to(torch.bfloat16)
    w3 = torch.randn((E, F, D), generator=g, device="cuda").to(torch.bfloat16)
    w13 = torch.empty((E, 2 * F, D), dtype=torch.bfloat16, device="cuda")
    mx.pack_w13(w1, w3, w13, E, F, D)
    a = torch.empty_like(w1)
    b = torch.empty_like(w3)
    mx.unpack_w13(w13, a, b, E, F, D)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), w1.view(torch.int16)) and torch.equal(b.view(torch.int16), w3.view(torch.int16))
    ref = om.pack_w13(bits(w1), bits(w3))
    assert np.array_equal(bits(w13), ref)


@pytest.mark.parametrize("case", [
    None,                                                             # tiny, pad 128
    dict(counts=[0, 200, 0, 57], E=4, D=256, F=384, pad=256),        # zero-token experts, pad 256
])
def test_unfused_plan_against_oracle(case):
    """The unfused plan's standalone SwiGLU and dSwiGLU + dual-quantization kernels (the
    standalone-cast side of torchtitan PR #2 "Numerics and tests") against the oracle fed the
    same upstream tensors: h from the plan's own BF16 FC1 output, dH13 from its own BF16 dh.
    Fused-code tolerance: each code within one E4M3 step, at most 0.1% differing."""
    mx = require_gpu()
    if case is None:
        prob = workloads.mlp_problem("tiny", m_capacity=1536)
    else:
        prob = workloads.mlp_problem(None, seed=5, counts=case["counts"], E=case["E"], D=case["D"], F=case["F"],
                                     pad=case["pad"],
                                     m_capacity=workloads.padded_offsets(case["counts"], case["pad"])[-1])
    E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
    print(f"\nunfused plan vs oracle: E={E} D={D} F={F} pad={pad}", flush=True)
    ctx = mx.MlpContext(E, D, F, pad, mcap, flags=mx.UNFUSED | mx.OUT_F32)
    offs = torch.tensor(prob["offs"], dtype=torch.int32, device="cuda")
    cnt = torch.tensor(prob["counts"], dtype=torch.int32, device="cuda")
    x, w1, w3, w2, dy = (prob[k].cuda() for k in ("x", "w1", "w3", "w2", "dy"))
    y = torch.empty((mcap, D), dtype=torch.float32, device="cuda")
    dx = torch.empty_like(y)
    dw1 = torch.empty((E, F, D), dtype=torch.float32, device="cuda")
    dw3, dw2 = torch.empty_like(dw1), torch.empty((E, D, F), dtype=torch.float32, device="cuda")
    ctx.fwd(offs, cnt, x, w1, w3, w2, y)
    torch.cuda.synchronize()
    # forward-only tensors share workspace bytes with the backward's: read them now
    fw = {n: ctx.view(n).cpu() for n in ("H13", "HQ_R", "HS_R", "HQ_C", "HS_C")}
    ctx.bwd(offs, cnt, dy, dx, dw1, dw3, dw2)
    torch.cuda.synchronize()
    assert ctx.status() == mx.DEV_OK
    bw = {n: ctx.view(n).cpu() for n in ("DH16", "DHQ_R", "DHS_R", "DHQ_C", "DHS_C")}
    m = prob["offs"][-1]
    h13_bits = bits(fw["H13"])[:m]
    _, hq_r, hs_r, hq_c, hs_c = om.swiglu_quant_from_h13(h13_bits)
    f1 = check_fused_codes(u(fw["HQ_R"])[:m], u(fw["HS_R"])[:m], hq_r, hs_r, label="hq_r")
    f2 = check_fused_codes(u(fw["HQ_C"])[:, :m], u(fw["HS_C"])[:, :m // 32], hq_c, hs_c, label="hq_c")
    dh = bf16_bits_to_f64(bits(bw["DH16"])[:m])
    _, dq_r, ds_r, dq_c, ds_c = om.dswiglu_quant(dh, h13_bits)
    f3 = check_fused_codes(u(bw["DHQ_R"])[:m], u(bw["DHS_R"])[:m], dq_r, ds_r, label="dhq_r")
    f4 = check_fused_codes(u(bw["DHQ_C"])[:, :m], u(bw["DHS_C"])[:, :m // 32], dq_c, ds_c, label="dhq_c")
    print(f"standalone SwiGLU codes differing: row {f1:.2e} col {f2:.2e}; dSwiGLU: row {f3:.2e} col {f4:.2e}")


def _graph_kernel_nodes(mx, prob, flags, direction):
    """Capture one grouped_mlp_fwd (or _bwd) call on a fresh stream into a HIP graph and return
    the types of the graph's nodes: an independent count of the kernels the call launches."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
    ctx = mx.MlpContext(E, D, F, pad, mcap, flags=flags)
    offs = torch.tensor(prob["offs"], dtype=torch.int32, device="cuda")
    cnt = torch.tensor(prob["counts"], dtype=torch.int32, device="cuda")
    x, w1, w3, w2, dy = (prob[k].cuda() for k in ("x", "w1", "w3", "w2", "dy"))
    y = torch.empty((mcap, D), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    dw1 = torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda")
    dw3, dw2 = torch.empty_like(dw1), torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")
    ctx.fwd(offs, cnt, x, w1, w3, w2, y)         # the backward's saved tensors exist
    torch.cuda.synchronize()
    st = ctypes.c_void_p()
    assert hip.hipStreamCreateWithFlags(ctypes.byref(st), 1) == 0          # non-blocking
    graph = ctypes.c_void_p()
    assert hip.hipStreamBeginCapture(st, 2) == 0                           # relaxed mode
    try:
        if direction == "fwd":
            ctx.fwd(offs, cnt, x, w1, w3, w2, y, stream=st.value)
        else:
            ctx.bwd(offs, cnt, dy, dx, dw1, dw3, dw2, stream=st.value)
    finally:
        assert hip.hipStreamEndCapture(st, ctypes.byref(graph)) == 0
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    types = []
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
        types.append(t.value)
    hip.hipGraphDestroy(graph)
    hip.hipStreamDestroy(st)
    return types


@pytest.mark.parametrize("shape", ["tiny", "pad256"])
@pytest.mark.parametrize("plan", ["fused", "unfused"])
def test_launch_counts(plan, shape):
    """Launch-count contract (torchtitan PR #2 "Summary": the fused plan removes the standalone
    activation casts; "Numerics and tests": profiler op-count contracts). Forward: 3 kernels
    for the fused plan (one launch quantizing W13, W2 and X; FC1 + SwiGLU + dual quantization;
    FC2), 4 for the unfused plan (plain FC1, then the standalone SwiGLU quantizer). Backward,
    fused: the dY quantizer, FC2 dgrad + dSwiGLU + dual quantization, then FC1 wgrad, FC2 wgrad
    and FC1 dgrad -- one launch on 256-row tiles (pad 256), three otherwise (pad 128): 3 or 5;
    unfused: plain FC2 dgrad and the standalone dSwiGLU quantizer in place of the fused GEMM,
    4 or 6. Counted twice: by the library's per-launch events and as kernel nodes of a
    captured HIP graph (which must hold nothing but kernels: no memset or copy nodes)."""
    mx = require_gpu()
    prob = workloads.mlp_problem("tiny", m_capacity=1536) if shape == "tiny" else _merged_problem(MERGED_BWD)
    flags = mx.UNFUSED if plan == "unfused" else 0
    tail = {"fc2_wgrad", "fc1_wgrad", "fc1_dgrad"} if shape == "tiny" else {"bwd_gemms"}
    want = {"fused": ({"quant_fwd", "fc1_swiglu", "fc2"}, {"quant_dy", "fc2_dgrad_dswiglu"} | tail),
            "unfused": ({"quant_fwd", "fc1", "swiglu_quant", "fc2"},
                        {"quant_dy", "fc2_dgrad", "dswiglu_quant"} | tail)}[plan]
    E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
    ctx = mx.MlpContext(E, D, F, pad, mcap, flags=flags)
    offs = torch.tensor(prob["offs"], dtype=torch.int32, device="cuda")
    cnt = torch.tensor(prob["counts"], dtype=torch.int32, device="cuda")
    x, w1, w3, w2, dy = (prob[k].cuda() for k in ("x", "w1", "w3", "w2", "dy"))
    y = torch.empty((mcap, D), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    dw1 = torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda")
    dw3, dw2 = torch.empty_like(dw1), torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")
    for direction, names in zip(("fwd", "bwd"), want):
        mx.profile_begin(64)
        if direction == "fwd":
            ctx.fwd(offs, cnt, x, w1, w3, w2, y)
        else:
            ctx.bwd(offs, cnt, dy, dx, dw1, dw3, dw2)
        prof = mx.profile_end()
        assert set(prof) == names and all(n == 1 for n, _ in prof.values()), (direction, prof)
        types = _graph_kernel_nodes(mx, prob, flags, direction)
        assert types == [0] * len(names), (direction, types)   # hipGraphNodeTypeKernel == 0


def test_graph_replay_equals_eager():
    """The whole fwd + bwd captured in a graph and replayed gives the eager call's outputs and
    all three weight gradients bit for bit (the compiled-vs-eager check of torchtitan PR #12
    "Evidence", here as graph replay vs eager launches). Replayed several times, alternating
    two input sets, with eager work of the library and host synchronisation between replays."""
    mx = require_gpu()
    prob = workloads.mlp_problem("tiny", m_capacity=1536)
    E, D, F, pad, mcap = prob["E"], prob["D"], prob["F"], prob["pad"], prob["m_capacity"]
    other = workloads.mlp_problem("tiny", seed=7, m_capacity=1536)
    offs = torch.tensor(prob["offs"], dtype=torch.int32, device="cuda")
    cnt = torch.tensor(prob["counts"], dtype=torch.int32, device="cuda")
    names = ("x", "w1", "w3", "w2", "dy")
    sets = [{k: p[k].cuda() for k in names} for p in (prob, other)]
    outs = ("y", "dx", "dw1", "dw3", "dw2")

    def buffers():
        y = torch.empty((mcap, D), dtype=torch.bfloat16, device="cuda")
        return {"y": y, "dx": torch.empty_like(y), "dw1": torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda"),
                "dw3": torch.empty((E, F, D), dtype=torch.bfloat16, device="cuda"),
                "dw2": torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")}

    def run(ctx, inp, o):
        ctx.fwd(offs, cnt, inp["x"], inp["w1"], inp["w3"], inp["w2"], o["y"])
        ctx.bwd(offs, cnt, inp["dy"], o["dx"], o["dw1"], o["dw3"], o["dw2"])

    m = prob["offs"][-1]
    eager_ctx = mx.MlpContext(E, D, F, pad, mcap)
    ref = []
    for s in sets:
        o = buffers()
        run(eager_ctx, s, o)
        torch.cuda.synchronize()
        ref.append({k: o[k].clone() for k in outs})
    gctx = mx.MlpContext(E, D, F, pad, mcap)
    static_in = {k: sets[0][k].clone() for k in names}
    static_out = buffers()
    run(gctx, static_in, static_out)                        # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(gctx, static_in, static_out)
    scratch = buffers()
    for rep in range(4):
        i = rep % 2
        for k in names:
            static_in[k].copy_(sets[i][k])
        g.replay()
        run(eager_ctx, sets[1 - i], scratch)                # eager work between replays
        torch.cuda.synchronize()
        for k in outs:
            a, b = static_out[k], ref[i][k]
            if k in ("y", "dx"):
                a, b = a[:m], b[:m]
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, k)
        assert gctx.status() == mx.DEV_OK
