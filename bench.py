#!/usr/bin/env python3
"""Benchmark of the MXFP8 routed-experts SwiGLU MLP on one MI355X.

One step = grouped_mlp_fwd + grouped_mlp_bwd (every kernel of the path: weight dual
quantization and packing, token dual quantization, FC1 + SwiGLU + dual quantization, FC2,
dY quantization, FC2 dgrad + dSwiGLU + dual quantization, both wgrads, FC1 dgrad) on the
DeepSeek-V3-16B-like expert-parallel rank: 16 local experts, D=2048, F=1408, 24576 routed
rows (Zipf(1.1) counts with 2 zero-token experts) padded to 256 per expert. Inputs are
synthetic (seeded), resident in HBM before timing; three input sets rotate so that the
256 MB last-level cache cannot hold a step's operands.

value = useful TFLOP/s = 18 * M_real * D * F / step time (pad rows are not counted).
The line also reports, for the dominant kernel, its roofline fraction (per-kernel HIP
event timing inside the library, on the launch stream), the standalone quantizer's GB/s
on BF16 [16384, 7168] dual quantization, and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "grouped-MLP fwd+bwd MXFP8 TFLOP/s & quantize GB/s, % of MI355X roofline"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense MXFP8 / FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def gemm_flops(name, m_real, D, F):
    """Useful FLOPs of one launch of each GEMM kernel (2 per multiply-add, real rows only)."""
    per = {"fc1_swiglu": 2 * 2 * F * D, "fc2": 2 * D * F, "fc2_dgrad_dswiglu": 2 * F * D,
           "fc2_wgrad": 2 * D * F, "fc1_dgrad": 2 * D * 2 * F, "fc1_wgrad": 2 * 2 * F * D,
           "bwd_gemms": 2 * D * F + 2 * D * 2 * F + 2 * 2 * F * D}  # FC2 wgrad + FC1 dgrad + FC1 wgrad
    return per[name] * m_real if name in per else None


def quant_bytes(name, m_pad, m_real, E, D, F):
    """Algorithmic HBM bytes of one launch of each quantization kernel: BF16 read of the real
    rows, codes in both directions (2 B/element) and scales (2/32 B/element) written.
    quant_fwd quantizes W13 (packed), W2 and X in one launch."""
    out = 2 + 2.0 / 32
    x = m_real * D * 2 + m_pad * D * out
    if name == "quant_dy":
        return x
    if name == "quant_fwd":
        return E * 2 * F * D * (2 + out) + E * D * F * (2 + out) + x
    return None


def traffic_for(kernel, workload, key="kernels"):
    """A per-launch figure from the committed rocprofv3 counter runs (key "kernels": HBM bytes;
    "mfma_busy": the matrix-core busy fraction), if they were taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        from mxfp8_mixed_precision_amd.prof_summary import source_sha256
        with open(path) as f:
            t = json.load(f)
        if t.get("source_sha256") != source_sha256(ROOT):
            return None
        return t.get(key, {}).get(workload, {}).get(kernel)
    except Exception:
        return None


def cpu_baseline(prob):
    """The oracle (as it stands) on a bounded sample of the same workload: the full fwd+bwd of
    the smallest non-empty experts holding at least 2500 routed rows together, timed on the
    host cores."""
    import numpy as np
    import workloads
    from oracle import mlp as om
    from oracle.formats import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    counts = prob["counts"]
    order = []
    for e in sorted([e for e in range(len(counts)) if counts[e] > 0], key=lambda e: counts[e]):
        order.append(e)
        if sum(counts[i] for i in order) >= 2500:
            break
    D, F, pad = prob["D"], prob["F"], prob["pad"]
    sub_counts = [counts[e] for e in order]
    sub_offs = workloads.padded_offsets(sub_counts, pad)
    offs = prob["offs"]
    x = np.concatenate([bf16_bits_to_f64(workloads.bf16_bits(prob["x_cpu"][offs[e]:offs[e + 1]])) for e in order])
    dy = np.concatenate([bf16_bits_to_f64(workloads.bf16_bits(prob["dy_cpu"][offs[e]:offs[e + 1]])) for e in order])
    w1 = bf16_bits_to_f64(workloads.bf16_bits(prob["w1_cpu"][order]))
    w3 = bf16_bits_to_f64(workloads.bf16_bits(prob["w3_cpu"][order]))
    w2 = bf16_bits_to_f64(workloads.bf16_bits(prob["w2_cpu"][order]))
    t0 = time.perf_counter()
    fwd = om.mlp_forward(x, w1, w3, w2, sub_offs, sub_counts)
    om.mlp_backward(fwd, dy)
    dt = time.perf_counter() - t0
    flops = 18.0 * sum(sub_counts) * D * F
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full fwd+bwd of experts {order} ({sum(sub_counts)} routed rows, "
                      f"{flops / 1e9:.1f} useful GFLOP) in {dt:.1f} s; numpy fp64, BLAS threads {threads}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 50 untimed steps (about 45 ms): after 5 the step still runs about 5% slower than after 60
    # or 200 (0.947 against 0.896 ms on one box) while the GPU's clocks settle under load
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="dsv3_rank", choices=["dsv3_rank", "dense", "large_expert", "tiny"])
    ap.add_argument("--sets", type=int, default=3, help="rotating input sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quant", action="store_true", help="skip the standalone quantizer measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference kernel for HBM byte counters)")
    ap.add_argument("--no-plans", action="store_true",
                    help="skip the fused/unfused plan and dispatch A/B legs (profiling runs: they launch other kernels)")
    ap.add_argument("--concurrent", action="store_true",
                    help="time the steps with MXF_CONCURRENT (helper streams) instead of serial launches")
    ap.add_argument("--serial", action="store_true",
                    help="launch with MXF_SERIAL stated explicitly (the default order; profiler runs)")
    ap.add_argument("--quant-only", action="store_true",
                    help="only measure the standalone quantizer and dequantizer (for a profiler run of those kernels alone)")
    ap.add_argument("--mfma-only", action="store_true",
                    help="only run the matrix-core ceiling kernels (for a profiler run of those kernels alone)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "the library runs one expert-parallel rank's share on one GPU and has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mxfp8_mixed_precision_amd as mx
    import workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 3}), flush=True)
        return
    if args.mfma_only:
        mx.lib()
        print(json.dumps({"mfma_ceilings": bench_mfma_ceilings(mx, torch, dev, args)}), flush=True)
        return
    if args.quant_only:
        mx.lib()
        print(json.dumps({"quantize": bench_quantize(mx, torch, dev, args),
                          "dequantize": bench_dequantize(mx, torch, dev, args)}), flush=True)
        return
    mx.lib()
    cfg = workloads.MLP_CONFIGS[args.workload]
    E, D, F, pad = cfg["E"], cfg["D"], cfg["F"], cfg["pad"]
    counts = workloads.expert_counts(args.workload)
    offs = workloads.padded_offsets(counts, pad)
    m_pad, m_real = offs[-1], sum(counts)
    mcap = m_pad

    # input sets generated on the GPU (same recipe, GPU generator) and kept resident
    sets = []
    for s in range(args.sets):
        p = workloads.mlp_problem(args.workload, seed=42 + s, device=dev)
        sets.append({k: p[k] for k in ("x", "w1", "w3", "w2", "dy")})
    offs_t = torch.tensor(offs, dtype=torch.int32, device=dev)
    counts_t = torch.tensor(counts, dtype=torch.int32, device=dev)
    ctx = mx.MlpContext(E, D, F, pad, mcap, flags=mx.CONCURRENT if args.concurrent else (mx.SERIAL if args.serial else 0),
                        device=dev)
    y = torch.empty((mcap, D), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((mcap, D), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((E, F, D), dtype=torch.bfloat16, device=dev)
    dw3 = torch.empty((E, F, D), dtype=torch.bfloat16, device=dev)
    dw2 = torch.empty((E, D, F), dtype=torch.bfloat16, device=dev)

    def step(i):
        s = sets[i % len(sets)]
        ctx.fwd(offs_t, counts_t, s["x"], s["w1"], s["w3"], s["w2"], y)
        ctx.bwd(offs_t, counts_t, s["dy"], dx, dw1, dw3, dw2)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert ctx.status() == mx.DEV_OK
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    useful = 18.0 * m_real * D * F
    executed = 18.0 * m_pad * D * F
    value = useful / (ms_per_step / 1e3) / 1e12

    # Per-kernel timing: library-internal HIP events on each launch's stream, over the same
    # steps again with MXF_SERIAL, so that every kernel runs alone on the GPU (with
    # --concurrent some launches of the timed steps overlap on helper streams, which would
    # stretch each one's own duration; the events add a little time between launches).
    sctx = mx.MlpContext(E, D, F, pad, mcap, flags=mx.SERIAL, device=dev)

    def sstep(i):
        s = sets[i % len(sets)]
        sctx.fwd(offs_t, counts_t, s["x"], s["w1"], s["w3"], s["w2"], y)
        sctx.bwd(offs_t, counts_t, s["dy"], dx, dw1, dw3, dw2)

    for i in range(2):
        sstep(i)
    torch.cuda.synchronize()
    mx.profile_begin(12 * args.steps + 16)
    t2 = time.perf_counter()
    for i in range(args.steps):
        sstep(i)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    prof = mx.profile_end()
    del sctx
    kernels = {}
    for name, (n, tot) in prof.items():
        avg = tot / n
        k = {"launches": n, "avg_us": round(avg * 1e3, 2)}
        fl = gemm_flops(name, m_real, D, F)
        if fl is not None:
            k["tflops"] = round(fl / (avg / 1e3) / 1e12, 1)
            k["frac_of_peak"] = round(k["tflops"] / PEAK_FP8_TFLOPS, 4)
        by = quant_bytes(name, m_pad, m_real, E, D, F)
        if by is not None:
            k["gbs"] = round(by / (avg / 1e3) / 1e9, 1)
            k["frac_of_peak"] = round(k["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = k
    dom = max(prof.items(), key=lambda kv: kv[1][1])[0]
    dn, dtot = prof[dom]
    davg_s = dtot / dn / 1e3
    fl = gemm_flops(dom, m_real, D, F)
    if fl is not None:
        ach = fl / davg_s / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4),
                "traffic": traffic_for(dom, args.workload),
                "mfma_busy": traffic_for(dom, args.workload, "mfma_busy")}
    else:
        by = quant_bytes(dom, m_pad, m_real, E, D, F)
        ach = by / davg_s / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic_for(dom, args.workload)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "mxfp8-e4m3/fp32-acc",
        "data": "synthetic (seeded N(0,1) activations and gradients, N(0,0.02) weights, BF16)",
        "config": {"workload": f"{args.workload}: one expert-parallel rank, E={E} D={D} F={F}, "
                               f"{m_real} routed rows padded to {m_pad} (pad {pad}), fwd+bwd",
                   "E": E, "D": D, "F": F, "m_real": m_real, "m_padded": m_pad, "pad_multiple": pad,
                   "parallelism": "single GPU (one EP rank's share)"},
        "gpu_ms_per_step": round(gpu_ms_per_step, 4),
        "executed_tflops": round(executed / (ms_per_step / 1e3) / 1e12, 2),
        "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 4),
        "roofline": roof,
        "kernels": kernels,
        "launches": "concurrent where independent (MXF_CONCURRENT)" if args.concurrent else "serial (default)",
        "kernels_timing": "a second pass of the same steps with MXF_SERIAL (each kernel alone on the GPU)",
        "serial_ms_per_step": round((t3 - t2) * 1e3 / args.steps, 4),
    }

    if not args.no_plans:
        out["mfma_ceilings"] = bench_mfma_ceilings(mx, torch, dev, args)
        if roof["bound"] == "mfma":
            roof["frac_of_matrix_ceiling"] = round(roof["achieved"] / out["mfma_ceilings"]["matrix_only"]["value"], 4)
        out["dispatch"] = bench_dispatch(mx, torch, dev, args, kernels["quant_fwd"]["avg_us"], sets[0])
        out["plans"] = bench_plans(mx, torch, dev, args, sets, counts, E, D, F, y, dx, dw1, dw3, dw2)
    if not args.no_quant:
        out["quantize"] = bench_quantize(mx, torch, dev, args)
        out["dequantize"] = bench_dequantize(mx, torch, dev, args)

    if not args.no_cpu_baseline:
        cpu_prob = workloads.mlp_problem(args.workload, seed=42)
        prob = {"x_cpu": cpu_prob["x"], "dy_cpu": cpu_prob["dy"], "w1_cpu": cpu_prob["w1"],
                "w3_cpu": cpu_prob["w3"], "w2_cpu": cpu_prob["w2"], "counts": counts, "offs": offs,
                "D": D, "F": F, "pad": pad}
        out["cpu_baseline"] = cpu_baseline(prob)
        if "quantize" in out:
            out["quantize"]["cpu_baseline"] = cpu_baseline_quantize()
    print(json.dumps(out), flush=True)


def loop_seconds(torch, n, launch):
    """Average seconds per launch of n back-to-back launches of one kernel, from two HIP events
    on the launching (current) stream around the whole loop. An event recorded after every
    launch lengthens these 55-90 us kernels themselves (the dequantizer's kernel-trace duration
    goes from about 55 to 62 us), so the standalone kernels are timed as they run in a
    pipeline: back to back."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(n):
        launch(i)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / n


def bench_quantize(mx, torch, dev, args):
    """Standalone dual quantization of BF16 [16384, 7168] (3 rotating inputs)."""
    import workloads
    rows, cols = workloads.QUANT_CONFIG["rows"], workloads.QUANT_CONFIG["cols"]
    xs = [workloads.quant_matrix(rows, cols, seed=42 + s, device=dev) for s in range(3)]
    q_r = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    s_r = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    q_c = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    s_c = torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)
    n = max(args.steps, 10)
    # 100 untimed launches first (about 9 ms): run straight after the MLP legs, the first timed
    # loop was slower whichever variant it timed (measured in order: E4M3 87.8 us, E5M2 82.9,
    # E4M3 again 82.2, E5M2 again 81.6, with 20 warm-up launches)
    for i in range(100):
        mx.mxfp8_quantize(xs[i % 3], rows, cols, 3, q_r, s_r, q_c, s_c)
    avg_s = loop_seconds(torch, n, lambda i: mx.mxfp8_quantize(xs[i % 3], rows, cols, 3, q_r, s_r, q_c, s_c))
    nbytes = rows * cols * (2 + 2 + 2.0 / 32)
    gbs = nbytes / avg_s / 1e9
    # the E5M2 element variant of the same kernel, same workload
    avg5 = loop_seconds(torch, n, lambda i: mx.mxfp8_quantize(xs[i % 3], rows, cols, 3 | mx.E5M2, q_r, s_r, q_c, s_c))
    # measured ceiling: a plain device copy reading the quantizer's input bytes and writing as
    # many (torch's vectorised copy kernel), same rotation of 3 sources
    dst = torch.empty_like(xs[0])
    for i in range(3):
        dst.copy_(xs[i])
    cp_s = loop_seconds(torch, n, lambda i: dst.copy_(xs[i % 3]))
    cp_gbs = 2 * xs[0].numel() * 2 / cp_s / 1e9
    # the library's HBM ceiling kernels on the same bytes: a pure read of the input, a pure
    # write of as many bytes, and a copy (read + write) -- the fastest access patterns measured
    # on this chip, against which the quantizer's read + write traffic is reported
    nb = xs[0].numel() * 2
    xor = torch.zeros(1024, dtype=torch.uint8, device=dev)
    ceil = {}
    for name, mode, src, traffic in (("read", mx.HBM_READ, lambda i: xs[i % 3], nb),
                                     ("write", mx.HBM_WRITE, lambda i: None, nb),
                                     ("copy", mx.HBM_COPY, lambda i: xs[i % 3], 2 * nb)):
        out = xor if mode == mx.HBM_READ else dst
        for i in range(3):
            mx.hbm_probe(mode, src(i), out, nb)
        t = loop_seconds(torch, n, lambda i: mx.hbm_probe(mode, src(i), out, nb))
        ceil[name] = {"value": round(traffic / t / 1e9, 1), "unit": "GB/s", "avg_us": round(t * 1e6, 2)}
    del dst, xor
    return {"workload": f"quant: BF16 [{rows}, {cols}] dual (row-wise + column-wise) MXFP8", "value": round(gbs, 1),
            "unit": "GB/s", "avg_us": round(avg_s * 1e6, 2),
            "e5m2": {"value": round(nbytes / avg5 / 1e9, 1), "unit": "GB/s", "avg_us": round(avg5 * 1e6, 2)},
            "copy_ceiling": {"value": round(cp_gbs, 1), "unit": "GB/s", "avg_us": round(cp_s * 1e6, 2),
                             "kernel": f"device copy of BF16 [{rows}, {cols}] (read + write)",
                             "frac_of_copy": round(gbs / cp_gbs, 4)},
            "hbm_ceilings": dict(ceil, kernel=f"library HBM probe kernels (mxf_hbm_probe) on {nb} bytes: read, "
                                               "write, copy (read + write)",
                                 frac_of_copy=round(gbs / ceil["copy"]["value"], 4),
                                 copy_frac_of_peak=round(ceil["copy"]["value"] / PEAK_HBM_GBS, 4)),
            "roofline": {"bound": "hbm", "kernel": "quantize", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_for("quantize", "quant")}}


def bench_mfma_ceilings(mx, torch, dev, args):
    """The library's matrix-core ceiling kernels (mxf_mfma_probe), one block per CU on a 256 x 256
    tile per block: the matrix instructions alone, and the GEMM main loop's whole stage (direct
    global->LDS loads, LDS fragment reads, matrix instructions, a barrier per stage) over a 2 MB
    window of codes (held in each XCD's L2) and a 64 MB window (streamed from beyond the L2s).
    The codes are N(0, 64^2) samples cast to E4M3 (real operand bits; the scales are 1)."""
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device=dev).manual_seed(7)
    nb_big = 64 << 20
    codes = (torch.randn(nb_big, generator=g, device=dev) * 64).clamp_(-448, 448).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8)
    out = torch.empty(ncu * 256, dtype=torch.float32, device=dev)
    stages = 2000
    flop = ncu * stages * 256 * 256 * 64 * 2
    n = 5
    res = {}
    for name, mode, nbytes in (("matrix_only", mx.MFMA_MATRIX, 2 << 20), ("stage_l2", mx.MFMA_STAGE, 2 << 20),
                               ("stage_streamed", mx.MFMA_STAGE, nb_big)):
        for _ in range(2):
            mx.mfma_probe(mode, codes, nbytes, stages, ncu, out)
        t = loop_seconds(torch, n, lambda i: mx.mfma_probe(mode, codes, nbytes, stages, ncu, out))
        tf = flop / t / 1e12
        res[name] = {"value": round(tf, 1), "unit": "TFLOP/s", "avg_us": round(t * 1e6, 1),
                     "us_per_stage": round(t * 1e6 / stages, 4), "frac_of_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
    del codes, out
    res["kernel"] = (f"library matrix-core probe kernels (mxf_mfma_probe): {ncu} blocks x {stages} stages of a "
                     "256 x 256 x 64 block tile; matrix_only = the matrix instructions alone, stage_l2 / "
                     "stage_streamed = the GEMM main-loop stage over a 2 MB / 64 MB window of E4M3 codes")
    return res


def cpu_baseline_quantize(rows_sample=8192):
    """The oracle's dual quantizer (numpy, one thread: no BLAS involved) on the first
    rows_sample rows of the quantizer workload, reported on the same 4.0625 B/element."""
    import numpy as np
    import workloads
    from oracle.formats import bf16_bits_to_f64
    from oracle.mx import quantize_colwise, quantize_rowwise
    cols = workloads.QUANT_CONFIG["cols"]
    x = bf16_bits_to_f64(workloads.bf16_bits(workloads.quant_matrix(seed=42)[:rows_sample]))
    t0 = time.perf_counter()
    quantize_rowwise(x)
    quantize_colwise(x)
    dt = time.perf_counter() - t0
    nel = rows_sample * cols
    return {"value": round(nel * (2 + 2 + 2.0 / 32) / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"dual quantization of rows 0..{rows_sample - 1} of the [16384, {cols}] workload "
                      f"({nel} elements) in {dt:.1f} s; numpy fp64 table search, one thread"}


def bench_plans(mx, torch, dev, args, sets, counts, E, D, F, y, dx, dw1, dw3, dw2):
    """Fused vs unfused plan (MXF_UNFUSED: plain GEMMs + standalone SwiGLU / dSwiGLU
    quantization kernels), each at pad_multiple 256 and 128, on the same routed rows."""
    import workloads
    m_real = sum(counts)
    res = {}
    for plan, flags in (("fused", 0), ("unfused", mx.UNFUSED)):
        for pad in (256, 128):
            offs = workloads.padded_offsets(counts, pad)
            mcap = offs[-1]
            offs_t = torch.tensor(offs, dtype=torch.int32, device=dev)
            counts_t = torch.tensor(counts, dtype=torch.int32, device=dev)
            ctx = mx.MlpContext(E, D, F, pad, mcap, flags=flags, device=dev)

            def step(i):
                s = sets[i % len(sets)]
                ctx.fwd(offs_t, counts_t, s["x"], s["w1"], s["w3"], s["w2"], y)
                ctx.bwd(offs_t, counts_t, s["dy"], dx, dw1, dw3, dw2)

            for i in range(10):  # untimed: a fresh context, and the clocks of the leg before
                step(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                step(i)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / args.steps
            res[f"{plan}_pad{pad}"] = {"ms_per_step": round(ms, 4), "m_padded": mcap,
                                       "useful_tflops": round(18.0 * m_real * D * F / (ms / 1e3) / 1e12, 1),
                                       # pad 256 (256-row tiles): FC1 wgrad, FC2 wgrad and FC1
                                       # dgrad share one launch
                                       "launches_fwd_bwd": ("3 + " if plan == "fused" else "4 + ") +
                                                           (("3" if plan == "fused" else "4") if pad == 256
                                                            else ("5" if plan == "fused" else "6"))}
            del ctx
    return res


def bench_dequantize(mx, torch, dev, args):
    """MXFP8 -> BF16 decode of the quantizer workload's row-wise output (3 rotating inputs)."""
    import workloads
    rows, cols = workloads.QUANT_CONFIG["rows"], workloads.QUANT_CONFIG["cols"]
    qs = []
    for s in range(3):
        q, sc, _, _ = mx.quantize(workloads.quant_matrix(rows, cols, seed=42 + s, device=dev), mx.ROW)
        qs.append((q, sc))
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
    n = max(args.steps, 10)
    for i in range(3):
        mx.mxfp8_dequantize(qs[i][0], qs[i][1], rows, cols, mx.DEQ_BF16, out)
    avg_s = loop_seconds(torch, n, lambda i: mx.mxfp8_dequantize(qs[i % 3][0], qs[i % 3][1], rows, cols,
                                                                 mx.DEQ_BF16, out))
    nbytes = rows * cols * (1 + 1.0 / 32 + 2)
    gbs = nbytes / avg_s / 1e9
    return {"workload": f"E4M3 + E8M0 [{rows}, {cols}] row-wise -> BF16", "value": round(gbs, 1),
            "unit": "GB/s", "avg_us": round(avg_s * 1e6, 2),
            "roofline": {"bound": "hbm", "kernel": "dequantize", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_for("dequantize", "quant")}}


def bench_dispatch(mx, torch, dev, args, quant_fwd_us, weights):
    """Dispatch of the workload's routed tokens into the padded layout: the routing plan, then
    either the BF16 permute (followed by the forward's quantization of X: the forward quantizer's
    time with X minus its time without X) or the fused gather + dual quantization of X."""
    import workloads
    tok, ids = workloads.routed_tokens(args.workload, device="cpu")
    cfg = workloads.MLP_CONFIGS[args.workload]
    E, D, F, pad = cfg["E"], cfg["D"], cfg["F"], cfg["pad"]
    tokens, topk = ids.shape
    counts = workloads.expert_counts(args.workload)
    mcap = workloads.padded_offsets(counts, pad)[-1]
    m_real = sum(counts)
    toks = [tok.to(dev)] + [workloads.randn_bf16(tuple(tok.shape), 1.0, workloads._gen(43 + s, dev), dev)
                            for s in range(2)]
    ids_t = torch.from_numpy(ids).to(dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    ra = torch.empty(mcap, dtype=torch.int32, device=dev)
    ar = torch.empty(tokens * topk, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    pws = torch.empty(mx.route_plan_workspace_bytes(tokens, topk, E), dtype=torch.uint8, device=dev)
    xp = torch.empty((mcap, D), dtype=torch.bfloat16, device=dev)
    ctx = mx.MlpContext(E, D, F, pad, mcap, device=dev)
    n = max(args.steps, 10)

    def one(i):
        mx.mxf_route_plan(ids_t, tokens, topk, E, pad, mcap, offs, cnt, ra, ar, status, pws)
        mx.mxf_dispatch_permute(toks[i % 3], tokens, topk, D, E, offs, ra, mcap, xp)
        ctx.dispatch_quantize(offs, cnt, ra, toks[i % 3], topk)

    for i in range(3):
        one(i)
    torch.cuda.synchronize()
    assert int(status.item()) == mx.DEV_OK and ctx.status() == mx.DEV_OK
    y = torch.empty((mcap, D), dtype=torch.bfloat16, device=dev)

    def fwd_xq(i):  # the forward with X's codes from the fused dispatch: W13 and W2 only
        ctx.fwd(offs, cnt, None, weights["w1"], weights["w3"], weights["w2"], y)

    for i in range(2):
        fwd_xq(i)
    torch.cuda.synchronize()
    mx.profile_begin(6 * n)
    for i in range(n):
        one(i)
        fwd_xq(i)
    torch.cuda.synchronize()
    prof = mx.profile_end()
    us = {k: prof[k][1] / prof[k][0] * 1e3 for k in ("route_plan", "permute", "dispatch_quant_x", "quant_fwd")}
    quant_x_us = quant_fwd_us - us["quant_fwd"]
    # compulsory HBM bytes: each token row read once (its topk copies come from cache), every
    # padded row written, the row indices read
    rd = tokens * D * 2
    perm_bytes = rd + mcap * D * 2 + mcap * 4
    dq_bytes = rd + mcap * D * (2 + 2.0 / 32) + m_real * 4
    gbs = lambda b, u: round(b / (u * 1e-6) / 1e9, 1)
    return {"workload": f"{tokens} tokens x top-{topk} -> {m_real} rows of {E} experts padded to {mcap} (pad {pad}), "
                        f"D={D}",
            "route_plan_us": round(us["route_plan"], 2),
            "permute_us": round(us["permute"], 2), "permute_gbs": gbs(perm_bytes, us["permute"]),
            "dispatch_quant_x_us": round(us["dispatch_quant_x"], 2),
            "dispatch_quant_x_gbs": gbs(dq_bytes, us["dispatch_quant_x"]),
            "quant_x_us": round(quant_x_us, 2),
            "unfused_us": round(us["permute"] + quant_x_us, 2),
            "fused_us": round(us["dispatch_quant_x"], 2),
            "note": "unfused = permute + the forward quantizer's X share (its time with X, main serial pass, "
                    "minus its time without X); fused = dispatch_quant_x"}


if __name__ == "__main__":
    main()
