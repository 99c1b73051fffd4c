"""Summarise rocprofv3 CSV output of bench.py runs into the text kept under profiles/.

Usage (paths are rocprofv3 output directories written with --output-format csv):

  python -m mxfp8_mixed_precision_amd.prof_summary --workload dsv3_rank \
      --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
      --commands FILE --out OUTDIR

Inputs:
  --trace       rocprofv3 --kernel-trace --stats run of `bench.py` (per-dispatch durations)
  --fetch/write rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of the same command
  --copy-*      the same counters for `bench.py --calibrate-copy` (a 1 GiB device copy), which
                give the factor from counter units to bytes
  --compute     (optional) a rocprofv3 --pmc run of the same command with COMPUTE_COUNTERS:
                per kernel, the matrix-core busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over the
                kernel's active cycles times the SIMD count, rocprofv3's own MfmaUtil), the
                FP8 matrix math the hardware counted, the L2 hit rate and the LDS activity
  --commands    text file holding the exact commands that produced the inputs

Outputs (in OUTDIR): <kernel-group>_<workload>.md summaries and traffic.json (HBM bytes
per launch, with the sha256 of the kernel sources they were measured on; bench.py only
reports them while the sources are unchanged).

Kernel dispatches are named by their position in a bench.py step: the MLP step enqueues, in
order, quant_fwd (W13, W2 and X in one launch), fc1_swiglu, fc2, quant_dy, fc2_dgrad_dswiglu,
bwd_gemms (FC1 wgrad, FC2 wgrad and FC1 dgrad in one launch); a --quant-only run launches `quantize` (the dual quantizer), the HBM
ceiling kernels `hbm_read`, `hbm_write`, `hbm_copy` on the quantizer's input bytes, and then
`dequantize` (row-wise codes to BF16); a --mfma-only run launches the matrix-core ceiling kernels
(`mfma_matrix`, then `mfma_stage` over a 2 MB and then a 64 MB window of codes). Profile with
`bench.py --serial` so that every kernel runs alone (durations not stretched by overlap).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

MLP_SEQUENCE = ["quant_fwd", "fc1_swiglu", "fc2", "quant_dy", "fc2_dgrad_dswiglu", "bwd_gemms"]
# expected kernel template per logical name: a piece of the kernel's name (GEMMs: ", SCHED, EPI, "
# of gemm_mx_kernel<BM, BN, WM, WN, SCHED, EPI, OCC>; quantizers: the kernel and its KIND)
EXPECT = {
    "quant_fwd": "quant_fwd_kernel",
    "quant_dy": "quant_dual_kernel<1,", "fc1_swiglu": ", 0, 1, ", "fc2": ", 0, 0, ", "fc2_dgrad_dswiglu": ", 0, 2, ",
    "bwd_gemms": "gemm_bwd3_kernel", "quantize": "quant_dual_kernel<0,true,true,0>",
    "dequantize": "dequant_kernel<true,0>",
    "hbm_read": "hbm_read_kernel", "hbm_write": "hbm_write_kernel", "hbm_copy": "hbm_copy_kernel",
    "mfma_matrix": "mfma_probe_kernel<0>", "mfma_stage": "mfma_probe_kernel<1>",
}
# a --quant-only run: the dual quantizer, the dequantizer, then the HBM ceiling kernels timed
# beside the quantizer (read, write, copy of the quantizer's input bytes)
QUANT_ONLY = ["quantize", "dequantize", "hbm_read", "hbm_write", "hbm_copy"]
# a --mfma-only run: the matrix-core ceiling kernels, the matrix instructions alone, then the
# whole GEMM stage over a 2 MB window (L2-resident) and, with as many launches, a 64 MB window
MFMA_ONLY = ["mfma_matrix", "mfma_stage_l2", "mfma_stage_streamed"]
COMPUTE_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_LDS_IDX_ACTIVE",
                    "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "TCC_HIT_sum", "TCC_MISS_sum"]
SIMDS = 1024   # 256 compute units x 4 SIMDs
XCCS = 8       # GRBM_GUI_ACTIVE is reported per XCC; the CSV value is their sum


def code_only(text):
    """C/C++ source with comments removed and whitespace runs collapsed (string and character
    literals kept as written): what the compiler sees, so that edits to comments or layout do
    not count as kernel changes."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_sha256(root):
    """sha256 over the kernel sources (file names and code without comments) and the compiler
    flags they are built with."""
    from mxfp8_mixed_precision_amd import build
    h = hashlib.sha256()
    csrc = os.path.join(root, "mxfp8_mixed_precision_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, n), encoding="utf-8") as f:
            h.update(n.encode() + b"\0" + code_only(f.read()).encode())
        h.update(" ".join(build.SOURCE_FLAGS.get(n, [])).encode() + b"\0")
    h.update(" ".join(f for f in build.HIPCC_FLAGS if not f.startswith("-I")).encode())
    return h.hexdigest()


def _one(d, pattern):
    files = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not files:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return files[0]


def mxf_dispatches(rows, dispatch_key="Dispatch_Id"):
    """The library's dispatches in launch order: list of (dispatch id, kernel name, row)."""
    seen = {}
    for r in rows:
        name = r["Kernel_Name"]
        if "mxf::" not in name:
            continue
        seen.setdefault(int(r[dispatch_key]), (name, r))
    return [(k, v[0], v[1]) for k, v in sorted(seen.items())]


def _matches(name, logical):
    return re.sub(r"\s+", "", EXPECT[logical]) in re.sub(r"\s+", "", name)


def label(dispatches, group):
    """Attach logical kernel names (see the module docstring). For an MLP run, every window of
    consecutive dispatches whose templates match the step sequence is one step; other
    dispatches (e.g. a trailing standalone-quantizer measurement) are left out."""
    out = []
    if group == "quant":
        return [(did, k, r) for did, name, r in dispatches for k in QUANT_ONLY if _matches(name, k)]
    if group == "mfma":
        mat = [(did, "mfma_matrix", r) for did, name, r in dispatches if _matches(name, "mfma_matrix")]
        st = [(did, r) for did, name, r in dispatches if _matches(name, "mfma_stage")]
        half = len(st) // 2  # the same launch count on each window, 2 MB first
        return mat + [(did, "mfma_stage_l2" if i < half else "mfma_stage_streamed", r)
                      for i, (did, r) in enumerate(st)]
    i, n = 0, len(MLP_SEQUENCE)
    while i + n <= len(dispatches):
        window = dispatches[i:i + n]
        if all(_matches(name, MLP_SEQUENCE[j]) for j, (_, name, _) in enumerate(window)):
            out += [(did, MLP_SEQUENCE[j], r) for j, (did, _, r) in enumerate(window)]
            i += n
        else:
            i += 1
    return out


def per_kernel_durations(trace_dir, group):
    rows = list(csv.DictReader(open(_one(trace_dir, "*kernel_trace.csv"))))
    disp = label(mxf_dispatches(rows), group)
    dur = defaultdict(list)
    for _, logical, r in disp:
        dur[logical].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return dur


def per_kernel_counter(pmc_dir, counter, group):
    rows = [r for r in csv.DictReader(open(_one(pmc_dir, "*counter_collection.csv"))) if r["Counter_Name"] == counter]
    disp = label(mxf_dispatches(rows), group)
    vals = defaultdict(list)
    for _, logical, r in disp:
        vals[logical].append(float(r["Counter_Value"]))
    return vals


def per_kernel_compute(pmc_dir, group):
    """Per logical kernel, the mean over launches of each COMPUTE_COUNTERS value."""
    rows = list(csv.DictReader(open(_one(pmc_dir, "*counter_collection.csv"))))
    out = {}
    for counter in COMPUTE_COUNTERS:
        sel = [r for r in rows if r["Counter_Name"] == counter]
        disp = label(mxf_dispatches(sel), group)
        vals = defaultdict(list)
        for _, logical, r in disp:
            vals[logical].append(float(r["Counter_Value"]))
        for k, v in vals.items():
            out.setdefault(k, {})[counter] = sum(v) / len(v)
    derived = {}
    for k, c in out.items():
        if not all(n in c for n in COMPUTE_COUNTERS):
            continue
        active = c["GRBM_GUI_ACTIVE"] / XCCS  # cycles the GPU was active during the dispatch
        hits, miss = c["TCC_HIT_sum"], c["TCC_MISS_sum"]
        derived[k] = {"mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * SIMDS),
                      "f8_flop": c["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512,
                      "l2_hit": hits / (hits + miss) if hits + miss else None,
                      "lds_active": c["SQ_LDS_IDX_ACTIVE"] / (active * SIMDS / 4),
                      "lds_bank_conflict": c["SQ_LDS_BANK_CONFLICT"] / (active * SIMDS / 4),
                      "active_cycles": active}
    return derived


def copy_factor(pmc_dir, counter, nbytes=1 << 30):
    rows = [r for r in csv.DictReader(open(_one(pmc_dir, "*counter_collection.csv"))) if r["Counter_Name"] == counter]
    vals = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()]
    if not vals:
        raise ValueError(f"no copy kernel in {pmc_dir}")
    v = sorted(vals)[len(vals) // 2]
    return nbytes / v, v


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--compute")
    ap.add_argument("--quant-only", action="store_true")
    ap.add_argument("--mfma-only", action="store_true")
    ap.add_argument("--commands", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--tail", type=int, default=20,
                    help="launches at the end of the trace averaged apart (the serial pass bench.py times)")
    args = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    os.makedirs(args.out, exist_ok=True)
    group = "quant" if args.quant_only else "mfma" if args.mfma_only else "mlp"
    dur = per_kernel_durations(args.trace, group)
    traffic = {}
    lines = []
    ff = wf = None
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        ff, fraw = copy_factor(args.copy_fetch, "FETCH_SIZE")
        wf, wraw = copy_factor(args.copy_write, "WRITE_SIZE")
        fetch = per_kernel_counter(args.fetch, "FETCH_SIZE", group)
        write = per_kernel_counter(args.write, "WRITE_SIZE", group)
        for k in dur:
            if k in fetch and k in write:
                fb = sum(fetch[k]) / len(fetch[k]) * ff
                wb = sum(write[k]) / len(write[k]) * wf
                traffic[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes": round(fb + wb)}
        lines.append(f"Counter calibration (1 GiB device copy): FETCH_SIZE reads {fraw:.0f} -> x{ff:.4f} bytes per unit; "
                     f"WRITE_SIZE reads {wraw:.0f} -> x{wf:.4f} bytes per unit.")
        lines.append("")
    comp = per_kernel_compute(args.compute, group) if args.compute else {}
    cmds = open(args.commands).read().strip()
    name = {"quant": "quantize", "mfma": "mfma_ceilings", "mlp": "mlp_fwd_bwd"}[group]
    md = [f"# {name} kernels, workload `{args.workload}` (rocprofv3)", "", "Commands (run from the repository root):",
          "", "```", cmds, "```", ""] + lines
    md.append(f"| kernel | launches | avg us | avg us, last {args.tail} | median us | min us | max us | "
              "HBM read MB/launch | HBM write MB/launch |")
    md.append("|---|---|---|---|---|---|---|---|---|")
    order = {"quant": QUANT_ONLY, "mfma": MFMA_ONLY, "mlp": MLP_SEQUENCE}[group]
    for k in order:
        if k not in dur:
            continue
        v = dur[k]
        t = traffic.get(k)
        rd = f"{t['fetch_bytes'] / 1e6:.1f}" if t else "-"
        wr = f"{t['write_bytes'] / 1e6:.1f}" if t else "-"
        med = sorted(v)[len(v) // 2]
        tl = v[-args.tail:] if args.tail > 0 else v
        md.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {sum(tl) / len(tl):.2f} | {med:.2f} | {min(v):.2f} | "
                  f"{max(v):.2f} | {rd} | {wr} |")
    md.append("")
    if comp:
        md.append("Compute counters (one rocprofv3 --pmc pass, " + ", ".join(COMPUTE_COUNTERS) + "): MFMA busy = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCC x 1024 SIMDs), as rocprofv3's MfmaUtil; "
                  "F8 math = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 (executed, pad rows included); L2 hit = "
                  "TCC_HIT / (TCC_HIT + TCC_MISS); LDS active and bank-conflict cycles per CU over the "
                  "kernel's active cycles.")
        md.append("")
        md.append("Clock = active cycles (counter pass) over the kernel's mean duration (trace pass): an estimate "
                  "of the shader clock the kernel ran at (2.4 GHz is the maximum; the MXFP8 peak scales with it, "
                  "5.0 PF at 2.4 GHz). The counter pass's window around a dispatch is a few microseconds longer "
                  "than the kernel, so short kernels read high (above 2.4 GHz for the 40 us dY quantizer).")
        md.append("")
        md.append("| kernel | MFMA busy | F8 math TFLOP/launch | L2 hit | LDS active | LDS bank conflict | active cycles | clock GHz |")
        md.append("|---|---|---|---|---|---|---|---|")
        for k in order:
            if k not in comp:
                continue
            c = comp[k]
            hit = f"{c['l2_hit']:.3f}" if c["l2_hit"] is not None else "-"
            ghz = f"{c['active_cycles'] / (sum(dur[k]) / len(dur[k])) / 1e3:.2f}" if k in dur else "-"
            md.append(f"| {k} | {c['mfma_busy']:.3f} | {c['f8_flop'] / 1e12:.4f} | {hit} | {c['lds_active']:.3f} | "
                      f"{c['lds_bank_conflict']:.4f} | {c['active_cycles']:.0f} | {ghz} |")
        md.append("")
    path = os.path.join(args.out, f"{name}_{args.workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(md) + "\n")
    if not traffic and not comp:  # a trace alone: no counters to store beside the source hash
        print(open(path).read())
        return
    tpath = os.path.join(args.out, "traffic.json")
    t = {"kernels": {}}
    if os.path.exists(tpath):
        t = json.load(open(tpath))
    t["source_sha256"] = source_sha256(root)
    t.setdefault("kernels", {})[args.workload] = {k: v["bytes"] for k, v in traffic.items()}
    t.setdefault("detail", {})[args.workload] = traffic
    if ff:
        t["copy_calibration"] = {"fetch_factor": ff, "write_factor": wf}
    if comp:
        t.setdefault("mfma_busy", {})[args.workload] = {k: round(v["mfma_busy"], 4) for k, v in comp.items()}
        t.setdefault("compute", {})[args.workload] = comp
    with open(tpath, "w") as f:
        json.dump(t, f, indent=1)
    print(open(path).read())


if __name__ == "__main__":
    main()
