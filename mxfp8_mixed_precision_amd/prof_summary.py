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
  --commands    text file holding the exact commands that produced the inputs

Outputs (in OUTDIR): <kernel-group>_<workload>.md summaries and traffic.json (HBM bytes
per launch, with the sha256 of the kernel sources they were measured on; bench.py only
reports them while the sources are unchanged).

Kernel dispatches are named by their position in a bench.py step: the MLP step enqueues, in
order, quant_w13, quant_x, quant_w2, fc1_swiglu, fc2, quant_dy, fc2_wgrad, fc2_dgrad_dswiglu,
fc1_wgrad, fc1_dgrad; a --quant-only run launches `quantize` (the dual quantizer) and then
`dequantize` (row-wise codes to BF16). Profile with
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

MLP_SEQUENCE = ["quant_w13", "quant_x", "quant_w2", "fc1_swiglu", "fc2", "quant_dy", "fc2_wgrad",
                "fc2_dgrad_dswiglu", "fc1_wgrad", "fc1_dgrad"]
# expected kernel template per logical name: (kernel family, SCHED/KIND, EPI/ROW,COL)
EXPECT = {
    "quant_w13": "quant_dual_kernel<2,", "quant_w2": "quant_dual_kernel<0,", "quant_x": "quant_dual_kernel<1,",
    "quant_dy": "quant_dual_kernel<1,", "fc1_swiglu": ", 0, 1>", "fc2": ", 0, 0>", "fc2_dgrad_dswiglu": ", 0, 2>",
    "fc2_wgrad": ", 1, 0>", "fc1_dgrad": ", 0, 0>", "fc1_wgrad": ", 1, 3>", "quantize": "quant_dual_kernel<0,true,true,0>",
    "dequantize": "dequant_kernel<true,0>",
}
QUANT_ONLY = ["quantize", "dequantize"]


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
    """sha256 over the kernel sources (file names and code without comments)."""
    h = hashlib.sha256()
    csrc = os.path.join(root, "mxfp8_mixed_precision_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, n), encoding="utf-8") as f:
            h.update(n.encode() + b"\0" + code_only(f.read()).encode())
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


def label(dispatches, quant_only):
    """Attach logical kernel names (see the module docstring). For an MLP run, every window of
    ten consecutive dispatches whose templates match the step sequence is one step; other
    dispatches (e.g. a trailing standalone-quantizer measurement) are left out."""
    out = []
    if quant_only:
        return [(did, k, r) for did, name, r in dispatches for k in QUANT_ONLY if _matches(name, k)]
    i, n = 0, len(MLP_SEQUENCE)
    while i + n <= len(dispatches):
        window = dispatches[i:i + n]
        if all(_matches(name, MLP_SEQUENCE[j]) for j, (_, name, _) in enumerate(window)):
            out += [(did, MLP_SEQUENCE[j], r) for j, (did, _, r) in enumerate(window)]
            i += n
        else:
            i += 1
    return out


def per_kernel_durations(trace_dir, quant_only):
    rows = list(csv.DictReader(open(_one(trace_dir, "*kernel_trace.csv"))))
    disp = label(mxf_dispatches(rows), quant_only)
    dur = defaultdict(list)
    for _, logical, r in disp:
        dur[logical].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return dur


def per_kernel_counter(pmc_dir, counter, quant_only):
    rows = [r for r in csv.DictReader(open(_one(pmc_dir, "*counter_collection.csv"))) if r["Counter_Name"] == counter]
    disp = label(mxf_dispatches(rows), quant_only)
    vals = defaultdict(list)
    for _, logical, r in disp:
        vals[logical].append(float(r["Counter_Value"]))
    return vals


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
    ap.add_argument("--quant-only", action="store_true")
    ap.add_argument("--commands", required=True)
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    os.makedirs(args.out, exist_ok=True)
    dur = per_kernel_durations(args.trace, args.quant_only)
    traffic = {}
    lines = []
    ff = wf = None
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        ff, fraw = copy_factor(args.copy_fetch, "FETCH_SIZE")
        wf, wraw = copy_factor(args.copy_write, "WRITE_SIZE")
        fetch = per_kernel_counter(args.fetch, "FETCH_SIZE", args.quant_only)
        write = per_kernel_counter(args.write, "WRITE_SIZE", args.quant_only)
        for k in dur:
            if k in fetch and k in write:
                fb = sum(fetch[k]) / len(fetch[k]) * ff
                wb = sum(write[k]) / len(write[k]) * wf
                traffic[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes": round(fb + wb)}
        lines.append(f"Counter calibration (1 GiB device copy): FETCH_SIZE reads {fraw:.0f} -> x{ff:.4f} bytes per unit; "
                     f"WRITE_SIZE reads {wraw:.0f} -> x{wf:.4f} bytes per unit.")
        lines.append("")
    cmds = open(args.commands).read().strip()
    name = "quantize" if args.quant_only else "mlp_fwd_bwd"
    md = [f"# {name} kernels, workload `{args.workload}` (rocprofv3)", "", "Commands (run from the repository root):",
          "", "```", cmds, "```", ""] + lines
    md.append("| kernel | launches | avg us | median us | min us | max us | HBM read MB/launch | HBM write MB/launch |")
    md.append("|---|---|---|---|---|---|---|---|")
    order = QUANT_ONLY if args.quant_only else MLP_SEQUENCE
    for k in order:
        if k not in dur:
            continue
        v = dur[k]
        t = traffic.get(k)
        rd = f"{t['fetch_bytes'] / 1e6:.1f}" if t else "-"
        wr = f"{t['write_bytes'] / 1e6:.1f}" if t else "-"
        med = sorted(v)[len(v) // 2]
        md.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {med:.2f} | {min(v):.2f} | {max(v):.2f} | {rd} | {wr} |")
    md.append("")
    path = os.path.join(args.out, f"{name}_{args.workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(md) + "\n")
    tpath = os.path.join(args.out, "traffic.json")
    t = {"kernels": {}}
    if os.path.exists(tpath):
        t = json.load(open(tpath))
    t["source_sha256"] = source_sha256(root)
    t.setdefault("kernels", {})[args.workload] = {k: v["bytes"] for k, v in traffic.items()}
    t.setdefault("detail", {})[args.workload] = traffic
    if ff:
        t["copy_calibration"] = {"fetch_factor": ff, "write_factor": wf}
    with open(tpath, "w") as f:
        json.dump(t, f, indent=1)
    print(open(path).read())


if __name__ == "__main__":
    main()
