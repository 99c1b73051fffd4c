"""bench.py end to end on the tiny workload (a few steps): one JSON line with the fields the
benchmark contract names, a positive throughput consistent with its step time, and the roofline
and per-kernel objects."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_tiny_json_line():
    require_gpu()
    print("bench.py --workload tiny", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
                        "--warmup", "2", "--no-cpu-baseline", "--no-quant", "--no-plans"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "kernels"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["unit"] == "TFLOP/s" and d["value"] > 0
    cfg = d["config"]
    assert cfg["workload"].startswith("tiny") and cfg["E"] == 4 and cfg["m_real"] == 1024
    # value is the useful FLOPs (18 M_real D F) over the step time
    useful = 18.0 * cfg["m_real"] * cfg["D"] * cfg["F"]
    assert d["value"] == pytest.approx(useful / (d["ms_per_step"] / 1e3) / 1e12, rel=5e-3, abs=0.01)
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-3, abs=6e-5)  # 4 decimals
    assert set(d["kernels"]) >= {"quant_fwd", "fc1_swiglu", "fc2", "quant_dy", "fc2_dgrad_dswiglu"}
