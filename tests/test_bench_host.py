"""Host-side logic of bench.py (no GPU): the per-launch algorithmic work it divides by the
measured times, checked against the totals the workload fixes, and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_gemm_flops_sum_to_the_step():
    """The six GEMMs of a step (FC1, FC2, FC2 dgrad, and the merged FC2 wgrad + FC1 dgrad + FC1
    wgrad) add up to 18 M_real D F; on the DSv3 rank workload that is 1.2756 TFLOP."""
    counts = workloads.expert_counts("dsv3_rank")
    m_real, D, F = sum(counts), 2048, 1408
    names = ["fc1_swiglu", "fc2", "fc2_dgrad_dswiglu", "bwd_gemms"]
    total = sum(bench.gemm_flops(n, m_real, D, F) for n in names)
    assert total == 18 * m_real * D * F
    assert abs(total / 1e12 - 1.2756) < 5e-4
    separate = sum(bench.gemm_flops(n, m_real, D, F) for n in ("fc2_wgrad", "fc1_dgrad", "fc1_wgrad"))
    assert separate == bench.gemm_flops("bwd_gemms", m_real, D, F)
    assert bench.gemm_flops("quant_fwd", m_real, D, F) is None


def test_quant_bytes():
    """Dual quantization moves 2 B in and 2 + 2/32 B out per element: the standalone workload
    [16384, 7168] is 477.1 MB; the dY quantizer reads the real rows and writes every padded row."""
    rows, cols = workloads.QUANT_CONFIG["rows"], workloads.QUANT_CONFIG["cols"]
    assert abs(rows * cols * (2 + 2 + 2.0 / 32) / 1e6 - 477.1) < 0.05
    m_pad, m_real, E, D, F = 26112, 24576, 16, 2048, 1408
    dy = bench.quant_bytes("quant_dy", m_pad, m_real, E, D, F)
    assert dy == m_real * D * 2 + m_pad * D * (2 + 2.0 / 32)
    fwd = bench.quant_bytes("quant_fwd", m_pad, m_real, E, D, F)
    weights = (E * 2 * F * D + E * D * F) * (2 + 2 + 2.0 / 32)
    assert fwd == pytest.approx(weights + dy)
    assert bench.quant_bytes("fc2", m_pad, m_real, E, D, F) is None


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
