"""Resource checks on the compiled gfx950 kernels (host only: hipcc cross-compiles here).

Every kernel of the library must run without scratch memory: a register spill turns into
per-lane private-segment traffic through HBM (a spilled accumulator fragment in the GEMM store
epilogue once added 16 KB of scratch writes per tile). Each kernel's LDS must also fit the
CU's 160 KB. The sources are compiled to AMDGPU assembly with the library's own flags (per source) and the
code-object metadata is read back.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from mxfp8_mixed_precision_amd import build

SOURCES = ["gemm.hip", "quantize.hip", "dispatch.hip", "hbm.hip", "mfma_probe.hip"]
LDS_LIMIT = 160 * 1024


def _kernel_metadata(src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc] + build.HIPCC_FLAGS + build.SOURCE_FLAGS.get(src, []) + ["-I", build.CSRC, "--cuda-device-only", "-S",
                                             os.path.join(build.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    kernels = []
    for block in re.split(r"\n\s+- \.", text.split("amdhsa.kernels:", 1)[1])[1:]:
        fields = dict(re.findall(r"\.?([a-z_]+):\s+(\S+)", block))
        if "name" in fields:
            kernels.append(fields)
    assert kernels, f"no kernel metadata in {src}"
    return kernels


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch_and_lds_fits(src):
    for k in _kernel_metadata(src):
        name = k["name"]
        assert int(k.get("private_segment_fixed_size", 0)) == 0, (name, "uses scratch")
        assert int(k.get("vgpr_spill_count", 0)) == 0, (name, "spills VGPRs")
        assert int(k.get("group_segment_fixed_size", 0)) <= LDS_LIMIT, (name, "LDS over 160 KB")
