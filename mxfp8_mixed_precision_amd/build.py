"""Build the gfx950 HIP library ``libmxfp8.so`` in-tree with hipcc.

Usage: ``python -m mxfp8_mixed_precision_amd.build`` (or ``build()`` from Python).
Each source is compiled to an object in ``_build/`` in parallel, then linked into
``mxfp8_mixed_precision_amd/libmxfp8.so``.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp8.so")
SOURCES = ["abi.hip", "quantize.hip", "gemm.hip", "dispatch.hip", "hbm.hip", "mfma_probe.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 vector ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source flags. gemm.hip: the machine scheduler's max-ILP strategy (measured on the DSv3
# rank step, four A/B pairs: FC2 dgrad + dSwiGLU 127.7-128.0 against 129.3-129.7 us, FC1 + SwiGLU
# about 1 us faster, the step about 4 us; applied to every source it made the quantizers 2-3 us
# slower, so it stays on the GEMM source).
SOURCE_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmxfp8.so")
    return path


def _compile(src, obj, extra):
    cmd = [_hipcc()] + HIPCC_FLAGS + SOURCE_FLAGS.get(src, []) + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(verbose=False, extra_flags=()):
    """Compile every HIP source for gfx950 and link libmxfp8.so. Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        futs = [ex.submit(_compile, s, o, list(extra_flags)) for s, o in zip(SOURCES, objs)]
        for f in futs:
            msg = f.result()
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
