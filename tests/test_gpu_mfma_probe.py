"""Matrix-core ceiling kernels (mxf_mfma_probe) through the C ABI: with every operand code 0x38
(E4M3 1.0) and unit scales each 32x32x64 matrix instruction adds 64 to every accumulator, so
every thread's output (the sum of the first accumulator of its 16 fragments) is exactly
1024 * stages; a window of other codes gives the same, finite output on repeated launches."""
import pytest
import torch

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("nbytes,stages,blocks", [(131072, 2, 1), (1 << 21, 64, 37), (5 * 32768, 130, 300)])
def test_unit_codes_closed_form(mode, nbytes, stages, blocks):
    mx = require_gpu()
    src = torch.full((nbytes,), 0x38, dtype=torch.uint8, device="cuda")
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device="cuda")
    print(f"mfma probe mode {mode} bytes {nbytes} stages {stages} blocks {blocks}", flush=True)
    mx.mfma_probe(mode, src, nbytes, stages, blocks, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.full((blocks * 256,), 1024.0 * stages))


@pytest.mark.parametrize("mode", [0, 1])
def test_random_codes_deterministic(mode):
    mx = require_gpu()
    g = torch.Generator().manual_seed(5)
    # finite E4M3 codes of both signs with exponents up to 7 (|value| < 2): no overflow in 16 stages
    codes = torch.randint(0, 256, (1 << 20,), dtype=torch.uint8, generator=g) & 0xBF
    src = codes.cuda()
    outs = []
    for _ in range(2):
        out = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
        mx.mfma_probe(mode, src, 1 << 20, 16, 256, out)
        outs.append(out.cpu())
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1])
