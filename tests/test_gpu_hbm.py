"""HBM ceiling kernels (mxf_hbm_probe) through the C ABI: each mode computes exactly what the
header documents, on sizes that are not a multiple of the launch's per-iteration span (ragged
last grid-stride round) and on a single 16-byte word."""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

SIZES = [16, 4096 + 48, (1 << 22) + 16 * 37]


@pytest.mark.parametrize("nbytes", SIZES)
def test_read_xor(nbytes):
    mx = require_gpu()
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    src = host.cuda()
    dst = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    mx.hbm_probe(mx.HBM_READ, src, dst, nbytes)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32).reshape(-1, 4), axis=0)
    got = np.bitwise_xor.reduce(dst.cpu().numpy().view(np.uint32).reshape(64, 4), axis=0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nbytes", SIZES)
def test_write_pattern(nbytes):
    mx = require_gpu()
    dst = torch.full((nbytes + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    mx.hbm_probe(mx.HBM_WRITE, None, dst, nbytes)
    got = dst.cpu().numpy()
    words = got[:nbytes].view(np.uint32).reshape(-1, 4)
    idx = np.arange(nbytes // 16, dtype=np.uint32)
    assert np.array_equal(words, np.repeat(idx[:, None], 4, axis=1))
    assert (got[nbytes:] == 0xAB).all()  # nothing past the end


@pytest.mark.parametrize("nbytes", SIZES)
def test_copy(nbytes):
    mx = require_gpu()
    g = torch.Generator().manual_seed(nbytes + 1)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full((nbytes + 64,), 0xCD, dtype=torch.uint8, device="cuda")
    mx.hbm_probe(mx.HBM_COPY, src, dst, nbytes)
    assert torch.equal(dst[:nbytes], src)
    assert (dst[nbytes:] == 0xCD).all()
