"""The device-side token-offset check against the oracle's contract check.

Every kernel of an MLP call validates offs / counts on the device and, on a violation, writes
nothing and sets the workspace status word (torchtitan PR #2, section "Fail-loud contract": the
data-dependent counts are checked without a host synchronisation). Random valid layouts and
random single violations of the contract are run through grouped_mlp_fwd and grouped_mlp_bwd;
the status word after each must be MXF_DEV_BAD_OFFSETS exactly when oracle.mlp.check_offsets
rejects the layout, and a rejected call must leave every output untouched. Expert counts below
and above 64 cover both of the kernels' code paths (one lane per expert, and the looping check).
"""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu
from oracle.mlp import check_offsets

pytestmark = pytest.mark.gpu

SENT = 7.0
KINDS = ["valid", "valid_no_counts", "unaligned", "decreasing", "first_nonzero", "over_capacity", "count_over",
         "count_negative", "negative_offset", "real_row_in_empty"]


def _layout(rng, E, pad, mcap, kind):
    """A random layout for E experts within mcap rows, then one contract violation of `kind`."""
    nseg = mcap // pad - 1                                   # leave one spare segment of capacity
    lens = np.zeros(E, dtype=np.int64)
    for _ in range(int(rng.integers(0, nseg + 1))):
        lens[rng.integers(0, E)] += pad
    counts = np.array([int(rng.integers(0, L + 1)) if L else 0 for L in lens], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    nz = [e for e in range(E) if lens[e] > 0]
    e = int(rng.integers(1, E + 1))
    if kind == "unaligned":
        offs[e] += pad // 2
    elif kind == "decreasing" and nz:
        k = nz[int(rng.integers(0, len(nz)))]
        offs[k] = offs[k + 1] + pad                           # segment k now ends before it starts
    elif kind == "first_nonzero":
        offs[0] = pad
    elif kind == "over_capacity":
        offs[E] = mcap + pad
    elif kind == "count_over" and nz:
        k = nz[int(rng.integers(0, len(nz)))]
        counts[k] = lens[k] + 1
    elif kind == "count_negative":
        counts[int(rng.integers(0, E))] = -1
    elif kind == "negative_offset":
        offs[e] = -pad
    elif kind == "real_row_in_empty":
        z = [k for k in range(E) if lens[k] == 0]
        if z:
            counts[z[int(rng.integers(0, len(z)))]] = 1
    return offs.astype(np.int32), counts.astype(np.int32)


@pytest.mark.parametrize("E", [4, 63, 64, 72, 300, 1024])
def test_device_status_word_matches_oracle_check(E):
    mx = require_gpu()
    D, F, pad, mcap = 128, 128, 128, 1024
    rng = np.random.default_rng(1000 + E)
    ctx = mx.MlpContext(E, D, F, pad, mcap, flags=mx.OUT_F32)
    g = torch.Generator(device="cuda")
    g.manual_seed(E)
    x = torch.randn((mcap, D), generator=g, device="cuda").to(torch.bfloat16)
    dy = torch.randn((mcap, D), generator=g, device="cuda").to(torch.bfloat16)
    w1 = (0.02 * torch.randn((E, F, D), generator=g, device="cuda")).to(torch.bfloat16)
    w3 = (0.02 * torch.randn((E, F, D), generator=g, device="cuda")).to(torch.bfloat16)
    w2 = (0.02 * torch.randn((E, D, F), generator=g, device="cuda")).to(torch.bfloat16)
    seen = {True: 0, False: 0}
    for rep in range(2):
        for kind in KINDS:
            offs, counts = _layout(rng, E, pad, mcap, kind)
            use_counts = kind != "valid_no_counts"
            want_ok = check_offsets(offs, counts if use_counts else None, pad, mcap)
            seen[want_ok] += 1
            print(f"E={E} rep {rep} {kind}: offs[E]={int(offs[-1])} oracle valid={want_ok}", flush=True)
            offs_t = torch.from_numpy(offs).cuda()
            cnt_t = torch.from_numpy(counts).cuda() if use_counts else None
            y = torch.full((mcap, D), SENT, device="cuda")
            dx = torch.full((mcap, D), SENT, device="cuda")
            dw1 = torch.full((E, F, D), SENT, device="cuda")
            dw3 = torch.full((E, F, D), SENT, device="cuda")
            dw2 = torch.full((E, D, F), SENT, device="cuda")
            ctx.fwd(offs_t, cnt_t, x, w1, w3, w2, y)
            st_f = ctx.status()
            ctx.bwd(offs_t, cnt_t, dy, dx, dw1, dw3, dw2)
            st_b = ctx.status()
            want = mx.DEV_OK if want_ok else mx.DEV_BAD_OFFSETS
            assert st_f == want and st_b == want, (kind, offs.tolist(), counts.tolist(), st_f, st_b)
            if not want_ok:
                for t in (y, dx, dw1, dw3, dw2):
                    assert torch.all(t == SENT), kind
            else:
                assert not torch.any(dw1 == SENT)
    assert seen[True] >= 4 and seen[False] >= 10
