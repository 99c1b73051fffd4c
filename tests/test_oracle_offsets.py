"""Pins for the oracle's token-offset contract check, oracle.mlp.check_offsets (CPU only).

The contract (torchtitan PR #12, section "What it adds": every expert's segment of the padded
expert-major layout is hard-aligned to pad_multiple) is pinned two ways that do not restate
the function's own tests:

* hand cases, each one statement of the contract with its expected answer;
* a constructive enumeration: every layout that can be built from segment lengths that are
  non-negative multiples of pad_multiple, laid end to end from row 0 within the capacity, with
  real-row counts in [0, length], is generated, and the check must accept exactly those among
  all offset/count vectors of a small range (negative values included).
"""
import itertools

import pytest

from oracle.mlp import check_offsets

HAND = [
    # (offs, counts, pad, capacity, valid, what)
    ([0, 128, 256], [100, 128], 128, 256, True, "aligned, counts within segments, exactly at capacity"),
    ([0, 128, 256], None, 128, 512, True, "counts omitted: every row real"),
    ([0, 0, 0], [0, 0], 128, 0, True, "no routed token at all"),
    ([0, 128, 128, 256], [5, 0, 128], 128, 256, True, "zero-token expert between two others"),
    ([0, 0, 256], [0, 200], 256, 256, True, "zero-token expert first"),
    ([0], None, 128, 0, True, "degenerate: no expert rows"),
    ([128, 256], [1], 128, 256, False, "first offset not 0"),
    ([0, 256, 128], [1, 0], 128, 256, False, "decreasing offsets"),
    ([0, 64, 256], [10, 10], 128, 256, False, "offset not a multiple of pad_multiple"),
    ([0, 128, 256], [10, 10], 256, 256, False, "multiple of 128 but pad_multiple is 256"),
    ([0, 128, 384], [10, 10], 128, 256, False, "layout exceeds capacity"),
    ([0, 128, 256], [129, 100], 128, 256, False, "more real rows than the segment holds"),
    ([0, 128, 256], [-1, 100], 128, 256, False, "negative count"),
    ([0, -128], None, 128, 256, False, "negative offset"),
    ([0, 0, 128], [1, 0], 128, 128, False, "real row in an empty segment"),
]


@pytest.mark.parametrize("offs,counts,pad,cap,valid,what", HAND, ids=[h[5] for h in HAND])
def test_hand_cases(offs, counts, pad, cap, valid, what):
    assert check_offsets(offs, counts, pad, cap) == valid, what


def _constructed(E, pad, cap, cmax):
    """Every (offs, counts) a dispatcher can produce: segments of pad-multiple lengths laid end
    to end from row 0 within cap, each holding 0..length real rows (counts capped at cmax to
    keep the enumeration small), plus the same offsets with counts omitted."""
    out = set()
    lengths = range(0, cap + 1, pad)
    for L in itertools.product(lengths, repeat=E):
        if sum(L) > cap:
            continue
        offs = [0]
        for x in L:
            offs.append(offs[-1] + x)
        out.add((tuple(offs), None))
        for c in itertools.product(*[range(0, min(x, cmax) + 1) for x in L]):
            out.add((tuple(offs), tuple(c)))
    return out


@pytest.mark.parametrize("E,pad,cap,orange,crange", [
    (2, 2, 6, range(-2, 9), range(-1, 6)),
    (3, 1, 3, range(-1, 5), range(-1, 3)),
])
def test_accepts_exactly_the_constructed_layouts(E, pad, cap, orange, crange):
    valid = _constructed(E, pad, cap, max(crange))
    seen = 0
    for offs in itertools.product(orange, repeat=E + 1):
        for counts in [None] + list(itertools.product(crange, repeat=E)):
            want = (offs, counts) in valid
            got = check_offsets(list(offs), None if counts is None else list(counts), pad, cap)
            assert got == want, (offs, counts, pad, cap)
            seen += want
    # every constructed layout lies inside the enumerated range
    assert seen == len(valid)
