"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle (via monkeypatch, on the CPU) and
checks that at least one of the pinning tests then fails.
"""
import numpy as np
import pytest

import test_oracle_mlp as tm
import test_oracle_quant as tq
from oracle import mlp, mx


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_dswiglu_mutations_are_caught(monkeypatch):
    sig = mlp.sigmoid
    muts = [
        lambda dh, g, u: (dh * u * sig(g) * (1 - g * (1 - sig(g))), dh * g * sig(g)),   # sign
        lambda dh, g, u: (dh * u * sig(g), dh * g * sig(g)),                           # dropped term
        lambda dh, g, u: (dh * g * sig(g), dh * u * sig(g) * (1 + g * (1 - sig(g)))),  # swapped outputs
    ]
    for m in muts:
        monkeypatch.setattr(mlp, "dswiglu", m)
        assert _fails(tm.test_exact_backward_matches_finite_differences)


def test_layout_mutations_are_caught(monkeypatch):
    split = mlp.split_gu
    monkeypatch.setattr(mlp, "split_gu", lambda h: split(h)[::-1])
    assert _fails(tm.test_exact_backward_matches_finite_differences)
    monkeypatch.undo()
    monkeypatch.setattr(mlp, "pack_w13", lambda a, b: np.concatenate([a, b], axis=1))
    assert _fails(tm.test_pack_layout_and_round_trip)


def test_scale_rule_mutations_are_caught(monkeypatch):
    good = mx.scale_byte
    monkeypatch.setattr(mx, "scale_byte", lambda a: np.minimum(good(a).astype(int) + 1, 254).astype(np.uint8))
    assert _fails(tq.test_power_of_two_amax, 0)
    monkeypatch.setattr(mx, "scale_byte", lambda a: np.where(np.asarray(a) == 0, 127, good(a)).astype(np.uint8))
    assert _fails(tq.test_all_zero_block)


def test_rounding_mutations_are_caught(monkeypatch):
    vals = mx._POS_VALUES

    def half_up(y):
        a = np.minimum(np.abs(y), 448.0)
        idx = np.searchsorted(vals, a, side="right") - 1
        idx = np.clip(idx, 0, len(vals) - 1)
        nxt = np.clip(idx + 1, 0, len(vals) - 1)
        up = (vals[nxt] - a) <= (a - vals[idx])
        c = np.where(up, nxt, idx).astype(np.uint8)
        return np.where(np.signbit(y), c | 0x80, c).astype(np.uint8)

    monkeypatch.setattr(mx, "e4m3_rne_sat", half_up)
    monkeypatch.setattr(tq, "e4m3_rne_sat", half_up)
    assert _fails(tq.test_subnormal_codes, 0)
    assert _fails(tq.test_brute_force_all_bf16_against_bit_level_rne, 127)

    monkeypatch.undo()
    good = tq.e4m3_rne_sat

    def no_sat(y):
        c = good(y)
        return np.where(np.abs(y) > 464, c | 0x7F, c).astype(np.uint8)

    monkeypatch.setattr(tq, "e4m3_rne_sat", no_sat)
    assert _fails(tq.test_brute_force_all_bf16_against_torch_cast, 127)
