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


def test_dispatch_mutations_are_caught(monkeypatch):
    import test_oracle_dispatch as td
    from oracle import dispatch
    good_plan, good_perm = dispatch.route_plan, dispatch.permute

    def reversed_segments(ids, E, pad, cap):
        p = good_plan(ids, E, pad, cap)
        ra = p["row_assign"].copy()
        for e in range(E):
            a, c = int(p["offs"][e]), int(p["counts"][e])
            ra[a:a + c] = ra[a:a + c][::-1].copy()
        ar = p["assign_row"].copy()
        ar[ra[ra >= 0]] = np.nonzero(ra >= 0)[0]
        return dict(p, row_assign=ra, assign_row=ar)

    def always_one_more_block(ids, E, pad, cap):
        p = good_plan(ids, E, pad, cap)
        offs = np.concatenate([[0], np.cumsum(np.diff(p["offs"]) + np.where(p["counts"] % pad == 0, pad, 0))])
        return dict(p, offs=offs)

    for m in (reversed_segments, always_one_more_block):
        monkeypatch.setattr(dispatch, "route_plan", m)
        assert _fails(td.test_hand_worked_dispatch) or _fails(td.test_plan_invariants_and_stable_order, 1, 5000, 16, 256)
        assert _fails(td.test_tiny_workload_layout_is_the_dispatch_of_its_tokens) or m is always_one_more_block
    monkeypatch.setattr(dispatch, "route_plan", good_plan)

    def k_major(x, ra, k, m):          # assignments read as a = k * tokens + t (transposed routing)
        x = np.asarray(x)
        out = np.zeros((m, x.shape[1]), dtype=x.dtype)
        for r, a in enumerate(ra):
            if a >= 0:
                out[r] = x[a % x.shape[0]]
        return out

    monkeypatch.setattr(dispatch, "permute", k_major)
    assert _fails(td.test_tiny_workload_layout_is_the_dispatch_of_its_tokens)
    assert _fails(td.test_hand_worked_dispatch)


def test_e5m2_mutations_are_caught(monkeypatch):
    import test_oracle_e5m2 as te
    good = mx.e5m2_rne_sat

    def to_inf(y):                      # overflow to infinity instead of saturating
        c = good(y)
        big = np.abs(np.asarray(y, dtype=np.float64)) > 57344.0
        return np.where(big, (c & 0x80) | 0x7C, c).astype(np.uint8)

    monkeypatch.setattr(mx, "e5m2_rne_sat", to_inf)
    monkeypatch.setattr(te, "e5m2_rne_sat", to_inf)
    assert _fails(te.test_brute_force_all_bf16, 239) or _fails(te.test_saturation_beyond_top_binade)
    monkeypatch.undo()
    sb = mx.scale_byte
    monkeypatch.setattr(mx, "scale_byte", lambda a, emax=8: sb(a, 14 if emax == 15 else emax))   # E4M3-like emax slip
    assert _fails(te.test_closed_forms, 0)


def test_offsets_check_mutations_are_caught(monkeypatch):
    import test_oracle_offsets as to
    good = mlp.check_offsets
    muts = [
        lambda o, c, p, m: good([x - x % p for x in o], c, p, m),                 # alignment ignored
        lambda o, c, p, m: good(o, None, p, m),                                   # counts ignored
        lambda o, c, p, m: good(o, c, p, m + p),                                  # capacity off by a segment
        lambda o, c, p, m: good(sorted(o), c, p, m),                              # order ignored
    ]
    cases = [(2, 2, 6, range(-2, 9), range(-1, 6))]
    for mut in muts:
        monkeypatch.setattr(to, "check_offsets", mut)
        caught = any(_fails(to.test_hand_cases, *h) for h in to.HAND) or \
            any(_fails(to.test_accepts_exactly_the_constructed_layouts, *c) for c in cases)
        assert caught
    monkeypatch.undo()
