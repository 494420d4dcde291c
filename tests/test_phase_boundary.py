"""kap_choose_plan (the library's full-context fallback decision) against the
cost-model oracle (oracle/costmodel.py: the KAP tutorial's phase-boundary
equations) and the KAP paper's Table 5 break-even points.  Host-only: no GPU."""
import math
import os

import numpy as np
import pytest

import block_sparse_paged_page_amd as kap
from oracle import costmodel as cm

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
OK, INVALID = 0, 1


def _table5():
    rows = []
    for line in open(os.path.join(GOLDEN, "table5_phase.txt")):
        if line.startswith("#") or not line.strip():
            continue
        ctx, s, margin, h, be = line.split()
        rows.append((ctx, float(s), float(margin), float(h), float(be)))
    return rows


def test_choice_and_speedup_match_the_cost_model_on_a_grid():
    rng = np.random.default_rng(7)
    seen = set()
    for _ in range(4000):
        h = float(rng.choice([rng.random(), 0.0, 1.0, 0.952, 0.958]))
        s = float(rng.choice([rng.random(), 0.0, 1.0, h, 0.055, 0.401]))
        kv = float(rng.choice([rng.random() * 1e9, 0.0, 2.0 ** 31]))
        w = float(rng.choice([rng.random() * 1e10, 0.0, 6.4e10]))
        k = int(rng.integers(1, 9))
        cap = int(rng.integers(0, 600))
        budget = int(rng.integers(0, 600))
        choice, sp = kap.choose_plan(h, s, w, kv, k, budget, cap)
        if budget > cap:
            want = kap.PLAN_FULL_CAPACITY
        elif not h > s:
            want = kap.PLAN_FULL_MARGIN
        elif not cm.phase_boundary_holds(h, s, w, kv):
            want = kap.PLAN_FULL_BOUNDARY
        else:
            want = kap.PLAN_SELECTED
        assert choice == want, (h, s, w, kv, k, budget, cap, choice)
        seen.add(choice)
        base, plan = cm.cost_base(k, h, w, kv), cm.cost_plan(k, s, w, w, kv)
        ref = base / plan if plan > 0 else 1.0
        assert sp == pytest.approx(ref, rel=1e-12, abs=1e-300)
        if want == kap.PLAN_SELECTED:
            assert sp > 1.0          # the boundary is exactly Cost_plan < Cost_base
    assert seen == {0, 1, 2, 3}


@pytest.mark.parametrize("row", _table5(), ids=lambda r: r[0])
def test_table5_break_even(row):
    """At the pages' h and s, the plan is kept just below the break-even
    W_main / KV = (h - s) / (1 - h) and dropped just above it."""
    ctx, s, margin, h, be = row
    assert cm.break_even_w_over_kv(h, s) == pytest.approx(be, rel=1e-12)
    kv = 1.0e9
    for k in (1, 4, 6):
        c_lo, sp_lo = kap.choose_plan(h, s, be * kv * (1 - 1e-6), kv, k, 451, 451)
        c_hi, sp_hi = kap.choose_plan(h, s, be * kv * (1 + 1e-6), kv, k, 451, 451)
        assert c_lo == kap.PLAN_SELECTED and sp_lo > 1.0
        assert c_hi == kap.PLAN_FULL_BOUNDARY and sp_hi < 1.0
    # the 128K selection of the benchmark (451 pages) overflowing a smaller compact view
    assert kap.choose_plan(h, s, 0.0, kv, 4, 451, 450)[0] == kap.PLAN_FULL_CAPACITY


def test_closed_forms():
    # s = 1: every proposal reads the full KV, so the plan can never pay off
    assert kap.choose_plan(0.99, 1.0, 1.0, 1.0, 4, 1, 1)[0] == kap.PLAN_FULL_MARGIN
    # h = 1 (every draft accepted): any s < 1 pays off, and the speedup is
    # (1 + k)(W + KV) / (k (W + s KV) + W + KV)
    c, sp = kap.choose_plan(1.0, 0.055, 8e9, 2e9, 4, 451, 451)
    assert c == kap.PLAN_SELECTED
    assert sp == pytest.approx(5 * 10e9 / (4 * (8e9 + 0.055 * 2e9) + 10e9), rel=1e-12)
    # no KV and no weights: nothing to save, speedup 1 by convention
    assert kap.choose_plan(0.5, 0.1, 0.0, 0.0, 4, 1, 1) == (kap.PLAN_FULL_BOUNDARY, 1.0)


def test_rejects_out_of_range_inputs():
    lib = kap.load()
    import ctypes
    ch = ctypes.c_int32()
    bad = [(-0.1, 0.1, 1, 1, 1, 1, 1), (1.1, 0.1, 1, 1, 1, 1, 1), (0.5, math.nan, 1, 1, 1, 1, 1),
           (0.5, 0.1, -1.0, 1, 1, 1, 1), (0.5, 0.1, 1, math.inf, 1, 1, 1), (0.5, 0.1, 1, 1, 0, 1, 1),
           (0.5, 0.1, 1, 1, 1, -1, 1), (0.5, 0.1, 1, 1, 1, 1, -1)]
    for a in bad:
        assert lib.kap_choose_plan(*a, ctypes.byref(ch), None) == INVALID, a
    assert lib.kap_choose_plan(0.5, 0.1, 1.0, 1.0, 1, 1, 1, None, None) == INVALID
