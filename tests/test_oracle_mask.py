"""Pins for the oracle mask (CPU only).

The pages print no worked mask, so the oracle is pinned by:

* the invariants the pages state (anchor count constant across steps; every
  frame an anchor once per Tper steps, a few twice when Tper does not divide
  T; |A(t)| at the budget; C ≥ T is dense) -- [gist] Technical Summary §2
  "Core Mechanism", TechWalker §二/§三;
* an independent, sort-based definition of the expanded window (the C − n_g
  non-anchor frames nearest to t, ties to the lower index), written here and
  not in the oracle;
* examples worked by hand from the readings, written out below;
* mutation tests: plausible mistakes planted in the oracle (on the CPU) must
  make at least one pin fail.
"""

import math

import pytest

import oracle.mask as om

# ---------------------------------------------------------------- helpers --


def indep_anchor_count(T, C, W):
    """n_g from the readings, restated: Tper = ⌈T/(C−W)⌉, n_g = ⌈T/Tper⌉."""
    t_per = math.ceil(T / (C - W))
    return t_per, math.ceil(T / t_per)


def indep_rows(T, C, W, anchors):
    """Sort-based definition of A(t) given the anchor set (independent of the
    oracle's walk): G ∪ first (C − |G|) of the non-anchors sorted by
    (|f − t|, f)."""
    if T <= C:
        return [list(range(T)) for _ in range(T)]
    g = set(anchors)
    rows = []
    for t in range(T):
        non = sorted((f for f in range(T) if f not in g), key=lambda f: (abs(f - t), f))
        rows.append(sorted(g.union(non[:C - len(g)])))
    return rows


def pin_failures(T, C, W, flags, steps):
    """Run every pin on (T, C, W, flags) over ``steps``; return a list of failures."""
    fails = []
    ceff = min(C, T)
    prev_count = None
    hits = {}
    for s in steps:
        g = om.anchors(T, C, W, s, flags)
        rows = om.key_frames(T, C, W, s, flags)
        if T <= C:
            if rows != [list(range(T))] * T:  # I4
                fails.append(("I4 dense", s))
            continue
        t_per, n_g = indep_anchor_count(T, C, W)
        if len(g) != n_g:  # I1 (count from the readings)
            fails.append(("I1 count", s, len(g), n_g))
        if prev_count is not None and len(g) != prev_count:  # I1 constant
            fails.append(("I1 constant", s))
        prev_count = len(g)
        if C - len(g) < W:  # R1: the window never shrinks below W
            fails.append(("window below W", s))
        for t, r in enumerate(rows):
            if len(r) != ceff:  # I3
                fails.append(("I3 size", s, t, len(r)))
            if r != sorted(set(r)):
                fails.append(("sorted unique", s, t))
            if any(f < 0 or f >= T for f in r):
                fails.append(("range", s, t))
            if t not in r:  # I5
                fails.append(("I5 self", s, t))
            if not set(g) <= set(r):  # I6
                fails.append(("I6 anchors", s, t))
        if rows != indep_rows(T, C, W, g):  # I7
            fails.append(("I7 sort-based window", s))
        for f in g:
            hits.setdefault(s, []).append(f)
    if T > C:
        t_per, n_g = indep_anchor_count(T, C, W)
        # I2: over any Tper consecutive steps each frame is an anchor once or
        # twice, and exactly n_g·Tper − T frames twice.  Not for the
        # fixed-grid ablation, which does not rotate.
        if flags != om.FIXED_GRID:
            ss = sorted(hits)
            for i in range(len(ss) - t_per + 1):
                win = ss[i:i + t_per]
                if win[-1] - win[0] != t_per - 1:
                    continue
                cnt = [0] * T
                for s in win:
                    for f in hits[s]:
                        cnt[f] += 1
                if min(cnt) < 1 or max(cnt) > 2 or cnt.count(2) != n_g * t_per - T:
                    fails.append(("I2 coverage", win[0]))
                    break
        for s in steps:
            g0 = om.anchors(T, C, W, s, flags)
            if flags == om.ROT_MOD_TPER and om.anchors(T, C, W, s + t_per, flags) != g0:
                fails.append(("I8 period", s))
            if flags == om.ROT_MOD_T:
                g1 = om.anchors(T, C, W, s + 1, flags)
                if g1 != sorted((f + 1) % T for f in g0):
                    fails.append(("I9 shift", s))
            if flags == om.ROT_MOD_TPER and T % t_per == 0 and s % t_per != t_per - 1:
                g1 = om.anchors(T, C, W, s + 1, flags)
                if g1 != sorted((f + 1) % T for f in g0):
                    fails.append(("I9 shift (Tper | T)", s))
            if flags == om.FIXED_GRID and g0 != om.anchors(T, C, W, 0, flags):
                fails.append(("fixed grid moves", s))
    return fails


# Hand-worked examples (readings R1–R5 applied by hand; not printed by the
# pages).  Tiny: T=8, C=4, W=2 → Tper = ⌈8/2⌉ = 4, n_g = 2, window budget 2.
TINY_ANCHORS = {0: [0, 4], 1: [1, 5], 2: [2, 6], 3: [3, 7], 4: [0, 4]}
TINY_ROWS_S0 = [
    [0, 1, 2, 4],  # t=0: walk 0,(−1),1 → {0,1}; 0 is an anchor so 1, 2
    [0, 1, 2, 4],  # t=1: 1, 0 is an anchor, 2
    [0, 1, 2, 4],  # t=2: 2, 1
    [0, 2, 3, 4],  # t=3: 3, 2
    [0, 3, 4, 5],  # t=4: 4 is an anchor; 3, 5
    [0, 4, 5, 6],  # t=5: 5, 4 is an anchor, 6
    [0, 4, 5, 6],  # t=6: 6, 5
    [0, 4, 6, 7],  # t=7: 7, 6
]
# Wan-1.3B 6× shape: T=121, C=21, W=9 → Tper = ⌈121/12⌉ = 11, n_g = 11,
# G_0 = {0, 11, ..., 110}, window budget 10.
C3_G0 = list(range(0, 121, 11))


def c3_rows_expected():
    g = set(C3_G0)
    return {
        0: sorted(g | set(range(0, 12))),           # 1..10 plus 12 (11 is an anchor)
        60: sorted(g | set(range(56, 66))),          # 60,59,61,...,56,64; 55 anchor → 65
        120: sorted(g | set(range(111, 121))),       # slides inward from the end
    }


# ------------------------------------------------------------------ tests --


def test_validate_rejects_bad_arguments():
    for args in [(0, 4, 2, 0), (8, 1, 1, 0), (8, 4, 0, 0), (8, 4, 4, 0), (8, 4, 2, -1)]:
        with pytest.raises(om.OracleArgError):
            om.build_mask(*args)
    with pytest.raises(om.OracleArgError):
        om.build_mask(8, 4, 2, 0, flags=7)


def test_tiny_hand_example():
    for s, g in TINY_ANCHORS.items():
        assert om.anchors(8, 4, 2, s) == g
    assert om.key_frames(8, 4, 2, 0) == TINY_ROWS_S0
    rows3 = om.key_frames(8, 4, 2, 3)
    assert rows3[0] == [0, 1, 3, 7]
    assert rows3[7] == [3, 5, 6, 7]


def test_wan_6x_hand_example():
    assert om.anchors(121, 21, 9, 0) == C3_G0
    rows = om.key_frames(121, 21, 9, 0)
    for t, r in c3_rows_expected().items():
        assert rows[t] == r, t
    rp, ci, info = om.build_mask(121, 21, 9, 0)
    assert info.c_eff == 21 and info.t_per == 11 and info.n_anchor == 11 and info.nnz == 121 * 21
    assert rp == [21 * t for t in range(122)]


def test_workload_schedules():
    # Tper and n_g at the workload shapes (restated from the readings).
    assert om.schedule(8, 4, 2) == (4, 2)
    assert om.schedule(121, 21, 9) == (11, 11)
    assert om.schedule(49, 33, 13) == (3, 17)
    assert om.schedule(65, 33, 13) == (4, 17)
    rp, ci, info = om.build_mask(21, 21, 9, 5)
    assert info.c_eff == 21 and info.t_per == 0 and info.n_anchor == 0
    assert ci == list(range(21)) * 21


def test_rotations_differ_only_when_tper_does_not_divide_t():
    for T, C, W in [(8, 4, 2), (121, 21, 9)]:
        for s in range(50):
            assert om.anchors(T, C, W, s, om.ROT_MOD_TPER) == om.anchors(T, C, W, s, om.ROT_MOD_T)
    diff = sum(om.anchors(49, 33, 13, s, om.ROT_MOD_TPER) != om.anchors(49, 33, 13, s, om.ROT_MOD_T)
               for s in range(50))
    assert diff > 0


@pytest.mark.parametrize("flags", [om.ROT_MOD_TPER, om.ROT_MOD_T, om.FIXED_GRID])
def test_invariants_at_workload_shapes(flags):
    for T, C, W in [(8, 4, 2), (21, 21, 9), (121, 21, 9), (49, 33, 13), (65, 33, 13)]:
        assert pin_failures(T, C, W, flags, range(50)) == [], (T, C, W)


@pytest.mark.parametrize("flags", [om.ROT_MOD_TPER, om.ROT_MOD_T])
def test_invariants_sweep(flags):
    cases = []
    for T in list(range(1, 40)) + [63, 64, 65, 97, 128, 150]:
        for C in ((2, 3, 5, 8, 13, 21, 33) if T < 40 else (8, 13, 21, 33)):
            for W in sorted({1, C // 2, C - 1}):
                if 1 <= W <= C - 1:
                    cases.append((T, C, W))
    for T, C, W in cases:
        t_per = math.ceil(T / (C - W)) if T > C else 1
        # one full period plus a wrap for long periods, two for short ones
        steps = range(0, (2 * t_per + 3) if t_per <= 16 else (t_per + 2))
        assert pin_failures(T, C, W, flags, steps) == [], (T, C, W)


def test_invariants_large_sequence():
    # Long horizon well beyond the workloads (a 600-frame sequence).
    assert pin_failures(600, 64, 20, om.ROT_MOD_TPER, range(0, 16)) == []


# ------------------------------------------------------ mutation tests --


def _all_pins(monkeypatch_ctx=None):
    """Every mask pin; returns True when all pass."""
    try:
        test_tiny_hand_example()
        test_wan_6x_hand_example()
    except AssertionError:
        return False
    for T, C, W in [(8, 4, 2), (121, 21, 9), (49, 33, 13), (65, 33, 13), (37, 8, 3), (29, 13, 6)]:
        for flags in (om.ROT_MOD_TPER, om.ROT_MOD_T):
            try:
                if pin_failures(T, C, W, flags, range(12)):
                    return False
            except AssertionError:
                return False
    return True


def test_pins_pass_on_unmodified_oracle():
    assert _all_pins()


def test_mutation_off_by_one_anchor_offset(monkeypatch):
    orig = om.anchor_offset
    monkeypatch.setattr(om, "anchor_offset", lambda T, tp, s, f: orig(T, tp, s, f) + 1)
    assert not _all_pins()


def test_mutation_reversed_rotation(monkeypatch):
    monkeypatch.setattr(om, "anchor_offset", lambda T, tp, s, f: (-s) % tp)
    assert not _all_pins()


def test_mutation_floor_rounding_of_tper(monkeypatch):
    def sched(T, C, W):
        t_per = max(1, T // (C - W))
        return t_per, -(-T // t_per)
    monkeypatch.setattr(om, "schedule", sched)
    assert not _all_pins()


def test_mutation_ties_to_higher_index(monkeypatch):
    def window(T, t, budget, gs):
        taken, dist = [], 0
        while len(taken) < budget:
            for f in ([t] if dist == 0 else [t + dist, t - dist]):
                if 0 <= f < T and f not in gs and len(taken) < budget:
                    taken.append(f)
            dist += 1
        return taken
    monkeypatch.setattr(om, "_window", window)
    assert not _all_pins()


def test_mutation_window_not_extended(monkeypatch):
    # Window of fixed extent around t; anchors inside it are not compensated.
    def window(T, t, budget, gs):
        near = sorted(range(T), key=lambda f: (abs(f - t), f))[:budget]
        return [f for f in near if f not in gs]
    monkeypatch.setattr(om, "_window", window)
    assert not _all_pins()


def test_mutation_anchor_positions_not_wrapped(monkeypatch):
    orig_anchors = om.anchors

    def anchors(T, C, W, step, flags=om.ROT_MOD_TPER):
        return [f for f in orig_anchors(T, C, W, step, flags) if f >= (step % max(1, om.schedule(T, C, W)[0]) if T > C else 0)]
    monkeypatch.setattr(om, "anchors", anchors)
    assert not _all_pins()


def window_only_closed_form(T, C, t):
    """Sliding window of min(C, T) frames centred on t (lower side first on
    ties), slid inward at the sequence ends."""
    n = min(C, T)
    lo = t - (n // 2)
    hi = lo + n - 1
    if lo < 0:
        lo, hi = 0, n - 1
    if hi > T - 1:
        lo, hi = T - n, T - 1
    return list(range(lo, hi + 1))


def test_window_only_ablation_is_a_sliding_window():
    for T in (1, 2, 5, 8, 21, 49, 121):
        for C in (2, 3, 4, 21, 33):
            for W in sorted({1, C - 1}):
                rows = om.key_frames(T, C, W, 3, om.WINDOW_ONLY)
                assert om.anchors(T, C, W, 3, om.WINDOW_ONLY) == []
                for t in range(T):
                    assert rows[t] == window_only_closed_form(T, C, t), (T, C, t)
    # the window does not move with the step
    assert om.key_frames(121, 21, 9, 0, om.WINDOW_ONLY) == om.key_frames(121, 21, 9, 17, om.WINDOW_ONLY)
