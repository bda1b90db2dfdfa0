"""Pins of the oracle's allocator variants (A JoLT for the KV Cache, Sec. 3 "Solving the allocation": the
pages' greedy per-cell search; Sec. 4.4: K/V-decoupled budgets, uniform ranks, rank-only; Appendix A:
the token-rank cap).  Each test names the fact that pins it: the pages' statement that the greedy rule
is exact for a single truncated mode, Everett's theorem (optimality for the budget actually attained,
checked by brute force), hand-worked walks, and invariances of the definitions."""
import itertools

import numpy as np
import pytest

import oracle
import synth

EPS2 = {0: 1.0, 2: 0.5149, 3: 0.06313, 4: 0.01158}


def _tiny(rT=(8, 16, 24, 32, 40, 48, 56, 64), rd=(8, 16, 24, 32, 40, 48, 56, 64), bits=(0, 2, 3, 4), seed=0):
    K, V = synth.per_head_lowrank(seed=seed)
    tabs = []
    for Z in (K, V):
        X = oracle.to_f64(Z.numpy()[0], "f32")
        _, sT = oracle.token_factors_exact(oracle.token_unfolding(X))
        tabs.append(oracle.cell_table(oracle.CellShape(*X.shape), 4, sT, oracle.feature_spectrum(X),
                                      float(np.sum(X * X)), list(rT), list(rd), list(bits), EPS2))
    return tabs


def _cost(t, i, lam):
    return float(t["e"][i]) + lam * float(t["s"][i])


# --------------------------------------------------------------------------- greedy search
def test_greedy_is_exact_for_a_single_truncated_mode():
    """Sec. 3: the rule is exact for a single truncated mode (convex: the left-out energy per step
    falls while the bytes per step stay fixed), so with one feature rank it equals the exact argmin."""
    tabs = _tiny(rT=tuple(range(8, 129, 8)), rd=(64,))
    for t in tabs:
        for lam in np.logspace(-14, -3, 80):
            i = oracle.argmin_cell_greedy(t, lam, 16, 1)
            j = oracle.argmin_cell(t, lam)
            assert _cost(t, i, lam) == pytest.approx(_cost(t, j, lam), rel=1e-12, abs=0)


def test_greedy_never_beats_the_exact_minimum_and_stops_where_no_step_helps():
    tabs = _tiny()
    nT = nD = 8
    for t in tabs:
        for lam in np.logspace(-14, -3, 60):
            i = oracle.argmin_cell_greedy(t, lam, nT, nD)
            j = oracle.argmin_cell(t, lam)
            assert _cost(t, i, lam) >= _cost(t, j, lam) * (1 - 1e-12)
            bi, rem = divmod(i, nT * nD)
            iT, iD = divmod(rem, nD)
            for nxt in ([(bi * nT + iT + 1) * nD + iD] if iT + 1 < nT else []) + \
                       ([(bi * nT + iT) * nD + iD + 1] if iD + 1 < nD else []):
                assert _cost(t, nxt, lam) >= _cost(t, i, lam) * (1 - 1e-12)


def test_greedy_walk_by_hand():
    """One bit-width, grid 2 x 2: e(rT, rd) and s given; at lambda = 0.1 the token step removes 0.5 for
    2 bytes (0.25 per byte > 0.1) and the feature step 0.3 for 1 byte (0.3 per byte): the steeper
    feature step is taken first, then the token step (0.5 - ... per byte) as long as it pays."""
    e = np.array([1.0, 0.7, 0.5, 0.15])      # (rT0, rd0), (rT0, rd1), (rT1, rd0), (rT1, rd1)
    s = np.array([10, 11, 12, 14])
    t = {"e": e, "s": s, "b": np.zeros(4, int), "rT": np.array([8, 8, 16, 16]), "rd": np.array([8, 16, 8, 16])}
    # from (0,0): token step 0.5/2 = 0.25, feature step 0.3/1 = 0.3 -> feature; from (0,1): token step
    # (0.7 - 0.15)/3 = 0.183 > 0.1 -> (1,1)
    assert oracle.argmin_cell_greedy(t, 0.1, 2, 2) == 3
    # at lambda = 0.2: feature step 0.3 > 0.2 -> (0,1); token step 0.183 < 0.2 -> stop at (0,1)
    assert oracle.argmin_cell_greedy(t, 0.2, 2, 2) == 1
    # at lambda = 0.4 neither first step pays
    assert oracle.argmin_cell_greedy(t, 0.4, 2, 2) == 0


def test_greedy_allocation_respects_budget_and_window():
    tabs = _tiny()
    dense = 2 * 1 * 2 * 128 * 64 * 4
    for C in (1.5, 2.0, 3.0, 5.0):
        r = oracle.allocate_greedy(tabs, dense / C, 8, 8)
        assert r["status"] == 0 and r["S"] <= dense / C
        if 0 < r["iters"] < 50:
            assert r["S"] >= 0.995 * dense / C
        ex = oracle.allocate(tabs, dense / C)
        assert r["E"] >= 0 and ex["E"] >= 0


# --------------------------------------------------------------------------- K/V-decoupled budgets
def test_kv_decoupled_each_kind_within_its_share_and_everett_optimal():
    """Each of K and V gets half the budget (equal dense bytes); each allocation is optimal for the
    bytes it attains (Everett), checked by brute force over the cell's grid."""
    tabs = _tiny()
    dense_cell = 1 * 2 * 128 * 64 * 4
    for C in (1.5, 2.0, 3.0, 5.0):
        B = 2 * dense_cell / C
        r = oracle.allocate_kv_decoupled(tabs, B, [dense_cell, dense_cell])
        assert r["status"] == 0
        for c, t in enumerate(tabs):
            i = r["picks"][c]
            assert int(t["s"][i]) <= B / 2
            feasible = t["s"] <= t["s"][i]
            assert float(t["e"][i]) <= float(np.min(t["e"][feasible])) * (1 + 1e-12)


# --------------------------------------------------------------------------- uniform ranks
def test_uniform_ranks_equal_joint_allocation_on_identical_cells():
    """With identical cells the joint allocation already gives every cell the same pick, so the
    uniform-rank variant must reach the same total error and bytes."""
    t = _tiny()[0]
    tabs = [t, t, t]
    dense = 3 * 1 * 2 * 128 * 64 * 4
    for C in (1.5, 2.5, 4.0):
        j = oracle.allocate(tabs, dense / C)
        u = oracle.allocate_uniform_ranks(tabs, dense / C, 8, 8)
        assert u["status"] == 0
        assert u["E"] <= j["E"] * (1 + 1e-12)
        assert u["S"] <= dense / C


def test_uniform_ranks_share_one_rank_pair():
    tabs = _tiny()
    dense = 2 * 1 * 2 * 128 * 64 * 4
    for C in (1.5, 2.5, 4.0):
        u = oracle.allocate_uniform_ranks(tabs, dense / C, 8, 8)
        assert u["status"] == 0 and u["S"] <= dense / C
        pairs = {(int(t["rT"][i]), int(t["rd"][i])) for t, i in zip(tabs, u["picks"])}
        assert len(pairs) == 1
        # Everett at the chosen pair: no choice of the cells' bit-widths at that pair reaches a smaller
        # total error within the total bytes attained (brute force over the bit combinations)
        iT, iD = u["pair"]
        opts = [[(bi * 8 + iT) * 8 + iD for bi in range(4)] for _ in tabs]
        best = min(sum(float(t["e"][i]) for t, i in zip(tabs, combo))
                   for combo in itertools.product(*opts)
                   if sum(int(t["s"][i]) for t, i in zip(tabs, combo)) <= u["S"])
        assert u["E"] <= best * (1 + 1e-12)


# --------------------------------------------------------------------------- grid restrictions
def test_rank_only_and_token_rank_cap_are_grid_restrictions():
    """Rank-only compression (Sec. 4.4) is the bit set {0}; the exact solver with the token rank capped
    at 32 (Appendix A) is the token grid cut at 32: the allocation then never leaves those grids."""
    tabs = _tiny(bits=(0,))
    dense = 2 * 1 * 2 * 128 * 64 * 4
    r = oracle.allocate(tabs, dense / 2.0)
    assert r["status"] == 0 and all(int(t["b"][i]) == 0 for t, i in zip(tabs, r["picks"]))
    tabs = _tiny(rT=(8, 16, 24, 32))
    r = oracle.allocate(tabs, dense / 2.0)
    assert all(int(t["rT"][i]) <= 32 for t, i in zip(tabs, r["picks"]))
