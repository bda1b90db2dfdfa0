"""Pins of the oracle's distortion/byte table (Eq. (2)) and of its bisection stop rule.

Source: Krishnan & Schulz, "A JoLT for the KV Cache" (arXiv 2607.12550v2), Sec. 3:
  * Eq. (2): the surrogate error of a grid point is eps^2(b) times the token-mode and feature-mode
    energy left out by the truncation, relative to ||X||_F^2 (unprojected spectra; in FlashJoLT the
    token spectrum ends with the synthetic tail entry, which every grid rank discards, Sec. 3.1);
  * "Solving the allocation": geometric bisection on lambda that stops once the total bytes are
    within 0.5% of the budget (from below), else after 50 steps.

The expected values do not come from the oracle's own formula: they are worked by hand from small
spectra, or measured directly as projection residuals ||X - P X||^2 (Eckart-Young), or are the
closed-form switching point of a two-option table.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _table(specT, specD, norm2, rT_grid, rd_grid, bits, eps2, sh=None, c=2):
    sh = sh or oracle.CellShape(1, 1, 64, 64)
    return oracle.cell_table(sh, c, np.asarray(specT, float), np.asarray(specD, float), norm2, rT_grid, rd_grid,
                             bits, eps2)


def _lookup(tab, b, rT, rd):
    i = np.flatnonzero((tab["b"] == b) & (tab["rT"] == rT) & (tab["rd"] == rd))
    assert len(i) == 1
    return float(tab["e"][i[0]]), int(tab["s"][i[0]])


# --------------------------------------------------------------------------- Eq. (2), by hand
def test_eq2_hand_worked_flash_spectrum_with_tail_entry():
    # FlashJoLT cell with q_cap = 2: two computed token values and the tail entry (last).
    # ||X||^2 = 5 + 3 + 2 = 10 = 6 + 3 + 1 (both spectra carry all of the energy).
    specT = [5.0, 3.0, 2.0]
    specD = [6.0, 3.0, 1.0]
    eps2 = {0: 1.0, 4: 0.25}
    tab = _table(specT, specD, 10.0, [1, 2], [1, 2, 3], [0, 4], eps2)
    # left-out energy: token mode keeps the first r_T values; feature mode the first r_d
    want_tau = {
        (1, 1): (3.0 + 2.0 + 3.0 + 1.0) / 10.0,   # 0.9
        (1, 2): (3.0 + 2.0 + 1.0) / 10.0,         # 0.6
        (1, 3): (3.0 + 2.0) / 10.0,               # 0.5
        (2, 1): (2.0 + 3.0 + 1.0) / 10.0,         # r_T = q_cap: only the tail entry is left out
        (2, 2): (2.0 + 1.0) / 10.0,               # 0.3
        (2, 3): 2.0 / 10.0,                       # 0.2
    }
    for (rT, rd), tau in want_tau.items():
        for b in (0, 4):
            e, _ = _lookup(tab, b, rT, rd)
            assert e == pytest.approx(eps2[b] * tau, rel=1e-15, abs=0.0), (b, rT, rd, e)


def test_eq2_hand_worked_exact_spectrum_and_zero_norm():
    # exact cell (no tail entry): r_T at the full length leaves nothing of the token mode out
    specT = [8.0, 1.5, 0.5]
    specD = [7.0, 2.0, 1.0]
    tab = _table(specT, specD, 10.0, [1, 3], [2, 3], [0, 2], {0: 1.0, 2: 0.5})
    assert _lookup(tab, 0, 1, 2)[0] == pytest.approx((1.5 + 0.5 + 1.0) / 10.0, rel=1e-15)
    assert _lookup(tab, 2, 1, 3)[0] == pytest.approx(0.5 * (1.5 + 0.5) / 10.0, rel=1e-15)
    assert _lookup(tab, 0, 3, 2)[0] == pytest.approx(1.0 / 10.0, rel=1e-15)
    assert _lookup(tab, 2, 3, 3)[0] == 0.0
    # a cell without energy has no error to report at any grid point
    tz = _table([0.0, 0.0, 0.0], [0.0, 0.0, 0.0], 0.0, [1, 3], [2, 3], [0, 2], {0: 1.0, 2: 0.5})
    assert np.all(tz["e"] == 0.0)


# --------------------------------------------------------------------------- Eq. (2), measured
def _unfold_token(X):
    G, H, T, D = X.shape
    out = np.empty((T, G * H * D))
    for g in range(G):
        for h in range(H):
            out[:, (g * H + h) * D:(g * H + h + 1) * D] = X[g, h]
    return out


def _proj_residual(A, k):
    """||A - U_k U_k^T A||_F^2 for the leading k left singular vectors of A (a projection, no spectrum)."""
    U, _, _ = np.linalg.svd(A, full_matrices=False)
    Uk = U[:, :k]
    R = A - Uk @ (Uk.T @ A)
    return float(np.sum(R * R))


@pytest.mark.parametrize("noise", [False, True])
def test_eq2_equals_left_out_energy_measured_by_projection(noise):
    """On the tiny cell: with one mode untruncated, tau ||X||^2 must equal the squared distance of the
    unfolding from its rank-r projection (Eckart-Young), measured directly in each unfolding."""
    K, V = synth.per_head_lowrank(noise=noise, seed=0)
    for Z in (K, V):
        X = oracle.to_f64(Z.numpy()[0], "f32")
        G, H, T, D = X.shape
        n2 = float(np.sum(X * X))
        At = _unfold_token(X)                 # T x (G H D)
        Ad = X.reshape(-1, D).T               # D x (G H T): feature mode as rows
        specT = np.linalg.svd(At, compute_uv=False) ** 2
        specD = np.linalg.svd(Ad, compute_uv=False) ** 2
        rT_grid, rd_grid = [8, 16, 32, 64], [8, 16, 32, 64]
        sh = oracle.CellShape(G, H, T, D)
        tab = oracle.cell_table(sh, 4, specT, specD, n2, rT_grid + [T], rd_grid, [0], {0: 1.0})
        for rT in rT_grid:   # r_d = D: no feature truncation
            tab_full = oracle.cell_table(sh, 4, specT, specD, n2, [rT], [D], [0], {0: 1.0})
            e, _ = _lookup(tab_full, 0, rT, D)
            assert e * n2 == pytest.approx(_proj_residual(At, rT), rel=1e-9, abs=1e-12 * n2)
        for rd in rd_grid:   # r_T = T: no token truncation
            e, _ = _lookup(tab, 0, T, rd)
            want = _proj_residual(Ad, rd)
            assert e * n2 == pytest.approx(want, rel=1e-9, abs=1e-12 * n2)
        # both modes truncated: the two left-out energies add
        for rT, rd in [(8, 8), (16, 32), (32, 16)]:
            e, _ = _lookup(tab, 0, rT, rd)
            assert e * n2 == pytest.approx(_proj_residual(At, rT) + _proj_residual(Ad, rd), rel=1e-9,
                                           abs=1e-12 * n2)


def test_eq2_flash_tail_entry_is_the_energy_outside_the_captured_subspace():
    """Sec. 3.1: the tail entry holds the energy the q_cap computed vectors miss, so at r_T = q_cap and
    r_d = d_h the table's tau ||X||^2 is ||X - U U^T X||^2 for the randomized factor U (T x q_cap)."""
    K, V = synth.power_law(L=4, H=2, T=256, D=64, dtype="f16", seed=5)
    X = oracle.to_f64(K.numpy()[0], "f16")
    At = _unfold_token(X)
    n2 = float(np.sum(X * X))
    q, ell = 32, 42
    Om = oracle.sketch_matrix(At.shape[1], ell, 0, "f16")
    U, spec = oracle.token_factors_flash(At, Om, q, 1, n2)
    assert len(spec) == q + 1
    specD = np.linalg.svd(X.reshape(-1, 64), compute_uv=False) ** 2
    sh = oracle.CellShape(*X.shape)
    tab = oracle.cell_table(sh, 2, spec, specD, n2, [8, q], [64], [0], {0: 1.0})
    R = At - U @ (U.T @ At)
    want = float(np.sum(R * R))
    e, _ = _lookup(tab, 0, q, 64)
    assert e * n2 == pytest.approx(want, rel=1e-8, abs=1e-12 * n2)
    # at r_T = 8 the values 9..q_cap are left out as well: the residual of the first 8 columns
    R8 = At - U[:, :8] @ (U[:, :8].T @ At)
    e8, _ = _lookup(tab, 0, 8, 64)
    assert e8 * n2 == pytest.approx(float(np.sum(R8 * R8)), rel=1e-8, abs=1e-12 * n2)


# --------------------------------------------------------------------------- bisection stop rule
def _two_option_tables(n_cells, e_lo, s_lo, e_hi, s_hi):
    """Cells with two grid points each: (error e_lo, bytes s_lo) and (e_hi, s_hi), s_lo < s_hi."""
    tabs = []
    for _ in range(n_cells):
        tabs.append({"b": np.array([0, 0]), "rT": np.array([8, 16]), "rd": np.array([8, 8]),
                     "e": np.array([e_lo, e_hi], dtype=np.float64), "s": np.array([s_lo, s_hi], dtype=np.int64)})
    return tabs


def test_bisection_runs_fifty_steps_when_no_total_lands_in_the_window():
    """Two identical cells whose only totals are 2 s_hi (over budget) and 2 s_lo (far under it):
    no lambda gives a total within 0.5% of B, so the bisection takes all 50 steps and returns the
    feasible end of its bracket, which must sit at the closed-form switching point
    lambda* = (e_lo - e_hi) / (s_hi - s_lo) (where e + lambda s ties), to the precision that 50
    halvings of log(1e10 / 1e-30) leave."""
    e_lo, s_lo, e_hi, s_hi = 1.0, 100, 0.0, 1000
    tabs = _two_option_tables(2, e_lo, s_lo, e_hi, s_hi)
    lam_star = (e_lo - e_hi) / (s_hi - s_lo)
    res = oracle.allocate(tabs, 1050.0)
    assert res["status"] == 0
    assert res["iters"] == 50
    assert res["S"] == 2 * s_lo and res["picks"] == [0, 0]
    width = math.log(1e10 / 1e-30) / 2 ** 50          # final bracket width in log(lambda)
    assert abs(math.log(res["lam"] / lam_star)) <= 2 * width + 1e-15
    assert res["lam"] >= lam_star * (1 - 1e-15)         # the returned end is the feasible one


def test_bisection_accepts_the_first_total_inside_the_window():
    """Two cells whose totals at the switching point are 2 s_lo = 0.997 B (inside the window): the
    bisection accepts before 50 steps with 0.995 B <= S <= B."""
    tabs = _two_option_tables(2, 1.0, 997, 0.0, 4000)
    res = oracle.allocate(tabs, 2000.0)
    assert res["status"] == 0
    assert res["iters"] < 50
    assert 0.995 * 2000.0 <= res["S"] <= 2000.0


def _tiny_tables():
    K, V = synth.per_head_lowrank(seed=0)
    eps2 = {0: 1.0, 2: 0.5149, 3: 0.06313, 4: 0.01158}
    tabs = []
    for Z in (K, V):
        X = oracle.to_f64(Z.numpy()[0], "f32")
        sh = oracle.CellShape(*X.shape)
        _, specT = oracle.token_factors_exact(oracle.token_unfolding(X))
        tabs.append(oracle.cell_table(sh, 4, specT, oracle.feature_spectrum(X), float(np.sum(X * X)),
                                      [8, 16, 24, 32, 40, 48, 56, 64], [8, 16, 24, 32, 40, 48, 56, 64],
                                      [0, 2, 3, 4], eps2))
    return tabs


def test_bisection_early_stop_only_inside_the_half_percent_window():
    """Over a sweep of budgets: every call that stops before 50 steps above lambda_lo holds
    0.995 B <= S <= B; every call stays within B; and where S(lambda) does reach the window some budgets
    do stop early (so the check is not vacuous)."""
    tabs = _tiny_tables()
    smin = sum(int(t["s"].min()) for t in tabs)
    smax = sum(int(t["s"].max()) for t in tabs)
    early = 0
    for B in np.linspace(smin * 1.001, smax * 0.999, 400):
        res = oracle.allocate(tabs, float(B))
        assert res["status"] == 0
        assert res["S"] <= B
        if res["iters"] < 50 and res["lam"] != oracle.jolt.LAMBDA_LO:
            early += 1
            assert 0.995 * B <= res["S"], (B, res["S"], res["iters"])
        if res["iters"] == 50:
            # no accept: the returned picks are those of the feasible bracket end
            idx = [oracle.argmin_cell(t, res["lam"]) for t in tabs]
            assert idx == res["picks"]
    assert early > 10
