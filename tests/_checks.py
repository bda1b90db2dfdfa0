"""Shared checks of the GPU tests (imported by the test modules; not collected itself)."""
import numpy as np

import oracle


def lambda_consistency(picks, lam, gpu_spectra, ref_cells, shape, c, rT, rd, bits, eps2):
    """Sec. 3, Eq. (3): the per-cell picks are the exact argmin of e + lambda s at the returned lambda.

    * On tables built from the GPU's own spectra the GPU's picks are that argmin exactly (the
      allocation is bit-exact against the oracle's on identical spectra).
    * On the oracle's tables (its own spectra) the GPU's pick is the argmin too, or its cost lies
      within twice the largest difference between the two tables' errors (spectra that agree only to
      rounding can move a near-tie); such cells are returned for reporting.
    """
    sT, sD, n2 = gpu_spectra
    allbits = sorted(set(bits) | {0})
    near_ties = []
    for i, (p, x) in enumerate(zip(picks, ref_cells)):
        tg = oracle.cell_table(shape, c, sT[i], sD[i], float(n2[i]), rT, rd, allbits, eps2)
        j = oracle.argmin_cell(tg, lam)
        assert (int(tg["rT"][j]), int(tg["rd"][j]), int(tg["b"][j])) == (p["rT"], p["rd"], p["bits"]), i
        to = oracle.cell_table(shape, c, x["specT"], x["specD"], x["norm2"], rT, rd, allbits, eps2)
        cost = to["e"] + lam * to["s"].astype(np.float64)
        delta = float(np.max(np.abs(tg["e"] - to["e"])))
        k = oracle.argmin_cell(to, lam)
        if k != j:
            assert cost[j] - cost[k] <= 2 * delta + 1e-15 * abs(cost[k]), (i, cost[j], cost[k], delta)
            near_ties.append(i)
    return near_ties
