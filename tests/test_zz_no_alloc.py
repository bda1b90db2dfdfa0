"""jolt_allocate_static (the allocation with no workspace argument, for callers that cannot allocate
device memory) against jolt_allocate on the same spectra: status, lambda, picks, bytes and predicted
errors identical, on two calls in a row (the second smaller, so stale scratch contents from the first
would show), on both allocation kernels; and the refusal of a table larger than the scratch."""
import numpy as np
import pytest
import torch

import synth
from kv_cache_compression_layer_amd import jolt

pytestmark = pytest.mark.gpu


def _spectra(n_groups2, T, D, seed):
    """Token and feature spectra of a small exact-mode cache of 2 n_groups2 layers in groups of 4
    (computed by the library itself)."""
    L = 2 * n_groups2
    K, V = synth.power_law(L=L, H=2, T=T, D=D, dtype="f16", seed=seed)
    groups = list(range(0, L + 1, 4))
    cfg = jolt.Config(1, L, 2, T, D, jolt.F16, groups, jolt.EXACT, [8, 16], [8, 16], [2, 4], 3.0)
    sT, sD, n2, _ = jolt.spectra(K.cuda(), V.cuda(), cfg)
    torch.cuda.synchronize()
    shapes = [(4, 2, T, D)] * cfg.n_cells
    return shapes, list(sT.cpu().numpy()), list(sD.cpu().numpy()), list(n2.cpu().numpy())


def _both(args, rT, rd, bits, budget, eps2):
    shapes, sT, sD, n2 = args
    a = jolt.allocate(shapes, 2, sT, sD, n2, rT, rd, bits, budget, eps2=eps2)
    b = jolt.allocate(shapes, 2, sT, sD, n2, rT, rd, bits, budget, eps2=eps2, static_scratch=True)
    return a, b


@pytest.mark.parametrize("rT", [[8, 16, 24, 32], list(range(8, 257, 8))])  # one-workgroup, per-cell kernel
def test_static_scratch_allocation_matches_workspace_allocation(rT):
    eps2 = {0: 1.0, 2: 0.5149, 4: 0.01158, 8: 3.52e-5}
    rd, bits = [8, 16, 32, 48, 64], [2, 4, 8]
    big = _spectra(8, 256, 64, seed=3)            # 16 layers in 4 groups -> 8 cells
    small = _spectra(2, 256, 64, seed=4)          # 4 layers in 1 group -> 2 cells
    for args in (big, small, big):
        dense = len(args[0]) * 4 * 2 * 256 * 64 * 2
        for C in (1.5, 3.0, 6.0, 1e6):
            (st1, p1, l1), (st2, p2, l2) = _both(args, rT, rd, bits, dense / C, eps2)
            assert st1 == st2, (C, st1, st2)
            if st1 != 0:
                assert st1 == -2
                continue
            assert l1 == l2
            assert p1 == p2


def test_static_scratch_refuses_tables_beyond_its_size():
    shapes, sT, sD, n2 = _spectra(2, 256, 64, seed=5)
    n = 1500                                       # 1500 cells x 3 bits x 32 x 8 grid points x 16 B > 16 MiB
    rT, rd, bits = list(range(8, 257, 8)), list(range(8, 65, 8)), [2, 4]
    st, _, _ = jolt.allocate(shapes[:1] * n, 2, sT[:1] * n, sD[:1] * n, n2[:1] * n, rT, rd, bits, 1e9,
                             eps2={0: 1.0, 2: 0.5149, 4: 0.01158}, static_scratch=True)
    assert st == -3
    assert "static scratch" in jolt.load().jolt_last_error().decode()
    # the scratch still serves a call that fits
    st, picks, _ = jolt.allocate(shapes, 2, sT, sD, n2, rT, rd, bits, 1e9, eps2={0: 1.0, 2: 0.5149, 4: 0.01158},
                                 static_scratch=True)
    assert st == 0 and len(picks) == len(shapes)
