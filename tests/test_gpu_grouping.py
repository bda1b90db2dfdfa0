"""GPU layer grouping (A JoLT for the KV Cache, Sec. 3 "Method" and its footnote on group sizes) and
compression over layer groups of different sizes, against the oracle.

Bars: alignment scores within 1e-4 of the oracle's (exact SVD of every layer's token unfolding; the
library uses randomized subspace iteration converged well below that); groups identical unless a score
lies within that difference of the median (reported); compression of unequal groups: picks equal to
the oracle's, lambda within 1%, Eq. (1) bytes with each cell's own group size, reconstructions within
the bar the code bar implies (xhat_tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kv_cache_compression_layer_amd import jolt
from test_gpu_parity_ranks import xhat_tolerance

pytestmark = pytest.mark.gpu


def _check_groups(K, tol=1e-4):
    starts, sc = jolt.layer_groups(K.cuda())
    torch.cuda.synchronize()
    ref = oracle.alignment_scores(oracle.to_f64(K.numpy()[0], "f16"))
    diff = np.abs(sc - ref)
    med = float(np.median(ref))
    print(f"scores max |diff| {diff.max():.2e}; median {med:.4f}; groups {starts}")
    assert diff.max() <= tol
    want = oracle.group_layers(ref)
    if starts != want:
        near = np.abs(ref - med) <= diff.max() + 1e-12
        assert near.any(), (starts, want)
        print("groups differ at a score within the scores' difference of the median:", starts, want)
    return starts, ref


def test_layer_groups_small_ragged():
    K, _ = synth.power_law(L=9, H=2, T=300, D=64, dtype="f16", seed=5, group=3)
    starts, _ = _check_groups(K)
    sizes = np.diff(starts)
    assert starts[0] == 0 and starts[-1] == 9 and np.all(sizes >= 2) and np.all(sizes <= 9)


def test_layer_groups_mistral7b_shape():
    K, _ = synth.power_law(L=32, H=8, T=1024, D=128, dtype="f16", seed=0)
    _check_groups(K)


def _compare_unequal(K, V, groups, dt, mode, rT, bits, C, T, D, H):
    eps2 = oracle.eps2_calibrate(D, [0] + bits, rows=1 << 15)
    rd = [r for r in [8, 16, 24, 32, 48, 64, 96, 128] if r <= D]
    p = dict(mode=mode, oversample=10, power_iters=1, qcap=None, rT_grid=rT, rd_grid=rd, bits=bits, eps2=eps2,
             target_ratio=C)
    ref = oracle.compress(K.numpy(), V.numpy(), groups, dt, p, keep=True)
    assert ref["status"] == 0
    L = K.shape[1]
    cfg = jolt.Config(1, L, H, T, D, {"f16": jolt.F16}[dt], groups, jolt.FLASH if mode == "flash" else jolt.EXACT, rT,
                      rd, bits, C, eps2=eps2)
    Kd, Vd = K.cuda(), V.cuda()
    blob, picks, lam = jolt.compress(Kd, Vd, cfg)
    Ko, Vo = torch.empty_like(Kd), torch.empty_like(Vd)
    jolt.reconstruct(blob, cfg, picks, Ko, Vo)
    torch.cuda.synchronize()
    got_p = [(q["rT"], q["rd"], q["bits"]) for q in picks]
    want_p = [(x["rT"], x["rd"], x["b"]) for x in ref["cells"]]
    print("picks", got_p, "lambda", lam, ref["lam"])
    assert sum(q["bytes"] for q in picks) <= ref["budget"]
    assert abs(lam - ref["lam"]) <= 1e-2 * ref["lam"]
    # sizes of every section follow Eq. (1) with the cell's own group size
    for q, x in zip(picks, ref["cells"]):
        G = groups[x["group"] + 1] - groups[x["group"]]
        assert q["bytes"] == oracle.cell_bytes(oracle.CellShape(G, H, T, D), 2, q["rT"], q["rd"], q["bits"])
    assert got_p == want_p
    for x in ref["cells"]:
        g0, g1 = groups[x["group"]], groups[x["group"] + 1]
        got = (Ko if x["kv"] == 0 else Vo)[0, g0:g1].double().cpu().numpy()
        want = oracle.round_to_dtype(x["Xhat"], dt)
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        tol = xhat_tolerance(x["enc"].get("scales"), D, np.linalg.norm(want), x["b"]) + 3e-4
        assert rel <= tol, (x["group"], x["kv"], rel, tol)
    return picks


@pytest.mark.parametrize("mode", ["flash", "exact"])
def test_compress_unequal_groups_matches_oracle(mode):
    """Groups of 3, 2 and 4 layers (three partitions of the batched stages, one joint allocation)."""
    L, H, T, D = 9, 2, 200 if mode == "exact" else 700, 64  # exact mode: T <= |g| n_h d_h = 256 for 2 layers
    K, V = synth.power_law(L=L, H=H, T=T, D=D, dtype="f16", seed=7)
    groups = [0, 3, 5, 9]
    rT = list(range(8, 201, 8)) if mode == "exact" else [8, 16, 24, 32]
    _compare_unequal(K, V, groups, "f16", mode, rT, [2, 4, 8], 3.0, T, D, H)


def test_grouping_feeds_compress_mistral7b_shape():
    """The alignment groups of the Mistral-7B-shaped cache passed to FlashJoLT compression: the
    reconstruction of every cell against the oracle's compression over the same groups."""
    L, H, T, D = 32, 8, 1024, 128
    K, V = synth.power_law(L=L, H=H, T=T, D=D, dtype="f16", seed=0)
    starts, _ = jolt.layer_groups(K.cuda())
    torch.cuda.synchronize()
    print("groups", starts)
    assert len(set(np.diff(starts))) >= 1
    _compare_unequal(K, V, starts, "f16", "flash", [8, 16, 24, 32], [2, 4, 8], 2.0, T, D, H)
