"""Pins of the CPU oracle against facts fixed by the pages or by mathematics.

Each test names what pins it.  None of them retypes the oracle's own formula:
expected values come from the pages (tests/golden/), from published generator
outputs, from closed forms (Eckart-Young, ST-HOSVD identities), or from brute
force on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import rng

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- rng
def test_splitmix64_matches_published_outputs():
    want = [int(l, 16) for l in open(os.path.join(GOLD, "splitmix64_seed0.txt")) if l.startswith("0x")]
    got = [int(rng.splitmix_words(0, i)) for i in range(3)]
    assert got == want


def test_box_muller_gaussians_are_standard_normal():
    from scipy import stats
    g = rng.gaussians(7, rng.STREAM_SKETCH, 200000)
    assert abs(g.mean()) < 5 / math.sqrt(len(g))
    assert abs(g.var() - 1.0) < 5 * math.sqrt(2.0 / len(g))
    assert stats.kstest(g, "norm").pvalue > 1e-3
    # counter-based: any window equals the same slice of a longer draw
    assert np.array_equal(rng.gaussians(7, rng.STREAM_SKETCH, 100, start=1001), g[1001:1101])
    # even/odd elements of a pair share the radius (Box-Muller)
    u = rng.uniforms(rng.splitmix_words(rng.stream_key(7, rng.STREAM_SKETCH), np.arange(2, dtype=np.uint64)))
    assert math.isclose(g[0] ** 2 + g[1] ** 2, -2.0 * math.log(u[0]), rel_tol=1e-12)


# --------------------------------------------------------------------------- quantizer
def test_eps2_calibration_reproduces_printed_values():
    gold = _gold("eps2_pages.json")
    bits = [int(b) for b in gold["eps2"]]
    got = oracle.eps2_calibrate(gold["d_head"], bits)
    for b in bits:
        assert abs(got[b] - gold["eps2"][str(b)]) <= gold["tolerance"][str(b)], (b, got[b])


@pytest.mark.parametrize("b", [2, 3, 4, 8])
def test_quantizer_is_nearest_level_bruteforce(b):
    r = np.random.default_rng(b)
    x = r.standard_normal((64, 16)) * np.exp(r.standard_normal((64, 1)))
    x[3] = 0.0
    u, s = oracle.quantize_rows(x, b)
    qm = 2 ** (b - 1) - 1
    xf = x.astype(np.float32)
    deq = oracle.dequantize_rows(u, s, b)
    for i in range(x.shape[0]):
        a = np.max(np.abs(xf[i]))
        assert s[i] == np.float32(a / np.float32(qm))
        if a == 0:
            assert np.all(deq[i] == 0)
            continue
        levels = np.arange(-qm, qm + 1, dtype=np.float32) * s[i]
        for j in range(x.shape[1]):
            dist = np.abs(levels.astype(np.float64) - float(xf[i, j]))
            assert abs(float(deq[i, j]) - float(xf[i, j])) <= dist.min() * (1 + 1e-6) + 1e-12
            # half-step bound
            assert abs(float(deq[i, j]) - float(xf[i, j])) <= 0.5 * float(s[i]) * (1 + 1e-6)


def test_quantizer_one_bit_is_sign_code():
    x = np.array([[0.5, -2.0, 1.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    u, s = oracle.quantize_rows(x, 1)
    deq = oracle.dequantize_rows(u, s, 1)
    assert s[0] == 2.0 and s[1] == 0.0
    assert np.array_equal(deq[0], np.array([2.0, -2.0, 2.0, 2.0], dtype=np.float32))
    assert np.all(np.abs(deq[0] - x[0]) <= 2.0 + 1e-12)   # error at most absmax


@pytest.mark.parametrize("b", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
def test_pack_rows_bitstream_bruteforce(b, D):
    r = np.random.default_rng(10 * b + D)
    u = r.integers(0, 2 ** b, size=(5, D)).astype(np.uint8)
    packed = oracle.pack_rows(u, b)
    assert packed.shape == (5, D * b // 8)
    for i in range(5):
        stream = 0
        for j in range(D):
            stream |= int(u[i, j]) << (j * b)   # element j at stream bits [j*b, (j+1)*b)
        want = stream.to_bytes(D * b // 8, "little")
        assert bytes(packed[i]) == want
    assert np.array_equal(oracle.unpack_rows(packed, b, D), u)


# --------------------------------------------------------------------------- Eq. (1)
def test_eq1_effective_bits_printed():
    for case in _gold("eq1_effective_bits.json")["cases"]:
        D, b = case["d_head"], case["b"]
        sh = oracle.CellShape(2, 3, 50, D)
        extra = oracle.cell_bytes(sh, 2, 4, 4, b) - oracle.cell_bytes(sh, 2, 4, 4, 0)
        assert extra * 8 / (sh.R * D) == case["bits_per_element"]


def test_eq1_tucker_term_counts_scalars():
    sh = oracle.CellShape(4, 8, 1024, 128)
    for c in (2, 4):
        got = oracle.cell_bytes(sh, c, 24, 40, 0)
        # core G x H x rT x rd, U_T T x rT, U_d D x rd scalars of c bytes each
        assert got == c * (np.prod([4, 8, 24, 40]) + 1024 * 24 + 128 * 40)


def test_blob_sections_hold_eq1_bytes_plus_padding():
    sh = oracle.CellShape(4, 8, 100, 64)
    for (rT, rd, b) in [(8, 8, 0), (16, 24, 3), (40, 64, 8)]:
        lay = oracle.section_layout(sh, 2, rT, rd, b)
        eq1 = oracle.cell_bytes(sh, 2, rT, rd, b)
        nsec = 5 if b > 0 else 3
        assert lay["end"] - oracle.jolt.HEADER_BYTES >= eq1
        assert lay["end"] - oracle.jolt.HEADER_BYTES - eq1 < 256 * nsec
        assert all(v % 256 == 0 for v in lay.values())


def test_qcap_eq5_cases():
    for case in _gold("qcap_eq5.json")["cases"]:
        assert oracle.qcap_eq5(case["T"], case["C"]) == case["qcap"]


# --------------------------------------------------------------------------- dtypes
def test_round_to_dtype_f16_matches_ieee_half():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(20000) * 10 ** r.uniform(-9, 4, 20000), [0.0, 65504.0, 2 ** -24, 3 * 2 ** -25]])
    assert np.array_equal(oracle.round_to_dtype(x, "f16"), x.astype(np.float16).astype(np.float64))


def test_round_to_dtype_bf16_matches_torch_on_f32_inputs():
    r = np.random.default_rng(1)
    x = (r.standard_normal(20000) * 10 ** r.uniform(-30, 30, 20000)).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_to_dtype(x, "bf16"), want)


# --------------------------------------------------------------------------- rotation
@pytest.mark.parametrize("D", [64, 128])
def test_rotation_is_haar_qr_with_positive_diagonal(D):
    Q = oracle.rotation(D, 0)
    assert np.abs(Q.T @ Q - np.eye(D)).max() < 1e-12
    G = rng.gaussians(0, rng.STREAM_ROTATION, D * D).reshape(D, D)
    R = Q.T @ G
    assert np.abs(np.tril(R, -1)).max() < 1e-10
    assert np.all(np.diag(R) > 0)
    x = np.random.default_rng(2).standard_normal((10, D))
    assert np.allclose(np.linalg.norm(x @ Q, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert not np.allclose(oracle.rotation(D, 1), Q)


# --------------------------------------------------------------------------- fit
def _tiny(noise=True, seed=0):
    K, V = synth.per_head_lowrank(noise=noise, seed=seed)
    return oracle.to_f64(K.numpy()[0], "f32"), oracle.to_f64(V.numpy()[0], "f32")


def test_fit_full_rank_is_exact_and_factors_orthonormal():
    X, _ = _tiny()
    Xt = oracle.token_unfolding(X)
    U, _ = oracle.token_factors_exact(Xt)
    UT, Ud, core, _ = oracle.fit_cell(X, U[:, :128], 64)
    assert np.abs(UT.T @ UT - np.eye(128)).max() < 1e-12
    assert np.abs(Ud.T @ Ud - np.eye(64)).max() < 1e-12
    Xr = np.einsum("tr,ghrk,dk->ghtd", UT, core, Ud)
    assert np.abs(Xr - X).max() < 1e-12 * np.abs(X).max()


@pytest.mark.parametrize("rT,rd", [(8, 8), (16, 32), (32, 16), (64, 64), (128, 8), (5, 63)])
def test_sthosvd_error_identity_and_bounds(rT, rd):
    X, V = _tiny()
    for Z in (X, V):
        Xt = oracle.token_unfolding(Z)
        U, specT = oracle.token_factors_exact(Xt)
        specD = oracle.feature_spectrum(Z)
        UT, Ud, core, wproj = oracle.fit_cell(Z, U[:, :rT], rd)
        Zr = np.einsum("tr,ghrk,dk->ghtd", UT, core, Ud)
        err2 = float(np.sum((Z - Zr) ** 2))
        # ST-HOSVD: error = discarded token mass + discarded projected feature mass (orthogonal parts)
        ident = float(np.sum(specT[rT:]) + np.sum(wproj[rd:]))
        assert math.isclose(err2, ident, rel_tol=1e-9, abs_tol=1e-9 * float(np.sum(Z * Z)))
        # upper bound by the unprojected discarded masses (tau), lower bound by Eckart-Young per mode
        assert err2 <= float(np.sum(specT[rT:]) + np.sum(specD[rd:])) * (1 + 1e-9)
        assert err2 >= max(float(np.sum(specT[rT:])), float(np.sum(specD[rd:]))) * (1 - 1e-9)


def test_zero_noise_tiny_is_exactly_rank_32():
    for Z in _tiny(noise=False):
        Xt = oracle.token_unfolding(Z)
        U, specT = oracle.token_factors_exact(Xt)
        specD = oracle.feature_spectrum(Z)
        n2 = float(np.sum(Z * Z))
        for rT, rd in itertools.product([8, 16, 32, 64], [8, 16, 32, 64]):
            UT, Ud, core, wproj = oracle.fit_cell(Z, U[:, :rT], rd)
            err2 = float(np.sum((Z - np.einsum("tr,ghrk,dk->ghtd", UT, core, Ud)) ** 2))
            if rT >= 32 and rd >= 32:   # only the fp32 storage rounding of the input remains
                assert err2 < 1e-14 * n2
            if rd >= 32:   # only the token mode truncates: Eckart-Young, error = discarded energy
                assert math.isclose(err2, float(np.sum(specT[rT:])), rel_tol=1e-8, abs_tol=1e-14 * n2)
        assert specT[32] < 1e-14 * n2 and specD[32] < 1e-14 * n2 and specT[31] > 1e-6 * n2


def test_flash_equals_exact_on_low_rank_input():
    X, _ = _tiny(noise=False)       # token rank 32 <= ell
    Xt = oracle.token_unfolding(X)
    n2 = float(np.sum(X * X))
    Om = oracle.sketch_matrix(Xt.shape[1], 42, 3, "f32")
    Uf, specf = oracle.token_factors_flash(Xt, Om, 32, 1, n2)
    Ue, spece = oracle.token_factors_exact(Xt)
    P1, P2 = Uf @ Uf.T, Ue[:, :32] @ Ue[:, :32].T
    assert np.linalg.norm(P1 - P2, 2) < 1e-9
    assert np.allclose(specf[:32], spece[:32], rtol=1e-9)
    assert specf[32] < 1e-9 * n2
    assert math.isclose(float(np.sum(specf)), n2, rel_tol=1e-12)


def test_flash_tail_entry_restores_total_energy():
    K, V = synth.power_law(L=4, H=2, T=256, D=64, dtype="f16", seed=3)
    X = oracle.to_f64(K.numpy()[0], "f16")
    Xt = oracle.token_unfolding(X)
    n2 = float(np.sum(X * X))
    Om = oracle.sketch_matrix(Xt.shape[1], 42, 0, "f16")
    U, spec = oracle.token_factors_flash(Xt, Om, 32, 1, n2)
    assert math.isclose(float(np.sum(spec)), n2, rel_tol=1e-12)
    assert np.abs(U.T @ U - np.eye(32)).max() < 1e-12
    # randomized values never exceed the exact ones (Rayleigh-Ritz interlacing)
    _, se = oracle.token_factors_exact(Xt)
    assert np.all(spec[:32] <= se[:32] * (1 + 1e-10))
    assert np.allclose(spec[:8], se[:8], rtol=1e-3)


def test_sketch_is_rounded_gaussian_stream():
    Om = oracle.sketch_matrix(64, 10, 5, "f16")
    g = rng.gaussians(5, rng.STREAM_SKETCH, 640).reshape(64, 10)
    assert np.array_equal(Om, g.astype(np.float16).astype(np.float64))


# --------------------------------------------------------------------------- allocator
def _tiny_tables():
    X, V = _tiny()
    eps2 = {0: 1.0, 2: 0.5149, 3: 0.06313, 4: 0.01158}
    tabs, shapes = [], []
    for Z in (X, V):
        sh = oracle.CellShape(*Z.shape)
        _, specT = oracle.token_factors_exact(oracle.token_unfolding(Z))
        tabs.append(oracle.cell_table(sh, 4, specT, oracle.feature_spectrum(Z), float(np.sum(Z * Z)),
                                      [8, 16, 32, 64], [8, 16, 32, 64], [0, 2, 3, 4], eps2))
        shapes.append(sh)
    return tabs, shapes


def test_allocator_matches_bruteforce_enumeration_everett():
    tabs, shapes = _tiny_tables()
    dense = sum(sh.R * sh.D * 4 for sh in shapes)
    for C in (1.5, 2.0, 3.0, 5.0, 8.0):
        res = oracle.allocate(tabs, dense / C)
        assert res["status"] == 0
        lam = res["lam"]
        # per cell: the pick minimises e + lam s over the whole grid (brute force in python)
        for t, i in zip(tabs, res["picks"]):
            costs = [float(t["e"][j]) + lam * float(t["s"][j]) for j in range(len(t["e"]))]
            assert costs[i] == min(costs)
        # Everett: no combination with the same or smaller total bytes has smaller total error
        S = res["S"]
        best = min(float(tabs[0]["e"][i]) + float(tabs[1]["e"][j])
                   for i in range(len(tabs[0]["e"])) for j in range(len(tabs[1]["e"]))
                   if int(tabs[0]["s"][i]) + int(tabs[1]["s"][j]) <= S)
        assert res["E"] <= best * (1 + 1e-12)
        assert S <= dense / C


def test_allocator_monotone_in_lambda():
    tabs, _ = _tiny_tables()
    prevS, prevE = None, None
    for lam in np.logspace(-14, -2, 60):
        idx = [oracle.argmin_cell(t, lam) for t in tabs]
        S = sum(int(t["s"][i]) for t, i in zip(tabs, idx))
        E = sum(float(t["e"][i]) for t, i in zip(tabs, idx))
        if prevS is not None:
            assert S <= prevS and E >= prevE - 1e-15
        prevS, prevE = S, E


def test_allocator_budget_edges():
    tabs, shapes = _tiny_tables()
    smin = sum(int(t["s"].min()) for t in tabs)
    smax = sum(int(t["s"].max()) for t in tabs)
    assert oracle.allocate(tabs, smin - 1)["status"] == -2
    res = oracle.allocate(tabs, smax * 10)
    assert res["status"] == 0 and res["iters"] == 0 and res["lam"] == oracle.jolt.LAMBDA_LO
    res = oracle.allocate(tabs, smin)
    assert res["status"] == 0 and res["S"] <= smin


# --------------------------------------------------------------------------- end to end
def test_tiny_compress_blob_roundtrip_and_half_step():
    K, V = synth.per_head_lowrank()
    eps2 = {0: 1.0, 2: 0.5149, 3: 0.06313, 4: 0.01158}
    p = dict(mode="exact", oversample=10, power_iters=1, qcap=None, rT_grid=[8, 16, 32, 64],
             rd_grid=[8, 16, 32, 64], bits=[2, 3, 4], eps2=eps2, target_ratio=2.0)
    r = oracle.compress(K.numpy(), V.numpy(), [0, 1], "f32", p, keep=True)
    assert r["status"] == 0 and r["S"] <= r["budget"]
    rec = oracle.reconstruct(r["blob"], r["offsets"], "f32", 0, 64)
    Q = oracle.rotation(64, 0)
    for cell, xh in zip(r["cells"], rec):
        assert np.array_equal(xh, cell["Xhat"])
        X = cell["X"]
        if cell["b"] > 0:
            # every rotated coordinate is within half a step of the residual
            Erot = ((X - cell["enc"]["backbone"]).reshape(-1, 64) @ Q).astype(np.float32)
            D_rot = ((X - xh).reshape(-1, 64) @ Q)
            s = cell["enc"]["scales"].astype(np.float64)
            assert np.all(np.abs(D_rot) <= 0.5 * s[:, None] * (1 + 1e-5) + 1e-6 * np.abs(Erot).max())
        hdr = np.frombuffer(r["blob"], dtype=np.uint32, count=10, offset=cell["offset"])
        assert list(hdr[2:9]) == [1, 2, 128, 64, cell["rT"], cell["rd"], cell["b"]]
