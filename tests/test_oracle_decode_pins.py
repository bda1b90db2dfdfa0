"""Pins of the oracle's decode-time attention (A JoLT for the KV Cache, Sec. 4.5 "Fused decode
kernel"): RoPE by hand-worked values, the identity at position 0, norm preservation and the
relative-position property on exactly representable angles; attention against the library's
scaled dot-product attention, the uniform-weight and single-key limits, the grouped-query head
mapping; the layer slice of a blob against the compressor's own reconstruction."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import decode as od


def test_rope_inverse_frequencies_and_hand_worked_rotation():
    f = od.rope_inv_freq(4, 10000.0)
    assert f.dtype == np.float32 and f[0] == 1.0 and f[1] == np.float32(0.01)
    y = od.apply_rope(np.array([[1.0, 0.0, 0.0, 0.0]]), [1], f)[0]
    assert np.allclose(y, [math.cos(1.0), 0.0, math.sin(1.0), 0.0], rtol=0, atol=1e-15)
    a = float(np.float32(3) * np.float32(0.01))  # the fp32 angle of position 3, pair 1
    y = od.apply_rope(np.array([[0.0, 2.0, 0.0, -1.0]]), [3], f)[0]
    assert np.allclose(y, [0.0, 2 * math.cos(a) + math.sin(a), 0.0, -math.cos(a) + 2 * math.sin(a)], rtol=0,
                       atol=1e-15)


def test_rope_identity_at_zero_and_norms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 16))
    f = od.rope_inv_freq(16, 500000.0)
    assert np.array_equal(od.apply_rope(x, np.zeros(5, int), f), x)
    y = od.apply_rope(x, np.arange(5) * 977, f)
    h = 8
    assert np.allclose(x[:, :h] ** 2 + x[:, h:] ** 2, y[:, :h] ** 2 + y[:, h:] ** 2, rtol=1e-13)


def test_rope_depends_on_relative_position_only():
    """With inverse frequencies that are powers of two (D = 8, base 16) and integer positions, every
    fp32 angle is exact, so rope(q, m) . rope(k, n) = rope(q, m - n) . k to fp64 rounding."""
    f = od.rope_inv_freq(8, 16.0)
    assert list(f) == [1.0, 0.5, 0.25, 0.125]
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(8), rng.standard_normal(8)
    for m, n in [(5, 2), (1000, 37), (70000, 69999)]:
        a = od.apply_rope(q[None], [m], f)[0] @ od.apply_rope(k[None], [n], f)[0]
        b = od.apply_rope(q[None], [m - n], f)[0] @ k
        assert abs(a - b) <= 1e-12 * np.linalg.norm(q) * np.linalg.norm(k)


def _dense_case(seed=0, H=2, T=37, n=3, D=8, nq=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((nq, D)), rng.standard_normal((H, T, D)), rng.standard_normal((H, T, D)),
            rng.standard_normal((H, n, D)), rng.standard_normal((H, n, D)))


def test_attention_equals_library_sdpa():
    q, K, V, kt, vt = _dense_case()
    f = od.rope_inv_freq(8, 16.0)
    out = od.decode_attention(q, K, V, kt, vt, f)
    Kall = np.concatenate([K, kt], 1)
    Vall = np.concatenate([V, vt], 1)
    Kr = od.apply_rope(Kall, np.arange(Kall.shape[1]), f)
    g = q.shape[0] // K.shape[0]
    Kq = torch.from_numpy(np.repeat(Kr, g, axis=0))          # [nq, T+n, D]
    Vq = torch.from_numpy(np.repeat(Vall, g, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], Kq, Vq)[:, 0]
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_limits_and_head_mapping():
    q, K, V, kt, vt = _dense_case(seed=2)
    f = od.rope_inv_freq(8, 16.0)
    # a zero query weighs every token equally: the mean of the values (tail included)
    out = od.decode_attention(np.zeros_like(q), K, V, kt, vt, f)
    want = np.concatenate([V, vt], 1).mean(axis=1)
    assert np.allclose(out, np.repeat(want, 2, axis=0), rtol=1e-13, atol=1e-13)
    # one key far along its query dominates
    Kd = K.copy()
    Kd[0, 11] = 200.0 * od.apply_rope(q[0][None], [-11], f)[0]
    out = od.decode_attention(q, Kd, V, kt[:, :0], vt[:, :0], f)
    assert np.allclose(out[0], V[0, 11], atol=1e-9)
    # grouped-query mapping: constant values per KV head come back on that head's queries
    Vc = np.stack([np.full((K.shape[1], 8), 1.0), np.full((K.shape[1], 8), 2.0)])
    out = od.decode_attention(q, K, Vc, kt[:, :0], vt[:, :0], f)
    assert np.allclose(out[:2], 1.0) and np.allclose(out[2:], 2.0)


def test_layer_from_blob_is_the_compressor_reconstruction():
    K, V = synth.power_law(L=4, H=2, T=96, D=64, dtype="f16", seed=3)
    groups = [0, 2, 4]
    p = dict(mode="exact", oversample=10, power_iters=1, qcap=None, rT_grid=[8, 16], rd_grid=[16, 32], bits=[2, 4],
             eps2=oracle.eps2_calibrate(64, [0, 2, 4], rows=1 << 12), target_ratio=2.5)
    ref = oracle.compress(K.numpy(), V.numpy(), groups, "f16", p, keep=True)
    assert ref["status"] == 0
    for layer in range(4):
        Kl, Vl = od.layer_from_blob(ref["blob"], ref["offsets"], "f16", 0, 64, 2, groups, 0, layer)
        g = 0 if layer < 2 else 1
        for x in ref["cells"]:
            if x["group"] == g:
                want = x["Xhat"][layer - groups[g]]
                assert np.array_equal(Kl if x["kv"] == 0 else Vl, want)
