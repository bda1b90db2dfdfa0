"""Pins of the oracle's layer grouping (A JoLT for the KV Cache, Sec. 3 "Method": layers are grouped
by how well their top-8 token-mode singular vectors align, scored on consecutive layers by the mean
squared cosine between the bases, with a new group below the network median; the footnote's size
bounds: at least two layers before a new group opens, at most eight, a trailing single layer merged).

Expected values are closed forms of constructed caches (identical, orthogonal and partly rotated token
subspaces, whose principal angles are known) and groupings worked by hand from score sequences."""
import math

import numpy as np
import pytest

import oracle


def _haar(n, k, rng):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))[None, :]


def _layer(Ut, rng, H=2, D=16, decay=None):
    """A layer's key cache (H x T x D) whose token unfolding is Ut diag(s) W^T: its top-k token basis
    is span(Ut) (well separated singular values)."""
    T, k = Ut.shape
    s = decay if decay is not None else 10.0 / np.arange(1, k + 1)
    W = _haar(H * D, k, rng)
    A = (Ut * s[None, :]) @ W.T          # T x (H D)
    return A.reshape(T, H, D).transpose(1, 0, 2)


def test_basis_is_the_leading_token_subspace():
    rng = np.random.default_rng(0)
    Ut = _haar(64, 8, rng)
    B = oracle.layer_token_basis(_layer(Ut, rng), 8)
    assert np.linalg.norm(B @ B.T - Ut @ Ut.T, 2) < 1e-10
    assert np.abs(B.T @ B - np.eye(8)).max() < 1e-12


def test_scores_closed_forms():
    """Same subspace (any basis inside it): 1; orthogonal subspaces: 0; one of the k directions turned
    by theta within a plane orthogonal to the rest: (k - 1 + cos^2 theta) / k."""
    rng = np.random.default_rng(1)
    T, k = 96, 8
    Q = _haar(T, 2 * k + 1, rng)
    U0 = Q[:, :k]
    U_same = U0 @ _haar(k, k, rng)                       # another basis of the same subspace
    U_orth = Q[:, k:2 * k]
    th = 0.7
    U_rot = U0.copy()
    U_rot[:, 3] = math.cos(th) * U0[:, 3] + math.sin(th) * Q[:, 2 * k]
    K = np.stack([_layer(U, rng) for U in (U0, U_same, U_orth, U_rot)])
    K[3] = _layer(U_rot, rng)
    sc = oracle.alignment_scores(np.stack([K[0], K[1], K[2]]), k)
    assert sc[0] == pytest.approx(1.0, abs=1e-10)
    assert sc[1] == pytest.approx(0.0, abs=1e-10)
    sc2 = oracle.alignment_scores(np.stack([K[0], K[3]]), k)
    assert sc2[0] == pytest.approx((k - 1 + math.cos(th) ** 2) / k, abs=1e-10)


@pytest.mark.parametrize("scores,want", [
    # every score equal to the median never falls below it: groups close at eight layers
    ([0.5] * 31, [0, 8, 16, 24, 32]),
    # a drop below the median after layer 2 (score index 2 -> new group at layer 3), then high scores
    ([0.9, 0.9, 0.1, 0.9, 0.9, 0.9, 0.9], [0, 3, 8]),
    # a drop right after the first layer is ignored (the group needs two layers first)
    ([0.1, 0.9, 0.9, 0.1, 0.9, 0.9], [0, 4, 7]),
    # a drop before the last layer would leave a single layer: it joins its predecessor
    ([0.9, 0.9, 0.9, 0.1], [0, 5]),
    # drops every other pair of layers: groups of two
    ([0.9, 0.1, 0.9, 0.1, 0.9, 0.1, 0.9], [0, 2, 4, 6, 8]),
    # ten layers of high alignment: closed at eight, the trailing two form their own group
    ([0.9] * 9, [0, 8, 10]),
    # nine layers of equal score: closed at eight, the trailing single layer is merged (nine layers)
    ([0.5] * 8, [0, 9]),
])
def test_grouping_rules_by_hand(scores, want):
    assert oracle.group_layers(scores) == want


def test_grouping_median_of_the_whole_network():
    # median of [0.2, 0.4, 0.6, 0.8, 1.0] is 0.6: the scores 0.2 (layers 1-2) and 0.4 (layers 3-4) fall
    # below it, each after a group of two layers; 0.6 itself does not
    assert oracle.group_layers([1.0, 0.2, 0.8, 0.4, 0.6]) == [0, 2, 4, 6]
    assert oracle.group_layers([1.0, 0.2, 0.8, 0.4, 0.59]) == [0, 2, 4, 6]
    assert oracle.group_layers([1.0, 0.2, 0.8, 0.4, 0.7, 0.3, 0.9]) == [0, 2, 4, 6, 8]


def test_grouping_sizes_always_within_bounds():
    rng = np.random.default_rng(3)
    for L in (2, 3, 9, 17, 32, 40, 80):
        for _ in range(20):
            g = oracle.group_layers(rng.random(L - 1))
            sizes = np.diff(g)
            assert g[0] == 0 and g[-1] == L and np.all(sizes >= 1)
            assert np.all(sizes[:-1] <= 8) and sizes[-1] <= 9
            if len(sizes) > 1:
                assert np.all(sizes >= 2)
