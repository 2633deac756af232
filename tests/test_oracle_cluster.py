"""Pins of the balanced spherical k-means oracle (oracle/cluster_oracle.py)
against hand-worked examples, closed forms, brute force and invariants."""

import json
import os

import numpy as np
import pytest
from scipy.stats import chisquare

from oracle import cluster_oracle as co

HERE = os.path.dirname(__file__)


def _golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def test_balanced_assign_hand_worked_rounds():
    g = _golden("balanced_assign.json")
    asg = co.balanced_assign(np.array(g["sims"]), g["b"])
    assert asg.tolist() == g["assign"]
    _, c2t = co.update_centroids(np.eye(6), asg, 3)
    assert c2t.tolist() == g["c2t"]


def _rounds_by_loops(S, b):
    """The same reading written as plain per-token loops (no numpy ranking)."""
    v, c = len(S), len(S[0])
    asg = [-1] * v
    fill = [0] * c
    while -1 in asg:
        props = {}
        for t in range(v):
            if asg[t] >= 0:
                continue
            best, bv = -1, None
            for k in range(c):
                if fill[k] < b and (bv is None or S[t][k] > bv):
                    best, bv = k, S[t][k]
            props.setdefault(best, []).append((bv, t))
        for k, lst in props.items():
            lst.sort(key=lambda x: (-x[0], x[1]))
            for bv, t in lst[: b - fill[k]]:
                asg[t] = k
            fill[k] += min(len(lst), b - fill[k])
    return asg


@pytest.mark.parametrize("seed,v,c", [(0, 12, 3), (1, 20, 5), (2, 24, 8), (3, 30, 30), (4, 16, 1)])
def test_balanced_assign_matches_loop_form_and_is_balanced(seed, v, c):
    rng = np.random.default_rng(seed)
    # values on a coarse grid, so that equal similarities (ties) occur
    S = np.round(rng.random((v, c)) * 8) / 8
    b = v // c
    asg = co.balanced_assign(S, b)
    assert asg.tolist() == _rounds_by_loops(S.tolist(), b)
    assert np.all(np.bincount(asg, minlength=c) == b)


def test_balanced_assign_is_argmax_when_capacity_never_binds():
    rng = np.random.default_rng(5)
    c, b = 6, 4
    S = rng.random((c * b, c)) * 0.5
    for t in range(c * b):
        S[t, t % c] = 1.0 + rng.random()  # each cluster is the favourite of exactly b tokens
    asg = co.balanced_assign(S, b)
    assert np.array_equal(asg, S.argmax(axis=1))


def test_kmeanspp_hand_worked():
    g = _golden("kmeanspp.json")
    Xn = co.normalize_rows(np.array(g["E"]))
    assert co.kmeanspp(Xn, 2, g["u"]).tolist() == g["centers"]


def test_kmeanspp_second_centre_follows_squared_distance():
    """With many uniforms the second centre's frequencies match D^2 / sum D^2."""
    rng = np.random.default_rng(7)
    Xn = co.normalize_rows(rng.standard_normal((12, 3)))
    first = 4
    w = co.pp_weights(Xn, [first])
    n = 40000
    u = rng.random(n)
    picks = np.array([co.pp_pick(w, x) for x in u])
    counts = np.bincount(picks, minlength=12)
    expected = w / w.sum() * n
    mask = expected > 0
    assert counts[~mask].sum() == 0  # the chosen centre itself has D = 0
    assert chisquare(counts[mask], expected[mask]).pvalue > 1e-4
    u0 = (first + 0.5) / 12
    assert co.kmeanspp(Xn, 1, [u0]).tolist() == [first]


def test_update_is_normalised_sum_and_c2t_ascending():
    rng = np.random.default_rng(8)
    Xn = co.normalize_rows(rng.standard_normal((12, 4)))
    asg = np.array([2, 0, 1, 2, 0, 1, 1, 0, 2, 2, 1, 0])
    C, c2t = co.update_centroids(Xn, asg, 3)
    for k in range(3):
        members = [t for t in range(12) if asg[t] == k]
        s = sum(Xn[t] for t in members)
        assert np.allclose(C[k], s / np.linalg.norm(s), atol=1e-14)
        assert c2t[k].tolist() == members
    same = np.tile(Xn[:1], (4, 1))
    C1, _ = co.update_centroids(same, np.array([0, 0, 1, 1]), 2)
    assert np.allclose(C1, np.tile(Xn[:1], (2, 1)), atol=1e-14)


def test_adjusted_rand_index_closed_forms():
    a = np.repeat(np.arange(4), 5)
    assert co.adjusted_rand_index(a, a) == pytest.approx(1.0)
    assert co.adjusted_rand_index(a, (a + 1) % 4) == pytest.approx(1.0)  # relabelled
    # worked by hand: contingency [[2, 1, 0], [0, 1, 2]] gives sum C(n_ij, 2) = 2,
    # row sums C(3, 2) + C(3, 2) = 6, column sums 3 * C(2, 2) = 3, C(6, 2) = 15:
    # ARI = (2 - 6*3/15) / (0.5*(6 + 3) - 6*3/15) = 0.8 / 3.3
    x = [0, 0, 0, 1, 1, 1]
    y = [0, 0, 1, 1, 2, 2]
    assert co.adjusted_rand_index(x, y) == pytest.approx(0.8 / 3.3)
    rng = np.random.default_rng(9)
    r = rng.integers(0, 10, 5000)
    assert abs(co.adjusted_rand_index(r, rng.integers(0, 10, 5000))) < 0.01


def test_balanced_kmeans_recovers_planted_clusters():
    """Planted, well separated clusters of exactly b tokens are recovered
    (ARI 1), every cluster is exactly b, and the pages' quality check holds
    (mean intra-cluster cosine above 0.6, explainer §5.3)."""
    rng = np.random.default_rng(10)
    c, b, d = 16, 32, 48
    mu = co.normalize_rows(rng.standard_normal((c, d)))
    truth = rng.permutation(np.repeat(np.arange(c), b))
    E = mu[truth] + 0.3 * rng.standard_normal((c * b, d)) / np.sqrt(d)
    res = co.balanced_kmeans(E, c, iters=5, u=rng.random(c))
    assert np.all(np.bincount(res.assign, minlength=c) == b)
    assert sorted(res.c2t.ravel().tolist()) == list(range(c * b))
    assert co.adjusted_rand_index(res.assign, truth) > 0.99
    assert co.intra_cluster_cosine(co.normalize_rows(E), res.c2t).min() > 0.6
