"""Pins of the oracle's adaptive probe count (select_adaptive) against values
fixed by hand, by brute force over subsets and by the exact distribution of
sequential draws without replacement.

The rule (explainer §1.2.2 dynamic adjustment, §4.2 fewer probes for
confident queries; the reading of the design notes): clusters in key order,
stop at the first count whose softmax(s/T) mass reaches tau, clamp to
[p_min, p_max]."""

import itertools
import math

import numpy as np
import pytest

from oracle import select, select_adaptive


def _row(vals):
    return np.log(np.asarray(vals, dtype=np.float64))[None, :]


@pytest.mark.parametrize("tau,n", [(0.4, 1), (0.6, 2), (0.8, 3), (0.9, 4)])
def test_hand_worked_t1(tau, n):
    # softmax(ln [4, 2, 1, 1]) = [1/2, 1/4, 1/8, 1/8]: masses 0.5, 0.75, 0.875, 1
    a = select_adaptive(_row([4, 2, 1, 1]), 4, tau)
    assert int(a.n[0]) == n
    assert list(a.S[0]) == list(range(n)) + [-1] * (4 - n)
    np.testing.assert_allclose(a.mass[0], [0.5, 0.75, 0.875, 1.0], rtol=1e-12)


def test_hand_worked_permuted_ids():
    # the same weights on clusters 1, 3, 0, 2: order 1, 3, then the tie 0 / 2
    # goes to the smaller id; 0.8 needs three clusters, listed ascending
    a = select_adaptive(_row([1, 4, 1, 2]), 4, 0.8)
    assert list(a.order[0]) == [1, 3, 0, 2]
    assert int(a.n[0]) == 3
    assert list(a.S[0]) == [0, 1, 3, -1]


@pytest.mark.parametrize("T,tau,n", [(2.0, 0.6, 2), (2.0, 0.65, 3), (0.5, 0.7, 1),
                                     (0.5, 0.9, 2), (0.5, 0.95, 3)])
def test_hand_worked_temperature(T, tau, n):
    # softmax(ln [4, 2, 1, 1] / T) is proportional to [4, 2, 1, 1] ** (1/T):
    # T = 2: [2, sqrt 2, 1, 1] / (4 + sqrt 2): masses .369, .631, .815, 1
    # T = 1/2: [16, 4, 1, 1] / 22: masses .727, .909, .955, 1
    a = select_adaptive(_row([4, 2, 1, 1]), 4, tau, temperature=T)
    w = np.array([4.0, 2.0, 1.0, 1.0]) ** (1.0 / T)
    np.testing.assert_allclose(a.mass[0], np.cumsum(w) / w.sum(), rtol=1e-12)
    assert int(a.n[0]) == n


def test_brute_force_smallest_subset():
    """Greedy probes: the first n clusters by score are the heaviest n-set, so
    n is the size of the smallest subset of clusters whose mass reaches tau,
    and the chosen set is the heaviest subset of that size."""
    rng = np.random.default_rng(5)
    checked = 0
    for trial in range(60):
        c = 7
        s = rng.normal(0, 1.5, size=c)
        T = float(rng.choice([0.5, 1.0, 2.0]))
        tau = float(rng.uniform(0.2, 0.97))
        w = np.exp(s / T) / np.exp(s / T).sum()
        best = None
        near = False
        for n in range(1, c + 1):
            heavy = max(itertools.combinations(range(c), n), key=lambda idx: w[list(idx)].sum())
            m = w[list(heavy)].sum()
            near |= abs(m - tau) < 1e-9
            if m >= tau:
                best = (n, sorted(heavy))
                break
        if near:
            continue
        a = select_adaptive(s[None, :], c, tau, temperature=T)
        assert int(a.n[0]) == best[0], trial
        assert list(a.S[0, :best[0]]) == best[1], trial
        checked += 1
    assert checked >= 50


def test_tau_one_probes_up_to_p_max():
    rng = np.random.default_rng(11)
    s = rng.uniform(-3, 3, size=(4, 64))
    for p_max in (64, 40):
        a = select_adaptive(s, p_max, 1.0 - 1e-12)
        assert np.all(a.n == p_max)
        ref = select(s, p_max)
        np.testing.assert_array_equal(a.S, ref.S)


@pytest.mark.parametrize("mode", [0, 1])
def test_fixed_count_reduces_to_select(mode):
    # p_min = p_max = p: the adaptive rule picks the same set as a fixed p
    rng = np.random.default_rng(2 + mode)
    s = rng.normal(0, 2, size=(6, 300))
    for p in (1, 17, 128):
        a = select_adaptive(s, p, 0.5, p_min=p, mode=mode, temperature=0.8, seed=9)
        ref = select(s, p, mode=mode, temperature=0.8, seed=9)
        assert np.all(a.n == p)
        np.testing.assert_array_equal(a.S, ref.S)


def test_clamps():
    rng = np.random.default_rng(4)
    s = rng.normal(0, 1, size=(5, 200))  # flat: 0.99 of the mass needs most clusters
    a = select_adaptive(s, 32, 0.99, p_min=4)
    assert np.all(a.n == 32)
    a = select_adaptive(s, 32, 1e-9, p_min=4)  # one cluster would do: clamped up
    assert np.all(a.n == 4)
    np.testing.assert_array_equal(a.S[:, :4], select(s, 4).S)
    assert np.all(a.S[:, 4:] == -1)


def test_peaked_rows_stop_earlier():
    # the point of the rule: a confident (peaked) query needs fewer probes
    rng = np.random.default_rng(8)
    base = rng.normal(0, 1, size=256)
    peaked = base.copy()
    peaked[17] += 12.0
    a = select_adaptive(np.stack([base, peaked]), 128, 0.9)
    assert a.n[1] < a.n[0]
    assert a.n[1] == 1 and a.S[1, 0] == 17


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_sampled_count_distribution(T):
    """Sampled probes: the order is a sequence of draws without replacement
    from softmax(s/T), and the count depends on which clusters came first.
    For c = 3 the law of n follows from the six draw orders; 20000 rows
    (independent noise per row) must match it within 4 sigma."""
    s = np.array([1.0, 0.5, -0.5])
    w = np.exp(s / T) / np.exp(s / T).sum()
    tau = 0.6
    law = np.zeros(4)
    for perm in itertools.permutations(range(3)):
        pr, left = 1.0, 1.0
        for k in perm:
            pr *= w[k] / left
            left -= w[k]
        m = np.cumsum(w[list(perm)])
        law[int(np.nonzero(m >= tau)[0][0]) + 1] += pr
    B = 20000
    a = select_adaptive(np.tile(s, (B, 1)), 3, tau, mode=1, temperature=T, seed=123)
    freq = np.bincount(a.n, minlength=4) / B
    for n in range(1, 4):
        sigma = math.sqrt(max(law[n] * (1 - law[n]), 1e-12) / B)
        assert abs(freq[n] - law[n]) <= 4 * sigma + 1e-12, (n, freq, law)
    assert np.sum(law > 0.05) >= 2  # the case is not degenerate


def test_argument_checks():
    s = np.zeros((1, 8))
    for kw in (dict(p_max=9, tau=0.5), dict(p_max=4, tau=0.0), dict(p_max=4, tau=1.5),
               dict(p_max=4, tau=0.5, p_min=5)):
        with pytest.raises(ValueError):
            select_adaptive(s, **kw)
    with pytest.raises(ValueError):
        select_adaptive(s, 4, 0.5, mode=4)
