"""Pins of the speculative-sampling oracle (oracle/spec_oracle.py): the
standard rule's guarantees, checked by closed forms and by distribution
tests over many independent rows (each row of a batch draws its own Philox
noise, so B copies of one hidden state are B independent trials)."""

import numpy as np
import pytest
from scipy.stats import binomtest, chisquare

import oracle
from oracle import spec_oracle as so

TSAMPLE, PSAMPLE = oracle.MODE_TOKEN_SAMPLE, oracle.MODE_PROBE_SAMPLE


def _tiny(seed=0, v=24, c=6, d=8, scale=1.5):
    rng = np.random.default_rng(seed)
    E = rng.standard_normal((v, d))
    C = rng.standard_normal((c, d))
    c2t = rng.permutation(v).reshape(c, v // c)
    h = scale * rng.standard_normal(d)
    return E, C, c2t, h


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


def _draft(E, C, c2t, h, n, p, mode, T, seed):
    head = oracle.OracleHead(E, C, c2t)
    H = np.repeat(h[None, :], n, axis=0)
    r = head.forward(H, p, mode, T, seed)
    return H, r.sel.S, r.fin.token, r.fin.lse


def _chi2(counts, probs, min_expected=5.0):
    """Chi-square p-value with bins of small expectation merged into one."""
    n = counts.sum()
    exp = probs * n
    big = exp >= min_expected
    obs = np.append(counts[big], counts[~big].sum())
    ex = np.append(exp[big], exp[~big].sum())
    keep = ex > 0
    return chisquare(obs[keep], ex[keep]).pvalue


def test_ratio_is_target_mass_of_the_probes():
    """With the draft scoring the same logits as the target, p(x)/q(x) =
    exp(LSE_S - LSE_full) = p(S) for every x in S, whatever x is."""
    E, C, c2t, h = _tiny(1)
    T = 0.8
    H, S, tok, _ = _draft(E, C, c2t, h, 64, 2, TSAMPLE, T, seed=3)
    r = so.spec_verify(E, c2t, H, S, tok, T, seed=4)
    p = _softmax(E @ h / T)
    mass = p[c2t[S[0]].ravel()].sum()
    assert np.allclose(r.ratio, mass, rtol=1e-12)


@pytest.mark.parametrize("p_probes,mode", [(1, TSAMPLE), (2, TSAMPLE), (2, PSAMPLE | TSAMPLE)])
def test_output_is_distributed_as_the_target(p_probes, mode):
    """The theorem of speculative sampling: the verified token is a draw from
    the dense head's softmax(E h / T), for top-p and for sampled probes."""
    E, C, c2t, h = _tiny(2)
    T = 1.0
    n = 30000
    H, S, tok, _ = _draft(E, C, c2t, h, n, p_probes, mode, T, seed=11)
    r = so.spec_verify(E, c2t, H, S, tok, T, seed=12)
    counts = np.bincount(r.token, minlength=E.shape[0])
    assert _chi2(counts, _softmax(E @ h / T)) > 1e-4
    # and the draft alone is not (it never leaves its probes' tokens)
    if p_probes == 1 and mode == TSAMPLE:
        assert _chi2(np.bincount(tok, minlength=E.shape[0]), _softmax(E @ h / T)) < 1e-6


def test_acceptance_rate_and_rejections():
    """Accepted with probability p(S); a rejected row's token lies outside
    the probes' tokens and follows p restricted to them."""
    E, C, c2t, h = _tiny(3)
    T = 1.2
    n = 30000
    H, S, tok, _ = _draft(E, C, c2t, h, n, 2, TSAMPLE, T, seed=21)
    r = so.spec_verify(E, c2t, H, S, tok, T, seed=22)
    p = _softmax(E @ h / T)
    inside = c2t[S[0]].ravel()
    mass = p[inside].sum()
    assert binomtest(int(r.accepted.sum()), n, mass).pvalue > 1e-4
    assert np.all(r.token[r.accepted] == tok[r.accepted])
    rej = r.token[~r.accepted]
    assert not np.isin(rej, inside).any()
    outside = np.setdiff1d(np.arange(E.shape[0]), inside)
    q_out = p[outside] / p[outside].sum()
    counts = np.array([(rej == t).sum() for t in outside])
    assert _chi2(counts, q_out) > 1e-4


def test_all_clusters_probed_always_accepts():
    """p = c: the draft is the target, the ratio is 1 and every draft is kept."""
    E, C, c2t, h = _tiny(4)
    H, S, tok, _ = _draft(E, C, c2t, h, 256, C.shape[0], TSAMPLE, 0.9, seed=31)
    r = so.spec_verify(E, c2t, H, S, tok, 0.9, seed=32)
    assert np.all(r.accepted) and np.array_equal(r.token, tok)
    assert np.allclose(r.ratio, 1.0)


def test_draft_outside_its_probes_is_accepted_and_bad_temperature_rejected():
    """q(x) = 0 makes the ratio infinite (min(1, .) = 1): accepted.  T must be > 0."""
    E, C, c2t, h = _tiny(5)
    S = np.array([[0]])
    x = np.array([c2t[1, 0]])
    r = so.spec_verify(E, c2t, h[None, :], S, x, 1.0, seed=1)
    assert r.accepted[0] and r.token[0] == x[0]
    with pytest.raises(ValueError):
        so.spec_verify(E, c2t, h[None, :], S, x, 0.0, seed=1)
