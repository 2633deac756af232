"""Distribution pins for the oracle's sampling stages.

Probe sampling (FlashHead explainer, framerc.cn, §1.2.3: multinomial
sampling over clusters with temperature) is read as p draws without
replacement from softmax(s/T).  Its closed form is the Plackett-Luce set
probability, enumerated here on tiny inputs.  Token sampling draws from
softmax(z/T) over the retrieved set, so the token marginal is
sum_S P(S) softmax_{R(S)}(z/T)_t.  Each test draws many independent samples
(the rows of one batched call get independent Philox streams), and checks
the frequencies with a chi-square test at fixed seeds.
"""

import itertools

import numpy as np
from scipy import stats

import oracle
from oracle import flashhead_oracle as fo

N = 1 << 16
PMIN = 1e-4


def _pl_set_prob(w, S):
    W = w.sum()
    total = 0.0
    for order in itertools.permutations(S):
        pr, used = 1.0, 0.0
        for k in order:
            pr *= w[k] / (W - used)
            used += w[k]
        total += pr
    return total


def _chi2_ok(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    exp = np.asarray(probs, dtype=np.float64) * counts.sum()
    keep = exp > 0
    assert counts[~keep].sum() == 0, "mass on an impossible outcome"
    pv = stats.chisquare(counts[keep], exp[keep]).pvalue
    assert pv > PMIN, f"chi-square p-value {pv}"
    return pv


def test_probe_sampling_p1_is_softmax():
    s = np.array([0.3, -1.0, 1.2, 0.0, 0.8, -0.4])
    T = 0.7
    rows = np.tile(s, (N, 1))
    sel = oracle.select(rows, 1, mode=fo.MODE_PROBE_SAMPLE, temperature=T, seed=11)
    counts = np.bincount(sel.S[:, 0], minlength=6)
    _chi2_ok(counts, scipy_softmax(s / T))


def test_probe_sampling_sets_follow_plackett_luce():
    s = np.array([0.9, -0.2, 0.4, 1.5, 0.0])
    T = 1.0
    w = np.exp(s / T)
    for p in (2, 3):
        rows = np.tile(s, (N, 1))
        sel = oracle.select(rows, p, mode=fo.MODE_PROBE_SAMPLE, temperature=T, seed=100 + p)
        sets = list(itertools.combinations(range(5), p))
        index = {S: i for i, S in enumerate(sets)}
        counts = np.zeros(len(sets))
        for r in sel.S:
            counts[index[tuple(r.tolist())]] += 1
        probs = [_pl_set_prob(w, S) for S in sets]
        assert abs(sum(probs) - 1) < 1e-12
        _chi2_ok(counts, probs)


def _tiny_head(seed):
    rng = np.random.default_rng(seed)
    v, d, c = 12, 4, 6
    b = v // c
    E = rng.standard_normal((v, d)).astype(np.float32) * 0.8
    C = rng.standard_normal((c, d)).astype(np.float32) * 0.6
    c2t = rng.permutation(v).reshape(c, b)
    h = rng.standard_normal(d)
    return oracle.OracleHead(E, C, c2t), h


def test_sampled_probes_then_sampled_token_marginal():
    """P(t) = sum_S PL(S) * softmax over S's tokens of z/T (c=6, b=2, p=2)."""
    head, h = _tiny_head(21)
    T, p = 0.9, 2
    s = oracle.score(head.C_hat, h)[0]
    z = np.asarray(head.E, dtype=np.float64) @ h
    w = np.exp(s / T)
    probs = np.zeros(head.v)
    for S in itertools.combinations(range(head.c), p):
        toks = head.c2t[list(S)].reshape(-1)
        probs[toks] += _pl_set_prob(w, S) * scipy_softmax(z[toks] / T)
    mode = fo.MODE_PROBE_SAMPLE | fo.MODE_TOKEN_SAMPLE
    r = head.forward(np.tile(h, (N, 1)), p, mode=mode, temperature=T, seed=5)
    counts = np.bincount(r.fin.token, minlength=head.v)
    _chi2_ok(counts, probs)


def test_topk_probes_then_sampled_token():
    """Deterministic top-p clusters, then softmax(z/T) over their tokens."""
    head, h = _tiny_head(22)
    T, p = 0.7, 3
    s = oracle.score(head.C_hat, h)[0]
    S = sorted(sorted(range(head.c), key=lambda k: (-s[k], k))[:p])
    toks = head.c2t[S].reshape(-1)
    z = np.asarray(head.E, dtype=np.float64) @ h
    probs = np.zeros(head.v)
    probs[toks] = scipy_softmax(z[toks] / T)
    r = head.forward(np.tile(h, (N, 1)), p, mode=fo.MODE_TOKEN_SAMPLE, temperature=T, seed=6)
    _chi2_ok(np.bincount(r.fin.token, minlength=head.v), probs)


def test_all_probes_sampling_is_dense_softmax():
    """With p = c every token is retrieved: the draw is softmax(E h / T)."""
    head, h = _tiny_head(23)
    T = 1.3
    z = np.asarray(head.E, dtype=np.float64) @ h
    mode = fo.MODE_PROBE_SAMPLE | fo.MODE_TOKEN_SAMPLE
    r = head.forward(np.tile(h, (N, 1)), head.c, mode=mode, temperature=T, seed=7)
    _chi2_ok(np.bincount(r.fin.token, minlength=head.v), scipy_softmax(z / T))
    dn = head.dense(np.tile(h, (N, 1)), mode=fo.MODE_TOKEN_SAMPLE, temperature=T, seed=8)
    _chi2_ok(np.bincount(dn.token, minlength=head.v), scipy_softmax(z / T))


def scipy_softmax(x):
    from scipy.special import softmax
    return softmax(np.asarray(x, dtype=np.float64))
