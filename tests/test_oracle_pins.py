"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks an oracle function against something other than itself:
hand-worked fixtures, closed forms, brute-force enumeration or a library
routine.  Citations name the FlashHead explainer (framerc.cn) section whose
definition the pin follows.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import flashhead_oracle as fo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- fixtures --

def test_toy_two_stage_fixture():
    """Hand-worked toy head (§1.2.1, §1.2.2, §1.2.4, §1.1)."""
    g = _load("toy_two_stage.json")
    E = np.array(g["E"], dtype=np.float64)
    C = np.array(g["C"], dtype=np.float32)
    c2t = np.array(g["C2T"])
    head = oracle.OracleHead(E, C, c2t)
    for case in g["cases"]:
        h = np.array(case["h"], dtype=np.float64)
        s = oracle.score(head.C_hat, h)[0]
        assert s.tolist() == case["scores"]
        dn = head.dense(h)
        assert dn.token[0] == case["dense_token"]
        for p, want in case["by_p"].items():
            r = head.forward(h, int(p))
            assert r.sel.S[0].tolist() == want["S"]
            assert r.ids[0].tolist() == want["ids"]
            assert r.z[0].tolist() == want["z"]
            assert r.fin.token[0] == want["token"]
            assert r.fin.token_logit[0] == want["token_logit"]
            lse = math.log(math.fsum(math.exp(x) for x in want["z"]))
            assert abs(r.fin.lse[0] - lse) < 1e-12


def test_int4_fixture_codes():
    """Hand-worked INT4 codes and scales (§1.2.4, §2.3)."""
    g = _load("int4_groups.json")
    rows = [grp["x"] for grp in g["groups"]]
    C = np.array(rows, dtype=np.float32)
    q, sigma = oracle.quantize_int4_g32(C)
    for r, grp in enumerate(g["groups"]):
        assert float(sigma[r, 0]) == grp["sigma"]
        assert q[r].tolist() == grp["q"]


# ------------------------------------------------------------------ C2T ----

def test_validate_c2t_accepts_permutation_and_rejects_others():
    """Balanced clusters: exactly b tokens each, each token once (§1.2.1)."""
    rng = np.random.default_rng(3)
    v, c = 64, 16
    b = v // c
    good = rng.permutation(v).reshape(c, b)
    assert oracle.validate_c2t(good, v, c, b).shape == (c, b)
    dup = good.copy()
    dup[0, 0] = dup[0, 1]
    with pytest.raises(ValueError):
        oracle.validate_c2t(dup, v, c, b)
    oob = good.copy()
    oob[1, 1] = v
    with pytest.raises(ValueError):
        oracle.validate_c2t(oob, v, c, b)
    neg = good.copy()
    neg[2, 2] = -1
    with pytest.raises(ValueError):
        oracle.validate_c2t(neg, v, c, b)
    with pytest.raises(ValueError):
        oracle.validate_c2t(good.reshape(b, c), v, c, b)
    with pytest.raises(ValueError):
        oracle.validate_c2t(good, v + 1, c, b)


# ------------------------------------------------------------ quantiser ----

def test_int4_exact_round_trip_on_representable_rows():
    """Rows made of q*sigma with max|q| = 7 quantise back exactly."""
    rng = np.random.default_rng(5)
    c, d = 16, 128
    sig = rng.uniform(1e-3, 2.0, size=(c, d // 32)).astype(np.float16)
    assert np.all(sig > 0)
    qs = rng.integers(-7, 8, size=(c, d // 32, 32))
    qs[:, :, 0] = rng.choice([-7, 7], size=(c, d // 32))  # amax = 7 sigma
    C = (sig.astype(np.float32)[..., None] * qs.astype(np.float32)).reshape(c, d)
    q, sigma = oracle.quantize_int4_g32(C)
    assert np.array_equal(sigma, sig)
    assert np.array_equal(q.reshape(c, d // 32, 32), qs)
    assert np.array_equal(oracle.dequantize_int4(q, sigma), C.astype(np.float64))


def test_int4_error_bound_and_amax():
    """|C - C_hat| <= sigma/2 (plus fp16 scale rounding); amax maps to +-7."""
    rng = np.random.default_rng(6)
    C = rng.standard_normal((32, 256)).astype(np.float32)
    q, sigma = oracle.quantize_int4_g32(C)
    Ch = oracle.dequantize_int4(q, sigma)
    s = sigma.astype(np.float64).repeat(32, axis=1)
    err = np.abs(C.astype(np.float64) - Ch)
    # the scale is amax/7 rounded to fp16 (relative error <= 2^-11), so the
    # clamped top code can miss amax by at most 7 * sigma * 2^-11 beyond sigma/2
    assert np.all(err <= s / 2 + 7 * s * 2.0 ** -10)
    g = np.abs(C).reshape(32, 8, 32)
    arg = g.argmax(axis=2)
    top = np.take_along_axis(q.reshape(32, 8, 32), arg[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 7)
    assert q.min() >= -7 and q.max() <= 7


def test_int4_pack_unpack_brute_force():
    """Low nibble first, two's complement (element 2m -> low nibble of byte m)."""
    rng = np.random.default_rng(7)
    q = rng.integers(-8, 8, size=(4, 64)).astype(np.int8)
    packed = oracle.pack_int4(q)
    for r in range(4):
        for m in range(32):
            lo = int(q[r, 2 * m]) & 0xF
            hi = int(q[r, 2 * m + 1]) & 0xF
            assert packed[r, m] == lo | (hi << 4)
    assert np.array_equal(oracle.unpack_int4(packed), q)


def test_int4_rejects_bad_shapes_and_overflow():
    with pytest.raises(ValueError):
        oracle.quantize_int4_g32(np.ones((2, 48), dtype=np.float32))
    with pytest.raises(OverflowError):
        oracle.quantize_int4_g32(np.full((1, 32), 1e6, dtype=np.float32))


def test_int8_fixture_codes():
    """Hand-worked INT8 codes and scales (W8A16, §5.2; scheme as INT4 with 127)."""
    g = _load("int8_groups.json")
    C = np.array([grp["x"] for grp in g["groups"]], dtype=np.float32)
    q, sigma = oracle.quantize_int8_g32(C)
    for r, grp in enumerate(g["groups"]):
        assert float(sigma[r, 0]) == grp["sigma"]
        assert q[r].tolist() == grp["q"]


def test_int8_exact_round_trip_on_representable_rows():
    """Rows of q*sigma with a power-of-two sigma and max|q| = 127 quantise
    back exactly (amax/127 = sigma exactly, and every quotient is an
    integer)."""
    rng = np.random.default_rng(15)
    c, d = 8, 128
    sig = (2.0 ** rng.integers(-12, 2, size=(c, d // 32))).astype(np.float16)
    qs = rng.integers(-127, 128, size=(c, d // 32, 32))
    qs[:, :, 3] = rng.choice([-127, 127], size=(c, d // 32))
    C = (sig.astype(np.float32)[..., None] * qs.astype(np.float32)).reshape(c, d)
    q, sigma = oracle.quantize_int8_g32(C)
    assert np.array_equal(sigma, sig)
    assert np.array_equal(q.reshape(c, d // 32, 32), qs)
    assert np.array_equal(oracle.dequantize_int8(q, sigma), C.astype(np.float64))


def test_int8_error_bound_and_amax():
    """|C - C_hat| <= sigma/2 (plus fp16 scale rounding); amax maps to +-127;
    and INT8 is closer to C than INT4 on the same rows."""
    rng = np.random.default_rng(16)
    C = rng.standard_normal((32, 256)).astype(np.float32)
    q, sigma = oracle.quantize_int8_g32(C)
    Ch = oracle.dequantize_int8(q, sigma)
    s = sigma.astype(np.float64).repeat(32, axis=1)
    err = np.abs(C.astype(np.float64) - Ch)
    assert np.all(err <= s / 2 + 127 * s * 2.0 ** -10)
    g = np.abs(C).reshape(32, 8, 32)
    arg = g.argmax(axis=2)
    top = np.take_along_axis(q.reshape(32, 8, 32), arg[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert q.min() >= -127 and q.max() <= 127
    q4, s4 = oracle.quantize_int4_g32(C)
    assert err.max() < np.abs(C - oracle.dequantize_int4(q4, s4)).max() / 8


def test_int8_rejects_bad_shapes_and_overflow():
    with pytest.raises(ValueError):
        oracle.quantize_int8_g32(np.ones((2, 48), dtype=np.float32))
    with pytest.raises(OverflowError):  # 1e7 / 127 exceeds the largest fp16
        oracle.quantize_int8_g32(np.full((1, 32), 1e7, dtype=np.float32))


def test_int8_head_scores_are_the_group_sums():
    """Stage-1 scores of an INT8 head: sum_g sigma_g sum_{i in g} q_i h_i,
    written out with math.fsum."""
    rng = np.random.default_rng(17)
    c, d, v = 4, 64, 8
    C = rng.standard_normal((c, d)).astype(np.float32)
    E = rng.standard_normal((v, d)).astype(np.float32)
    H = rng.standard_normal((2, d)).astype(np.float32)
    head = oracle.OracleHead(E, C, np.arange(v).reshape(c, 2), "int8")
    q, sigma = oracle.quantize_int8_g32(C)
    s = oracle.score(head.C_hat, H)
    for b in range(2):
        for k in range(c):
            want = math.fsum(float(sigma[k, g]) * math.fsum(int(q[k, 32 * g + i]) * float(H[b, 32 * g + i])
                                                            for i in range(32))
                             for g in range(d // 32))
            assert abs(s[b, k] - want) <= 1e-12 * (1 + abs(want))


# ---------------------------------------------------------------- stage 1 --

def test_score_matches_fsum_on_tiny_inputs():
    """s = C h as a textbook dot product, compared with math.fsum."""
    rng = np.random.default_rng(8)
    C = rng.standard_normal((5, 7))
    H = rng.standard_normal((3, 7))
    s = oracle.score(C, H)
    for b in range(3):
        for k in range(5):
            want = math.fsum(float(C[k, i]) * float(H[b, i]) for i in range(7))
            assert abs(s[b, k] - want) <= 1e-14 * max(1.0, abs(want))


def test_score_on_basis_rows_returns_h_entries():
    """Centroid rows that are basis vectors read out the entries of h."""
    d = 16
    C = np.eye(d)[[3, 0, 15, 7]]
    h = np.arange(d, dtype=np.float64) * 0.25 - 1.0
    assert oracle.score(C, h)[0].tolist() == [h[3], h[0], h[15], h[7]]


# ---------------------------------------------------------------- select ---

def test_select_topk_matches_brute_force_sort():
    """Top-p by score, ascending ids, ties to the smaller id (§1.2.2)."""
    rng = np.random.default_rng(9)
    # few distinct values force many ties
    s = rng.integers(-3, 4, size=(6, 40)).astype(np.float64) * 0.5
    for p in (1, 5, 17, 40):
        sel = oracle.select(s, p)
        for r in range(6):
            ranked = sorted(range(40), key=lambda k: (-s[r, k], k))
            assert sel.S[r].tolist() == sorted(ranked[:p])
            assert sel.theta[r] == np.float32(s[r, ranked[p - 1]])


def test_select_p1_is_argmax_and_p_eq_c_is_everything():
    rng = np.random.default_rng(10)
    s = rng.standard_normal((4, 33))
    assert oracle.select(s, 1).S[:, 0].tolist() == np.argmax(s, axis=1).tolist()
    assert np.array_equal(oracle.select(s, 33).S, np.tile(np.arange(33), (4, 1)))
    with pytest.raises(ValueError):
        oracle.select(s, 0)
    with pytest.raises(ValueError):
        oracle.select(s, 34)


def test_select_decides_in_float32():
    """Keys that differ only below float32 resolution tie, so the smaller id wins."""
    s = np.array([[1.0, 1.0 + 1e-12, 0.5]])
    assert oracle.select(s, 1).S[0].tolist() == [0]


# ---------------------------------------------------------------- stage 2 --

def test_p_equals_c_reproduces_dense_head():
    """With every cluster probed the retrieved logits are the dense logits,
    permuted by C2T, and the token is the dense argmax (§1.2, §1.1)."""
    rng = np.random.default_rng(11)
    v, d, c = 96, 24, 12
    b = v // c
    E = rng.standard_normal((v, d)).astype(np.float32)
    C = rng.standard_normal((c, d)).astype(np.float32)
    c2t = rng.permutation(v).reshape(c, b)
    H = rng.standard_normal((5, d))
    head = oracle.OracleHead(E, C, c2t)
    r = head.forward(H, c)
    zd = H @ E.astype(np.float64).T  # brute force, all tokens
    for q in range(5):
        assert r.ids[q].tolist() == c2t.reshape(-1).tolist()
        assert np.allclose(r.z[q], zd[q, c2t.reshape(-1)], rtol=0, atol=1e-12)
        assert r.fin.token[q] == int(np.argmax(zd[q]))
        assert abs(r.fin.lse[q] - scipy.special.logsumexp(zd[q])) < 1e-12
    dn = head.dense(H)
    assert dn.token.tolist() == np.argmax(zd, axis=1).tolist()


def test_gather_brute_force_loop():
    rng = np.random.default_rng(12)
    v, d, c = 40, 8, 10
    b = v // c
    E = rng.standard_normal((v, d))
    c2t = rng.permutation(v).reshape(c, b)
    H = rng.standard_normal((2, d))
    S = np.array([[1, 4, 9], [0, 2, 3]])
    ids, z = oracle.gather(E, c2t, S, H)
    for q in range(2):
        pos = 0
        for k in S[q]:
            for j in range(b):
                t = c2t[k, j]
                assert ids[q, pos] == t
                want = math.fsum(E[t, i] * H[q, i] for i in range(d))
                assert abs(z[q, pos] - want) < 1e-13
                pos += 1


# ---------------------------------------------------------------- finish ---

def test_finish_argmax_ties_and_lse():
    ids = np.array([[7, 3, 9, 1]])
    z = np.array([[2.0, 5.0, 5.0, -1.0]])
    f = oracle.finish(ids, z)
    assert f.token[0] == 3 and f.token_logit[0] == 5.0
    assert abs(f.lse[0] - scipy.special.logsumexp(z[0])) < 1e-14
    ids2 = np.array([[9, 3]])
    f2 = oracle.finish(ids2, np.array([[5.0, 5.0]]))
    assert f2.token[0] == 3  # smaller token id, not the first position


def test_finish_lse_uses_temperature_only_when_sampling():
    ids = np.arange(6)[None]
    z = np.linspace(-2, 3, 6)[None]
    g = oracle.finish(ids, z, mode=0, temperature=0.5)
    assert abs(g.lse[0] - scipy.special.logsumexp(z[0])) < 1e-13
    s = oracle.finish(ids, z, mode=fo.MODE_TOKEN_SAMPLE, temperature=0.5, seed=1)
    assert abs(s.lse[0] - scipy.special.logsumexp(z[0] / 0.5)) < 1e-13


def test_small_temperature_sampling_reduces_to_argmax():
    """As T -> 0 temperature sampling becomes greedy (top-2 gap >> 20 T)."""
    rng = np.random.default_rng(13)
    z = rng.standard_normal((200, 50))
    ids = np.tile(np.arange(50), (200, 1))
    top2 = np.sort(z, axis=1)[:, -2:]
    keep = (top2[:, 1] - top2[:, 0]) > 0.05
    f = oracle.finish(ids, z, mode=fo.MODE_TOKEN_SAMPLE, temperature=1e-3, seed=4)
    assert np.array_equal(f.token[keep], np.argmax(z, axis=1)[keep])


def test_sampling_rejects_nonpositive_temperature():
    s = np.zeros((1, 4))
    with pytest.raises(ValueError):
        oracle.select(s, 2, mode=fo.MODE_PROBE_SAMPLE, temperature=0.0)
    with pytest.raises(ValueError):
        oracle.finish(np.arange(4)[None], s, mode=fo.MODE_TOKEN_SAMPLE, temperature=-1.0)


def test_gumbel_keys_depend_on_token_id_not_position():
    """Token noise is keyed by token id: permuting candidates permutes nothing else."""
    rng = np.random.default_rng(14)
    z = rng.standard_normal((1, 30))
    ids = np.arange(30)[None]
    perm = rng.permutation(30)
    a = oracle.finish(ids, z, mode=fo.MODE_TOKEN_SAMPLE, temperature=0.8, seed=77)
    b = oracle.finish(ids[:, perm], z[:, perm], mode=fo.MODE_TOKEN_SAMPLE, temperature=0.8, seed=77)
    assert a.token[0] == b.token[0]
    assert abs(a.lse[0] - b.lse[0]) < 1e-12


def test_enumerated_plackett_luce_helper_is_a_distribution():
    """Sanity of the closed form the sampling tests use."""
    w = np.array([0.1, 0.5, 1.3, 0.7, 2.0])
    tot = 0.0
    for S in itertools.combinations(range(5), 3):
        tot += _pl_set_prob(w, S)
    assert abs(tot - 1.0) < 1e-12


def _pl_set_prob(w, S):
    """P(set S) for sequential draws without replacement with weights w."""
    W = w.sum()
    total = 0.0
    for order in itertools.permutations(S):
        pr, used = 1.0, 0.0
        for k in order:
            pr *= w[k] / (W - used)
            used += w[k]
        total += pr
    return total


# ------------------------------------------------------ batch-shared probes --

def test_shared_selection_hand_worked():
    """Summed scores (explainer §4.2, read as the top p of sum_b s[b, k]):
    rows (1, 0, 3, 2, 0), (0, 4, 0, 1, 1), (2, 0, 0, 0, 1) sum to
    (3, 4, 3, 3, 2); p = 3 takes cluster 1 and then two of the three tied at 3,
    by the smaller id: {0, 1, 2}."""
    s = np.array([[1, 0, 3, 2, 0], [0, 4, 0, 1, 1], [2, 0, 0, 0, 1]], dtype=np.float64)
    sel = oracle.select(s, 3, oracle.MODE_PROBE_SHARED)
    assert sel.S.tolist() == [[0, 1, 2]] * 3
    assert float(sel.theta[0]) == 3.0


def test_shared_selection_reductions_and_invariances():
    rng = np.random.default_rng(21)
    s = rng.standard_normal((6, 40))
    one = oracle.select(s[2:3], 7, oracle.MODE_PROBE_SHARED)
    assert np.array_equal(one.S, oracle.select(s[2:3], 7).S)  # B = 1: per-query top-p
    sh = oracle.select(s, 7, oracle.MODE_PROBE_SHARED).S
    assert np.all(sh == sh[0])                                 # one set for every row
    perm = rng.permutation(6)
    assert np.array_equal(oracle.select(s[perm], 7, oracle.MODE_PROBE_SHARED).S, sh)
    top = np.argsort(-s.sum(axis=0), kind="stable")[:7]
    assert sorted(top.tolist()) == sh[0].tolist()
    with pytest.raises(ValueError):
        oracle.select(s, 7, oracle.MODE_PROBE_SHARED | oracle.MODE_PROBE_SAMPLE, 1.0)


def test_shared_probes_with_all_clusters_reproduce_the_dense_head():
    """p = c: every row retrieves every token, as the dense head does."""
    rng = np.random.default_rng(22)
    v, c, d = 48, 6, 8
    E = rng.standard_normal((v, d))
    C = rng.standard_normal((c, d))
    c2t = rng.permutation(v).reshape(c, v // c)
    H = rng.standard_normal((3, d))
    head = oracle.OracleHead(E, C, c2t)
    r = head.forward(H, c, oracle.MODE_PROBE_SHARED)
    dn = oracle.dense(E, H)
    assert np.array_equal(r.fin.token, dn.token)
    assert np.allclose(r.fin.lse, dn.lse, rtol=1e-12)
