"""The parity checker itself, pinned: it must reject each plausible GPU
mistake and accept exactly the near-ties the rule certifies.

The rule (oracle/parity.py) encodes the targets of the FlashHead explainer
(framerc.cn): probe clusters by top-p score (§1.2.2) with ties at the
boundary certified when the keys differ by less than 1e-3, retrieved tokens
through C2T (§1.2.1), and logits, the token and the LSE within 2e-3 of the
oracle.  Each case builds a "GPU" result from the oracle's own answer and
plants one mistake in it (on the CPU; nothing here runs a kernel).
"""

import numpy as np
import pytest

import oracle
from oracle import parity
from oracle.flashhead_oracle import gather

# Eight clusters of two tokens in d = 8.  C is the identity, so s = h; token t
# of cluster k is E_t = a_t e_k, so z_t = a_t h_k: every key is chosen.
C = np.eye(8, dtype=np.float32)
C2T = np.array([[3, 12], [0, 9], [14, 5], [7, 1], [10, 4], [2, 15], [11, 6], [8, 13]],
               dtype=np.int32)
A = np.array([1.0, 0.5, 1.1, 2.0, 0.8, 1.3, 0.6, 0.9, 1.2, 0.7, 1.5, 0.4, 1.0, 0.3, 0.2, 1.4],
             dtype=np.float32)
E = np.zeros((16, 8), dtype=np.float32)
for k in range(8):
    for t in C2T[k]:
        E[t, k] = A[t]
# scores: cluster 1 (0.3004) is the 3rd largest, cluster 2 (0.3000) the 4th,
# 0.4 ms apart: a certified near-tie at p = 3; cluster 4 (0.1) is far below
H = np.array([[0.9, 0.3004, 0.3, 0.2, 0.1, -0.2, 0.7, -0.5]], dtype=np.float32)
P = 3


@pytest.fixture(scope="module")
def head():
    return oracle.OracleHead(E, C, C2T)


def result_for(head, S, h=H):
    """The exact answer on probe set S, keyed like FlashHead.forward."""
    ids, z = gather(head.E, head.c2t, np.asarray(S)[None, :], np.asarray(h, np.float64))
    fin = oracle.finish(ids, z, 0, 1.0, 0)
    return {"clusters": np.asarray(S, np.int32)[None, :], "ids": ids.astype(np.int32),
            "logits": z.astype(np.float32), "token": fin.token.astype(np.int32),
            "token_logit": fin.token_logit.astype(np.float32), "lse": fin.lse.astype(np.float32)}


def check(head, gpu):
    return parity.check_forward(head, H, P, 0, 1.0, 0, gpu)


def exact(head):
    return result_for(head, head.forward(H, P).sel.S[0])


def test_the_exact_answer_passes(head):
    ref = head.forward(H, P)
    assert ref.sel.S[0].tolist() == [0, 1, 6]
    rep = check(head, exact(head))
    assert rep.ok(), rep.failures
    assert rep.cluster_ties == 0 and rep.token_ties == 0


def test_probe_inside_the_tie_band_passes_and_is_counted(head):
    rep = check(head, result_for(head, [0, 2, 6]))  # cluster 2 for 1: keys 4e-4 apart
    assert rep.ok(), rep.failures
    assert rep.cluster_ties == 1


def test_probe_outside_the_tie_band_fails(head):
    rep = check(head, result_for(head, [0, 4, 6]))  # cluster 4 (0.1) for 1 (0.3004)
    assert not rep.ok()
    assert "beyond near-ties" in rep.failures[0]


def test_a_band_just_too_wide_fails(head):
    # the same swap with a gap of 1.2e-3: beyond the 1e-3 band
    h = H.copy()
    h[0, 1] = 0.3012
    ref = parity.check_forward(head, h, P, 0, 1.0, 0, result_for(head, [0, 2, 6], h))
    assert not ref.ok()


def test_probe_sets_that_are_not_p_ascending_ids_fail(head):
    for S in ([0, 1, 1], [6, 1, 0], [0, 1, 8]):
        gpu = exact(head)
        gpu["clusters"] = np.array([S], np.int32)
        assert not check(head, gpu).ok(), S


def test_swapped_ids_fail(head):
    gpu = exact(head)
    gpu["ids"][0, [0, 1]] = gpu["ids"][0, [1, 0]]
    gpu["logits"][0, [0, 1]] = gpu["logits"][0, [1, 0]]
    rep = check(head, gpu)
    assert not rep.ok() and "retrieved ids differ" in rep.failures[0]


def test_logits_one_percent_off_fail_and_within_tolerance_pass(head):
    gpu = exact(head)
    gpu["logits"][0, 3] *= np.float32(1.01)  # 5x the 2e-3 tolerance
    rep = check(head, gpu)
    assert not rep.ok() and "retrieved logit error" in rep.failures[0]
    gpu = exact(head)
    gpu["logits"][0, 3] *= np.float32(1.0005)  # a quarter of it
    assert check(head, gpu).ok()


def test_nan_outputs_fail(head):
    for key in ("logits", "token_logit", "lse"):
        gpu = exact(head)
        gpu[key].reshape(-1)[0] = np.nan
        assert not check(head, gpu).ok(), key


def test_token_not_retrieved_fails(head):
    gpu = exact(head)
    outside = sorted(set(range(16)) - set(gpu["ids"][0].tolist()))[0]
    gpu["token"][0] = outside
    rep = check(head, gpu)
    assert not rep.ok() and "not a candidate" in rep.failures[0]


def test_token_minus_one_fails(head):
    gpu = exact(head)
    gpu["token"][0] = -1  # what the single launch writes after a given-up wait
    assert not check(head, gpu).ok()


def test_wrong_token_beyond_a_tie_fails_and_a_certified_tie_passes():
    # tokens 3 and 12 (cluster 0): z = a_t * 0.9; a near-tie when a_12 is
    # within 1e-3 / 0.9 of a_3
    a = A.copy()
    a[12] = a[3] - np.float32(5e-4)  # z gap 4.5e-4 < 1e-3
    E2 = np.zeros_like(E)
    for k in range(8):
        for t in C2T[k]:
            E2[t, k] = a[t]
    head2 = oracle.OracleHead(E2, C, C2T)
    gpu = result_for(head2, [0, 1, 6])
    assert gpu["token"][0] == 3
    gpu["token"][0] = 12
    gpu["token_logit"][0] = gpu["logits"][0, list(gpu["ids"][0]).index(12)]
    rep = parity.check_forward(head2, H, P, 0, 1.0, 0, gpu)
    assert rep.ok(), rep.failures
    assert rep.token_ties == 1
    # the next best token (1: 2.0 * 0.3004 = 0.60) is 0.3 below: not a tie
    gpu["token"][0] = 7 if 7 in gpu["ids"][0] else 9
    gpu["token_logit"][0] = gpu["logits"][0, list(gpu["ids"][0]).index(int(gpu["token"][0]))]
    assert not parity.check_forward(head2, H, P, 0, 1.0, 0, gpu).ok()


def test_token_logit_and_lse_beyond_tolerance_fail(head):
    gpu = exact(head)
    gpu["token_logit"][0] *= np.float32(1.01)
    assert not check(head, gpu).ok()
    gpu = exact(head)
    lse = float(gpu["lse"][0])
    gpu["lse"][0] = np.float32(lse + 3e-3 * max(1.0, abs(lse)))
    rep = check(head, gpu)
    assert not rep.ok() and "lse error" in rep.failures[0]
    gpu = exact(head)
    gpu["lse"][0] = np.float32(lse + 1e-3 * max(1.0, abs(lse)))
    assert check(head, gpu).ok()


@pytest.mark.parametrize("key", parity.FORWARD_KEYS)
def test_a_missing_output_fails(head, key):
    gpu = exact(head)
    del gpu[key]
    rep = check(head, gpu)
    assert not rep.ok() and "lacks" in rep.failures[0]


def test_dense_checker_requires_the_token_and_rejects_a_wrong_one(head):
    z = (H.astype(np.float64) @ E.astype(np.float64).T)
    fin = oracle.dense(E, H)
    gpu = {"token": fin.token.astype(np.int32), "token_logit": fin.token_logit.astype(np.float32),
           "lse": fin.lse.astype(np.float32), "logits": z.astype(np.float32)}
    assert parity.check_dense(E, H, 0, 1.0, 0, gpu).ok()
    bad = dict(gpu, token=np.array([int(np.argsort(z[0])[-2])], np.int32))
    assert not parity.check_dense(E, H, 0, 1.0, 0, bad).ok()
    for key in parity.DENSE_KEYS:
        assert not parity.check_dense(E, H, 0, 1.0, 0, {k: v for k, v in gpu.items() if k != key}).ok()


# ---- adaptive probe count (check_adaptive): a count is certified when the
# oracle's mass at the GPU's cut is within mass_gap (1e-4) of tau

PMAX = 6


def adaptive_result(head, n, tau, p_max=PMAX):
    """The exact answer with the first n clusters of the oracle's key order."""
    a = oracle.select_adaptive(H @ head.C_hat.T, p_max, tau)
    S = np.sort(a.order[0, :n])
    out = result_for(head, S)
    b = head.b
    row = np.full((1, p_max), -1, np.int32)
    row[0, :n] = S
    ids = np.full((1, p_max * b), -1, np.int32)
    ids[0, :n * b] = out["ids"][0]
    z = np.full((1, p_max * b), -np.inf, np.float32)
    z[0, :n * b] = out["logits"][0]
    out.update(clusters=row, ids=ids, logits=z, nprobe=np.array([n], np.int32))
    return out, a


def check_a(head, gpu, tau):
    return parity.check_adaptive(head, H, PMAX, 1, tau, 0, 1.0, 0, gpu)


def test_adaptive_exact_answer_passes(head):
    a = oracle.select_adaptive(H @ head.C_hat.T, PMAX, 0.5)
    gpu, _ = adaptive_result(head, int(a.n[0]), 0.5)
    rep = check_a(head, gpu, 0.5)
    assert rep.ok(), rep.failures
    assert rep.count_ties == 0


def test_adaptive_count_off_by_one_fails(head):
    a = oracle.select_adaptive(H @ head.C_hat.T, PMAX, 0.5)
    n = int(a.n[0])
    for m in (n - 1, n + 1):
        gpu, _ = adaptive_result(head, m, 0.5)
        rep = check_a(head, gpu, 0.5)
        assert not rep.ok()
        assert "the oracle's mass allows" in rep.failures[0]


def test_adaptive_count_at_a_mass_near_tie_passes(head):
    a = oracle.select_adaptive(H @ head.C_hat.T, PMAX, 0.5)
    j = 1
    tau = float(a.mass[0, j]) + 5e-5  # the oracle needs j + 2; j + 1 falls short by 5e-5
    assert int(oracle.select_adaptive(H @ head.C_hat.T, PMAX, tau).n[0]) == j + 2
    gpu, _ = adaptive_result(head, j + 1, tau)
    rep = check_a(head, gpu, tau)
    assert rep.ok(), rep.failures
    assert rep.count_ties == 1
    tau = float(a.mass[0, j]) + 5e-4  # short by 5e-4: beyond the band
    gpu, _ = adaptive_result(head, j + 1, tau)
    assert not check_a(head, gpu, tau).ok()


@pytest.mark.parametrize("what", ["clusters", "ids", "logits", "set"])
def test_adaptive_planted_mistakes_fail(head, what):
    a = oracle.select_adaptive(H @ head.C_hat.T, PMAX, 0.5)
    n = int(a.n[0])
    gpu, _ = adaptive_result(head, n, 0.5)
    if what == "clusters":
        gpu["clusters"][0, n] = 0  # padding must be -1
    elif what == "ids":
        gpu["ids"][0, -1] = 0
    elif what == "logits":
        gpu["logits"][0, -1] = 0.0  # padding must be -inf
    else:  # a cluster far below the n-th key instead of the n-th
        S = np.sort(np.r_[a.order[0, :n - 1], 7])
        gpu2 = result_for(head, S)
        gpu["clusters"][0, :n] = S
        gpu["ids"][0, :n * head.b] = gpu2["ids"][0]
        gpu["logits"][0, :n * head.b] = gpu2["logits"][0]
    rep = check_a(head, gpu, 0.5)
    assert not rep.ok(), what


def test_adaptive_needs_the_count(head):
    gpu, _ = adaptive_result(head, 2, 0.5)
    del gpu["nprobe"]
    rep = check_a(head, gpu, 0.5)
    assert not rep.ok() and "nprobe" in rep.failures[0]


# ---- fp8 probabilities (check_probs_fp8)

def _fp8_case():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 2, size=(2, 300))
    lse = np.log(np.exp(z).sum(1))
    return z, lse


def test_fp8_exact_bytes_pass():
    z, lse = _fp8_case()
    want, k, _ = oracle.probs_fp8(z, lse, 1.0)
    assert parity.check_probs_fp8(z, lse, 1.0, want, k).ok()


def test_fp8_one_code_off_fails_away_from_a_midpoint():
    z, lse = _fp8_case()
    want, k, p = oracle.probs_fp8(z, lse, 1.0)
    got = want.copy()
    got[0, int(np.argmax(p[0]))] += 1
    rep = parity.check_probs_fp8(z, lse, 1.0, got, k)
    assert not rep.ok() and "not a midpoint near-tie" in rep.failures[0]


def test_fp8_wrong_scale_fails():
    z, lse = _fp8_case()
    want, k, _ = oracle.probs_fp8(z, lse, 1.0)
    rep = parity.check_probs_fp8(z, lse, 1.0, want, k + 1)
    assert not rep.ok() and "scale exponent" in rep.failures[0]


def test_fp8_neighbour_at_a_midpoint_passes():
    # row [1/2, q, 1/2 - q]: p_max = 1/2 gives k = 8, and q 2^8 = 68 (1 + 1e-7)
    # lies a hair above 68, the midpoint of codes 0x68 (64) and 0x69 (72): the
    # oracle rounds up, and the other code is certified
    q = 68.0 / 256 * (1 + 1e-7)
    z = np.log(np.array([[0.5, q, 0.5 - q]]))
    lse = np.array([0.0])
    want, k, _ = oracle.probs_fp8(z, lse, 1.0)
    assert int(k[0]) == 8 and int(want[0, 1]) == 0x69
    got = want.copy()
    got[0, 1] = 0x68
    rep = parity.check_probs_fp8(z, lse, 1.0, got, k)
    assert rep.ok() and rep.token_ties == 1
    # the same swap 1e-3 above the midpoint fails
    q = 68.0 / 256 * (1 + 1e-3)
    z = np.log(np.array([[0.5, q, 0.5 - q]]))
    assert not parity.check_probs_fp8(z, lse, 1.0, got, k).ok()


def test_fp8_scale_at_a_power_of_two_is_certified():
    # p_max a hair above 1/2: the oracle takes k = 8; a float32 p_max a hair
    # below 1/2 would take k = 9, and that is certified
    row = np.array([[0.5 * (1 + 1e-7), 0.5 * (1 - 1e-7)]])
    z = np.log(row)
    lse = np.array([0.0])
    want, k, p = oracle.probs_fp8(z, lse, 1.0)
    assert int(k[0]) == 8
    from oracle.flashhead_oracle import e4m3_encode
    got = e4m3_encode(np.ldexp(p, 9))
    rep = parity.check_probs_fp8(z, lse, 1.0, got, k + 1)
    assert rep.ok(), rep.failures
    assert rep.cluster_ties == 1
