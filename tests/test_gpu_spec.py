"""GPU parity of the speculative verification (fh_spec_verify) against the
float64 oracle (oracle/spec_oracle.py), and its guarantee measured on the
GPU: verified tokens follow the dense head's softmax.

Element-wise rule: the acceptance decision must match the oracle's unless
|u - ratio| < 1e-4 (the GPU's ratio comes from float32 LSEs); a kept draft
is the draft token; a rejected one is the oracle's residual draw, or a
certified near-tie of it (residual keys within 1e-3); the full LSE within
2e-3 relative.
"""

import numpy as np
import pytest
import torch
from scipy.stats import binomtest, chisquare

from oracle import spec_oracle as so
from synth import Shape, make_problem

from _gpu import host, need_gpu, problem_tensors, say

pytestmark = pytest.mark.gpu

PSAMPLE, TSAMPLE = 1, 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    from lm_output_head_amd import load_library
    load_library()


def _check(pb, H, draft, ver, T, seed):
    clusters = draft["clusters"]
    ref = so.spec_verify(pb.E, pb.C2T, H, clusters, draft["token"], T, seed)
    B = H.shape[0]
    ties = 0
    for r in range(B):
        acc = bool(ver["accepted"][r])
        if acc != ref.accepted[r]:
            assert abs(ref.u[r] - ref.ratio[r]) < 1e-4, (r, ref.u[r], ref.ratio[r])
            ties += 1
            continue
        if acc:
            assert ver["token"][r] == draft["token"][r], r
        else:
            g, o = int(ver["token"][r]), int(ref.token[r])
            if g != o:
                k = ref.rkey32[r]
                assert np.isfinite(k[g]) and abs(float(k[g]) - float(k[o])) < 1e-3, (r, g, o)
                ties += 1
        assert abs(ver["lse"][r] - ref.lse[r]) <= 2e-3 * max(1.0, abs(ref.lse[r])), r
    say("spec rows", B, "accepted", int(ver["accepted"].sum()), "certified ties", ties)
    return ref


def _run(head, H_dev, p, mode, T, seed_draft, seed_verify):
    draft = head.forward(H_dev, p, mode=mode, temperature=T, seed=seed_draft, want_clusters=True)
    ver = head.spec_verify(H_dev, draft, p, T, seed_verify)
    return host(draft), host(ver)


@pytest.mark.parametrize("mode", [TSAMPLE, PSAMPLE | TSAMPLE])
def test_tiny_matches_oracle(mode):
    from lm_output_head_amd import FlashHead
    pb = make_problem("tiny", nq=64)
    E, C, H = problem_tensors(pb)
    head = FlashHead(E, C, pb.C2T, max_batch=64)
    say("spec tiny", mode)
    draft, ver = _run(head, H, 16, mode, 0.8, 7, 9)
    ref = _check(pb, pb.H, draft, ver, 0.8, 9)
    assert 0 < ref.accepted.sum() < 64  # both branches are exercised
    head.close()


@pytest.mark.parametrize("T,B", [(1.0, 8), (0.25, 8), (1.0, 3)])
def test_llama_matches_oracle(T, B):
    """Full size: at T = 1 the probes hold little of the target's mass (most
    drafts are refused and redrawn outside them); at T = 0.25 most are kept.
    B = 8 runs the dense pass as the matrix-core GEMM, B = 3 split over d."""
    from lm_output_head_amd import FlashHead
    pb = make_problem("llama32_1b", nq=B)
    E, C, H = problem_tensors(pb)
    head = FlashHead(E, C, pb.C2T, max_batch=B)
    say("spec llama B", B, "T", T)
    draft, ver = _run(head, H, 512, PSAMPLE | TSAMPLE, T, 21, 22)
    _check(pb, pb.H, draft, ver, T, 22)
    head.close()


def test_verified_tokens_follow_the_dense_softmax():
    """8192 verifications of one hidden state (each row draws its own noise):
    the verified tokens follow softmax(E h / T) (chi-square), the drafts do
    not, and the acceptance rate is the target mass of the probes."""
    from lm_output_head_amd import FlashHead
    pb = make_problem(Shape("spec_small", 256, 64, 16, 2, "f32", 1.5, 1), seed_data=5)
    n, p, T = 8192, 2, 1.0
    h = np.repeat(pb.H[:1], n, axis=0)
    E, C, _ = problem_tensors(pb)
    head = FlashHead(E, C, pb.C2T, max_batch=n)
    H = torch.from_numpy(np.ascontiguousarray(h, dtype=np.float32)).cuda()
    say("spec distribution", n)
    draft, ver = _run(head, H, p, TSAMPLE, T, 31, 32)
    z = pb.E.astype(np.float64) @ pb.H[0].astype(np.float64) / T
    prob = np.exp(z - z.max())
    prob /= prob.sum()

    def pval(tokens):
        counts = np.bincount(tokens, minlength=pb.E.shape[0]).astype(np.float64)
        exp = prob * n
        big = exp >= 5
        obs = np.append(counts[big], counts[~big].sum())
        ex = np.append(exp[big], exp[~big].sum())
        return chisquare(obs[ex > 0], ex[ex > 0]).pvalue

    assert pval(ver["token"]) > 1e-4
    assert pval(draft["token"]) < 1e-6
    S = draft["clusters"][0]
    assert np.all(draft["clusters"] == S)  # top-p probes: the same for every row
    mass = prob[pb.C2T[S].ravel()].sum()
    assert binomtest(int(ver["accepted"].sum()), n, mass).pvalue > 1e-4
    head.close()


def test_bad_arguments():
    from lm_output_head_amd import FlashHead, FlashHeadError
    pb = make_problem("tiny", nq=2)
    E, C, H = problem_tensors(pb)
    head = FlashHead(E, C, pb.C2T, max_batch=2)
    draft = head.forward(H, 4, mode=TSAMPLE, temperature=1.0, want_clusters=True)
    with pytest.raises(FlashHeadError):
        head.spec_verify(H, draft, 4, 0.0)
    with pytest.raises(FlashHeadError):
        head.spec_verify(H, {**draft, "clusters": torch.zeros((2, 300), dtype=torch.int32,
                                                             device="cuda")}, 300, 1.0)
    head.close()
