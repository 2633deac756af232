"""GPU parity of the fp8 probability format (fh_probs_fp8) against the
oracle's E4M3 encoding of exp(z / T' - LSE), on the GPU's own logits and LSE
(checked against the oracle first), so that every byte is decided from the
same inputs: bytes equal, or one code apart within 1e-5 of a midpoint
(oracle/parity.check_probs_fp8)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth import make_graded_queries, make_problem

from _gpu import assert_report, host, need_gpu, problem_tensors, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    from lm_output_head_amd import load_library
    load_library()


@pytest.fixture(scope="module")
def llama():
    from lm_output_head_amd import FlashHead
    pb = make_problem("llama32_1b", nq=8)
    E, C, H = problem_tensors(pb)
    head = FlashHead(E, C, pb.C2T, max_batch=8)
    yield pb, head, H
    head.close()


@pytest.mark.parametrize("B,mode,T", [(1, 0, 1.0), (4, 0, 1.0), (4, 2, 0.7), (8, 3, 0.5)])
def test_forward_probabilities(llama, B, mode, T):
    pb, head, H = llama
    ref = oracle.OracleHead(pb.E, pb.C, pb.C2T)
    say("fp8 probs B", B, "mode", mode, "T", T)
    o = head.forward(H[:B], 512, mode=mode, temperature=T, seed=4, want_clusters=True,
                     want_retrieved=True)
    tp = T if mode & 2 else 1.0
    out = host(dict(o, **head.probs_fp8(o, tp)))
    assert_report(parity.check_forward(ref, pb.H[:B], 512, mode, T, 4, out), "forward")
    rep = parity.check_probs_fp8(out["logits"], out["lse"], tp, out["probs"], out["scale_exp"])
    say("midpoint near-ties", rep.token_ties, "scale near-ties", rep.cluster_ties, "of",
        out["probs"].size)
    assert rep.ok(), rep.failures
    q = np.ldexp(oracle.e4m3_decode(out["probs"]), -out["scale_exp"][:, None])
    assert np.all(np.abs(q.sum(1) - 1.0) < 0.03)


def test_adaptive_padding_is_zero():
    from lm_output_head_amd import FlashHead
    pb = make_problem("tiny")
    E, C, _ = problem_tensors(pb)
    Hf, _, _ = make_graded_queries(pb, np.linspace(0, 4, 16), seed=2)
    head = FlashHead(E, C, pb.C2T, max_batch=16)
    say("fp8 probs of an adaptive call")
    o = head.forward_adaptive(to_dev(Hf, torch.float32), 200, 0.9, temperature=0.5,
                              want_clusters=True, want_retrieved=True)
    out = host(dict(o, **head.probs_fp8(o, 1.0)))
    rep = parity.check_probs_fp8(out["logits"], out["lse"], 1.0, out["probs"], out["scale_exp"])
    assert rep.ok(), rep.failures
    for r in range(16):
        assert np.all(out["probs"][r, out["nprobe"][r] * pb.b:] == 0)
    head.close()


@pytest.mark.parametrize("B,n", [(1, 1), (3, 1001), (2, 70000)])
def test_ragged_sizes(B, n):
    from lm_output_head_amd import fh_probs_fp8
    rng = np.random.default_rng(n)
    z = rng.normal(0, 4, size=(B, n)).astype(np.float32)
    z[:, ::7] = -np.inf if n > 1 else z[:, ::7]
    zt = torch.from_numpy(z).cuda()
    lse = torch.logsumexp(zt / 0.8, dim=1).contiguous()
    out = torch.empty((B, n), dtype=torch.uint8, device="cuda")
    k = torch.empty(B, dtype=torch.int32, device="cuda")
    say("fp8 probs ragged", B, n)
    fh_probs_fp8(zt, lse, 0.8, out, k)
    got = host({"p": out, "k": k, "lse": lse})
    rep = parity.check_probs_fp8(z, got["lse"], 0.8, got["p"], got["k"])
    assert rep.ok(), rep.failures


def test_argument_errors():
    from lm_output_head_amd import FlashHeadError, fh_probs_fp8
    z = torch.zeros((2, 8), device="cuda")
    lse = torch.zeros(2, device="cuda")
    out = torch.empty((2, 8), dtype=torch.uint8, device="cuda")
    k = torch.empty(2, dtype=torch.int32, device="cuda")
    for T in (0.0, float("inf"), float("nan")):
        with pytest.raises(FlashHeadError):
            fh_probs_fp8(z, lse, T, out, k)
    with pytest.raises(ValueError):
        fh_probs_fp8(z, lse, 1.0, out[:1], k)
    with pytest.raises(ValueError):
        fh_probs_fp8(z, lse, 1.0, out, k[:1])
