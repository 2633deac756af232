"""GPU parity of the adaptive probe count (fh_forward_adaptive) against the
oracle's select_adaptive, through the C ABI.

Queries of graded confidence (synth.make_graded_queries: alpha from 0, a
diffuse query, to 4, a confident one) make the count vary inside one batch;
the temperature is chosen per head so that it does (the Llama-3.2-1B head,
c = 8016, splits into one-probe queries and p_max ones; the tiny head spreads
over 1 .. p_max).  The parity rule is oracle/parity.check_adaptive: the count
within a mass band of 1e-4 around tau, the probe set exact up to key
near-ties, then stage 2 and the finish as for fixed p."""

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


def _setup(name, nq, quant="none", max_batch=64, seed=7):
    from lm_output_head_amd import FlashHead
    pb = make_problem(name) if name == "tiny" else make_problem(name, nq=8)
    E, C, _ = problem_tensors(pb)
    Hf, Hbits, _ = make_graded_queries(pb, np.linspace(0.0, 4.0, nq), seed=seed)
    if pb.shape.dtype == "bf16":
        H = to_dev(Hbits, torch.bfloat16)
    else:
        H = to_dev(Hf, torch.float32)
    head = FlashHead(E, C, pb.C2T, quant=quant, max_batch=max_batch)
    return pb, head, H, Hf, oracle.OracleHead(pb.E, pb.C, pb.C2T, quant)


def _run(head, ref, H, Hf, p_max, p_min, tau, mode, T, seed, what):
    say(what, "p_max", p_max, "p_min", p_min, "tau", tau, "mode", mode, "T", T)
    out = host(head.forward_adaptive(H, p_max, tau, p_min=p_min, mode=mode, temperature=T,
                                     seed=seed, want_clusters=True, want_retrieved=True))
    rep = parity.check_adaptive(ref, Hf, p_max, p_min, tau, mode, T, seed, out)
    say(what, "counts", out["nprobe"].tolist(), "count near-ties", rep.count_ties)
    assert_report(rep, what)
    return out


@pytest.mark.parametrize("mode,T,tau", [(0, 0.3, 0.5), (0, 0.5, 0.9), (1, 0.5, 0.9),
                                        (2, 0.3, 0.5), (3, 0.5, 0.9), (0, 1.0, 1.0)])
def test_tiny_graded_batch(mode, T, tau):
    pb, head, H, Hf, ref = _setup("tiny", 32)
    out = _run(head, ref, H, Hf, 250, 1, tau, mode, T, 5, f"tiny mode={mode}")
    if tau < 1.0 and mode == 0:
        assert len(set(out["nprobe"].tolist())) > 4  # the count does vary
    head.close()


def test_tiny_clamps_and_batch1():
    pb, head, H, Hf, ref = _setup("tiny", 32)
    _run(head, ref, H, Hf, 64, 8, 0.9, 0, 0.3, 0, "tiny clamp [8, 64]")
    # B = 1: the single launch (its selector takes the count), then the
    # per-stage launches
    for path in ("auto", "multi"):
        head.set_path(path)
        for q in (0, 13, 31):
            for mode, T in ((0, 0.3), (3, 0.5)):
                _run(head, ref, H[q:q + 1], Hf[q:q + 1], 128, 1, 0.9, mode, T, 9 + q,
                     f"tiny B=1 {path} row {q}")
    head.close()


def test_tiny_fixed_count_equals_forward():
    """p_min = p_max = p: the same probes, retrieved tokens and results as
    fh_forward with p, bit for bit (the same row-GEMV stage 2, B > 1)."""
    pb, head, H, Hf, ref = _setup("tiny", 8)
    for mode in (0, 2):
        say("tiny fixed p = 40, mode", mode)
        a = host(head.forward_adaptive(H, 40, 0.5, p_min=40, mode=mode, temperature=0.7, seed=3,
                                       want_clusters=True, want_retrieved=True))
        f = host(head.forward(H, 40, mode=mode, temperature=0.7, seed=3, want_clusters=True,
                              want_retrieved=True))
        assert np.all(a["nprobe"] == 40)
        for k in ("clusters", "ids", "logits", "token", "token_logit", "lse"):
            assert np.array_equal(a[k], f[k]), k
    head.close()


@pytest.mark.parametrize("quant,mode,T,tau", [("none", 0, 0.3, 0.5), ("none", 3, 0.2, 0.9),
                                              ("int4", 0, 0.3, 0.5), ("int8", 1, 0.2, 0.9)])
def test_llama_graded_batch(quant, mode, T, tau):
    pb, head, H, Hf, ref = _setup("llama32_1b", 32, quant=quant, max_batch=32)
    out = _run(head, ref, H, Hf, 512, 1, tau, mode, T, 21, f"llama {quant} mode={mode}")
    n = out["nprobe"]
    if mode == 0:
        assert n.min() == 1 and n.max() == 512  # both kinds of query in the batch
    head.close()


@pytest.mark.parametrize("quant", ["none", "int4"])
def test_llama_batch1_single_launch(quant):
    """B = 1 through the single launch at the Llama-3.2-1B shape: graded
    queries from diffuse (p_max probes) to confident (one probe), greedy and
    sampled; every row against the oracle."""
    pb, head, H, Hf, ref = _setup("llama32_1b", 12, quant=quant, max_batch=1)
    counts = []
    for q in range(12):
        mode = (0, 1, 3)[q % 3]
        out = _run(head, ref, H[q:q + 1], Hf[q:q + 1], 512, 1, 0.5, mode, 0.3, 40 + q,
                   f"llama {quant} B=1 row {q}")
        counts.append(int(out["nprobe"][0]))
    assert min(counts) == 1 and max(counts) == 512, counts
    head.close()


def test_llama_p_max_1024():
    pb, head, H, Hf, ref = _setup("llama32_1b", 8, max_batch=8)
    _run(head, ref, H, Hf, 1024, 1, 0.5, 0, 0.3, 0, "llama p_max=1024")
    head.close()


def test_argument_errors():
    from lm_output_head_amd import FlashHeadError
    pb, head, H, Hf, ref = _setup("tiny", 4)
    for kw in (dict(p_max=257, tau=0.5), dict(p_max=16, tau=0.0), dict(p_max=16, tau=1.5),
               dict(p_max=16, tau=0.5, p_min=17), dict(p_max=16, tau=0.5, mode=4),
               dict(p_max=16, tau=0.5, temperature=0.0)):
        with pytest.raises(FlashHeadError):
            head.forward_adaptive(H, **kw)
    head.close()
