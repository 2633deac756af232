"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case runs the engine (libflashhead via the thin binding) and the
float64 oracle on the same seeded inputs and applies the parity rule of
oracle/parity.py: exact ids up to certified near-ties (gap < 1e-3), logits
within 2e-3 relative (with a one-bfloat16-quantum Cauchy-Schwarz floor).
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth import SHAPES, Shape, make_problem

from _gpu import assert_report, host, need_gpu, problem_tensors, say, to_dev

pytestmark = pytest.mark.gpu

TOPK, PSAMPLE, TSAMPLE, SHARED = 0, 1, 2, 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    from lm_output_head_amd import load_library
    load_library()


def _engine(pb, quant="none", max_batch=1):
    from lm_output_head_amd import FlashHead
    E, C, H = problem_tensors(pb)
    return FlashHead(E, C, pb.C2T, quant=quant, max_batch=max_batch), H


def _oracle(pb, quant="none"):
    return oracle.OracleHead(pb.E, pb.C, pb.C2T, quant)


# ---------------------------------------------------------------- fixture ---

def test_toy_fixture_on_gpu():
    """The hand-worked toy head, padded to d = 4 with zero columns (fp32)."""
    from lm_output_head_amd import FlashHead
    with open(os.path.join(os.path.dirname(__file__), "golden", "toy_two_stage.json")) as f:
        g = json.load(f)
    pad = lambda a: np.pad(np.array(a, dtype=np.float32), ((0, 0), (0, 2)))  # noqa: E731
    E, C = torch.from_numpy(pad(g["E"])).cuda(), torch.from_numpy(pad(g["C"])).cuda()
    head = FlashHead(E, C, np.array(g["C2T"], dtype=np.int32), max_batch=1)
    for case in g["cases"]:
        h = torch.from_numpy(pad([case["h"]])).cuda()
        say("toy", case["h"])
        assert host({"s": head.score(h)})["s"][0].tolist() == case["scores"]
        dn = host(head.dense(h, want_logits=True))
        assert dn["token"][0] == case["dense_token"]
        assert dn["logits"][0].tolist() == case["dense_z"]
        for p, want in case["by_p"].items():
            out = host(head.forward(h, int(p), want_clusters=True, want_retrieved=True))
            assert out["clusters"][0].tolist() == want["S"]
            assert out["ids"][0].tolist() == want["ids"]
            assert out["logits"][0].tolist() == want["z"]
            assert out["token"][0] == want["token"]
            assert out["token_logit"][0] == want["token_logit"]
    head.close()


# -------------------------------------------------------------- tiny (fp32) --

def test_tiny_greedy_batch1_all_queries():
    pb = make_problem("tiny")
    head, H = _engine(pb)
    ref = _oracle(pb)
    outs = {k: [] for k in ("token", "token_logit", "lse", "clusters", "ids", "logits")}
    for q in range(H.shape[0]):
        o = host(head.forward(H[q:q + 1], 16, want_clusters=True, want_retrieved=True))
        for k in outs:
            outs[k].append(o[k][0])
    gpu = {k: np.stack(v) for k, v in outs.items()}
    say("tiny B=1 x 64")
    assert_report(parity.check_forward(ref, pb.H, 16, TOPK, 1.0, 0, gpu), "tiny greedy B=1")


def test_tiny_batched_scores_dense_and_determinism():
    pb = make_problem("tiny")
    head, H = _engine(pb, max_batch=64)
    ref = _oracle(pb)
    say("tiny scores B=64")
    s = host({"s": head.score(H)})["s"]
    assert_report(parity.check_scores(ref.C_hat, pb.H, s), "tiny scores")
    say("tiny forward B=64")
    a = host(head.forward(H, 16, want_clusters=True, want_retrieved=True))
    b = host(head.forward(H, 16, want_clusters=True, want_retrieved=True))
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{k} not bit-identical across runs"
    assert_report(parity.check_forward(ref, pb.H, 16, TOPK, 1.0, 0, a), "tiny greedy B=64")
    say("tiny dense B=64")
    d = host(head.dense(H, want_logits=True))
    assert_report(parity.check_dense(pb.E, pb.H, TOPK, 1.0, 0, d), "tiny dense")


@pytest.mark.parametrize("p", [1, 2, 255, 256])
def test_tiny_probe_counts_including_p_equals_c(p):
    pb = make_problem("tiny")
    head, H = _engine(pb, max_batch=8)
    say("tiny p", p)
    out = host(head.forward(H[:8], p, want_clusters=True, want_retrieved=True))
    assert_report(parity.check_forward(_oracle(pb), pb.H[:8], p, TOPK, 1.0, 0, out), f"tiny p={p}")
    if p == 256:  # every cluster probed: the dense head's token
        d = host(head.dense(H[:8]))
        assert np.array_equal(d["token"], out["token"])


@pytest.mark.parametrize("p", [129, 200, 255, 256])
def test_tiny_batch1_single_launch_large_p(p):
    """B = 1 through the single launch with the tiny head's p b rows spread
    over up to CUs - 1 stage-2 workgroups: the regime where the partial slots
    must cover every p, not only p = c."""
    pb = make_problem("tiny")
    head, H = _engine(pb, max_batch=1)
    ref = _oracle(pb)
    for q, (mode, T) in enumerate(((0, 1.0), (3, 0.8))):
        say("tiny B=1 single launch p", p, "mode", mode)
        out = host(head.forward(H[q:q + 1], p, mode=mode, temperature=T, seed=17,
                                want_clusters=True, want_retrieved=True))
        assert_report(parity.check_forward(ref, pb.H[q:q + 1], p, mode, T, 17, out),
                      f"tiny B=1 p={p} mode={mode}")
    head.sync_status()
    head.close()


@pytest.mark.parametrize("shape,quant,B,p,mode", [
    ("tiny", "none", 2, 16, 0), ("tiny", "none", 3, 100, 3), ("tiny", "none", 16, 255, 2),
    ("llama32_1b", "none", 4, 512, 0), ("llama32_1b", "int4", 8, 256, 1),
    ("llama32_1b", "int8", 3, 1024, 3), ("gemma3_1b", "none", 8, 512, 3),
])
def test_batched_launch_matches_per_stage(shape, quant, B, p, mode):
    """Small query-major batches (each probed cluster read by fewer than 1.2
    queries on average) run the selection, stage 2 and the finish in one
    launch after stage 1; the per-stage launches (FH_PATH_MULTI) give the
    same probes, retrieved ids and logits and tokens bit for bit, the LSE to
    rounding (the partials merge in another order), and both match the
    oracle."""
    pb = make_problem(shape) if shape == "tiny" else make_problem(shape, nq=16)
    head, H = _engine(pb, quant=quant, max_batch=B)
    say("batched launch", shape, quant, B, p, mode)
    one = host(head.forward(H[:B], p, mode=mode, temperature=0.8, seed=29, want_clusters=True,
                            want_retrieved=True))
    head.set_path("multi")
    per = host(head.forward(H[:B], p, mode=mode, temperature=0.8, seed=29, want_clusters=True,
                            want_retrieved=True))
    for k in ("clusters", "ids", "logits", "token", "token_logit"):
        assert np.array_equal(one[k], per[k]), k
    assert np.allclose(one["lse"], per["lse"], rtol=1e-5, atol=1e-6)
    assert_report(parity.check_forward(_oracle(pb, quant), pb.H[:B], p, mode, 0.8, 29, one),
                  f"batched {shape} {quant} B={B} p={p} mode={mode}")
    head.sync_status()
    head.close()


# ------------------------------------------------------- ragged / edge cases --

def _custom_problem(v, d, c, dtype, nq, seed=5):
    sh = Shape(f"custom{v}_{d}_{c}", v, d, c, 4, dtype, 4.0, nq)
    return make_problem(sh, seed_data=seed, seed_query=seed + 1)


@pytest.mark.parametrize("v,d,c,dtype", [
    (1500, 40, 300, "bf16"),     # d = 5 chunks: lanes 5..63 idle; c not a multiple of 1024
    (3000, 1032, 1000, "bf16"),  # d = 129 chunks: a ragged second chunk per lane
    (1200, 36, 100, "f32"),      # fp32, 9 chunks
    (20000, 264, 2000, "f32"),   # 66 chunks, b = 10
])
def test_ragged_shapes(v, d, c, dtype):
    pb = _custom_problem(v, d, c, dtype, 12)
    head, H = _engine(pb, max_batch=12)
    ref = _oracle(pb)
    for p in (1, 7, c // 3, c):
        say("ragged", v, d, c, dtype, "p", p)
        out = host(head.forward(H, p, want_clusters=True, want_retrieved=True))
        assert_report(parity.check_forward(ref, pb.H, p, TOPK, 1.0, 0, out), f"ragged p={p}")
    s = host({"s": head.score(H)})["s"]
    assert_report(parity.check_scores(ref.C_hat, pb.H, s), "ragged scores")
    dn = host(head.dense(H, want_logits=True))
    assert_report(parity.check_dense(pb.E, pb.H, TOPK, 1.0, 0, dn), "ragged dense")


@pytest.mark.parametrize("v,d,c,dtype,quant", [
    (4096, 4096, 256, "bf16", "none"),  # the largest bf16 d: 8 chunks per lane
    (4096, 4096, 256, "bf16", "int4"),  # 128 INT4 groups: two per lane
    (4096, 4096, 256, "bf16", "int8"),
    (2048, 2048, 128, "f32", "none"),   # the largest fp32 d
])
def test_maximum_hidden_size(v, d, c, dtype, quant):
    """d at the library's limit, through every path: the single launch (B = 1),
    per-stage launches, the matrix cores for stage 1 (INT4 and INT8 from B = 2, bf16
    from 8) and the dense head (from 2)."""
    pb = _custom_problem(v, d, c, dtype, 8, seed=13)
    head, H = _engine(pb, quant=quant, max_batch=8)
    ref = _oracle(pb, quant)
    for B in (1, 3, 8):
        say("max d", v, d, c, dtype, quant, "B", B)
        out = host(head.forward(H[:B], 32, want_clusters=True, want_retrieved=True))
        assert_report(parity.check_forward(ref, pb.H[:B], 32, TOPK, 1.0, 0, out), f"max d B={B}")
        s = host({"s": head.score(H[:B])})["s"]
        assert_report(parity.check_scores(ref.C_hat, pb.H[:B], s), f"max d scores B={B}")
        dn = host(head.dense(H[:B], mode=TSAMPLE, temperature=0.9, seed=2, want_logits=True))
        assert_report(parity.check_dense(pb.E, pb.H[:B], TSAMPLE, 0.9, 2, dn), f"max d dense B={B}")
    head.close()


def test_hidden_size_beyond_the_limit_is_unsupported():
    from lm_output_head_amd import FlashHead, FlashHeadError
    for d, dt in ((4104, torch.bfloat16), (2052, torch.float32)):
        E = torch.zeros((64, d), dtype=dt, device="cuda")
        C = torch.zeros((4, d), dtype=dt, device="cuda")
        with pytest.raises(FlashHeadError):
            FlashHead(E, C, np.arange(64, dtype=np.int32).reshape(4, 16))


@pytest.mark.parametrize("B", [256, 257])
def test_batches_at_the_cluster_major_limit(B):
    """256 queries: the cluster-major stage 2 (its LDS lists hold 256); 257:
    the query-major one.  Both against the oracle on a sample of rows."""
    pb = _custom_problem(8192, 128, 512, "bf16", 257, seed=17)
    head, H = _engine(pb, max_batch=257)
    ref = _oracle(pb)
    say("cm limit B", B)
    out = host(head.forward(H[:B], 96, want_clusters=True, want_retrieved=True))
    rows = sorted({0, 1, 100, 255, B - 1})
    assert_report(parity.check_forward(ref, pb.H[:B], 96, TOPK, 1.0, 0, out, queries=rows),
                  f"cm limit B={B}")
    # the matrix-core GEMMs at 128 queries per workgroup: dense head (sampled
    # tokens) and stage-1 scores, on the same rows
    dn = host(head.dense(H[:B], TSAMPLE, 0.9, 4))
    assert_report(parity.check_dense(pb.E, pb.H[:B], TSAMPLE, 0.9, 4, dn, queries=rows),
                  f"cm limit dense B={B}")
    s = host({"s": head.score(H[:B])})["s"]
    assert_report(parity.check_scores(ref.C_hat, pb.H[rows], s[rows]), f"cm limit scores B={B}")
    # stage 1 split over d with one and two 16-query tiles (ragged second tile)
    for nb in (16, 24, 32):
        s = host({"s": head.score(H[:nb])})["s"]
        assert_report(parity.check_scores(ref.C_hat, pb.H[:nb], s), f"split-d scores B={nb}")
    head.close()


@pytest.mark.parametrize("quant", ["none", "int4", "int8"])
def test_sampled_probes_over_two_query_tiles(quant):
    """24 queries with sampled probes and tokens: stage 1 split over d in two
    16-query tiles forms the Gumbel keys itself, keyed by each query's index
    in the batch (the second tile's 8 queries included)."""
    pb = _custom_problem(8192, 128, 512, "bf16", 24, seed=29)
    head, H = _engine(pb, quant=quant, max_batch=24)
    ref = _oracle(pb, quant)
    say("sampled probes two tiles", quant)
    out = host(head.forward(H, 32, mode=PSAMPLE | TSAMPLE, temperature=0.9, seed=11,
                            want_clusters=True, want_retrieved=True))
    assert_report(parity.check_forward(ref, pb.H, 32, PSAMPLE | TSAMPLE, 0.9, 11, out),
                  f"sampled probes B=24 {quant}")
    head.close()


@pytest.mark.parametrize("shape,quant,B,p,mode,T", [
    ("tiny", "none", 8, 16, SHARED, 1.0),               # fp32: query-major, one probe row
    ("tiny", "none", 64, 16, SHARED | TSAMPLE, 0.8),
    ("llama32_1b", "none", 8, 512, SHARED, 1.0),        # bf16: one GEMM over the probes' rows
    ("llama32_1b", "int4", 64, 512, SHARED | TSAMPLE, 0.7),
    ("llama32_1b", "none", 1, 512, SHARED, 1.0),        # B = 1: the single launch, top-p
])
def test_shared_probes(shape, quant, B, p, mode, T):
    """One probe set for the batch (the top p of the summed scores): the same
    set in every row, and every query's stage 2 and finish over it."""
    pb = make_problem(shape, nq=max(B, 8))
    head, H = _engine(pb, quant=quant, max_batch=B)
    ref = _oracle(pb, quant)
    say("shared", shape, quant, B, p, mode)
    out = host(head.forward(H[:B], p, mode=mode, temperature=T, seed=9, want_clusters=True,
                            want_retrieved=True))
    assert np.all(out["clusters"] == out["clusters"][0])
    assert_report(parity.check_forward(ref, pb.H[:B], p, mode, T, 9, out), f"shared {shape} B={B}")
    if B == 1:
        plain = host(head.forward(H[:1], p, mode=mode & TSAMPLE, temperature=T, seed=9,
                                  want_clusters=True))
        assert np.array_equal(plain["clusters"], out["clusters"])
        assert np.array_equal(plain["token"], out["token"])
    head.close()


def test_shared_probes_large_batch():
    """257 bf16 queries sharing one probe set (one GEMM over the probes' rows,
    no batch limit), checked on sampled rows; sampled shared probes are refused."""
    from lm_output_head_amd import FlashHeadError
    pb = _custom_problem(8192, 128, 512, "bf16", 257, seed=17)
    head, H = _engine(pb, max_batch=257)
    ref = _oracle(pb)
    say("shared B=257")
    out = host(head.forward(H, 96, mode=SHARED, want_clusters=True, want_retrieved=True))
    assert np.all(out["clusters"] == out["clusters"][0])
    assert_report(parity.check_forward(ref, pb.H, 96, SHARED, 1.0, 0, out,
                                       queries=[0, 1, 128, 256]), "shared B=257")
    with pytest.raises(FlashHeadError):
        head.forward(H[:4], 96, mode=SHARED | PSAMPLE, temperature=1.0)
    head.close()


def test_all_equal_scores_take_smallest_cluster_ids():
    """Degenerate: identical centroids give equal scores; ties go to small ids."""
    from lm_output_head_amd import FlashHead
    v, d, c = 640, 64, 40
    rng = np.random.default_rng(2)
    E = rng.standard_normal((v, d)).astype(np.float32)
    C = np.tile(rng.standard_normal((1, d)).astype(np.float32), (c, 1))
    c2t = rng.permutation(v).reshape(c, v // c).astype(np.int32)
    head = FlashHead(torch.from_numpy(E).cuda(), torch.from_numpy(C).cuda(), c2t, max_batch=3)
    H = rng.standard_normal((3, d)).astype(np.float32)
    for p in (1, 13, 39):
        say("all-equal p", p)
        out = host(head.forward(torch.from_numpy(H).cuda(), p, want_clusters=True))
        assert np.array_equal(out["clusters"], np.tile(np.arange(p), (3, 1)))


@pytest.mark.parametrize("layout", ["narrow_first_keys", "high_first_keys", "quantised_levels"])
def test_selection_with_misleading_key_statistics(layout):
    """Scores built exactly (h = a e0, so s[k] = a C[k, 0]) such that a
    threshold placed from the statistics of the first keys is far too low,
    far too high, or lands in heavy exact ties.  The selection must still be
    the exact top p with ties to the smaller id, at B = 1 (single launch) and
    B = 3 (per-stage launches)."""
    from lm_output_head_amd import FlashHead
    v, d, c = 16032, 8, 8016
    rng = np.random.default_rng(11)
    s = rng.standard_normal(c).astype(np.float32)
    if layout == "narrow_first_keys":
        s[:2048] *= np.float32(0.01)
    elif layout == "high_first_keys":
        s[:2048] += np.float32(6.0)
    else:
        s = (np.rint(s * np.float32(3.0)) / np.float32(3.0)).astype(np.float32)
    C = rng.standard_normal((c, d)).astype(np.float32)
    C[:, 0] = s
    E = rng.standard_normal((v, d)).astype(np.float32)
    c2t = rng.permutation(v).reshape(c, v // c).astype(np.int32)
    H = np.zeros((3, d), np.float32)
    H[:, 0] = [1.0, 0.5, 2.0]
    head = FlashHead(torch.from_numpy(E).cuda(), torch.from_numpy(C).cuda(), c2t, max_batch=3)
    ref = oracle.OracleHead(E, C, c2t, "none")
    Hd = torch.from_numpy(H).cuda()
    for p in (100, 512, 1500):
        say("misleading stats", layout, "p", p)
        out = host(head.forward(Hd, p, want_clusters=True, want_retrieved=True))
        assert_report(parity.check_forward(ref, H, p, TOPK, 1.0, 0, out), f"{layout} B=3 p={p}")
        for q in range(3):
            one = host(head.forward(Hd[q:q + 1], p, want_clusters=True, want_retrieved=True))
            assert np.array_equal(one["clusters"][0], out["clusters"][q]), (layout, p, q)
            assert np.array_equal(one["ids"][0], out["ids"][q]), (layout, p, q)
    head.sync_status()
    head.close()


# -------------------------------------------------------- Llama-3.2-1B shape --

@pytest.fixture(scope="module")
def llama():
    pb = make_problem("llama32_1b", nq=64)
    return pb


def test_llama_greedy_batch1(llama):
    pb = llama
    head, H = _engine(pb)
    ref = _oracle(pb)
    outs = {k: [] for k in ("token", "token_logit", "lse", "clusters", "ids", "logits")}
    nq = 16
    for q in range(nq):
        say("llama B=1 q", q)
        o = host(head.forward(H[q:q + 1], 512, want_clusters=True, want_retrieved=True))
        for k in outs:
            outs[k].append(o[k][0])
    gpu = {k: np.stack(v) for k, v in outs.items()}
    assert_report(parity.check_forward(ref, pb.H[:nq], 512, TOPK, 1.0, 0, gpu), "llama greedy")
    head.close()


def test_llama_scores_and_dense(llama):
    pb = llama
    head, H = _engine(pb, max_batch=4)
    ref = _oracle(pb)
    say("llama scores B=4")
    s = host({"s": head.score(H[:4])})["s"]
    assert_report(parity.check_scores(ref.C_hat, pb.H[:4], s), "llama scores")
    say("llama dense B=4")
    d = host(head.dense(H[:4], want_logits=True))
    assert_report(parity.check_dense(pb.E, pb.H[:4], TOPK, 1.0, 0, d), "llama dense")
    head.close()


# --------------------------------------------------------------- INT4 (cfg3) --

def test_int4_codes_bit_exact(llama):
    pb = llama
    head, _ = _engine(pb, quant="int4")
    say("int4 codes")
    packed, scales = head.int4()
    packed, scales = packed.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
    q, sigma = oracle.quantize_int4_g32(pb.C)
    assert np.array_equal(scales, sigma.view(np.uint16))
    assert np.array_equal(packed, oracle.pack_int4(q))
    head.close()


@pytest.mark.parametrize("quant,B,p", [
    ("int4", 1, 128), ("int4", 1, 1024), ("int4", 8, 256), ("int4", 8, 512),
    ("int4", 32, 128), ("int4", 32, 512), ("int4", 64, 512), ("int4", 64, 1024),
    ("none", 32, 512), ("none", 64, 512), ("none", 64, 1024),
])
def test_llama_batch_probe_sweep_every_row(llama, quant, B, p):
    """The batch sweep at the Llama-3.2-1B shape, B in {1, 8, 32, 64} x p in
    {128 ... 1024}, INT4 and bf16 centroids: every query of every call
    against the oracle (per-query probes; cluster-major stage 2 from B = 8 at p = 512)."""
    pb = llama
    head, H = _engine(pb, quant=quant, max_batch=64)
    ref = _oracle(pb, quant)
    say(quant, "B", B, "p", p)
    out = host(head.forward(H[:B], p, want_clusters=True, want_retrieved=True))
    assert_report(parity.check_forward(ref, pb.H[:B], p, TOPK, 1.0, 0, out), f"{quant} B={B} p={p}")
    s = host({"s": head.score(H[:B])})["s"]
    assert_report(parity.check_scores(ref.C_hat, pb.H[:B], s), f"{quant} scores B={B}")
    head.close()


# --------------------------------------------------------- INT8 (W8A16) ---

def test_int8_codes_bit_exact(llama):
    pb = llama
    head, _ = _engine(pb, quant="int8")
    say("int8 codes")
    codes, scales = head.int8()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
    q, sigma = oracle.quantize_int8_g32(pb.C)
    assert np.array_equal(scales, sigma.view(np.uint16))
    assert np.array_equal(codes, q)
    head.close()


@pytest.mark.parametrize("B,p", [(1, 512), (3, 64), (8, 512)])
def test_int8_batched_probe_sweep(llama, B, p):
    pb = llama
    head, H = _engine(pb, quant="int8", max_batch=8)
    ref = _oracle(pb, "int8")
    say("int8 B", B, "p", p)
    out = host(head.forward(H[:B], p, want_clusters=True, want_retrieved=True))
    assert_report(parity.check_forward(ref, pb.H[:B], p, TOPK, 1.0, 0, out), f"int8 B={B} p={p}")
    s = host({"s": head.score(H[:B])})["s"]
    assert_report(parity.check_scores(ref.C_hat, pb.H[:B], s), "int8 scores")
    head.close()


@pytest.mark.parametrize("v,d,c,quant", [
    (2000, 160, 250, "int4"),   # 5 INT4 groups (a partial block of 4); c not a multiple of 16
    (2000, 160, 250, "int8"),   # 5 INT8 groups of two 16-byte loads each (vector units at every B)
    (2560, 96, 160, "int4"),    # 3 groups: a single partial block
    (3000, 1032, 1000, "none"),  # bf16 d with a 8-element tail after 128-element blocks
    (1200, 40, 75, "none"),      # d below one 128-element block
])
def test_batched_matrix_core_paths(v, d, c, quant):
    """Batched stage 1 and the dense head on the matrix cores (bf16 queries,
    B above the thresholds), on ragged shapes, against the oracle; B = 1 and
    small B take the GEMV paths on the same engine."""
    pb = _custom_problem(v, d, c, "bf16", 40, seed=9)
    head, H = _engine(pb, quant=quant, max_batch=40)
    ref = _oracle(pb, quant)
    for B in (1, 2, 7, 8, 17, 40):
        say("mfma", v, d, c, quant, "B", B)
        s = host({"s": head.score(H[:B])})["s"]
        assert_report(parity.check_scores(ref.C_hat, pb.H[:B], s), f"scores B={B}")
        for mode, T in ((TOPK, 1.0), (PSAMPLE | TSAMPLE, 0.8)):
            out = host(head.forward(H[:B], max(1, c // 10), mode=mode, temperature=T, seed=5,
                                    want_clusters=True, want_retrieved=True))
            assert_report(parity.check_forward(ref, pb.H[:B], max(1, c // 10), mode, T, 5, out),
                          f"forward B={B} mode={mode}")
        for mode, T in ((TOPK, 1.0), (TSAMPLE, 0.7)):
            dn = host(head.dense(H[:B], mode=mode, temperature=T, seed=3, want_logits=True))
            assert_report(parity.check_dense(pb.E, pb.H[:B], mode, T, 3, dn), f"dense B={B} m={mode}")
    head.close()


# ------------------------------------------------ Gemma-3-1B shape (cfg4) ---

def test_gemma_sampled_probes_and_tokens():
    pb = make_problem("gemma3_1b", nq=16)
    head, H = _engine(pb, max_batch=16)
    ref = _oracle(pb)
    mode = PSAMPLE | TSAMPLE
    say("gemma B=16 sampled")
    out = host(head.forward(H, 512, mode=mode, temperature=1.0, seed=0x5EED,
                            want_clusters=True, want_retrieved=True))
    assert_report(parity.check_forward(ref, pb.H, 512, mode, 1.0, 0x5EED, out), "gemma sampled")
    say("gemma dense sampled B=16")
    d = host(head.dense(H, mode=TSAMPLE, temperature=1.0, seed=0x5EED))
    assert_report(parity.check_dense(pb.E, pb.H, TSAMPLE, 1.0, 0x5EED, d), "gemma dense")
    head.close()


# ------------------------------------------------- Qwen-3-4B shape (cfg5) ---

def test_qwen_int4_batch128_greedy_and_t07():
    pb = make_problem("qwen3_4b", nq=128)
    head, H = _engine(pb, quant="int4", max_batch=128)
    ref = _oracle(pb, "int4")
    rows = None  # every one of the 128 queries
    say("qwen B=128 greedy")
    out = host(head.forward(H, 1024, want_clusters=True, want_retrieved=True))
    assert_report(parity.check_forward(ref, pb.H, 1024, TOPK, 1.0, 0, out, queries=rows),
                  "qwen greedy")
    say("qwen B=128 T=0.7")
    out = host(head.forward(H, 1024, mode=TSAMPLE, temperature=0.7, seed=0x5EED + 1,
                            want_clusters=True, want_retrieved=True))
    assert_report(parity.check_forward(ref, pb.H, 1024, TSAMPLE, 0.7, 0x5EED + 1, out,
                                       queries=rows), "qwen T=0.7")
    head.close()


# ------------------------------------------------------------ argument errors --

def test_argument_errors_are_reported():
    from lm_output_head_amd import FlashHeadError
    pb = make_problem("tiny")
    head, H = _engine(pb, max_batch=2)
    for kwargs in ({"p": 0}, {"p": 257}, {"p": 4, "mode": TSAMPLE, "temperature": 0.0},
                   {"p": 4, "mode": 5}):
        with pytest.raises(FlashHeadError) as ei:
            head.forward(H[:1], **kwargs)
        assert ei.value.status == -1
    with pytest.raises(FlashHeadError):
        head.forward(H[:3], 4)  # B > max_batch
    from lm_output_head_amd import FlashHead
    E, C, _ = problem_tensors(pb)
    bad = pb.C2T.copy()
    bad[0, 0] = bad[0, 1]
    with pytest.raises(FlashHeadError):
        FlashHead(E, C, bad)
    head.close()


# ------------------------------------------- single-launch vs multi-launch ---

@pytest.mark.parametrize("shape,quant,mode,T", [
    ("tiny", "none", TOPK, 1.0),
    ("tiny", "none", PSAMPLE | TSAMPLE, 0.8),
    ("llama32_1b", "none", TOPK, 1.0),
    ("llama32_1b", "int4", TOPK, 1.0),
    ("llama32_1b", "int8", TOPK, 1.0),
    ("tiny", "int8", PSAMPLE | TSAMPLE, 0.8),
    ("llama32_1b", "none", TSAMPLE, 0.7),
    ("gemma3_1b", "none", PSAMPLE | TSAMPLE, 1.0),
])
def test_fused_batch1_matches_multi_launch_and_oracle(shape, quant, mode, T):
    """B=1 runs in one cooperative launch; it must agree with the per-stage
    launches (ids and logits bit-identical, LSE to rounding) and the oracle."""
    pb = make_problem(shape, nq=8)
    head, H = _engine(pb, quant=quant)
    ref = _oracle(pb, quant)
    p = pb.shape.p
    runs = {}
    for path in ("auto", "multi"):
        head.set_path(path)
        outs = {k: [] for k in ("token", "token_logit", "lse", "clusters", "ids", "logits")}
        for q in range(4):
            say("paths", shape, quant, mode, path, "q", q)
            o = host(head.forward(H[q:q + 1], p, mode=mode, temperature=T, seed=0x5EED + q,
                                  want_clusters=True, want_retrieved=True))
            for k in outs:
                outs[k].append(o[k][0])
        head.sync_status()
        runs[path] = {k: np.stack(v) for k, v in outs.items()}
    a, b = runs["auto"], runs["multi"]
    for k in ("token", "token_logit", "clusters", "ids", "logits"):
        assert np.array_equal(a[k], b[k]), k
    assert np.allclose(a["lse"], b["lse"], rtol=1e-5, atol=1e-5)
    for q in range(4):
        one = {k: v[q:q + 1] for k, v in a.items()}
        rep = parity.check_forward(ref, pb.H[q:q + 1], p, mode, T, 0x5EED + q, one)
        assert_report(rep, f"fused {shape} q{q}")
    head.close()
