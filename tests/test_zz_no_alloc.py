"""fh_forward_noalloc (the entry point that allocates nothing) against the
existing fh_forward, through the C ABI: two calls in a row on one GPU, the
second with a smaller input, so that the second runs on the first's leftover
workspace.  Outputs must equal fh_forward's per-stage path bit for bit and
pass the oracle's parity rule."""

import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from synth import make_problem

from _gpu import host, need_gpu, problem_tensors, say

pytestmark = pytest.mark.gpu

KEYS = ("token", "token_logit", "lse", "clusters", "ids", "logits")


def _noalloc(E, C, c2t, H, p, mode, T, seed):
    from lm_output_head_amd import fh_forward_noalloc
    B, b = H.shape[0], E.shape[0] // C.shape[0]
    dev = H.device
    out = {"token": torch.full((B,), -7, dtype=torch.int32, device=dev),
           "token_logit": torch.full((B,), np.nan, dtype=torch.float32, device=dev),
           "lse": torch.full((B,), np.nan, dtype=torch.float32, device=dev),
           "clusters": torch.full((B, p), -7, dtype=torch.int32, device=dev),
           "ids": torch.full((B, p * b), -7, dtype=torch.int32, device=dev),
           "logits": torch.full((B, p * b), np.nan, dtype=torch.float32, device=dev)}
    fh_forward_noalloc(E, C, c2t, H, p, mode, T, seed, out["token"], out["token_logit"],
                       out["lse"], out["clusters"], out["ids"], out["logits"])
    return host(out)


@pytest.mark.parametrize("mode,T", [(0, 1.0), (3, 0.8)])
def test_noalloc_matches_fh_forward_two_calls(mode, T):
    need_gpu()
    from lm_output_head_amd import FlashHead
    cases = [("llama32_1b", 1, 512), ("tiny", 4, 16)]  # the second is smaller
    for shape, B, p in cases:
        pb = make_problem(shape, nq=8)
        E, C, H = problem_tensors(pb)
        H = H[:B].contiguous()
        c2t = torch.from_numpy(np.ascontiguousarray(pb.C2T, dtype=np.int32)).cuda()
        say("no-alloc", shape, "B", B, "p", p, "mode", mode)
        got = _noalloc(E, C, c2t, H, p, mode, T, 0x5EED)
        head = FlashHead(E, C, pb.C2T, max_batch=B)
        head.set_path("multi")
        ref = host(head.forward(H, p, mode=mode, temperature=T, seed=0x5EED, want_clusters=True,
                                want_retrieved=True))
        head.close()
        for k in KEYS:
            assert np.array_equal(got[k], ref[k], equal_nan=False), (shape, k)
        rep = parity.check_forward(oracle.OracleHead(pb.E, pb.C, pb.C2T), pb.H[:B], p, mode, T,
                                   0x5EED, got)
        assert rep.ok(), rep.failures


def test_noalloc_refuses_a_workspace_beyond_its_array():
    need_gpu()
    from lm_output_head_amd import FlashHeadError, fh_forward_noalloc
    pb = make_problem("tiny", nq=64)
    E, C, H = problem_tensors(pb)
    c2t = torch.from_numpy(np.ascontiguousarray(pb.C2T, dtype=np.int32)).cuda()
    Hbig = H.repeat(1024, 1)  # 65536 queries: ~0.8 GB of workspace
    Hbig = Hbig[:65535].contiguous()
    tok = torch.empty(Hbig.shape[0], dtype=torch.int32, device="cuda")
    with pytest.raises(FlashHeadError) as ei:
        fh_forward_noalloc(E, C, c2t, Hbig, 256, 0, 1.0, 0, tok)
    assert ei.value.status == -1 and "workspace" in str(ei.value)
