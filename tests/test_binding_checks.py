"""The Python binding refuses queries and outputs that do not match the
engine before anything reaches the library (a bfloat16 h given to a float32
engine, or an h narrower than d, would make the kernels read past it; a
short output, write past it).  CPU only: the engine handle is registered by
hand and no library call is made."""

import pytest
import torch

from lm_output_head_amd import flashhead as fhb

V, D, C = 64, 32, 4  # b = 16
HANDLE = 0x5EED


@pytest.fixture
def eng():
    fhb._ENGINES[HANDLE] = (torch.bfloat16, V, D, C)
    yield HANDLE
    fhb._ENGINES.pop(HANDLE, None)


def out1(B, dt=torch.int32):
    return torch.zeros(B, dtype=dt)


@pytest.mark.parametrize("h,needle", [
    (torch.zeros(2, D, dtype=torch.float32), "h: expected torch.bfloat16"),
    (torch.zeros(2, D - 8, dtype=torch.bfloat16), "h: expected"),
    (torch.zeros(D, dtype=torch.bfloat16), "[B x d]"),
])
def test_forward_refuses_a_mismatched_query(eng, h, needle):
    with pytest.raises(ValueError, match=needle.replace("[", r"\[").replace("]", r"\]")):
        fhb.fh_forward(eng, h, 2, 0, 1.0, 0, out1(h.shape[0] if h.dim() == 2 else 1))


@pytest.mark.parametrize("which", ["token", "clusters", "ids", "logits"])
def test_forward_refuses_a_short_output(eng, which):
    B, p = 2, 3
    h = torch.zeros(B, D, dtype=torch.bfloat16)
    kw = {"out_token": out1(B), "out_clusters": torch.zeros(B, p, dtype=torch.int32),
          "out_ids": torch.zeros(B, p * 16, dtype=torch.int32),
          "out_logits": torch.zeros(B, p * 16, dtype=torch.float32)}
    short = {"token": out1(B - 1), "clusters": torch.zeros(B, p - 1, dtype=torch.int32),
             "ids": torch.zeros(B, p * 16 - 1, dtype=torch.int32),
             "logits": torch.zeros(B, p * 16, dtype=torch.float64)}
    kw["out_" + which] = short[which]
    with pytest.raises(ValueError, match="out_" + which):
        fhb.fh_forward(eng, h, p, 0, 1.0, 0, kw.pop("out_token"), **kw)


def test_score_dense_and_verify_refuse_mismatches(eng):
    h = torch.zeros(3, D, dtype=torch.float32)
    with pytest.raises(ValueError, match="h: expected"):
        fhb.fh_score(eng, h, torch.zeros(3, C))
    with pytest.raises(ValueError, match="h: expected"):
        fhb.fh_dense_forward(eng, h, 0, 1.0, 0, out1(3))
    hb = torch.zeros(3, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out_scores"):
        fhb.fh_score(eng, hb, torch.zeros(3, C - 1))
    with pytest.raises(ValueError, match="out_logits"):
        fhb.fh_dense_forward(eng, hb, 0, 1.0, 0, out1(3), out_logits=torch.zeros(3, V - 1))
    with pytest.raises(ValueError, match="draft_clusters"):
        fhb.fh_spec_verify(eng, hb, 2, torch.zeros(3, 1, dtype=torch.int32), out1(3),
                           torch.zeros(3), 1.0, 0, out1(3))


def test_unknown_engine_is_refused():
    with pytest.raises(ValueError, match="unknown engine"):
        fhb.fh_forward(0xBAD, torch.zeros(1, D, dtype=torch.bfloat16), 1, 0, 1.0, 0, out1(1))


@pytest.mark.parametrize("which", ["nprobe", "clusters", "ids", "logits"])
def test_adaptive_refuses_a_short_output(eng, which):
    # the adaptive outputs are sized by p_max: [B], [B x p_max], [B x p_max b]
    B, pmax = 2, 3
    h = torch.zeros(B, D, dtype=torch.bfloat16)
    kw = {"out_nprobe": out1(B), "out_clusters": torch.zeros(B, pmax, dtype=torch.int32),
          "out_ids": torch.zeros(B, pmax * 16, dtype=torch.int32),
          "out_logits": torch.zeros(B, pmax * 16, dtype=torch.float32)}
    short = {"nprobe": out1(B + 1), "clusters": torch.zeros(B, pmax - 1, dtype=torch.int32),
             "ids": torch.zeros(B, pmax * 16 - 16, dtype=torch.int32),
             "logits": torch.zeros(B, pmax * 16, dtype=torch.float16)}
    kw["out_" + which] = short[which]
    with pytest.raises(ValueError, match="out_" + which):
        fhb.fh_forward_adaptive(eng, h, pmax, 1, 0.9, 0, 1.0, 0, out1(B), **kw)
