"""Invariants of the seeded synthetic workloads (no method arithmetic here)."""

import numpy as np
import pytest
import torch

import oracle
from synth import SHAPES, bf16_bits_to_f32, f32_to_bf16_bits, make_problem


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0],
                                 dtype=np.float32)])
    mine = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(bf16_bits_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def _check(pb):
    s = pb.shape
    assert pb.E.shape == (s.v, s.d) and pb.C.shape == (s.c, s.d)
    assert pb.C2T.shape == (s.c, s.b) and pb.C2T.dtype == np.int32
    oracle.validate_c2t(pb.C2T, s.v, s.c, s.b)  # balanced, a permutation
    tol = 1e-5 if s.dtype == "f32" else 2e-2
    assert np.allclose(np.linalg.norm(pb.E, axis=1), 1.0, atol=tol)
    assert np.allclose(np.linalg.norm(pb.C, axis=1), 1.0, atol=tol)
    # cluster quality: mean cosine of each token with its cluster's centroid
    Et = pb.E[pb.C2T]  # [c, b, d]
    cos = np.einsum("kbd,kd->kb", Et.astype(np.float64), pb.C.astype(np.float64))
    assert cos.mean() > 0.6
    if s.dtype == "bf16":
        assert np.array_equal(bf16_bits_to_f32(pb.E_bits), pb.E)
        assert np.array_equal(bf16_bits_to_f32(pb.H_bits), pb.H)


def test_tiny_invariants_and_determinism():
    pb = make_problem("tiny")
    _check(pb)
    assert pb.H.shape == (64, 256)
    pb2 = make_problem(SHAPES["tiny"], seed_data=0, seed_query=1, nq=64)
    assert pb2 is pb  # memoised
    from synth.clustered import _make_problem_cached
    fresh = _make_problem_cached.__wrapped__(SHAPES["tiny"], 0, 1, 64)
    assert np.array_equal(fresh.E, pb.E) and np.array_equal(fresh.H, pb.H)
    other = _make_problem_cached.__wrapped__(SHAPES["tiny"], 1, 1, 64)
    assert not np.array_equal(other.E, pb.E)


@pytest.mark.slow
def test_llama_shape_invariants():
    pb = make_problem("llama32_1b", nq=8)
    _check(pb)
    assert pb.E_bits.dtype == np.uint16 and pb.E_bits.shape == (128256, 2048)
