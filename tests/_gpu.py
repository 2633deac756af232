"""Shared helpers for the GPU tests (not collected: no test_ prefix)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def say(*a):
    """Name the case before each GPU step, flushed, so a crash log points at it."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def to_dev(pb_array_bits_or_f32, dtype):
    """numpy uint16 bf16 bits or float32 -> contiguous GPU tensor of dtype."""
    if dtype == torch.bfloat16:
        t = torch.from_numpy(np.ascontiguousarray(pb_array_bits_or_f32).view(np.int16))
        return t.view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(pb_array_bits_or_f32, dtype=np.float32)).cuda()


def problem_tensors(pb):
    """Device copies of a synth Problem's E, C and H in its stored dtype."""
    if pb.shape.dtype == "bf16":
        dt = torch.bfloat16
        return to_dev(pb.E_bits, dt), to_dev(pb.C_bits, dt), to_dev(pb.H_bits, dt)
    dt = torch.float32
    return to_dev(pb.E, dt), to_dev(pb.C, dt), to_dev(pb.H, dt)


def host(out: dict) -> dict:
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def assert_report(rep, what):
    msg = (f"{what}: {rep.queries} queries, cluster near-ties {rep.cluster_ties}, "
           f"token near-ties {rep.token_ties}, max logit err {rep.max_logit_err:.3g} tol, "
           f"max lse err {rep.max_lse_err:.3g} tol")
    say(msg)
    assert rep.ok(), msg + "\n" + "\n".join(rep.failures)
