"""Pins of the oracle's fp8 E4M3 probability format (explainer §2.3, the
probability intermediate as fp8): hand-worked codes from the OCP E4M3
definition, torch's own float8_e4m3fn cast as an independent library, and
the round trip over every finite code."""

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode, probs_fp8


@pytest.mark.parametrize("x,code", [
    (1.0, 0x38),                # 1.000 * 2^0: field 7, mantissa 0
    (0.5, 0x30),
    (0.9375, 0x37),             # 1.111b * 2^-1
    (0.96875, 0x38),            # midway 0.9375 / 1.0: to the even code (mantissa 0)
    (2.0 ** -6, 0x08),          # smallest normal
    (7 * 2.0 ** -9, 0x07),      # largest subnormal
    (2.0 ** -9, 0x01),          # smallest subnormal
    (2.0 ** -10, 0x00),         # midway 0 / 2^-9: to the even code 0
    (3 * 2.0 ** -10, 0x02),     # midway 2^-9 / 2^-8: to the even code 2
    (1.2 * 2.0 ** -10, 0x01),   # above the midpoint
    (448.0, 0x7E),              # largest finite
    (1000.0, 0x7E),             # saturates
    (0.0, 0x00),
])
def test_hand_worked_codes(x, code):
    assert int(e4m3_encode(np.array([x]))[0]) == code
    if x < 448:  # 0x7F, the neighbour of 448's code, is NaN
        assert abs(e4m3_decode(code) - x) <= abs(e4m3_decode(code ^ 1) - x) + 1e-300


def test_round_trip_every_finite_code():
    codes = np.arange(0x7F)
    vals = e4m3_decode(codes)
    assert np.all(np.diff(vals) > 0)
    assert np.array_equal(e4m3_encode(vals), codes.astype(np.uint8))
    assert np.isnan(e4m3_decode(0x7F)) and vals[-1] == 448.0


def test_matches_torch_float8_e4m3fn():
    """torch's float32 -> float8_e4m3fn cast (round to nearest even) on
    random probabilities, every code value, and every midpoint between codes."""
    rng = np.random.default_rng(0)
    vals = e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([rng.uniform(0, 1, 20000), 10.0 ** rng.uniform(-4, 0, 20000), vals,
                        mids, np.nextafter(mids, 0), np.nextafter(mids, 1)]).astype(np.float32)
    x = x[x <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x.astype(np.float64)), ref)


def test_probs_hand_worked_row():
    # p = [1/2, 1/4, 1/4]: p_max = 1/2 = 0.5 * 2^0, so k = 8 and the scaled
    # row is [128, 64, 64]: codes 1.0 * 2^7 (field 14) and 1.0 * 2^6 (field 13)
    b, k, p = probs_fp8(np.log([[0.5, 0.25, 0.25]]), np.array([0.0]), 1.0)
    assert int(k[0]) == 8
    assert b[0].tolist() == [0x70, 0x68, 0x68]
    # p_max = 0.3 = 0.6 * 2^-1: k = 9, 0.3 * 512 = 153.6 -> 1.001b * 2^7 = 144
    # or 1.010b * 2^7 = 160; 153.6 is nearer 160 (field 14, mantissa 2)
    b, k, _ = probs_fp8(np.log([[0.3, 0.7 / 3, 0.7 / 3, 0.7 / 3]]), np.array([0.0]), 1.0)
    assert int(k[0]) == 9 and int(b[0, 0]) == 0x72


def test_probs_rows_sum_to_one_within_the_format():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3, size=(4, 5000))
    z[0, :10] = -np.inf
    z[3] = rng.normal(0, 0.01, size=5000)  # nearly flat: every p near 1/5000
    for T in (1.0, 0.6):
        x = z / T
        lse = x.max(1) + np.log(np.exp(x - x.max(1, keepdims=True)).sum(1))
        b, k, p = probs_fp8(z, lse, T)
        np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-12)
        assert np.all(b[0, :10] == 0)
        scaled_max = np.ldexp(p.max(1), k)
        assert np.all((scaled_max >= 128) & (scaled_max < 256))
        q = np.ldexp(e4m3_decode(b), -k[:, None])
        # within half a step of the scaled value: relative 2^-4 for normals,
        # absolute 2^-10 (scaled) below 2^-6
        assert np.all(np.abs(q - p) <= np.maximum(p * 2.0 ** -4, np.ldexp(2.0 ** -10, -k[:, None])))
        assert np.all(b[3] > 0)  # a flat row keeps all of its mass
        np.testing.assert_allclose(q.sum(1), 1.0, atol=0.03)
