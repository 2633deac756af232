"""Pins of the oracle's Philox4x32-10 and Gumbel noise.

The independent reference is rocRAND's header-only Philox4x32-10 engine,
compiled here for the host (it needs no GPU), driven through the counter
mapping stated in oracle/philox.py.  Uniformity and the Gumbel transform are
checked against their distributions.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("philox") / "rocrand_philox")
    src = os.path.join(HERE, "pins", "rocrand_philox.cpp")
    subprocess.run([hipcc, "-O1", "-o", exe, src], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)

    def run(seed, row, stage, nblocks):
        out = subprocess.run([exe, str(seed), str(row), str(stage), str(nblocks)],
                             check=True, stdout=subprocess.PIPE, text=True).stdout
        return np.array([[int(x) for x in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64).astype(np.uint32)
    return run


@pytest.mark.parametrize("seed,row,stage", [
    (0, 0, 0), (0x5EED, 0, 0), (0x5EED, 3, 1), (0xFFFFFFFFFFFFFFFF, 0x3FFFFFFF, 1),
    (123456789987654321, 77, 0), (1 << 32, 1, 1)])
def test_philox_matches_rocrand(rocrand_ref, seed, row, stage):
    nblocks = 64
    ref = rocrand_ref(seed, row, stage, nblocks)
    idx = np.arange(4 * nblocks)
    mine = philox.philox_words(seed, row, idx, stage).reshape(nblocks, 4)
    assert np.array_equal(mine, ref)


def test_philox_raw_function_matches_rocrand_zero_counter(rocrand_ref):
    ref = rocrand_ref(0, 0, 0, 1)[0]
    got = philox.philox4x32_10(np.zeros((1, 4), dtype=np.uint32), [0, 0])[0]
    assert np.array_equal(got, ref)


def test_uniform_mapping_is_exact_and_open():
    w = np.array([0, 511, 512, 0xFFFFFFFF], dtype=np.uint32)
    u = philox.uniform_from_word(w)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[2] == 3 * 2.0 ** -24
    assert u[3] == 1 - 2.0 ** -24
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)  # exact in float32


def test_words_uniform_and_bits_balanced():
    idx = np.arange(1 << 20)
    w = philox.philox_words(99, 5, idx, 0)
    counts = np.bincount((w >> np.uint32(24)).astype(np.int64), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-4
    bits = np.unpackbits(w.view(np.uint8)).reshape(-1, 32).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / np.sqrt(w.size))


def test_gumbel_distribution():
    g = philox.gumbel(7, np.arange(256)[:, None], np.arange(1024)[None, :], 1).reshape(-1)
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-4
    assert abs(g.mean() - np.euler_gamma) < 0.01


def test_streams_differ_by_row_stage_and_seed():
    idx = np.arange(64)
    a = philox.philox_words(1, 0, idx, 0)
    assert not np.array_equal(a, philox.philox_words(1, 1, idx, 0))
    assert not np.array_equal(a, philox.philox_words(1, 0, idx, 1))
    assert not np.array_equal(a, philox.philox_words(2, 0, idx, 0))
