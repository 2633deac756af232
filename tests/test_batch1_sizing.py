"""Host check of the single-launch batch-1 sizing: the hand-over words the
kernel writes fit the buffer the engine allocates for every probe count (the
stage-2 grid is not monotone in p, so each p is checked), the stage-1
workgroups cover every centroid row and each stage-2 workgroup's probe list
fits its LDS array (the C++ sizing header compiled with g++; no GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_output_head_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "pins", "batch1_sizing.cpp")

# (v, c): the configs' heads, the tiny head, ragged test heads, the limits
HEADS = [(4096, 256), (128256, 8016), (262144, 16384), (151936, 9496), (1500, 300),
         (3000, 1000), (1200, 100), (20000, 2000), (640, 40), (16032, 8016), (8192, 512),
         (4096, 4096), (16384, 16384), (1024, 1), (16, 16)]


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("sizing") / "batch1_sizing")
    subprocess.run([gxx, "-O1", "-std=c++17", "-I", CSRC, "-o", out, SRC], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return out


@pytest.mark.parametrize("cus", [256, 304, 80, 20, 10])
@pytest.mark.parametrize("v,c", HEADS)
def test_batch1_words_fit_for_every_p(exe, v, c, cus):
    r = subprocess.run([exe, str(v), str(c), str(cus)], stdout=subprocess.PIPE, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout
