"""The plain read probe (bench.py's fhb_read_probe) behind --burst: a search for
one 32-bit value, so it must see every word of the buffer, including the last
one of a ragged final workgroup."""

import numpy as np
import pytest
import torch

from _gpu import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16384, 16384 * 3 + 48, 32_869_696])
def test_read_probe_finds_every_word(nbytes):
    need_gpu()
    import ctypes

    import bench
    blib = bench.load_bench_lib()

    def fh_read_probe(b, key, f):
        st = torch.cuda.current_stream().cuda_stream
        assert blib.fhb_read_probe(ctypes.c_void_p(b.data_ptr()), b.numel() * 4, key & 0xFFFFFFFF,
                                   ctypes.c_void_p(f.data_ptr()), ctypes.c_void_p(st)) == 0
    say("read probe", nbytes)
    n = nbytes // 4
    # distinct words 1 .. n (a permutation), so a key is present exactly once
    words = np.random.default_rng(nbytes).permutation(n).astype(np.uint32) + 1
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    for pos in sorted({0, n // 2, n - 1}):
        found.zero_()
        fh_read_probe(buf, int(words[pos]), found)
        assert int(found.item()) == 1, pos
    found.zero_()
    fh_read_probe(buf, 0, found)          # absent: the words are 1 .. n
    fh_read_probe(buf, n + 1, found)
    assert int(found.item()) == 0
