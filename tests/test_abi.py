"""The C-ABI library: it loads, exports every declared symbol, and rejects
bad arguments on the host before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashhead.h")


@pytest.fixture(scope="module")
def lib():
    from lm_output_head_amd import _abi
    if not os.path.exists(_abi.lib_path()):
        from lm_output_head_amd.build import build
        build()
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fh_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    from lm_output_head_amd import _abi
    assert declared_functions() == sorted(_abi.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.fh_version().decode().startswith("flashhead")


P = ctypes.c_void_p


def _create(lib, E=P(4096), C=P(8192), c2t=None, dtype=1, v=64, d=16, c=8, quant=0, max_batch=1):
    if c2t is None:
        c2t = np.arange(v, dtype=np.int32)
    out = P()
    st = lib.fh_create(E, C, c2t.ctypes.data_as(P) if c2t is not False else None, dtype, v, d, c,
                       quant, max_batch, None, ctypes.byref(out))
    return st, out, lib.fh_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    ({"E": None}, -1, "non-NULL"),
    ({"c2t": False}, -1, "non-NULL"),
    ({"dtype": 7}, -1, "dtype"),
    ({"quant": 9}, -1, "quant"),
    ({"v": 65}, -1, "multiple of c"),
    ({"v": 0}, -1, "positive"),
    ({"d": 12}, -1, "d % 8"),
    ({"dtype": 0, "d": 6}, -1, "d % 4"),
    ({"quant": 1, "d": 48}, -4, "d % 32"),
    ({"d": 8192}, -4, "too large"),
    ({"v": 32768, "c": 32768}, -4, "16384"),
    ({"max_batch": 0}, -1, "max_batch"),
    ({"E": P(4100)}, -1, "aligned"),
])
def test_create_rejects_bad_arguments(lib, kw, status, needle):
    st, out, msg = _create(lib, **kw)
    assert st == status and needle in msg and not out.value


def test_create_rejects_unbalanced_c2t(lib):
    c2t = np.arange(64, dtype=np.int32)
    c2t[5] = 3  # token 3 twice, token 5 missing
    st, _, msg = _create(lib, c2t=c2t)
    assert st == -1 and "permutation" in msg
    c2t = np.arange(64, dtype=np.int32)
    c2t[0] = 64
    st, _, msg = _create(lib, c2t=c2t)
    assert st == -1 and "outside" in msg


def test_calls_on_null_engine_fail_cleanly(lib):
    h = P(4096)
    assert lib.fh_forward(None, h, 1, 1, 0, 1.0, 0, None, None, None, None, None, None, None) == -1
    assert lib.fh_score(None, h, 1, P(4096), None) == -1
    assert lib.fh_forward_adaptive(None, h, 1, 4, 1, 0.9, 0, 1.0, 0, None, None, None, None, None,
                                   None, None, None) == -1
    assert lib.fh_dense_forward(None, h, 1, 0, 1.0, 0, None, None, None, None, None) == -1
    assert lib.fh_get_int4(None, P(4096), P(4096), None) == -1
    assert lib.fh_profile_begin(None, 4) == -1
    n = ctypes.c_int(0)
    assert lib.fh_profile_end(None, None, 0, ctypes.byref(n)) == -1
    lib.fh_destroy(None)
    assert "NULL" in lib.fh_last_error().decode()


def test_bench_read_probe_rejects_bad_arguments():
    """bench.py's read probe (its own library, outside the product ABI)
    checks its arguments before anything is launched: NULL pointers, a
    misaligned buffer, sizes that are not a positive multiple of 16."""
    import bench
    blib = bench.load_bench_lib()
    buf, out = P(4096), P(4096)
    for args in [(None, 4096, 7, out), (buf, 4096, 7, None), (P(4104), 4096, 7, out),
                 (buf, 0, 7, out), (buf, 4100, 7, out), (buf, 1 << 41, 7, out)]:
        assert blib.fhb_read_probe(*args, None) == -1, args


def test_product_library_does_not_export_the_read_probe(lib):
    assert not hasattr(lib, "fh_read_probe")

