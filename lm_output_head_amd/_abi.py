"""ctypes declarations of libflashhead's C ABI (include/flashhead.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""

from __future__ import annotations

import ctypes
import os

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashhead.so")

FH_OK, FH_EINVAL, FH_ENOMEM, FH_EHIP, FH_EUNSUPPORTED = 0, -1, -2, -3, -4
FH_F32, FH_BF16 = 0, 1
FH_QUANT_NONE, FH_QUANT_INT4_G32, FH_QUANT_INT8_G32 = 0, 1, 2
FH_PROBE_TOPK, FH_PROBE_SAMPLE, FH_TOKEN_ARGMAX, FH_TOKEN_SAMPLE = 0, 1, 0, 2
FH_PROBE_SHARED = 4
FH_PATH_AUTO, FH_PATH_MULTI = 0, 1

# Every symbol the header declares.
EXPORTS = (
    "fh_create", "fh_destroy", "fh_forward", "fh_forward_adaptive", "fh_forward_noalloc", "fh_probs_fp8",
    "fh_score",
    "fh_dense_forward",
    "fh_get_int4", "fh_get_int8", "fh_spec_verify", "fh_profile_begin", "fh_profile_end",
    "fh_set_path", "fh_sync_status",
    "fh_balanced_assign", "fh_cluster", "fh_last_error", "fh_version",
)


class FhKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class FhClusterTimes(ctypes.Structure):
    _fields_ = [("init_ms", ctypes.c_float), ("sims_ms", ctypes.c_float),
                ("total_ms", ctypes.c_float), ("pp_step_us", ctypes.c_float),
                ("rounds", ctypes.c_int)]


class FlashHeadError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"flashhead status {status}: {message}")
        self.status = status


_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_int = ctypes.c_int
_f = ctypes.c_float

_SIGS = {
    "fh_create": ([_p, _p, _p, _int, _i64, _i64, _i64, _int, _i64, _p, ctypes.POINTER(_p)], _int),
    "fh_destroy": ([_p], None),
    "fh_forward": ([_p, _p, _i64, _i64, _int, _f, _u64, _p, _p, _p, _p, _p, _p, _p], _int),
    "fh_forward_adaptive": ([_p, _p, _i64, _i64, _i64, _f, _int, _f, _u64, _p, _p, _p, _p, _p,
                             _p, _p, _p], _int),
    "fh_probs_fp8": ([_p, _p, _i64, _i64, _f, _p, _p, _p], _int),
    "fh_forward_noalloc": ([_p, _p, _p, _int, _i64, _i64, _i64, _p, _i64, _i64, _int, _f, _u64,
                            _p, _p, _p, _p, _p, _p, _p], _int),
    "fh_score": ([_p, _p, _i64, _p, _p], _int),
    "fh_dense_forward": ([_p, _p, _i64, _int, _f, _u64, _p, _p, _p, _p, _p], _int),
    "fh_get_int4": ([_p, _p, _p, _p], _int),
    "fh_get_int8": ([_p, _p, _p, _p], _int),
    "fh_spec_verify": ([_p, _p, _i64, _i64, _p, _p, _p, _f, _u64, _p, _p, _p, _p], _int),
    "fh_profile_begin": ([_p, _i64], _int),
    "fh_profile_end": ([_p, ctypes.POINTER(FhKernelTime), _int, ctypes.POINTER(_int)], _int),
    "fh_set_path": ([_p, _int], _int),
    "fh_sync_status": ([_p, _p], _int),
    "fh_balanced_assign": ([_p, _i64, _i64, _p, ctypes.POINTER(_int), _p], _int),
    "fh_cluster": ([_p, _int, _i64, _i64, _i64, _int, ctypes.POINTER(ctypes.c_double), _p, _p, _p,
                    _p, ctypes.POINTER(FhClusterTimes), _p], _int),
    "fh_last_error": ([], ctypes.c_char_p),
    "fh_version": ([], ctypes.c_char_p),
}


def lib_path() -> str:
    return os.environ.get("FLASHHEAD_LIB", LIB)


def load() -> ctypes.CDLL:
    """Load libflashhead.so (built in-tree) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m lm_output_head_amd.build` "
            "(there is no fallback implementation)")
    # torch ships its own HIP runtime beside the system one this library
    # links.  Loaded after this library, torch's runtime was the one that saw
    # the GPU and ours reported no device (build() then smoke() in one
    # process); loaded first, both work.  Importing torch loads its libraries
    # without touching the GPU.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FH_OK:
        msg = load().fh_last_error().decode(errors="replace")
        raise FlashHeadError(status, msg)
