"""FlashHead inference for MI355X (gfx950): hand-written HIP kernels behind a
C ABI (include/flashhead.h), with this thin torch/ctypes binding on top."""

from ._abi import (FH_BF16, FH_F32, FH_PROBE_SAMPLE, FH_PROBE_TOPK,  # noqa: F401
                   FH_QUANT_INT4_G32, FH_QUANT_INT8_G32, FH_QUANT_NONE, FH_TOKEN_ARGMAX,
                   FH_TOKEN_SAMPLE,
                   FlashHeadError)
from ._abi import load as load_library  # noqa: F401


def __getattr__(name):
    # the torch-facing binding is imported lazily so that the ABI module and
    # the build script stay usable without initialising torch
    if name in ("FlashHead", "fh_create", "fh_destroy", "fh_forward", "fh_forward_adaptive", "fh_forward_noalloc", "fh_probs_fp8", "fh_score",
                "fh_dense_forward", "fh_get_int4", "fh_get_int8", "fh_spec_verify", "fh_profile_begin", "fh_profile_end",
                "fh_set_path", "fh_sync_status", "fh_balanced_assign", "fh_cluster",
                "fh_last_error", "fh_version"):
        from . import flashhead
        return getattr(flashhead, name)
    raise AttributeError(name)
