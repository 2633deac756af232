"""Thin Python binding of libflashhead: torch tensors in, C-ABI calls out.

Functions named like the C entry points (``fh_create``, ``fh_forward`` ...)
only marshal arguments: they check tensor placement and dtype, pass raw
pointers and the current HIP stream, and raise on a non-OK status.  All
computation runs in the library's HIP kernels.  ``FlashHead`` wraps an engine
with output allocation for convenience.
"""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import torch

from . import _abi
from ._abi import (FH_BF16, FH_F32, FH_PROBE_SAMPLE, FH_PROBE_TOPK, FH_QUANT_INT4_G32,  # noqa: F401
                   FH_QUANT_INT8_G32, FH_QUANT_NONE, FH_TOKEN_ARGMAX, FH_TOKEN_SAMPLE, FlashHeadError, check)

_DTYPES = {torch.float32: FH_F32, torch.bfloat16: FH_BF16}
_QUANTS = {"none": FH_QUANT_NONE, "int4": FH_QUANT_INT4_G32, "int8": FH_QUANT_INT8_G32}


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to libflashhead must be contiguous GPU tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(t, dtype, shape, name):
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


# What each engine was created with: h must have the engine's dtype and d
# columns and every output its size, or the kernels would read or write past
# them.  Keyed by the handle's value: (dtype, v, d, c).
_ENGINES = {}


def _engine_h(eng, h):
    """Check h [B x d] against the engine; returns (B, v, d, c)."""
    key = eng.value if isinstance(eng, ctypes.c_void_p) else eng
    info = _ENGINES.get(key)
    if info is None:
        raise ValueError("unknown engine handle (not created by fh_create, or destroyed)")
    dtype, v, d, c = info
    if h.dim() != 2:
        raise ValueError(f"h must be [B x d], got shape {tuple(h.shape)}")
    _require(h, dtype, (h.shape[0], d), "h")
    return h.shape[0], v, d, c


def fh_version() -> str:
    return _abi.load().fh_version().decode()


def fh_last_error() -> str:
    return _abi.load().fh_last_error().decode()


def fh_create(E: torch.Tensor, C: torch.Tensor, C2T, quant: str = "none", max_batch: int = 1,
              stream=None) -> ctypes.c_void_p:
    """Create an engine.  E [v x d] and C [c x d] on the GPU (float32 or
    bfloat16, same dtype); C2T [c x b] int32 on the host (numpy or CPU tensor)."""
    lib = _abi.load()
    if E.dtype not in _DTYPES or C.dtype != E.dtype:
        raise ValueError("E and C must share dtype float32 or bfloat16")
    c2t = np.ascontiguousarray(np.asarray(C2T), dtype=np.int32)
    v, d = E.shape
    c = C.shape[0]
    if C.shape[1] != d or c2t.size != v:
        raise ValueError("inconsistent shapes of E, C and C2T")
    eng = ctypes.c_void_p()
    check(lib.fh_create(_ptr(E), _ptr(C), c2t.ctypes.data_as(ctypes.c_void_p), _DTYPES[E.dtype],
                        v, d, c, _QUANTS[quant], max_batch, _stream(stream), ctypes.byref(eng)))
    _ENGINES[eng.value] = (E.dtype, v, d, c)
    return eng


def fh_destroy(eng) -> None:
    _abi.load().fh_destroy(eng)
    _ENGINES.pop(eng.value if isinstance(eng, ctypes.c_void_p) else eng, None)


def fh_forward(eng, h, p, mode, temperature, seed, out_token, out_token_logit=None, out_lse=None,
               out_clusters=None, out_ids=None, out_logits=None, stream=None) -> None:
    B, v, _, c = _engine_h(eng, h)
    b = v // c
    _require(out_token, torch.int32, (B,), "out_token")
    _require(out_token_logit, torch.float32, (B,), "out_token_logit")
    _require(out_lse, torch.float32, (B,), "out_lse")
    _require(out_clusters, torch.int32, (B, p), "out_clusters")
    _require(out_ids, torch.int32, (B, p * b), "out_ids")
    _require(out_logits, torch.float32, (B, p * b), "out_logits")
    check(_abi.load().fh_forward(eng, _ptr(h), h.shape[0], p, mode, temperature, seed,
                                 _ptr(out_token), _ptr(out_token_logit), _ptr(out_lse),
                                 _ptr(out_clusters), _ptr(out_ids), _ptr(out_logits),
                                 _stream(stream)))


def fh_forward_adaptive(eng, h, p_max, p_min, tau, mode, temperature, seed, out_token,
                        out_nprobe=None, out_token_logit=None, out_lse=None, out_clusters=None,
                        out_ids=None, out_logits=None, stream=None) -> None:
    B, v, _, c = _engine_h(eng, h)
    b = v // c
    _require(out_nprobe, torch.int32, (B,), "out_nprobe")
    _require(out_token, torch.int32, (B,), "out_token")
    _require(out_token_logit, torch.float32, (B,), "out_token_logit")
    _require(out_lse, torch.float32, (B,), "out_lse")
    _require(out_clusters, torch.int32, (B, p_max), "out_clusters")
    _require(out_ids, torch.int32, (B, p_max * b), "out_ids")
    _require(out_logits, torch.float32, (B, p_max * b), "out_logits")
    check(_abi.load().fh_forward_adaptive(eng, _ptr(h), B, p_max, p_min, tau, mode, temperature,
                                          seed, _ptr(out_nprobe), _ptr(out_token),
                                          _ptr(out_token_logit), _ptr(out_lse), _ptr(out_clusters),
                                          _ptr(out_ids), _ptr(out_logits), _stream(stream)))


def fh_forward_noalloc(E, C, c2t, h, p, mode, temperature, seed, out_token, out_token_logit=None,
                       out_lse=None, out_clusters=None, out_ids=None, out_logits=None,
                       stream=None) -> None:
    """fh_forward without an engine, on caller-owned tables (c2t: a device
    int32 [c x b] permutation of [0, v)), with the library's fixed workspace."""
    if E.dtype not in _DTYPES or C.dtype != E.dtype or h.dtype != E.dtype:
        raise ValueError("E, C and h must share dtype float32 or bfloat16")
    v, d = E.shape
    c = C.shape[0]
    if C.shape[1] != d or h.dim() != 2 or h.shape[1] != d or c < 1 or v % c:
        raise ValueError("inconsistent shapes of E, C and h")
    B, b = h.shape[0], v // c
    _require(c2t, torch.int32, (c, b), "c2t")
    _require(out_token, torch.int32, (B,), "out_token")
    _require(out_token_logit, torch.float32, (B,), "out_token_logit")
    _require(out_lse, torch.float32, (B,), "out_lse")
    _require(out_clusters, torch.int32, (B, p), "out_clusters")
    _require(out_ids, torch.int32, (B, p * b), "out_ids")
    _require(out_logits, torch.float32, (B, p * b), "out_logits")
    check(_abi.load().fh_forward_noalloc(_ptr(E), _ptr(C), _ptr(c2t), _DTYPES[E.dtype], v, d, c,
                                         _ptr(h), B, p, mode, temperature, seed, _ptr(out_token),
                                         _ptr(out_token_logit), _ptr(out_lse), _ptr(out_clusters),
                                         _ptr(out_ids), _ptr(out_logits), _stream(stream)))


def fh_probs_fp8(logits, lse, temperature, out_probs, out_scale_exp, stream=None) -> None:
    """fp8 E4M3 bytes of exp(logits / T' - lse) 2^k per row of [B x n] float32
    logits, with the row's power-of-two scale exponent k in out_scale_exp."""
    if logits is None or lse is None or out_probs is None or out_scale_exp is None:
        raise ValueError("logits, lse, out_probs and out_scale_exp are required")
    if logits.dim() != 2:
        raise ValueError(f"logits must be [B x n], got shape {tuple(logits.shape)}")
    B, n = logits.shape
    _require(logits, torch.float32, (B, n), "logits")
    _require(lse, torch.float32, (B,), "lse")
    _require(out_probs, torch.uint8, (B, n), "out_probs")
    _require(out_scale_exp, torch.int32, (B,), "out_scale_exp")
    check(_abi.load().fh_probs_fp8(_ptr(logits), _ptr(lse), B, n, temperature, _ptr(out_probs),
                                   _ptr(out_scale_exp), _stream(stream)))


def fh_score(eng, h, out_scores, stream=None) -> None:
    B, _, _, c = _engine_h(eng, h)
    _require(out_scores, torch.float32, (B, c), "out_scores")
    check(_abi.load().fh_score(eng, _ptr(h), h.shape[0], _ptr(out_scores), _stream(stream)))


def fh_dense_forward(eng, h, mode, temperature, seed, out_token, out_token_logit=None,
                     out_lse=None, out_logits=None, stream=None) -> None:
    B, v, _, _ = _engine_h(eng, h)
    _require(out_token, torch.int32, (B,), "out_token")
    _require(out_token_logit, torch.float32, (B,), "out_token_logit")
    _require(out_lse, torch.float32, (B,), "out_lse")
    _require(out_logits, torch.float32, (B, v), "out_logits")
    check(_abi.load().fh_dense_forward(eng, _ptr(h), h.shape[0], mode, temperature, seed,
                                       _ptr(out_token), _ptr(out_token_logit), _ptr(out_lse),
                                       _ptr(out_logits), _stream(stream)))


def fh_get_int4(eng, packed, scales, stream=None) -> None:
    check(_abi.load().fh_get_int4(eng, _ptr(packed), _ptr(scales), _stream(stream)))


def fh_get_int8(eng, codes, scales, stream=None) -> None:
    check(_abi.load().fh_get_int8(eng, _ptr(codes), _ptr(scales), _stream(stream)))


def fh_spec_verify(eng, h, p, draft_clusters, draft_token, draft_lse, temperature, seed,
                   out_token, out_accepted=None, out_lse=None, stream=None) -> None:
    B, _, _, _ = _engine_h(eng, h)
    _require(draft_clusters, torch.int32, (B, p), "draft_clusters")
    _require(draft_token, torch.int32, (B,), "draft_token")
    _require(draft_lse, torch.float32, (B,), "draft_lse")
    _require(out_token, torch.int32, (B,), "out_token")
    _require(out_accepted, torch.int32, (B,), "out_accepted")
    _require(out_lse, torch.float32, (B,), "out_lse")
    check(_abi.load().fh_spec_verify(eng, _ptr(h), h.shape[0], p, _ptr(draft_clusters),
                                     _ptr(draft_token), _ptr(draft_lse), temperature, seed,
                                     _ptr(out_token), _ptr(out_accepted), _ptr(out_lse),
                                     _stream(stream)))


def fh_set_path(eng, path: int) -> None:
    check(_abi.load().fh_set_path(eng, path))


def fh_sync_status(eng, stream=None) -> None:
    check(_abi.load().fh_sync_status(eng, _stream(stream)))


def fh_profile_begin(eng, max_launches: int) -> None:
    check(_abi.load().fh_profile_begin(eng, max_launches))


def fh_profile_end(eng) -> dict:
    """Per-kernel {name: (launches, total_ms)} since fh_profile_begin."""
    recs = (_abi.FhKernelTime * 64)()
    n = ctypes.c_int(0)
    check(_abi.load().fh_profile_end(eng, recs, 64, ctypes.byref(n)))
    return {recs[i].name.decode(): (recs[i].launches, recs[i].total_ms) for i in range(n.value)}


def fh_balanced_assign(sims: torch.Tensor, out_assign: torch.Tensor, stream=None) -> int:
    """Balanced assignment of v tokens to c clusters of v / c: sims [v x c]
    float32 on the GPU, out_assign [v] int32 on the GPU.  Returns the number
    of rounds."""
    v, c = sims.shape
    _require(sims, torch.float32, (v, c), "sims")
    _require(out_assign, torch.int32, (v,), "out_assign")
    rounds = ctypes.c_int(0)
    check(_abi.load().fh_balanced_assign(_ptr(sims), v, c, _ptr(out_assign), ctypes.byref(rounds),
                                         _stream(stream)))
    return rounds.value


def fh_cluster(E: torch.Tensor, c: int, iters: int, u, out_C: torch.Tensor, out_c2t: torch.Tensor,
               out_init=None, out_assign=None, stream=None) -> dict:
    """Balanced spherical k-means over E's rows (float32 or bfloat16 on the
    GPU) into c clusters; u holds the c k-means++ uniforms (host).  Fills
    out_C [c x d] float32 and out_c2t [c x v/c] int32 (and optionally
    out_init [c], out_assign [v] int32) and returns the call's timings."""
    if E.dtype not in _DTYPES:
        raise ValueError("E must be float32 or bfloat16")
    v, d = E.shape
    if c < 1 or v % c:
        raise ValueError("v must be a multiple of c")
    _require(out_C, torch.float32, (c, d), "out_C")
    _require(out_c2t, torch.int32, (c, v // c), "out_c2t")
    _require(out_init, torch.int32, (c,), "out_init")
    _require(out_assign, torch.int32, (v,), "out_assign")
    uu = np.ascontiguousarray(np.asarray(u, dtype=np.float64))
    if uu.shape != (c,):
        raise ValueError("u must hold c uniforms")
    t = _abi.FhClusterTimes()
    check(_abi.load().fh_cluster(_ptr(E), _DTYPES[E.dtype], v, d, c, iters,
                                 uu.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), _ptr(out_C),
                                 _ptr(out_c2t), _ptr(out_init), _ptr(out_assign), ctypes.byref(t),
                                 _stream(stream)))
    return {"init_ms": t.init_ms, "sims_ms": t.sims_ms, "total_ms": t.total_ms,
            "pp_step_us": t.pp_step_us, "rounds": t.rounds}


class FlashHead:
    """An engine over one head, with output allocation.

    ``E`` and ``C`` stay borrowed by the engine; this object keeps references
    to them so they outlive it.
    """

    def __init__(self, E: torch.Tensor, C: torch.Tensor, C2T, quant: str = "none",
                 max_batch: int = 1, stream=None):
        self.v, self.d = E.shape
        self.c = C.shape[0]
        self.b = self.v // self.c
        self.quant = quant
        self.max_batch = max_batch
        self.device = E.device
        self._E = E
        self._C = C if quant == "none" else None
        self.eng = fh_create(E, C, C2T, quant, max_batch, stream)

    def close(self):
        if getattr(self, "eng", None) is not None:
            fh_destroy(self.eng)
            self.eng = None

    def __del__(self):
        # not while the interpreter shuts down: the HIP runtime (and any
        # profiler wrapping it) may already be torn down, and a process that
        # ends frees the engine's memory anyway.  Close engines explicitly.
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def _alloc(self, shape, dtype):
        return torch.empty(shape, dtype=dtype, device=self.device)

    def forward(self, h: torch.Tensor, p: int, mode: int = 0, temperature: float = 1.0,
                seed: int = 0, want_clusters: bool = False, want_retrieved: bool = False,
                stream=None) -> dict:
        B = h.shape[0]
        out = {"token": self._alloc((B,), torch.int32),
               "token_logit": self._alloc((B,), torch.float32),
               "lse": self._alloc((B,), torch.float32)}
        if want_clusters:
            out["clusters"] = self._alloc((B, p), torch.int32)
        if want_retrieved:
            out["ids"] = self._alloc((B, p * self.b), torch.int32)
            out["logits"] = self._alloc((B, p * self.b), torch.float32)
        fh_forward(self.eng, h, p, mode, temperature, seed, out["token"], out["token_logit"],
                   out["lse"], out.get("clusters"), out.get("ids"), out.get("logits"), stream)
        return out

    def forward_adaptive(self, h: torch.Tensor, p_max: int, tau: float, p_min: int = 1,
                         mode: int = 0, temperature: float = 1.0, seed: int = 0,
                         want_clusters: bool = False, want_retrieved: bool = False,
                         stream=None) -> dict:
        """forward with a per-query probe count: the first clusters in key
        order whose softmax(s/T) mass reaches tau, clamped to [p_min, p_max]."""
        B = h.shape[0]
        out = {"nprobe": self._alloc((B,), torch.int32),
               "token": self._alloc((B,), torch.int32),
               "token_logit": self._alloc((B,), torch.float32),
               "lse": self._alloc((B,), torch.float32)}
        if want_clusters:
            out["clusters"] = self._alloc((B, p_max), torch.int32)
        if want_retrieved:
            out["ids"] = self._alloc((B, p_max * self.b), torch.int32)
            out["logits"] = self._alloc((B, p_max * self.b), torch.float32)
        fh_forward_adaptive(self.eng, h, p_max, p_min, tau, mode, temperature, seed, out["token"],
                            out["nprobe"], out["token_logit"], out["lse"], out.get("clusters"),
                            out.get("ids"), out.get("logits"), stream)
        return out

    def probs_fp8(self, out: dict, temperature: float = 1.0, stream=None) -> dict:
        """fp8 E4M3 probabilities of a forward's retrieved candidates (its
        "logits" and "lse"; temperature = the LSE's T': the call's temperature
        when tokens were sampled, else 1): {"probs": uint8 [B x n],
        "scale_exp": int32 [B]}, p = value(byte) 2^-scale_exp."""
        B = out["logits"].shape[0]
        res = {"probs": self._alloc(tuple(out["logits"].shape), torch.uint8),
               "scale_exp": self._alloc((B,), torch.int32)}
        fh_probs_fp8(out["logits"], out["lse"], temperature, res["probs"], res["scale_exp"], stream)
        return res

    def score(self, h: torch.Tensor, stream=None) -> torch.Tensor:
        out = self._alloc((h.shape[0], self.c), torch.float32)
        fh_score(self.eng, h, out, stream)
        return out

    def dense(self, h: torch.Tensor, mode: int = 0, temperature: float = 1.0, seed: int = 0,
              want_logits: bool = False, stream=None) -> dict:
        B = h.shape[0]
        out = {"token": self._alloc((B,), torch.int32),
               "token_logit": self._alloc((B,), torch.float32),
               "lse": self._alloc((B,), torch.float32)}
        if want_logits:
            out["logits"] = self._alloc((B, self.v), torch.float32)
        fh_dense_forward(self.eng, h, mode, temperature, seed, out["token"], out["token_logit"],
                         out["lse"], out.get("logits"), stream)
        return out

    def spec_verify(self, h: torch.Tensor, draft: dict, p: int, temperature: float,
                    seed: int = 0, stream=None) -> dict:
        """Verify the draft of ``forward(h, p, mode=...|FH_TOKEN_SAMPLE,
        temperature, want_clusters=True)`` against the dense head."""
        B = h.shape[0]
        _require(draft["clusters"], torch.int32, (B, p), "draft clusters")
        out = {"token": self._alloc((B,), torch.int32),
               "accepted": self._alloc((B,), torch.int32),
               "lse": self._alloc((B,), torch.float32)}
        fh_spec_verify(self.eng, h, p, draft["clusters"], draft["token"], draft["lse"],
                       temperature, seed, out["token"], out["accepted"], out["lse"], stream)
        return out

    def set_path(self, path: str) -> None:
        """"auto" (single launch at B=1) or "multi" (one launch per stage)."""
        fh_set_path(self.eng, {"auto": _abi.FH_PATH_AUTO, "multi": _abi.FH_PATH_MULTI}[path])

    def sync_status(self, stream=None) -> None:
        fh_sync_status(self.eng, stream)

    def int4(self, stream=None):
        packed = self._alloc((self.c, self.d // 2), torch.uint8)
        scales = self._alloc((self.c, self.d // 32), torch.int16)
        fh_get_int4(self.eng, packed, scales, stream)
        return packed, scales

    def int8(self, stream=None):
        codes = self._alloc((self.c, self.d), torch.int8)
        scales = self._alloc((self.c, self.d // 32), torch.int16)
        fh_get_int8(self.eng, codes, scales, stream)
        return codes, scales
