"""Seeded generator of balanced clustered output embeddings and decode queries.

The FlashHead pages (FlashHead explainer, framerc.cn, §1.2.1 "balanced
clustering"; arXiv 2603.14591 abstract, innovation (1)) describe a vocabulary
split into c clusters of exactly b = v/c tokens each, recorded in a dense
cluster-to-token table C2T[c x b], with c unit-norm centroids C.  Real output
embeddings and their clustering are not available here, so this module plants
such a structure directly:

1. ``rng = default_rng(seed_data)``.
2. ``mu``: c standard-normal float32 rows, each L2-normalised.
3. ``perm = rng.permutation(v)``; ``C2T = perm.reshape(c, b)``: token
   ``perm[k*b + j]`` sits in cluster k, slot j.
4. ``noise``: v x d standard-normal float32; ``E[t] = normalize(mu[k(t)] +
   spread * noise[t] / sqrt(d))`` where k(t) is t's cluster; spread = 0.3
   unless the shape sets another (a token's cosine to its cluster's
   direction is about 1 / sqrt(1 + spread^2)).
5. ``C[k] = normalize(mean_j E[C2T[k, j]])`` in float32.
6. E and C are rounded to bfloat16 (round to nearest, ties to even) unless the
   shape is float32.
7. Queries: ``rq = default_rng(seed_query)``; ``tok = rq.integers(0, v, nq)``;
   ``h = alpha * E_rounded[tok] + rq.standard_normal((nq, d)) / sqrt(d)``,
   then rounded like E.

All scalars are explicit float32 so that numpy does not promote to float64.
"""

from __future__ import annotations

import functools
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Shape:
    """A head shape: vocabulary v, hidden size d, clusters c, probes p."""

    name: str
    v: int
    d: int
    c: int
    p: int
    dtype: str  # "f32" or "bf16": the storage type of E, C and h
    alpha: float  # query scale on its source token's embedding
    nq: int  # number of generated queries
    spread: float = 0.3  # within-cluster noise scale of the embeddings

    @property
    def b(self) -> int:
        return self.v // self.c


# The five workloads share four shapes.  Shapes follow public model heads:
# Llama-3.2-1B (v=128256, d=2048), Gemma-3-1B (v=262144, d=1152) and
# Qwen-3-4B (v=151936, d=2560); c = v/16 in each, as the explainer recommends
# (§2.3: c about v/16; §1.2.1: c = 8016 for a 128K vocabulary).
SHAPES = {
    "tiny": Shape("tiny", 4096, 256, 256, 16, "f32", 4.0, 64),
    "llama32_1b": Shape("llama32_1b", 128256, 2048, 8016, 512, "bf16", 4.0, 256),
    "gemma3_1b": Shape("gemma3_1b", 262144, 1152, 16384, 512, "bf16", 2.0, 256),
    "qwen3_4b": Shape("qwen3_4b", 151936, 2560, 9496, 1024, "bf16", 4.0, 256),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normalize_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("ij,ij->i", x, x, dtype=np.float32))[:, None]
    return (x / n).astype(np.float32)


@dataclass
class Problem:
    """One generated workload.

    ``E``, ``C`` and ``H`` are float32 arrays holding exactly the values that
    the stored dtype represents (bfloat16 values widened, for bf16 shapes).
    ``E_bits``/``C_bits``/``H_bits`` hold the bfloat16 bit patterns (None for
    float32 shapes).  ``C2T`` is int32 [c x b]; ``tok`` the token each query
    was drawn around.
    """

    shape: Shape
    E: np.ndarray
    C: np.ndarray
    C2T: np.ndarray
    H: np.ndarray
    tok: np.ndarray
    E_bits: np.ndarray | None
    C_bits: np.ndarray | None
    H_bits: np.ndarray | None

    @property
    def v(self):
        return self.shape.v

    @property
    def d(self):
        return self.shape.d

    @property
    def c(self):
        return self.shape.c

    @property
    def b(self):
        return self.shape.b


def make_problem(shape: Shape | str, seed_data: int = 0, seed_query: int = 1,
                 nq: int | None = None) -> Problem:
    """Generate the clustered workload for ``shape`` (see module docstring)."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    return _make_problem_cached(shape, seed_data, seed_query,
                                shape.nq if nq is None else nq)


@functools.lru_cache(maxsize=2)
def _make_problem_cached(shape: Shape, seed_data: int, seed_query: int, nq: int) -> Problem:
    v, d, c = shape.v, shape.d, shape.c
    if v % c != 0:
        raise ValueError("v must be a multiple of c (balanced clusters)")
    b = v // c
    rng = np.random.default_rng(seed_data)
    mu = _normalize_rows(rng.standard_normal((c, d), dtype=np.float32))
    perm = rng.permutation(v)
    c2t = perm.reshape(c, b).astype(np.int32)
    cluster_of = np.empty(v, dtype=np.int64)
    cluster_of[perm] = np.arange(v, dtype=np.int64) // b
    noise = rng.standard_normal((v, d), dtype=np.float32)
    noise *= np.float32(shape.spread) / np.float32(np.sqrt(np.float32(d)))
    noise += mu[cluster_of]
    E32 = _normalize_rows(noise)
    del noise
    C32 = _normalize_rows(E32[c2t].mean(axis=1, dtype=np.float32))

    rq = np.random.default_rng(seed_query)
    tok = rq.integers(0, v, nq)
    if shape.dtype == "bf16":
        E_bits = f32_to_bf16_bits(E32)
        del E32
        E = bf16_bits_to_f32(E_bits)
        C_bits = f32_to_bf16_bits(C32)
        C = bf16_bits_to_f32(C_bits)
    elif shape.dtype == "f32":
        E, C, E_bits, C_bits = E32, C32, None, None
    else:
        raise ValueError(f"unknown dtype {shape.dtype}")
    H32 = (np.float32(shape.alpha) * E[tok]
           + rq.standard_normal((nq, d), dtype=np.float32) / np.float32(np.sqrt(np.float32(d))))
    H32 = H32.astype(np.float32)
    if shape.dtype == "bf16":
        H_bits = f32_to_bf16_bits(H32)
        H = bf16_bits_to_f32(H_bits)
    else:
        H_bits, H = None, H32
    return Problem(shape, E, C, c2t, H, tok, E_bits, C_bits, H_bits)


def make_graded_queries(pb: Problem, alphas, seed: int = 7):
    """Queries of graded confidence on pb's head: h_i = alphas[i] E[t_i] +
    n_i / sqrt(d) for a random token t_i and standard normal n_i (alpha = 0
    is pure noise, a diffuse query; the shape's own alpha gives pb's queries),
    rounded to the stored dtype.  Returns (H float32, H_bits or None, tokens)."""
    alphas = np.asarray(alphas, dtype=np.float32)
    nq, d = alphas.size, pb.shape.d
    rq = np.random.default_rng(seed)
    tok = rq.integers(0, pb.shape.v, nq)
    H32 = (alphas[:, None] * pb.E[tok]
           + rq.standard_normal((nq, d), dtype=np.float32) / np.float32(np.sqrt(np.float32(d))))
    H32 = H32.astype(np.float32)
    if pb.shape.dtype == "bf16":
        bits = f32_to_bf16_bits(H32)
        return bf16_bits_to_f32(bits), bits, tok
    return H32, None, tok
