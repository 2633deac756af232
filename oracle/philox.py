"""Philox4x32-10 counter-based generator and the Gumbel noise drawn from it.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Philox4x32-10 follows its publication: J. K. Salmon, M. A. Moraes,
R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC'11.  A 128-bit counter (four 32-bit words) and a 64-bit key (two words)
pass through ten rounds.  One round multiplies counter words 0 and 2 by the
constants 0xD2511F53 and 0xCD9E8D57 (64-bit products split into high and low
halves) and mixes the high halves with the odd counter words and the key;
between rounds each key word is incremented by a Weyl constant (0x9E3779B9,
0xBB67AE85).  The oracle evaluates it vectorised over counters in numpy.

The sampling stages of FlashHead (FlashHead explainer, framerc.cn, §1.2.3
"probabilistic sampling"; arXiv 2603.14591 abstract, innovation (3)) need
random numbers that the host cannot pass in per call, so each side of the
parity test implements this one generator from its definition.  The mapping
of (seed, row, index, stage) to a counter is fixed here:

    key     = (seed mod 2^32, seed >> 32)
    counter = (index // 4, row, stage, 0);  word = index mod 4
    u       = ((word >> 9) + 0.5) * 2^-23      in (0, 1), exact in float32
    G       = -ln(-ln u)                       a standard Gumbel variate

Stage 0 keys probe (cluster) sampling, stage 1 keys token sampling; the
speculative verification (spec_oracle) keys its acceptance uniform with
stage 2 and its residual draw with stage 3.
"""

from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter: np.ndarray, key) -> np.ndarray:
    """Apply Philox4x32 with 10 rounds.

    ``counter``: uint32 array of shape (..., 4).  ``key``: two uint32 words
    (broadcast over all counters) or an array of shape (..., 2).
    Returns uint32 array of shape (..., 4).
    """
    ctr = np.asarray(counter, dtype=np.uint32).astype(np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    k0 = k[..., 0] & _MASK32
    k1 = k[..., 1] & _MASK32
    x0, x1, x2, x3 = ctr[..., 0], ctr[..., 1], ctr[..., 2], ctr[..., 3]
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(_W0)) & _MASK32
            k1 = (k1 + np.uint64(_W1)) & _MASK32
        p0 = _M0 * x0  # < 2^64, exact in uint64
        p1 = _M1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    out = np.stack([x0, x1, x2, x3], axis=-1)
    return out.astype(np.uint32)


def philox_words(seed: int, row, index, stage: int) -> np.ndarray:
    """The 32-bit word that (seed, row, index, stage) maps to (see module doc)."""
    row = np.asarray(row, dtype=np.int64)
    index = np.asarray(index, dtype=np.int64)
    row, index = np.broadcast_arrays(row, index)
    shape = row.shape
    row, index = row.reshape(-1), index.reshape(-1)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
    out = np.empty(row.shape, dtype=np.uint32)
    step = 1 << 20  # bound the temporaries on large inputs
    for lo in range(0, row.size, step):
        r, i = row[lo:lo + step], index[lo:lo + step]
        ctr = np.zeros(r.shape + (4,), dtype=np.uint32)
        ctr[:, 0] = i // 4
        ctr[:, 1] = r
        ctr[:, 2] = stage
        words = philox4x32_10(ctr, key)
        out[lo:lo + step] = words[np.arange(r.size), i % 4]
    return out.reshape(shape)


def uniform_from_word(word: np.ndarray) -> np.ndarray:
    """Map a 32-bit word to u = ((w >> 9) + 1/2) / 2^23, in float64 (exact)."""
    w = np.asarray(word, dtype=np.uint32)
    return ((w >> np.uint32(9)).astype(np.float64) + 0.5) * (2.0 ** -23)


def gumbel(seed: int, row, index, stage: int) -> np.ndarray:
    """Standard Gumbel noise G = -ln(-ln u) in float64 for (seed, row, index, stage)."""
    u = uniform_from_word(philox_words(seed, row, index, stage))
    return -np.log(-np.log(u))
