"""Speculative sampling with a FlashHead draft verified by the dense head, in
float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages (FlashHead explainer, framerc.cn, §4.2 "speculative decoding
integration") outline it in three steps: draw a draft token with FlashHead at
temperature T, compute the full probabilities with the original (dense) head,
and accept or reject the draft.  They do not give the rule.  The plain
reading is the standard speculative-sampling rule (Leviathan, Kalman,
Matias, "Fast inference from transformers via speculative decoding", ICML
2023; Chen et al., "Accelerating large language model decoding with
speculative sampling", 2023), applied to one position per row:

- target   p(t) = softmax(E h / T) over all v tokens;
- draft    q(t) = softmax(z / T) over the retrieved tokens of the draft's
           probes (z = E_t . h, the logits FlashHead scored), 0 elsewhere:
           the distribution the draft token was drawn from, given its probes;
- accept   the draft token x when u < min(1, p(x) / q(x)), with
           u = uniform(seed, row, 0, stage 2);
- else     draw from the residual r(t) = max(0, p(t) - q(t)) normalised:
           Gumbel-max of log r(t) + G(seed, row, t, stage 3) over the tokens
           with r(t) > 0.

The result is distributed exactly as p, for every probe set, hence also when
the probes themselves were sampled.  Decisions (the acceptance test and the
residual argmax) are taken in float32, as the kernels take them.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import gumbel, philox_words, uniform_from_word

STAGE_ACCEPT = 2
STAGE_RESIDUAL = 3


@dataclass
class SpecResult:
    token: np.ndarray       # int64 [B] the output token
    accepted: np.ndarray    # bool [B]
    lse: np.ndarray         # float64 [B] log sum_t exp(z_t / T) over all v
    ratio: np.ndarray       # float64 [B] min(1, p(x) / q(x))
    u: np.ndarray           # float64 [B] the acceptance uniform
    residual: np.ndarray    # int64 [B] the residual draw (-1 where r = 0)
    rkey32: list            # per row: float32 residual keys over all v (-inf off the support)


def _lse(x: np.ndarray) -> float:
    m = x.max()
    return float(m + np.log(np.exp(x - m).sum()))


def spec_verify(E, c2t, H, probes, draft_token, temperature: float, seed: int) -> SpecResult:
    """The rule above for each row b: hidden state H[b], the draft's probe
    clusters probes[b] and its token draft_token[b]."""
    if not temperature > 0:
        raise ValueError("speculative sampling needs temperature > 0")
    E = np.asarray(E, dtype=np.float64)
    c2t = np.asarray(c2t, dtype=np.int64)
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    probes = np.atleast_2d(np.asarray(probes, dtype=np.int64))
    draft_token = np.asarray(draft_token, dtype=np.int64)
    B = H.shape[0]
    v = E.shape[0]
    T = float(temperature)
    rows = np.arange(B)
    u = uniform_from_word(philox_words(seed, rows, np.zeros(B, dtype=np.int64), STAGE_ACCEPT))
    out = SpecResult(np.empty(B, np.int64), np.empty(B, bool), np.empty(B), np.empty(B),
                     np.asarray(u, dtype=np.float64), np.empty(B, np.int64), [])
    tok = np.arange(v)
    for r in range(B):
        z = E @ H[r] / T
        lse = _lse(z)
        p = np.exp(z - lse)
        ids = c2t[probes[r]].ravel()
        q = np.zeros(v)
        q[ids] = np.exp(z[ids] - _lse(z[ids]))
        x = int(draft_token[r])
        ratio = min(1.0, p[x] / q[x]) if q[x] > 0 else 1.0
        res = np.maximum(p - q, 0.0)
        key = np.full(v, -np.inf)
        live = res > 0
        key[live] = np.log(res[live]) + gumbel(seed, np.full(int(live.sum()), r), tok[live],
                                               STAGE_RESIDUAL)
        key32 = key.astype(np.float32)
        if live.any():
            best = key32.max()
            residual = int(np.flatnonzero(key32 == best)[0])  # ties: the smaller token id
        else:
            residual = -1
        acc = bool(np.float32(out.u[r]) < np.float32(ratio)) or residual < 0
        out.token[r] = x if acc else residual
        out.accepted[r] = acc
        out.lse[r] = lse
        out.ratio[r] = ratio
        out.residual[r] = residual
        out.rkey32.append(key32)
    return out
