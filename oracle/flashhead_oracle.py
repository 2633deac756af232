"""FlashHead inference, stage by stage, in float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the method computes (FlashHead explainer, framerc.cn, §1.1, §1.2 and
§2.2.2; arXiv 2603.14591 abstract): a dense head scores every token,
z = E h.  FlashHead replaces this with a two-stage retrieval over a balanced
clustering of E's rows:

1. score h against the c centroids (optionally INT4-quantised, §1.2.4, or
   INT8-quantised, the W8A16 row of the tuning table, §5.2);
2. choose p probe clusters, by top-p score (§1.2.2) or by multinomial
   sampling with temperature (§1.2.3);
3. score only the b = v/c tokens of each chosen cluster, found through the
   dense cluster-to-token table C2T[c x b] (§1.2.1), in the embedding's own
   precision (§1.2.4);
4. finish with argmax or temperature sampling over the retrieved tokens.

Inside a stage nothing is approximated, so each stage is its plain
definition: float64 dot products over the exact stored values (bfloat16
widened exactly, or dequantised INT4 / INT8), a full lexicographic sort for
selection, and Gumbel-max for every draw.  Readings where the pages are
silent (the INT4 and INT8 schemes, tie-breaks, output order, sampling without
replacement, one temperature for both stages) are the ones listed under
"Readings" in the design notes and restated at each function.

Where a floating-point value decides an integer (a top-p cut, an argmax, an
INT4 or INT8 code), the decision is taken in float32, the precision the kernels
decide in; all other arithmetic is float64.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .philox import gumbel

# mode bits: probe stage (0 = top-p by score, 1 = sampled) | token stage
# (0 = argmax, 2 = sampled)
MODE_PROBE_SAMPLE = 1
MODE_TOKEN_SAMPLE = 2
MODE_PROBE_SHARED = 4


# ---------------------------------------------------------------------------
# Data structures (§1.2.1 balanced clustering; C2T is a dense c x b table)
# ---------------------------------------------------------------------------

def validate_c2t(c2t, v: int, c: int, b: int) -> np.ndarray:
    """Check C2T: c clusters of exactly b tokens covering [0, v) once each.

    Balanced clustering (explainer §1.2.1) gives every cluster exactly v/c
    tokens, stored as a dense [c x b] table; a token belongs to one cluster.
    Raises ValueError otherwise; returns C2T as int64 [c x b].
    """
    if c <= 0 or b <= 0 or c * b != v:
        raise ValueError(f"v={v} must equal c*b={c}*{b}")
    t = np.asarray(c2t)
    if t.shape != (c, b):
        raise ValueError(f"C2T shape {t.shape} != ({c}, {b})")
    flat = t.reshape(-1).astype(np.int64)
    if flat.min() < 0 or flat.max() >= v:
        raise ValueError("C2T holds a token id outside [0, v)")
    if np.bincount(flat, minlength=v).max() != 1:
        raise ValueError("C2T is not a permutation of [0, v)")
    return flat.reshape(c, b)


# ---------------------------------------------------------------------------
# Stage-1 quantisation (§1.2.4 selective quantisation; §2.3 quant config)
# ---------------------------------------------------------------------------

def _quantize_sym_g32(C: np.ndarray, qmax: int, name: str):
    """Symmetric integer codes with one fp16 scale per 32 consecutive row
    elements: for each centroid row k and group g (elements 32g..32g+31),
    sigma = fp16(amax / qmax) with the division in float32 and round-to-
    nearest-even to fp16; q = clamp(rint(x / sigma), -qmax, qmax) with
    float32 division and ties to even; q = 0 where sigma = 0.  Returns
    (q int8 [c x d], sigma float16 [c x d/32]).  Raises OverflowError if a
    scale is not a finite fp16 number and ValueError if d is not a multiple
    of 32."""
    C = np.asarray(C, dtype=np.float32)
    c, d = C.shape
    if d % 32 != 0:
        raise ValueError(f"{name} g32 needs d % 32 == 0")
    g = C.reshape(c, d // 32, 32)
    amax = np.abs(g).max(axis=2)
    with np.errstate(over="ignore"):
        sigma = (amax / np.float32(qmax)).astype(np.float16)
    if not np.all(np.isfinite(sigma)):
        raise OverflowError(f"a centroid group's {name} scale overflows fp16")
    s = sigma.astype(np.float32)[..., None]
    nz = s > 0
    q = np.rint(g / np.where(nz, s, np.float32(1.0)))
    q = np.where(nz, np.clip(q, -qmax, qmax), 0).astype(np.int8)
    return q.reshape(c, d), sigma


def quantize_int4_g32(C: np.ndarray):
    """INT4 stage-1 centroids (§1.2.4, §2.3 "centroid: int4"): the symmetric
    g32 scheme with qmax = 7."""
    return _quantize_sym_g32(C, 7, "INT4")


def quantize_int8_g32(C: np.ndarray):
    """INT8 stage-1 centroids, the W8A16 configuration of the tuning table
    (§5.2): the same symmetric g32 scheme with qmax = 127; queries stay in
    their 16-bit type."""
    return _quantize_sym_g32(C, 127, "INT8")


def dequantize_g32(q: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """C_hat = sigma * q in float64 (exact)."""
    c, d = q.shape
    return (sigma.astype(np.float64)[:, :, None]
            * q.reshape(c, d // 32, 32).astype(np.float64)).reshape(c, d)


dequantize_int4 = dequantize_g32
dequantize_int8 = dequantize_g32


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2m in the low nibble of byte m."""
    q = np.asarray(q, dtype=np.int8)
    lo = q[..., 0::2].astype(np.uint8) & np.uint8(0xF)
    hi = q[..., 1::2].astype(np.uint8) & np.uint8(0xF)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & np.uint8(0xF)).astype(np.int16)
    hi = (p >> np.uint8(4)).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------------------
# Stage 1: centroid scores (explainer §1.2.2, §1.2.4: c_logits = quantize(C) h)
# ---------------------------------------------------------------------------

def score(C_hat: np.ndarray, H: np.ndarray) -> np.ndarray:
    """s[b, k] = sum_i C_hat[k, i] * h[b, i] in float64 (a plain dot product)."""
    C_hat = np.asarray(C_hat, dtype=np.float64)
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    return H @ C_hat.T


# ---------------------------------------------------------------------------
# Probe selection (explainer §1.2.2 multi-probe; §1.2.3 multinomial probes)
# ---------------------------------------------------------------------------

@dataclass
class Selection:
    S: np.ndarray  # int64 [B x p], ascending cluster ids per row
    key: np.ndarray  # float64 [B x c] selection keys
    key32: np.ndarray  # float32 [B x c] the keys the decision is taken on
    theta: np.ndarray  # float32 [B] the p-th largest key32 per row


def probe_keys(s: np.ndarray, mode: int, temperature: float, seed: int,
               rows=None) -> np.ndarray:
    """Selection keys: the score itself, or score/T plus Gumbel noise.

    Drawing p distinct clusters one after another from softmax(s/T) without
    replacement is the same as taking the top p of s/T + G with independent
    standard Gumbel G (Gumbel-top-k: Yellott 1977; Kool, van Hoof and
    Welling 2019).  Noise for row b, cluster k is gumbel(seed, b, k, stage 0);
    ``rows`` gives the row indices b of s's rows (default 0..B-1).
    """
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    if not (mode & MODE_PROBE_SAMPLE):
        return s.copy()
    if not temperature > 0:
        raise ValueError("sampling needs temperature > 0")
    B, c = s.shape
    rows = np.arange(B) if rows is None else np.asarray(rows)
    g = gumbel(seed, rows[:, None], np.arange(c)[None, :], 0)
    return s / float(temperature) + g


def _top_ids(key32_row: np.ndarray, ids_row: np.ndarray, n: int) -> np.ndarray:
    """Positions of the n best entries: key descending, ties to the smaller id."""
    order = np.lexsort((ids_row, -key32_row.astype(np.float64)))
    return order[:n]


def select_shared(s: np.ndarray, p: int) -> Selection:
    """One probe set for the whole batch (explainer §4.2, server-side
    batching: share the cluster selection across the samples).  The pages
    give no rule; the reading here: the p clusters with the largest summed
    score sum_b s[b, k] (the top p for the batch's mean query), compared in
    float32, ties to the smaller id.  Every row gets the same set."""
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    B, c = s.shape
    if not 1 <= p <= c:
        raise ValueError(f"p={p} outside [1, c={c}]")
    key = s.sum(axis=0)
    key32 = key.astype(np.float32)
    top = _top_ids(key32, np.arange(c), p)
    S = np.tile(np.sort(top), (B, 1))
    return Selection(S, np.tile(key, (B, 1)), np.tile(key32, (B, 1)),
                     np.full(B, key32[top[-1]], dtype=np.float32))


def select(s: np.ndarray, p: int, mode: int = 0, temperature: float = 1.0,
           seed: int = 0, rows=None) -> Selection:
    """Pick p clusters per row: the p largest keys, returned in ascending id.

    Top-p here counts clusters (the pages' p probes), not nucleus mass.  Keys
    are compared in float32; equal keys go to the smaller cluster id.  With
    MODE_PROBE_SHARED the batch shares one set (select_shared).
    """
    if mode & MODE_PROBE_SHARED:
        if mode & MODE_PROBE_SAMPLE:
            raise ValueError("shared probes are chosen by score, not sampled")
        return select_shared(s, p)
    key = probe_keys(s, mode, temperature, seed, rows)
    B, c = key.shape
    if not 1 <= p <= c:
        raise ValueError(f"p={p} outside [1, c={c}]")
    key32 = key.astype(np.float32)
    ids = np.arange(c)
    S = np.empty((B, p), dtype=np.int64)
    theta = np.empty(B, dtype=np.float32)
    for r in range(B):
        top = _top_ids(key32[r], ids, p)
        theta[r] = key32[r, top[-1]]
        S[r] = np.sort(top)
    return Selection(S, key, key32, theta)


@dataclass
class AdaptiveSelection:
    S: np.ndarray  # int64 [B x p_max]: the n[b] probes of row b ascending, then -1
    n: np.ndarray  # int64 [B] probes per row
    order: np.ndarray  # int64 [B x c] every cluster by key32 descending, ties to the smaller id
    key: np.ndarray  # float64 [B x c] selection keys (as select)
    key32: np.ndarray  # float32 [B x c] the keys the order is taken on
    mass: np.ndarray  # float64 [B x c] softmax(s / T) mass of the first j+1 clusters of `order`


def select_adaptive(s: np.ndarray, p_max: int, tau: float, p_min: int = 1, mode: int = 0,
                    temperature: float = 1.0, seed: int = 0, rows=None) -> AdaptiveSelection:
    """Per-query probe count (explainer §1.2.2, dynamic adjustment: the number
    of probes follows the distribution of h; §4.2: fewer probes where the
    query is confident, e.g. for frequent tokens).

    The pages give no formula.  The reading here: the clusters are taken one
    after another in the order of the selection keys (the scores, or with
    MODE_PROBE_SAMPLE the Gumbel-perturbed keys, i.e. draws without
    replacement from softmax(s/T)), and a row stops at the first count n whose
    clusters together hold at least tau of the centroid distribution
    softmax(s/T) over all c clusters; n is then clamped to [p_min, p_max].
    A peaked distribution stops after few clusters, a flat one probes up to
    p_max.  The order is decided on float32 keys like select (ties to the
    smaller id); the mass is float64.
    """
    if mode & MODE_PROBE_SHARED:
        raise ValueError("the adaptive count is per query; shared probes are not adaptive")
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    B, c = s.shape
    if not 1 <= p_min <= p_max <= c:
        raise ValueError(f"need 1 <= p_min={p_min} <= p_max={p_max} <= c={c}")
    if not 0.0 < tau <= 1.0:
        raise ValueError(f"tau={tau} outside (0, 1]")
    if not temperature > 0:
        raise ValueError("the mass needs temperature > 0")
    key = probe_keys(s, mode, temperature, seed, rows)
    key32 = key.astype(np.float32)
    x = s / float(temperature)
    w = np.exp(x - x.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    ids = np.arange(c)
    order = np.empty((B, c), dtype=np.int64)
    mass = np.empty((B, c), dtype=np.float64)
    n = np.empty(B, dtype=np.int64)
    S = np.full((B, p_max), -1, dtype=np.int64)
    for r in range(B):
        order[r] = _top_ids(key32[r], ids, c)
        mass[r] = np.cumsum(w[r, order[r]])
        reach = np.nonzero(mass[r] >= tau)[0]
        n_raw = int(reach[0]) + 1 if reach.size else c
        n[r] = min(max(n_raw, p_min), p_max)
        S[r, :n[r]] = np.sort(order[r, :n[r]])
    return AdaptiveSelection(S, n, order, key, key32, mass)


# ---------------------------------------------------------------------------
# Stage 2: token scores of the probed clusters (explainer §1.2.4: E[top] h)
# ---------------------------------------------------------------------------

def gather(E: np.ndarray, c2t: np.ndarray, S: np.ndarray, H: np.ndarray):
    """Retrieved ids and logits per row.

    For row b, clusters k in S[b] (ascending) and slots j = 0..b-1 (that
    order): t = C2T[k, j], z = E[t] . h_b in float64.  Returns (ids int64
    [B x p*b], z float64 [B x p*b]).
    """
    c2t = np.asarray(c2t, dtype=np.int64)
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    S = np.atleast_2d(S)
    B = S.shape[0]
    ids = c2t[S].reshape(B, -1)
    z = np.empty(ids.shape, dtype=np.float64)
    for r in range(B):
        z[r] = np.asarray(E[ids[r]], dtype=np.float64) @ H[r]
    return ids, z


@dataclass
class Finish:
    token: np.ndarray  # int64 [B]
    token_logit: np.ndarray  # float64 [B] z of the chosen token
    lse: np.ndarray  # float64 [B] log sum exp(z / T') over the candidates
    key: np.ndarray  # float64 [B x n] the keys the choice maximised
    key32: np.ndarray  # float32 [B x n]


def finish(ids: np.ndarray, z: np.ndarray, mode: int = 0, temperature: float = 1.0,
           seed: int = 0, rows=None) -> Finish:
    """Argmax, or one draw from softmax(z/T), over each row's candidates.

    Sampling is Gumbel-max: argmax of z/T + gumbel(seed, b, t, stage 1),
    keyed by the token id t so that the draw does not depend on where t sits
    in the candidate list.  The choice is taken on float32 keys, ties to the
    smaller token id.  LSE = log sum_t exp(z_t / T') with T' = T when the
    token is sampled and 1 otherwise, computed with the max shifted out.
    ``rows`` gives the row indices b of the rows (default 0..B-1).
    """
    ids = np.atleast_2d(np.asarray(ids, dtype=np.int64))
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    B, n = z.shape
    sample = bool(mode & MODE_TOKEN_SAMPLE)
    if sample and not temperature > 0:
        raise ValueError("sampling needs temperature > 0")
    tp = float(temperature) if sample else 1.0
    if sample:
        rows = np.arange(B) if rows is None else np.asarray(rows)
        key = z / tp + gumbel(seed, rows[:, None], ids, 1)
    else:
        key = z.copy()
    key32 = key.astype(np.float32)
    token = np.empty(B, dtype=np.int64)
    token_logit = np.empty(B, dtype=np.float64)
    lse = np.empty(B, dtype=np.float64)
    for r in range(B):
        best = _top_ids(key32[r], ids[r], 1)[0]
        token[r] = ids[r, best]
        token_logit[r] = z[r, best]
        x = z[r] / tp
        m = x.max()
        lse[r] = m + np.log(np.exp(x - m).sum())
    return Finish(token, token_logit, lse, key, key32)


# ---------------------------------------------------------------------------
# fp8 probability format (explainer §2.3: the quantisation config gives the
# probability intermediate as fp8)
# ---------------------------------------------------------------------------

def e4m3_decode(code) -> np.ndarray:
    """Value of an fp8 E4M3 byte (OCP 8-bit floating point, E4M3: sign, four
    exponent bits with bias 7, three mantissa bits; exponent field 0 holds
    the subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


_E4M3_POS = e4m3_decode(np.arange(0x7F))  # codes 0 .. 126: the finite values >= 0, ascending


def e4m3_encode(x) -> np.ndarray:
    """Nearest fp8 E4M3 byte to each x >= 0, ties to the even code, values
    above the largest finite (448) saturating to it; NaN gives 0x7F.  Written
    as a search over the code table, not as bit manipulation."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0):
        raise ValueError("probabilities are non-negative")
    out = np.full(x.shape, 0x7F, dtype=np.uint8)
    ok = ~np.isnan(x)
    xv = np.minimum(x[ok], _E4M3_POS[-1])
    hi = np.searchsorted(_E4M3_POS, xv, side="left")  # first value >= x
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = xv - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - xv
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    out[ok] = pick.astype(np.uint8)
    return out


def probs_fp8(z, lse, temperature: float = 1.0):
    """fp8 probabilities of candidates, scaled per row.

    p = exp(z / T' - LSE) per row (LSE the row's log-sum-exp at the same T';
    a logit of -inf, an empty slot, gives 0).  The pages name fp8 for the
    probability intermediate but not its scaling; the reading here: a power of
    two per row, 2^k with k = 8 - e where p_max = f 2^e, f in [1/2, 1) (so the
    row's largest probability lands in [128, 256), below E4M3's largest finite
    448, and the scaling itself is exact), then byte = e4m3_encode(p 2^k).
    A row decodes as e4m3_decode(byte) 2^-k.  Returns (bytes uint8 [B x n],
    k int64 [B], p float64 [B x n]); a row with no mass gets k = 0."""
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    lse = np.asarray(lse, dtype=np.float64).reshape(-1, 1)
    if not temperature > 0:
        raise ValueError("temperature must be > 0")
    with np.errstate(under="ignore"):
        p = np.exp(z / float(temperature) - lse)
    pmax = p.max(axis=1)
    _, e = np.frexp(pmax)
    k = np.where(pmax > 0, 8 - e, 0).astype(np.int64)
    return e4m3_encode(np.ldexp(p, k[:, None])), k, p


# ---------------------------------------------------------------------------
# Whole paths
# ---------------------------------------------------------------------------

@dataclass
class ForwardResult:
    scores: np.ndarray  # float64 [B x c]
    sel: Selection
    ids: np.ndarray  # int64 [B x p*b]
    z: np.ndarray  # float64 [B x p*b]
    fin: Finish


class OracleHead:
    """The engine's state: E, C (or its INT4 / INT8 form) and C2T, validated once."""

    def __init__(self, E, C, c2t, quant: str = "none"):
        E = np.asarray(E)
        C = np.asarray(C, dtype=np.float32)
        self.v, self.d = E.shape
        self.c = C.shape[0]
        if self.v % self.c:
            raise ValueError("v must be a multiple of c")
        self.b = self.v // self.c
        self.c2t = validate_c2t(c2t, self.v, self.c, self.b)
        self.E = E
        self.quant = quant
        if quant == "none":
            self.q = self.sigma = None
            self.C_hat = C.astype(np.float64)
        elif quant == "int4":
            self.q, self.sigma = quantize_int4_g32(C)
            self.C_hat = dequantize_g32(self.q, self.sigma)
        elif quant == "int8":
            self.q, self.sigma = quantize_int8_g32(C)
            self.C_hat = dequantize_g32(self.q, self.sigma)
        else:
            raise ValueError(f"unknown quant {quant}")

    def forward(self, H, p: int, mode: int = 0, temperature: float = 1.0,
                seed: int = 0) -> ForwardResult:
        s = score(self.C_hat, H)
        sel = select(s, p, mode, temperature, seed)
        ids, z = gather(self.E, self.c2t, sel.S, H)
        fin = finish(ids, z, mode, temperature, seed)
        return ForwardResult(s, sel, ids, z, fin)

    def dense(self, H, mode: int = 0, temperature: float = 1.0, seed: int = 0) -> Finish:
        return dense(self.E, H, mode, temperature, seed)


def forward(E, C, c2t, H, p: int, mode: int = 0, temperature: float = 1.0,
            seed: int = 0, quant: str = "none") -> ForwardResult:
    """One FlashHead call on the CPU (see OracleHead.forward)."""
    return OracleHead(E, C, c2t, quant).forward(H, p, mode, temperature, seed)


def dense(E, H, mode: int = 0, temperature: float = 1.0, seed: int = 0) -> Finish:
    """The dense head z = E h over all v tokens, finished like FlashHead (§1.1)."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    z = H @ np.asarray(E, dtype=np.float64).T
    ids = np.broadcast_to(np.arange(z.shape[1]), z.shape)
    return finish(ids, z, mode, temperature, seed)
