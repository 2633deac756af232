"""Parity rule between a GPU result and the oracle — TEST INFRASTRUCTURE ONLY.

The rule (integer results exact, float results within a stated tolerance,
near-ties certified on the oracle's own keys):

* Clusters: the GPU's probe set must equal the oracle's, except that every
  cluster in the symmetric difference must have an oracle key within
  ``tie_gap`` of the oracle's p-th largest key.  Such a query is then checked
  from stage 2 on against the oracle run on the GPU's own probe set, so the
  later stages are still compared exactly.
* Retrieved ids: bit-exact (cluster ascending, slot order).
* Logits (retrieved, token, dense): |z_gpu - z_ref| <= rel * max(|z_ref|,
  2^-8 * ||E_t|| * ||h||).  The floor is one bfloat16 quantum of the
  Cauchy-Schwarz scale of the dot product, so that near-zero logits do not
  make a relative test meaningless.
* Token: equal ids, or a certified near-tie: the oracle's keys of the two ids
  differ by less than ``tie_gap``; the GPU's token must be a retrieved one.
* LSE: |lse_gpu - lse_ref| <= rel * max(1, |lse_ref|).

* Adaptive probe count: the GPU's count must be one that a cut within
  ``mass_gap`` of tau on the oracle's mass gives (check_adaptive).

Defaults follow the stated targets: rel = 2e-3 (bfloat16 inputs, float32
accumulation), tie_gap = 1e-3 and mass_gap = 1e-4.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .flashhead_oracle import (OracleHead, e4m3_decode, e4m3_encode, finish, gather, probs_fp8,
                               select, select_adaptive)

REL = 2e-3
TIE_GAP = 1e-3
# adaptive probe count: the GPU accumulates the softmax mass in float32 from
# float32 scores; a count is certified when the oracle's mass at the GPU's cut
# lies within MASS_GAP of tau
MASS_GAP = 1e-4
# fp8 probabilities: the GPU's exp runs in float32 (a few ulp); a byte may
# differ from the oracle's by one code when the probability lies within
# MID_GAP (relative) of the midpoint between the two codes
MID_GAP = 1e-5


@dataclass
class Report:
    queries: int = 0
    cluster_ties: int = 0  # queries whose probe set differed only at certified near-ties
    token_ties: int = 0
    count_ties: int = 0  # adaptive rows whose count differs at a certified mass near-tie
    max_logit_err: float = 0.0  # in units of the tolerance (<= 1 passes)
    max_lse_err: float = 0.0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def fail(self, msg):
        if len(self.failures) < 20:
            self.failures.append(msg)


def _logit_tol(E, ids, h, z_ref, rel):
    En = np.linalg.norm(np.asarray(E[ids], dtype=np.float64), axis=-1)
    floor = 2.0 ** -8 * En * np.linalg.norm(np.asarray(h, dtype=np.float64))
    return rel * np.maximum(np.abs(z_ref), floor)


FORWARD_KEYS = ("clusters", "ids", "logits", "token", "token_logit", "lse")
ADAPTIVE_KEYS = FORWARD_KEYS + ("nprobe",)
DENSE_KEYS = ("token", "token_logit", "lse")


def _missing(rep, gpu, keys):
    miss = [k for k in keys if k not in gpu]
    if miss:
        rep.fail(f"result lacks {', '.join(miss)}: nothing can be certified without them")
    return bool(miss)


def check_forward(head: OracleHead, H, p, mode, temperature, seed, gpu: dict, queries=None,
                  rel=REL, tie_gap=TIE_GAP) -> Report:
    """Compare a GPU forward result (numpy arrays keyed like FlashHead.forward)
    with the oracle, on all queries or on the listed row indices.  Every
    output is required: the probe set, the retrieved ids and logits, the
    token, its logit and the LSE (FORWARD_KEYS)."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    B = H.shape[0]
    rows = range(B) if queries is None else queries
    rep = Report()
    rows = list(rows)
    if _missing(rep, gpu, FORWARD_KEYS):
        return rep
    shared = bool(mode & 4)  # a shared probe set depends on every row of the batch
    s = (H if shared else H[rows]) @ head.C_hat.T  # float64 scores
    sel = select(s, p, mode, temperature, seed, rows=None if shared else rows)
    for pos, r in enumerate(rows):
        rep.queries += 1
        h = H[r]
        i = r if shared else pos
        keys_all = sel.key[i]
        S_ref = sel.S[i]
        theta = float(sel.theta[i])
        S_gpu = np.asarray(gpu["clusters"][r])
        if not np.array_equal(S_gpu, S_ref):
            if (len(S_gpu) != p or np.any(np.diff(S_gpu) <= 0) or S_gpu.min() < 0
                    or S_gpu.max() >= head.c):
                rep.fail(f"row {r}: GPU probe set is not {p} ascending valid ids")
                continue
            diff = np.setxor1d(S_gpu, S_ref)
            if np.all(np.abs(keys_all[diff] - theta) < tie_gap):
                rep.cluster_ties += 1
            else:
                rep.fail(f"row {r}: probe sets differ beyond near-ties at {diff[:8]}")
                continue
        # stage 2 and the finish, on the GPU's probe set
        ids, z = gather(head.E, head.c2t, S_gpu[None, :], h[None, :])
        ids, z = ids[0], z[0]
        fin = _finish_row(ids, z, mode, temperature, seed, r)
        if not np.array_equal(np.asarray(gpu["ids"][r]), ids):
            rep.fail(f"row {r}: retrieved ids differ")
            continue
        tol = _logit_tol(head.E, ids, h, z, rel)
        err = np.abs(np.asarray(gpu["logits"][r], dtype=np.float64) - z) / tol
        rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
        if not err.max() <= 1:  # a NaN logit fails too
            rep.fail(f"row {r}: retrieved logit error {err.max():.3g} x tol")
        _check_token(rep, head.E, ids, z, h, fin, gpu, r, rel, tie_gap)
    return rep


def _plausible_counts(mass, tau, p_min, p_max, gap):
    """Counts a float32 accumulation of the mass may stop at: the cut lands
    where the oracle's mass is within gap of tau, then the clamp."""
    lo = np.nonzero(mass >= tau - gap)[0]
    hi = np.nonzero(mass >= tau + gap)[0]
    n_lo = int(lo[0]) + 1 if lo.size else mass.size
    n_hi = int(hi[0]) + 1 if hi.size else mass.size
    return min(max(n_lo, p_min), p_max), min(max(n_hi, p_min), p_max)


def check_adaptive(head: OracleHead, H, p_max, p_min, tau, mode, temperature, seed, gpu: dict,
                   queries=None, rel=REL, tie_gap=TIE_GAP, mass_gap=MASS_GAP) -> Report:
    """Compare a GPU adaptive forward (FlashHead.forward_adaptive) with the
    oracle's select_adaptive.  Per row: the count n must lie in the range of
    counts the oracle's mass allows within mass_gap of tau; the first n
    entries of the probe row must be n ascending valid ids, equal to the
    oracle's first n clusters in key order up to certified key near-ties at
    the n-th key, and the rest -1; retrieved slots past n b hold id -1.  Stage
    2 and the finish are then checked on the GPU's probe set, as in
    check_forward.  Every output is required (ADAPTIVE_KEYS)."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    B = H.shape[0]
    rows = list(range(B) if queries is None else queries)
    rep = Report()
    if _missing(rep, gpu, ADAPTIVE_KEYS):
        return rep
    s = H[rows] @ head.C_hat.T
    a = select_adaptive(s, p_max, tau, p_min, mode, temperature, seed, rows=rows)
    b = head.b
    for pos, r in enumerate(rows):
        rep.queries += 1
        h = H[r]
        n = int(gpu["nprobe"][r])
        lo, hi = _plausible_counts(a.mass[pos], tau, p_min, p_max, mass_gap)
        if not lo <= n <= hi:
            rep.fail(f"row {r}: {n} probes, the oracle's mass allows {lo}..{hi}")
            continue
        if n != int(a.n[pos]):
            rep.count_ties += 1
        row = np.asarray(gpu["clusters"][r])
        S_gpu = row[:n]
        if (np.any(row[n:] != -1) or np.any(np.diff(S_gpu) <= 0) or S_gpu.min() < 0
                or S_gpu.max() >= head.c):
            rep.fail(f"row {r}: probe row is not {n} ascending valid ids followed by -1")
            continue
        S_ref = np.sort(a.order[pos, :n])
        if not np.array_equal(S_gpu, S_ref):
            theta = float(a.key32[pos, a.order[pos, n - 1]])
            diff = np.setxor1d(S_gpu, S_ref)
            if np.all(np.abs(a.key[pos, diff] - theta) < tie_gap):
                rep.cluster_ties += 1
            else:
                rep.fail(f"row {r}: probe sets differ beyond near-ties at {diff[:8]}")
                continue
        ids, z = gather(head.E, head.c2t, S_gpu[None, :], h[None, :])
        ids, z = ids[0], z[0]
        fin = _finish_row(ids, z, mode, temperature, seed, r)
        gid = np.asarray(gpu["ids"][r])
        if not np.array_equal(gid[:n * b], ids) or np.any(gid[n * b:] != -1):
            rep.fail(f"row {r}: retrieved ids differ")
            continue
        zg = np.asarray(gpu["logits"][r], dtype=np.float64)
        if not np.all(np.isneginf(zg[n * b:])):
            rep.fail(f"row {r}: retrieved logits past the {n} probes are not -inf")
            continue
        tol = _logit_tol(head.E, ids, h, z, rel)
        err = np.abs(zg[:n * b] - z) / tol
        rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
        if not err.max() <= 1:
            rep.fail(f"row {r}: retrieved logit error {err.max():.3g} x tol")
        _check_token(rep, head.E, ids, z, h, fin, gpu, r, rel, tie_gap)
    return rep


def _finish_row(ids, z, mode, temperature, seed, r):
    f = finish(ids[None, :], z[None, :], mode, temperature, seed, rows=[r])
    return {"token": int(f.token[0]), "token_logit": float(f.token_logit[0]),
            "lse": float(f.lse[0]), "key": f.key[0]}


def _check_token(rep, E, ids, z, h, fin, gpu, r, rel, tie_gap):
    y = int(gpu["token"][r])
    if y != fin["token"]:
        where = np.nonzero(ids == y)[0]
        if where.size != 1:
            rep.fail(f"row {r}: GPU token {y} is not a candidate")
            return
        k_ref = fin["key"][np.nonzero(ids == fin["token"])[0][0]]
        if abs(fin["key"][where[0]] - k_ref) < tie_gap:
            rep.token_ties += 1
        else:
            rep.fail(f"row {r}: token {y} != {fin['token']} beyond near-tie")
            return
    zi = float(z[np.nonzero(ids == y)[0][0]])
    tol = _logit_tol(E, np.array([y]), h, np.array([zi]), rel)[0]
    err = abs(float(gpu["token_logit"][r]) - zi) / tol
    rep.max_logit_err = max(rep.max_logit_err, err)
    if not err <= 1:
        rep.fail(f"row {r}: token logit error {err:.3g} x tol")
    err = abs(float(gpu["lse"][r]) - fin["lse"]) / (rel * max(1.0, abs(fin["lse"])))
    rep.max_lse_err = max(rep.max_lse_err, err)
    if not err <= 1:
        rep.fail(f"row {r}: lse error {err:.3g} x tol")


def check_dense(E, H, mode, temperature, seed, gpu: dict, queries=None, rel=REL,
                tie_gap=TIE_GAP) -> Report:
    """Compare a GPU dense-head result with the oracle's dense head.  The
    token, its logit and the LSE are required (DENSE_KEYS); the v logits are
    checked when the call asked for them."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    B = H.shape[0]
    rows = list(range(B) if queries is None else queries)
    rep = Report()
    if _missing(rep, gpu, DENSE_KEYS):
        return rep
    E64 = np.asarray(E, dtype=np.float64)
    v = E64.shape[0]
    ids = np.arange(v)
    for r in rows:
        rep.queries += 1
        h = H[r]
        z = E64 @ h
        fin = _finish_row(ids, z, mode, temperature, seed, r)
        if "logits" in gpu:
            tol = _logit_tol(E, ids, h, z, rel)
            err = np.abs(np.asarray(gpu["logits"][r], dtype=np.float64) - z) / tol
            rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
            if not err.max() <= 1:
                rep.fail(f"row {r}: dense logit error {err.max():.3g} x tol")
        _check_token(rep, E, ids, z, h, fin, gpu, r, rel, tie_gap)
    return rep


def check_scores(C_hat, H, s_gpu, rel=REL) -> Report:
    """Stage-1 scores within the logit tolerance (floor on ||C_k|| ||h||)."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    s = H @ np.asarray(C_hat, dtype=np.float64).T
    Cn = np.linalg.norm(C_hat, axis=1)
    rep = Report(queries=H.shape[0])
    for r in range(H.shape[0]):
        tol = rel * np.maximum(np.abs(s[r]), 2.0 ** -8 * Cn * np.linalg.norm(H[r]))
        err = np.abs(np.asarray(s_gpu[r], dtype=np.float64) - s[r]) / tol
        rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
        if not err.max() <= 1:
            rep.fail(f"row {r}: score error {err.max():.3g} x tol")
    return rep


def check_probs_fp8(z, lse, temperature, got, got_k, mid_gap=MID_GAP) -> Report:
    """fp8 E4M3 probabilities and their per-row scale exponents against the
    oracle's probs_fp8, taken on the same logits and LSE the GPU used (its
    own, already checked against the oracle), so that every byte is decided
    from the same inputs.  A row's exponent must equal the oracle's, or differ
    by one where the oracle's largest probability lies within mid_gap
    (relative) of the power of two between the two choices; bytes (at the
    GPU's exponent) must be equal, or adjacent codes with the scaled
    probability within mid_gap of their midpoint."""
    _, k_ref, p = probs_fp8(z, lse, temperature)
    got = np.asarray(got, dtype=np.uint8).reshape(p.shape)
    got_k = np.asarray(got_k, dtype=np.int64).reshape(-1)
    rep = Report(queries=p.shape[0])
    pmax = p.max(axis=1)
    for r in np.nonzero(got_k != k_ref)[0]:
        edge = 2.0 ** (7 - max(got_k[r], k_ref[r]) + 1)  # the binade boundary between the two
        if abs(int(got_k[r]) - int(k_ref[r])) != 1 or abs(pmax[r] - edge) > mid_gap * edge:
            rep.fail(f"row {r}: scale exponent {got_k[r]} != {k_ref[r]} (p_max = {pmax[r]:.8g})")
            return rep
        rep.cluster_ties += 1
    want = e4m3_encode(np.ldexp(p, got_k[:, None]))
    scaled = np.ldexp(p, got_k[:, None])
    bad = got != want
    if not bad.any():
        return rep
    g, w, pv = got[bad].astype(np.int64), want[bad].astype(np.int64), scaled[bad]
    adjacent = (np.abs(g - w) == 1) & (g < 0x7F) & (w < 0x7F)
    mid = (e4m3_decode(np.minimum(g, w)) + e4m3_decode(np.maximum(g, w))) / 2
    near = adjacent & (np.abs(pv - mid) <= mid_gap * np.maximum(mid, 2.0 ** -10))
    rep.token_ties = int(near.sum())
    if not near.all():
        rows, cols = np.nonzero(bad)
        i = int(np.nonzero(~near)[0][0])
        rep.fail(f"row {rows[i]} slot {cols[i]}: fp8 byte {g[i]:#04x} != {w[i]:#04x} "
                 f"(scaled p = {pv[i]:.6g}), not a midpoint near-tie; {int((~near).sum())} such bytes")
    return rep
