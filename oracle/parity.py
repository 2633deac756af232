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

Defaults follow the stated targets: rel = 2e-3 (bfloat16 inputs, float32
accumulation) and tie_gap = 1e-3.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .flashhead_oracle import OracleHead, finish, gather, select

REL = 2e-3
TIE_GAP = 1e-3


@dataclass
class Report:
    queries: int = 0
    cluster_ties: int = 0  # queries whose probe set differed only at certified near-ties
    token_ties: int = 0
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


def check_forward(head: OracleHead, H, p, mode, temperature, seed, gpu: dict, queries=None,
                  rel=REL, tie_gap=TIE_GAP) -> Report:
    """Compare a GPU forward result (numpy arrays keyed like FlashHead.forward)
    with the oracle, on all queries or on the listed row indices."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    B = H.shape[0]
    rows = range(B) if queries is None else queries
    rep = Report()
    rows = list(rows)
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
        S_gpu = np.asarray(gpu["clusters"][r]) if "clusters" in gpu else S_ref
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
        if "ids" in gpu and not np.array_equal(np.asarray(gpu["ids"][r]), ids):
            rep.fail(f"row {r}: retrieved ids differ")
            continue
        if "logits" in gpu:
            tol = _logit_tol(head.E, ids, h, z, rel)
            err = np.abs(np.asarray(gpu["logits"][r], dtype=np.float64) - z) / tol
            rep.max_logit_err = max(rep.max_logit_err, float(err.max()))
            if err.max() > 1:
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
    if "token_logit" in gpu:
        tol = _logit_tol(E, np.array([y]), h, np.array([zi]), rel)[0]
        err = abs(float(gpu["token_logit"][r]) - zi) / tol
        rep.max_logit_err = max(rep.max_logit_err, err)
        if err > 1:
            rep.fail(f"row {r}: token logit error {err:.3g} x tol")
    if "lse" in gpu:
        err = abs(float(gpu["lse"][r]) - fin["lse"]) / (rel * max(1.0, abs(fin["lse"])))
        rep.max_lse_err = max(rep.max_lse_err, err)
        if err > 1:
            rep.fail(f"row {r}: lse error {err:.3g} x tol")


def check_dense(E, H, mode, temperature, seed, gpu: dict, queries=None, rel=REL,
                tie_gap=TIE_GAP) -> Report:
    """Compare a GPU dense-head result with the oracle's dense head."""
    H = np.atleast_2d(np.asarray(H, dtype=np.float64))
    B = H.shape[0]
    rows = list(range(B) if queries is None else queries)
    rep = Report()
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
            if err.max() > 1:
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
        if err.max() > 1:
            rep.fail(f"row {r}: score error {err.max():.3g} x tol")
    return rep
