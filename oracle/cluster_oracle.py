"""Balanced spherical k-means, the offline step that produces C and C2T, in
float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages describe (FlashHead explainer, framerc.cn, §1.2.1 "balanced
clustering" and §2.1 "offline clustering"; arXiv 2603.14591 abstract,
innovation (1)): the v embedding rows are L2-normalised; c centres are seeded
with k-means++; then, repeatedly, cosine similarities between every token
and every centre are computed, tokens are assigned to clusters so that every
cluster holds exactly b = v / c tokens (a greedy re-assignment), and every
centre becomes the normalised mean of its tokens.  C2T lists each cluster's
tokens.

Readings where the pages leave a step open (restated in the design notes):

- k-means++ on the sphere: the distance of a token to the chosen centres is
  D(t) = 1 - max_j cos(E_t, C_j); the first centre is token floor(u_0 v);
  centre i is the first token (in id order) whose running sum of D^2 exceeds
  u_i * sum(D^2) (inverse-CDF sampling with P(t) proportional to D(t)^2).
  The uniforms u_i are inputs.  If every D is 0, token floor(u_i v) is taken.
- balanced assignment, "greedy re-assignment": rounds.  In a round every
  unassigned token proposes to its most similar cluster among those that
  are not full (ties to the smaller cluster id); every cluster accepts, up
  to its remaining room, the proposals with the highest similarity (ties to
  the smaller token id); accepted tokens are final, the others propose again
  in the next round.  Every cluster ends with exactly b tokens.
- update: C_k = normalise(sum of its tokens' normalised rows), which is the
  normalised mean.
- C2T[k] holds cluster k's tokens in ascending id.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def normalize_rows(E) -> np.ndarray:
    """L2-normalised rows in float64 (explainer §2.1: spherical k-means works
    on unit vectors).  A zero row stays zero."""
    X = np.asarray(E, dtype=np.float64)
    n = np.sqrt((X * X).sum(axis=1, keepdims=True))
    return np.divide(X, n, out=np.zeros_like(X), where=n > 0)


def pp_pick(w: np.ndarray, u: float) -> int:
    """Inverse-CDF draw over token order with weights w (k-means++ step):
    the first t whose running sum exceeds u * sum(w)."""
    v = w.shape[0]
    total = float(w.sum())
    if total <= 0.0:
        return min(int(np.floor(u * v)), v - 1)
    run = np.cumsum(w)
    t = int(np.searchsorted(run, u * total, side="right"))
    return min(t, v - 1)


def kmeanspp(Xn: np.ndarray, c: int, u) -> np.ndarray:
    """k-means++ seeding on the sphere (explainer §2.1): returns the c
    chosen token ids.  Xn holds unit rows; u holds c uniforms in [0, 1)."""
    v = Xn.shape[0]
    u = np.asarray(u, dtype=np.float64)
    centers = np.empty(c, dtype=np.int64)
    centers[0] = min(int(np.floor(u[0] * v)), v - 1)
    D = 1.0 - Xn @ Xn[centers[0]]
    for i in range(1, c):
        centers[i] = pp_pick(D * D, u[i])
        D = np.minimum(D, 1.0 - Xn @ Xn[centers[i]])
    return centers


def pp_weights(Xn: np.ndarray, centers) -> np.ndarray:
    """D(t)^2 for the centres chosen so far (used to certify a draw)."""
    sims = Xn @ Xn[np.asarray(centers, dtype=np.int64)].T
    D = 1.0 - sims.max(axis=1)
    return D * D


def balanced_assign(sims, b: int, margins: list | None = None) -> np.ndarray:
    """Greedy balanced assignment by rounds (the reading above): returns the
    cluster of every token; every cluster gets exactly b tokens.  The
    decisions compare the given similarity values as they are.

    If ``margins`` is a list, the smallest similarity gap that decided
    anything is appended to it: per proposal, best minus second-best open
    cluster; per cluster with more proposals than room, last accepted minus
    first refused.  A caller that computes the similarities differently
    (another precision) can expect the same assignment only when this gap
    is well above the difference."""
    S = np.asarray(sims, dtype=np.float64)
    v, c = S.shape
    if v != b * c:
        raise ValueError("v must equal b * c")
    asg = np.full(v, -1, dtype=np.int64)
    fill = np.zeros(c, dtype=np.int64)
    gap = np.inf
    while True:
        todo = np.flatnonzero(asg < 0)
        if todo.size == 0:
            if margins is not None:
                margins.append(gap)
            return asg
        open_k = np.flatnonzero(fill < b)
        sub = S[np.ix_(todo, open_k)]
        best = sub.argmax(axis=1)  # first maximum: the smaller cluster id
        prop = open_k[best]
        val = sub[np.arange(todo.size), best]
        if margins is not None and open_k.size > 1:
            top2 = -np.partition(-sub, 1, axis=1)[:, :2]
            gap = min(gap, float((top2[:, 0] - top2[:, 1]).min()))
        for k in np.unique(prop):
            mine = prop == k
            toks, vals = todo[mine], val[mine]
            order = np.lexsort((toks, -vals))  # similarity desc, then token id asc
            room = b - fill[k]
            if margins is not None and toks.size > room:
                gap = min(gap, float(vals[order[room - 1]] - vals[order[room]]))
            take = toks[order[:room]]
            asg[take] = k
            fill[k] += take.size


def update_centroids(Xn: np.ndarray, asg, c: int):
    """Normalised sums of each cluster's rows, and C2T with each cluster's
    tokens in ascending id."""
    asg = np.asarray(asg, dtype=np.int64)
    d = Xn.shape[1]
    C = np.zeros((c, d), dtype=np.float64)
    np.add.at(C, asg, Xn)
    C = normalize_rows(C)
    order = np.lexsort((np.arange(asg.size), asg))
    b = asg.size // c
    return C, order.reshape(c, b).astype(np.int32)


@dataclass
class Clustering:
    C: np.ndarray          # [c x d] float64 unit rows
    c2t: np.ndarray        # [c x b] int32
    assign: np.ndarray     # [v] cluster of each token
    init_centers: np.ndarray  # [c] k-means++ token ids


def balanced_kmeans(E, c: int, iters: int, u) -> Clustering:
    """The whole procedure: normalise, seed with k-means++ (uniforms u), then
    `iters` rounds of cosine similarity, balanced assignment and update."""
    Xn = normalize_rows(E)
    centers = kmeanspp(Xn, c, u)
    C = Xn[centers].copy()
    asg = None
    c2t = None
    for _ in range(iters):
        asg = balanced_assign(Xn @ C.T, Xn.shape[0] // c)
        C, c2t = update_centroids(Xn, asg, c)
    if asg is None:
        asg = balanced_assign(Xn @ C.T, Xn.shape[0] // c)
        _, c2t = update_centroids(Xn, asg, c)
    return Clustering(C, c2t, asg, centers)


def adjusted_rand_index(a, b) -> float:
    """Adjusted Rand index of two labelings (Hubert and Arabie, 1985), from
    the contingency table."""
    a = np.asarray(a)
    b = np.asarray(b)
    _, ai = np.unique(a, return_inverse=True)
    _, bi = np.unique(b, return_inverse=True)
    n = a.size
    M = np.zeros((ai.max() + 1, bi.max() + 1), dtype=np.int64)
    np.add.at(M, (ai, bi), 1)
    comb = lambda x: x * (x - 1) / 2.0  # noqa: E731
    s_ij = comb(M).sum()
    s_a = comb(M.sum(axis=1)).sum()
    s_b = comb(M.sum(axis=0)).sum()
    expected = s_a * s_b / comb(n)
    top = 0.5 * (s_a + s_b)
    if top == expected:
        return 1.0
    return float((s_ij - expected) / (top - expected))


def intra_cluster_cosine(Xn: np.ndarray, c2t) -> np.ndarray:
    """Mean cosine of each cluster's tokens to their normalised mean (the
    pages' quality check, explainer §5.3: above 0.6)."""
    c2t = np.asarray(c2t)
    out = np.empty(c2t.shape[0])
    for k in range(c2t.shape[0]):
        rows = Xn[c2t[k]]
        m = rows.sum(axis=0)
        n = np.linalg.norm(m)
        out[k] = float((rows @ (m / n)).mean()) if n > 0 else 0.0
    return out
