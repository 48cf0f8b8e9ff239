"""The DoSA pruning certificate in float64 (test infrastructure).

Follows the DoSA pages (podcast transcript of "DOSA: Dots Sparse Attention",
Method section; the zicq.com summary, "Technical Mechanism Analysis" items
1-2; the picx.dev item, section 03):

1. Seed threshold.  Score a subset of the visible keys exactly; the K-th
   largest seed score tau lower-bounds the K-th largest score over all
   visible keys (a subset's K-th largest can never exceed the full set's).
2. Omitted positive heads.  A few positive-weight heads (proxies P) are
   evaluated exactly.  Every other positive-weight head h is projected onto
   the proxies with nonnegative coefficients that minimise the residual norm:
   q_h = sum_p alpha_hp q_p + r_h, alpha >= 0.  Since ReLU is subadditive and
   positively homogeneous, ReLU(q_h.k) <= sum_p alpha_hp ReLU(q_p.k) + ReLU(r_h.k),
   so the proxies absorb these heads with weights c_p = w_p + sum_h w_h alpha_hp.
3. Joint residual bound.  sum_h w_h ReLU(r_h.k) = (sum_{h active} w_h r_h).k
   <= rho * ||k|| with rho^2 = sum_{h,j} w_h w_j max(0, <r_h, r_j>), which
   covers every possible active subset at once (never larger than the
   separable sum_h w_h ||r_h||, also provided).
4. Negative heads.  For any subset A of the negative-weight heads,
   sum_{h in H-} |w_h| ReLU(x_h) >= ReLU(a.k) with a = sum_{h in A} |w_h| q_h.
   A is chosen from activation statistics: the negative heads that are
   positive on at least half of the seed keys.
5. Certificate: UB(t,s) = sum_p c_p ReLU(q_p.k_s) + rho ||k_s|| - ReLU(a.k_s)
   >= S(t,s).  A key with UB < tau cannot enter the Top-K (K seed keys score
   at least tau > S), whatever the tie rule, so it is pruned.
6. Key blocks: a block's centre, radius and largest norm give one bound that
   dominates UB for every key of the block (block_upper_bound).
7. Refinement within a call (two_round_pruned): the stages repeat over key
   ranges, newest first; exactly scored survivors of the first range join the
   seed scores, and their K-th largest (K distinct keys reach it, so it still
   lower-bounds the K-th score) is the threshold for the second range.

None of the choices (seed set, proxy count, rho variant, support) affects the
selected set as long as each bound is valid; they only change how much is
pruned.
"""
from __future__ import annotations

import itertools

import numpy as np

from . import indexer


def seed_keys(pos: int, K: int, prefix: int = 64, window: int | None = None) -> np.ndarray:
    """Seed set: the first ``prefix`` keys and the last ``window`` visible keys (window defaults to K)."""
    W = K if window is None else window
    n = pos + 1
    a = np.arange(min(prefix, n))
    b = np.arange(max(0, n - W), n)
    return np.union1d(a, b)


def seed_threshold(S_seed: np.ndarray, K: int) -> float:
    """K-th largest seed score, -inf when fewer than K seeds."""
    if S_seed.size < K:
        return -np.inf
    return float(np.sort(S_seed)[::-1][K - 1])


def nnls(Q: np.ndarray, v: np.ndarray) -> np.ndarray:
    """argmin_{alpha >= 0} ||v - Q alpha||_2 for a handful of columns.

    Exhaustive over supports: for each subset of columns solve the
    unconstrained least squares; among the feasible (nonnegative) solutions
    keep the one of least residual.  Exact for the small column counts used.
    """
    p = Q.shape[1]
    best = np.zeros(p)
    best_r = float(v @ v)
    for size in range(1, p + 1):
        for sub in itertools.combinations(range(p), size):
            Qs = Q[:, sub]
            sol, *_ = np.linalg.lstsq(Qs, v, rcond=None)
            if np.any(sol < 0):
                continue
            res = v - Qs @ sol
            r = float(res @ res)
            if r < best_r:
                best_r = r
                best = np.zeros(p)
                best[list(sub)] = sol
    return best


def plan(q: np.ndarray, w: np.ndarray, x_seed: np.ndarray | None, num_proxies: int = 3,
         support_frac: float = 0.5, rho_kind: str = "joint", use_negative: bool = True):
    """Per-query certificate constants.

    q [H, d], w [H] float64; x_seed [H, m] head dots on the seed keys (for
    the negative support).  Returns a dict with proxies P, coefficients c,
    alpha, residuals, rho, support A and aggregate a.
    """
    H = w.shape[0]
    pos_h = np.nonzero(w > 0)[0]
    neg_h = np.nonzero(w < 0)[0]
    qn = np.linalg.norm(q, axis=1)
    strength = w[pos_h] * qn[pos_h]
    order = pos_h[np.lexsort((pos_h, -strength))]
    P = np.sort(order[: min(num_proxies, order.size)])
    O = np.setdiff1d(pos_h, P)
    QP = q[P].T                                          # [d, p]
    alpha = np.zeros((O.size, P.size))
    R = np.zeros((O.size, q.shape[1]))
    for i, h in enumerate(O):
        al = nnls(QP, q[h]) if P.size else np.zeros(0)
        alpha[i] = al
        R[i] = q[h] - QP @ al if P.size else q[h]
    c = w[P] + (w[O] @ alpha if O.size else 0.0)
    if O.size == 0:
        rho = 0.0
    elif rho_kind == "joint":
        G = R @ R.T
        rho = float(np.sqrt(max(0.0, np.einsum("i,j,ij->", w[O], w[O], np.maximum(G, 0.0)))))
    elif rho_kind == "separable":
        rho = float(np.sum(w[O] * np.linalg.norm(R, axis=1)))
    else:
        raise ValueError(rho_kind)
    if use_negative and neg_h.size and x_seed is not None and x_seed.shape[1] > 0:
        active = np.mean(x_seed[neg_h] > 0, axis=1)
        A = neg_h[active >= support_frac]
    else:
        A = np.zeros(0, dtype=np.int64)
    a = (np.abs(w[A]) @ q[A]) if A.size else np.zeros(q.shape[1])
    return {"P": P, "O": O, "alpha": alpha, "R": R, "c": np.asarray(c, dtype=np.float64),
            "rho": rho, "A": A, "a": a, "qP": q[P]}


def upper_bound(pl, k: np.ndarray) -> np.ndarray:
    """UB[s] = sum_p c_p ReLU(q_p . k_s) + rho ||k_s|| - ReLU(a . k_s), float64."""
    kn = np.linalg.norm(k, axis=1)
    ub = pl["rho"] * kn
    if pl["P"].size:
        ub = ub + np.maximum(pl["qP"] @ k.T, 0.0).T @ pl["c"]
    ub = ub - np.maximum(k @ pl["a"], 0.0)
    return ub


def block_summaries(k: np.ndarray, block: int = 64):
    """Summaries of the blocks of ``block`` consecutive keys (the last one may be short).

    Any centre works for the block bound; this one is the mean of the block's keys.
    Returns (centre [n_blocks, d], radius [n_blocks] = max_s ||k_s - centre||,
    maxnorm [n_blocks] = max_s ||k_s||), float64.
    """
    n = k.shape[0]
    nb = (n + block - 1) // block
    centre = np.zeros((nb, k.shape[1]))
    radius = np.zeros(nb)
    maxnorm = np.zeros(nb)
    for b in range(nb):
        kb = k[b * block:(b + 1) * block]
        centre[b] = kb.mean(axis=0)
        radius[b] = np.linalg.norm(kb - centre[b], axis=1).max()
        maxnorm[b] = np.linalg.norm(kb, axis=1).max()
    return centre, radius, maxnorm


def block_upper_bound(pl, centre, radius, maxnorm):
    """One bound for every key of a block (DoSA pages: the transcript's Conclusion
    names certificates over key blocks instead of individual keys).

    For a key s of a block with centre c and radius r (||k_s - c|| <= r) and
    N >= ||k_s||:  q_p.k_s <= q_p.c + ||q_p|| r, and ReLU and c_p >= 0 keep the
    order, so the proxy term is at most sum_p c_p ReLU(q_p.c + ||q_p|| r); the
    residual term rho ||k_s|| is at most rho N; a.k_s >= a.c - ||a|| r, so the
    negative aggregate subtracts at least ReLU(a.c - ||a|| r).  Hence
        BUB = sum_p c_p ReLU(q_p.c + ||q_p|| r) + rho N - ReLU(a.c - ||a|| r)
    is at least UB(t, s) for every key of the block, and a block with BUB < tau
    holds no key the per-key certificate would keep.
    """
    centre = np.atleast_2d(centre)
    ub = pl["rho"] * np.asarray(maxnorm, dtype=np.float64)
    if pl["P"].size:
        qn = np.linalg.norm(pl["qP"], axis=1)
        ub = ub + np.maximum(centre @ pl["qP"].T + np.outer(radius, qn), 0.0) @ pl["c"]
    ub = ub - np.maximum(centre @ pl["a"] - np.linalg.norm(pl["a"]) * np.asarray(radius), 0.0)
    return ub


def query_certificate(q, w, k_vis, pos, K, num_proxies=3, prefix=64, window=None,
                      support_frac=0.5, rho_kind="joint", use_negative=True):
    """Everything the certificate says about one query.

    k_vis: the query's visible keys [pos+1, d].  Returns dict with S (exact
    scores), seed indices, tau, UB (all visible keys), pruned mask (non-seed
    keys with UB < tau) and the plan.
    """
    S = indexer.scores(q[None], w[None], k_vis)[0]
    seeds = seed_keys(pos, K, prefix, window)
    tau = seed_threshold(S[seeds], K)
    x_seed = q @ k_vis[seeds].T
    pl = plan(q, w, x_seed, num_proxies, support_frac, rho_kind, use_negative)
    UB = upper_bound(pl, k_vis)
    is_seed = np.zeros(S.size, dtype=bool)
    is_seed[seeds] = True
    pruned = (~is_seed) & (UB < tau)
    return {"S": S, "seeds": seeds, "tau": tau, "UB": UB, "pruned": pruned, "plan": pl}


def two_round_pruned(cert: dict, K: int, align: int = 64):
    """The bounded keys of one query's certificate in two rounds.

    cert: a query_certificate result.  Bounded keys are the non-seed visible
    keys, one contiguous range [lo, hi) for the seed set of seed_keys.  The
    range splits at lo + align * floor((hi - lo) / 2 / align): round 1 takes
    the newer keys [mid, hi) against tau and its survivors (UB >= tau) are
    scored exactly; tau2 = K-th largest of the seed scores and those scores;
    round 2 prunes the older keys [lo, mid) with UB < tau2.
    Returns (pruned mask over the visible keys, tau2, mid).
    """
    S, UB, tau = cert["S"], cert["UB"], cert["tau"]
    n = S.size
    is_seed = np.zeros(n, dtype=bool)
    is_seed[cert["seeds"]] = True
    bounded = np.nonzero(~is_seed)[0]
    pruned = np.zeros(n, dtype=bool)
    if bounded.size == 0:
        return pruned, tau, 0
    lo, hi = int(bounded[0]), int(bounded[-1]) + 1
    assert hi - lo == bounded.size, "bounded keys form one range"
    mid = lo + align * (((hi - lo) // 2) // align)
    r1 = np.arange(mid, hi)
    pruned[r1] = UB[r1] < tau
    surv1 = r1[~pruned[r1]]
    tau2 = seed_threshold(np.concatenate([S[cert["seeds"]], S[surv1]]), K)
    r2 = np.arange(lo, mid)
    pruned[r2] = UB[r2] < tau2
    return pruned, tau2, mid


def filter_rate(wl, rows, **kw):
    """Fraction of bounded (non-seed visible) pairs pruned, over the given query rows."""
    seq, pos = indexer.query_positions(wl)
    bounded = 0
    pruned = 0
    for r in np.asarray(rows, dtype=np.int64):
        b, p = int(seq[r]), int(pos[r])
        kv = indexer.seq_keys(wl, b, p + 1)
        q = indexer.query_rows(wl, [r])[0]
        w = indexer.weights(wl, [r])[0]
        cert = query_certificate(q, w, kv, p, wl.topk, **kw)
        nb = int(np.sum(~np.isin(np.arange(p + 1), cert["seeds"])))
        bounded += nb
        pruned += int(cert["pruned"].sum())
    return pruned / max(bounded, 1), bounded, pruned
