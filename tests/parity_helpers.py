"""Comparison of GPU results with the oracle, and of the two GPU paths with each other.

Readings applied (the pages give the exact-selection claim and a 1e-3
relative score tolerance with fp32 accumulation; ties go to the lower index):
* a returned score passes if |S_gpu - S_ref| <= 1e-3 * max(|S_ref|, A), where
  A = sum_h |w_h| |q_h . k| is the scale of the terms that cancel in S;
* the GPU's set may differ from the oracle's only by keys whose oracle score
  lies within that tolerance of the oracle's K-th score (boundary ties);
* the pruned path must return exactly the dense path's keys with bit-identical scores.
"""
import numpy as np

from oracle import indexer

REL = 1e-3


def check_vs_oracle(wl, gidx, gsc, rows, rel=REL):
    """Returns (max relative score error vs A, number of boundary swaps)."""
    rows = np.asarray(rows, dtype=np.int64)
    o_idx, o_sc, theta = indexer.topk_rows(wl, rows)
    _, pos = indexer.query_positions(wl)
    K = wl.topk
    worst = 0.0
    swaps = 0
    for j, r in enumerate(rows):
        g = gidx[r]
        keep = g >= 0
        gv = g[keep]
        nvis = min(K, int(pos[r]) + 1)
        assert gv.size == nvis, (r, gv.size, nvis)
        assert np.all(g[:nvis] >= 0) and np.all(g[nvis:] == -1), f"row {r}: padding layout"
        assert np.unique(gv).size == gv.size, f"row {r}: duplicate keys"
        assert gv.min(initial=0) >= 0 and gv.max(initial=0) <= pos[r], f"row {r}: key out of range"
        S, A = indexer.score_pairs(wl, np.full(gv.size, r), gv)
        err = np.abs(gsc[r][keep].astype(np.float64) - S)
        tol = rel * np.maximum(np.abs(S), A) + 1e-30
        assert np.all(err <= tol), f"row {r}: score error {np.max(err / tol) * rel}"
        worst = max(worst, float(np.max(err / np.maximum(A, 1e-30))) if err.size else 0.0)
        ov = o_idx[j][o_idx[j] >= 0]
        diff = np.array(sorted(set(gv.tolist()) ^ set(ov.tolist())), dtype=np.int64)
        if diff.size:
            Sd, Ad = indexer.score_pairs(wl, np.full(diff.size, r), diff)
            th = theta[j]
            ok = np.abs(Sd - th) <= rel * np.maximum(np.abs(th), Ad)
            assert np.all(ok), f"row {r}: set differs beyond boundary ties: {diff[~ok][:5]}"
            swaps += diff.size // 2
    return worst, swaps


def assert_same_selection(idx_a, sc_a, idx_b, sc_b):
    """Same key set per row, and bit-identical scores for each key."""
    assert idx_a.shape == idx_b.shape
    oa = np.argsort(idx_a, axis=1, kind="stable")
    ob = np.argsort(idx_b, axis=1, kind="stable")
    ia = np.take_along_axis(idx_a, oa, 1)
    ib = np.take_along_axis(idx_b, ob, 1)
    bad = np.nonzero(~np.all(ia == ib, axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"
    sa = np.take_along_axis(sc_a, oa, 1).view(np.uint32)
    sb = np.take_along_axis(sc_b, ob, 1).view(np.uint32)
    assert np.array_equal(sa, sb), "scores of the same keys differ"


def sample_rows(wl, n=24, seed=0):
    """Spread sample of query rows incl. the first and last of every sequence."""
    cu = wl.cu_q()
    picks = set()
    for b in range(wl.batch):
        if cu[b + 1] > cu[b]:
            picks.update([int(cu[b]), int(cu[b + 1] - 1)])
    rng = np.random.default_rng(seed)
    if wl.total_q:
        picks.update(rng.choice(wl.total_q, size=min(n, wl.total_q), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)
