"""Dense DSA-indexer scores and exact Top-K in float64 (test infrastructure).

The plain definition, written out (DoSA pages: podcast transcript, Method
section, problem formulation -- a query carries several indexer heads, each
with its own query vector and weight, all heads share one key per token, and
the task is the K keys of highest score; the DSA indexer's score is the
weighted sum over heads of ReLU(q_h . k)):

    S(t, s) = sum_h w[t, h] * max(0, sum_i q[t, h, i] * k[s, i])

Causality: query i of sequence b sits at position kv_len - q_len + i and sees
keys 0..position (a chunk of new queries at the end of the context).
Selection: full sort by (S descending, key index ascending); the first
min(K, visible) keys, padded with -1.  Lower index wins a tie.
"""
from __future__ import annotations

import numpy as np

from .formats import decode


# ----------------------------------------------------------------------------
# inputs -> float64
# ----------------------------------------------------------------------------
def query_rows(wl, rows) -> np.ndarray:
    """Decoded queries [len(rows), H, d] float64."""
    rows = np.asarray(rows, dtype=np.int64)
    qs = None if wl.q_scale is None else wl.q_scale[rows]
    return decode(wl.q[rows], wl.q_dtype, qs, token_axes=1)


def weights(wl, rows) -> np.ndarray:
    return np.asarray(wl.w[np.asarray(rows, dtype=np.int64)], dtype=np.float32).astype(np.float64)


def seq_keys(wl, b: int, upto: int | None = None) -> np.ndarray:
    """Decoded logical keys 0..upto-1 of sequence b, [n, d] float64.

    Contiguous storage packs the sequences back to back; paged storage maps
    logical key j of sequence b to pool page page_table[b, j // P], slot j % P.
    """
    n = int(wl.kv_lens[b]) if upto is None else int(upto)
    if wl.page_table is None:
        base = int(np.sum(wl.kv_lens[:b], dtype=np.int64))
        raw = wl.k[base: base + n]
        sc = None if wl.k_scale is None else wl.k_scale[base: base + n]
        return decode(raw, wl.k_dtype, sc, token_axes=1)
    P = wl.page_size
    j = np.arange(n, dtype=np.int64)
    pg = wl.page_table[b, j // P].astype(np.int64)
    sl = j % P
    raw = wl.k[pg, sl]
    sc = None if wl.k_scale is None else wl.k_scale[pg, sl]
    return decode(raw, wl.k_dtype, sc, token_axes=1)


def query_positions(wl):
    """(sequence, position) of every query row."""
    seq = np.repeat(np.arange(wl.batch), wl.q_lens)
    cu = np.concatenate([[0], np.cumsum(wl.q_lens)])
    i = np.arange(wl.total_q) - cu[seq]
    pos = wl.kv_lens[seq].astype(np.int64) - wl.q_lens[seq].astype(np.int64) + i
    return seq.astype(np.int64), pos.astype(np.int64)


# ----------------------------------------------------------------------------
# the definition
# ----------------------------------------------------------------------------
def head_dots(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """x[.., h, s] = q[.., h, :] . k[s, :]  (float64 matmul)."""
    return q @ k.T


def scores(q: np.ndarray, w: np.ndarray, k: np.ndarray) -> np.ndarray:
    """S[.., s] = sum_h w[.., h] * max(0, q[.., h, :] . k[s, :]) in float64.

    q [..., H, d], w [..., H], k [n, d] -> [..., n].
    """
    x = head_dots(q, k)
    np.maximum(x, 0.0, out=x)
    return np.einsum("...h,...hs->...s", w, x)


def abs_mass(q: np.ndarray, w: np.ndarray, k: np.ndarray) -> np.ndarray:
    """A[.., s] = sum_h |w_h| * |q_h . k_s|: the scale against which cancellation is judged."""
    x = np.abs(head_dots(q, k))
    return np.einsum("...h,...hs->...s", np.abs(w), x)


def select_topk(S: np.ndarray, K: int):
    """Exact Top-K of one query's visible scores S[0..n-1].

    Full sort by (score descending, index ascending); returns (idx int64 [K],
    score float64 [K]) padded with -1 / -inf when n < K.
    """
    n = S.shape[0]
    order = np.lexsort((np.arange(n), -S))
    take = order[: min(K, n)]
    idx = np.full(K, -1, dtype=np.int64)
    sc = np.full(K, -np.inf, dtype=np.float64)
    idx[: take.size] = take
    sc[: take.size] = S[take]
    return idx, sc


def _block_rows(n_keys: int, H: int, budget: int = 1 << 24) -> int:
    return max(1, budget // max(1, n_keys * H))


def topk_rows(wl, rows=None, return_scores: bool = True):
    """Oracle Top-K for the given query rows (all rows by default).

    Returns idx [R, K] int64 (-1 padded), score [R, K] float64 (-inf padded),
    and the K-th score theta [R] (the smallest selected score; -inf if fewer
    than K keys are visible).
    """
    seq, pos = query_positions(wl)
    rows = np.arange(wl.total_q) if rows is None else np.asarray(rows, dtype=np.int64)
    K = wl.topk
    out_i = np.full((rows.size, K), -1, dtype=np.int64)
    out_s = np.full((rows.size, K), -np.inf, dtype=np.float64)
    theta = np.full(rows.size, -np.inf, dtype=np.float64)
    # group rows by sequence so each sequence's keys are decoded once
    for b in np.unique(seq[rows]):
        sel = np.nonzero(seq[rows] == b)[0]
        maxpos = int(pos[rows[sel]].max())
        kb = seq_keys(wl, int(b), maxpos + 1)
        step = _block_rows(maxpos + 1, wl.H)
        for a in range(0, sel.size, step):
            part = sel[a: a + step]
            r = rows[part]
            S = scores(query_rows(wl, r), weights(wl, r), kb)
            for j, rr in enumerate(part):
                p = int(pos[rows[rr]])
                i, s = select_topk(S[j, : p + 1], K)
                out_i[rr] = i
                out_s[rr] = s
                if p + 1 >= K:
                    theta[rr] = s[K - 1]
    return (out_i, out_s, theta) if return_scores else out_i


def score_pairs(wl, rows, keys):
    """S and A for explicit (row, key) pairs, float64.  rows/keys: same-length arrays."""
    seq, pos = query_positions(wl)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    S = np.empty(rows.size)
    A = np.empty(rows.size)
    for b in np.unique(seq[rows]):
        sel = np.nonzero(seq[rows] == b)[0]
        kb = seq_keys(wl, int(b), int(keys[sel].max()) + 1)
        q = query_rows(wl, rows[sel])
        w = weights(wl, rows[sel])
        kk = kb[keys[sel]]
        x = np.einsum("nhd,nd->nh", q, kk)
        S[sel] = np.sum(w * np.maximum(x, 0.0), axis=1)
        A[sel] = np.sum(np.abs(w) * np.abs(x), axis=1)
    return S, A
