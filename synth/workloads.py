"""Seeded input recipes for the DSA-indexer Top-K path.

Every recipe returns a :class:`Workload`: raw input buffers in the storage
formats the library consumes, plus sequence lengths and (for paged caches) a
page table.  Randomness comes from ``numpy.random.Generator(PCG64)`` streams
derived from ``SeedSequence([seed, recipe_id])``; blocks of tokens draw from
their own spawned child streams, so a block's values do not depend on how many
threads generate the others.

The recipes follow the workload descriptions of the DoSA pages (DSA-shaped
indexers: 64 heads, head dim 128, Top-K 2048, 128K..1M contexts, chunked
prefill) with the shapes and value structure stated for each recipe below.
Where the description is open, the reading taken is stated next to the code.

Nothing here scores, bounds or selects anything.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

FP8_MAX = 448.0  # largest finite OCP E4M3FN magnitude
_BLOCK = 4096    # tokens per generation block
_THREADS = 8


# ----------------------------------------------------------------------------
# storage-format encoders (generation side only; decoders live elsewhere)
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _fp8_bits(x: np.ndarray) -> np.ndarray:
    import torch

    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_MAX, FP8_MAX)
    t = torch.from_numpy(x)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_fp8_per_token(x: np.ndarray, token_axes: int = 1):
    """Per-token fp8 E4M3FN quantisation.

    ``x`` has ``token_axes`` leading token dimensions; one fp32 scale covers
    all remaining dimensions of a token (for queries: all heads and the head
    dimension).  scale = amax / 448 (1 for an all-zero token); stored code =
    RNE_e4m3(x / scale), saturating at +-448.
    """
    x = np.asarray(x, dtype=np.float32)
    red = tuple(range(token_axes, x.ndim))
    amax = np.abs(x).max(axis=red) if red else np.abs(x)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    bshape = scale.shape + (1,) * (x.ndim - token_axes)
    codes = _fp8_bits(x / scale.reshape(bshape))
    return codes, scale


def _encode(x: np.ndarray, dtype: str, token_axes: int = 1):
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32), None
    if dtype == "bf16":
        return to_bf16_bits(x), None
    if dtype == "fp8":
        return quantize_fp8_per_token(x, token_axes)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# the workload container
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    """Inputs of one indexer problem.

    q        [total_q, H, d]  storage of ``q_dtype`` (float32 | uint16 bf16 bits | uint8 fp8 bits)
    q_scale  [total_q] float32 or None (fp8 only)
    w        [total_q, H] float32
    k        contiguous [total_k, d] (sequence b's keys at rows cu_kv[b]..)
             or paged [num_pages, page_size, d]
    k_scale  [total_k] / [num_pages, page_size] float32 or None (fp8 only)
    q_lens, kv_lens  int32 [batch]; query i of sequence b sits at position
             kv_lens[b] - q_lens[b] + i and sees keys 0..position.
    page_table  int32 [batch, max_pages] or None (contiguous keys)
    """

    name: str
    H: int
    d: int
    topk: int
    q_dtype: str
    k_dtype: str
    q: np.ndarray
    q_scale: Optional[np.ndarray]
    w: np.ndarray
    k: np.ndarray
    k_scale: Optional[np.ndarray]
    q_lens: np.ndarray
    kv_lens: np.ndarray
    page_table: Optional[np.ndarray] = None
    page_size: int = 0
    chunk: int = 0          # >0: the workload is run as successive chunked-prefill calls
    recipe: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.q_lens))

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    def pairs(self) -> int:
        """Number of causal (query, visible key) pairs."""
        tot = 0
        for m, n in zip(self.q_lens.tolist(), self.kv_lens.tolist()):
            first = n - m + 1
            tot += m * first + m * (m - 1) // 2
        return int(tot)

    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int64)

    def cu_kv(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.kv_lens)]).astype(np.int64)

    def chunk_calls(self):
        """Split a single-sequence contiguous prefill into chunked calls.

        Yields dicts with q row range, q_len, kv_len: chunk c covers queries
        [c*chunk, (c+1)*chunk) and sees the first kv_len keys.
        """
        assert self.batch == 1 and self.page_table is None
        m = int(self.q_lens[0])
        n = int(self.kv_lens[0])
        step = self.chunk if self.chunk > 0 else m
        first_pos = n - m
        for q0 in range(0, m, step):
            ql = min(step, m - q0)
            yield {"q0": q0, "q_len": ql, "kv_len": first_pos + q0 + ql}


# ----------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------
def _streams(seed: int, recipe_id: int, n: int):
    ss = np.random.SeedSequence([int(seed), int(recipe_id)])
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(n)]


def _child_streams(rng: np.random.Generator, n: int):
    ss = np.random.SeedSequence(rng.integers(0, 2**63 - 1, size=4).tolist())
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(n)]


def _par_blocks(n: int, fn: Callable[[int, int, int], None], rngs_root, block: int = _BLOCK):
    nblk = (n + block - 1) // block
    rngs = _child_streams(rngs_root, max(nblk, 1))
    jobs = [(b * block, min(n, (b + 1) * block), rngs[b]) for b in range(nblk)]
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda j: fn(*j), jobs))


# ----------------------------------------------------------------------------
# value structure
# ----------------------------------------------------------------------------
RANK = 16
NOISE = 0.3
SINKS = 4
SINK_GAIN = 4.0
ANCHOR_WINDOW = 512
ANCHOR_COS = 0.5
NEG_FRAC = 0.3


def _low_rank_basis(rng, d):
    # U in R^{d x 16}, entries N(0, 1/16): ||U c|| ~ sqrt(d) for c ~ N(0, I_16)
    return (rng.standard_normal((d, RANK), dtype=np.float32) * np.float32(1.0 / math.sqrt(RANK)))


def _structured_keys(n, d, U, rng_root, sinks=True):
    """k_s = U c_s + eps_s, c_s ~ N(0, I_16), eps ~ N(0, 0.3^2 I); tokens 0..3 scaled by 4."""
    k = np.empty((n, d), dtype=np.float32)

    def blk(a, b, rng):
        c = rng.standard_normal((b - a, RANK), dtype=np.float32)
        e = rng.standard_normal((b - a, d), dtype=np.float32) * np.float32(NOISE)
        k[a:b] = c @ U.T + e

    _par_blocks(n, blk, rng_root)
    if sinks:
        k[: min(SINKS, n)] *= np.float32(SINK_GAIN)
    return k


def _iid(shape, rng_root, lead_block=_BLOCK):
    out = np.empty(shape, dtype=np.float32)
    n = shape[0]

    def blk(a, b, rng):
        out[a:b] = rng.standard_normal((b - a,) + tuple(shape[1:]), dtype=np.float32)

    _par_blocks(n, blk, rng_root, lead_block)
    return out


def _mixed_sign_weights(n, H, rng):
    """w = s*|g|, g ~ N(0,1), s = -1 with probability 0.3 (mixed-sign head weights)."""
    g = np.abs(rng.standard_normal((n, H), dtype=np.float32))
    s = np.where(rng.random((n, H)) < NEG_FRAC, np.float32(-1.0), np.float32(1.0))
    return (g * s).astype(np.float32)


def _anchored_queries(positions, H, d, keys, rng_root):
    """Queries correlated with the preceding keys.

    For each (t, h): an anchor j is drawn uniformly from the 512 positions
    before t (position 0 anchors to itself); q = sqrt(d)*(0.5*u + sqrt(0.75)*z)
    with u = k_j/||k_j|| and z a unit Gaussian direction orthogonal to u, so
    cos(q, k_j) = 0.5 and ||q|| = sqrt(d).
    """
    n = len(positions)
    q = np.empty((n, H, d), dtype=np.float32)
    sd = np.float32(math.sqrt(d))
    a_u = np.float32(ANCHOR_COS)
    a_z = np.float32(math.sqrt(1.0 - ANCHOR_COS**2))

    def blk(a, b, rng):
        t = positions[a:b].astype(np.int64)
        hi = np.maximum(t - 1, 0)
        lo = np.maximum(t - ANCHOR_WINDOW, 0)
        lo = np.minimum(lo, hi)
        j = rng.integers(lo[:, None], hi[:, None] + 1, size=(b - a, H))
        u = keys[j]                                          # [nb, H, d]
        u = u / np.linalg.norm(u, axis=-1, keepdims=True)
        z = rng.standard_normal((b - a, H, d), dtype=np.float32)
        z -= np.sum(z * u, axis=-1, keepdims=True) * u
        z /= np.linalg.norm(z, axis=-1, keepdims=True)
        q[a:b] = sd * (a_u * u + a_z * z)

    _par_blocks(n, blk, rng_root, 1024)
    return q


# ----------------------------------------------------------------------------
# recipes
# ----------------------------------------------------------------------------
def _contig(name, H, d, topk, qd, kd, q32, w, k32, q_lens, kv_lens, **kw):
    q, qs = _encode(q32, qd, 1)
    k, ks = _encode(k32, kd, 1)
    return Workload(name=name, H=H, d=d, topk=topk, q_dtype=qd, k_dtype=kd, q=q, q_scale=qs,
                    w=np.ascontiguousarray(w, dtype=np.float32), k=k, k_scale=ks,
                    q_lens=np.asarray(q_lens, np.int32), kv_lens=np.asarray(kv_lens, np.int32), **kw)


def tiny_prefill(seed: int = 0, L: int = 2048, H: int = 8, d: int = 64, topk: int = 256):
    """1 sequence, causal, fp32, q/k/w i.i.d. N(0,1) (mixed-sign w)."""
    r = _streams(seed, 1, 3)
    q = _iid((L, H, d), r[0])
    k = _iid((L, d), r[1])
    w = r[2].standard_normal((L, H), dtype=np.float32)
    return _contig("tiny_prefill", H, d, topk, "f32", "f32", q, w, k, [L], [L],
                   recipe="q,k,w iid N(0,1), fp32")


def _structured_prefill(name, recipe_id, seed, L, H, d, topk, qd, kd, chunk, q_len=None):
    r = _streams(seed, recipe_id, 4)
    U = _low_rank_basis(r[0], d)
    k32 = _structured_keys(L, d, U, r[1])
    m = L if q_len is None else q_len
    pos = np.arange(L - m, L, dtype=np.int64)
    w = _mixed_sign_weights(m, H, r[2])
    q32 = _anchored_queries(pos, H, d, k32, r[3])
    return _contig(name, H, d, topk, qd, kd, q32, w, k32, [m], [L], chunk=chunk,
                   recipe="rank-16 keys + N(0,0.3^2) noise, sinks 0..3 x4, queries cos 0.5 to an "
                          "anchor among the previous 512 keys, w 30% negative")


def dsa_prefill_32k(seed: int = 0, L: int = 32768, H: int = 64, d: int = 128, topk: int = 2048):
    """DSA-shaped prefill: 1 sequence of L tokens, bf16 q/k, fp32 w, structured values."""
    return _structured_prefill("dsa_prefill_32k", 2, seed, L, H, d, topk, "bf16", "bf16", 0)


def long_prefill_128k(seed: int = 0, L: int = 131072, H: int = 64, d: int = 128, topk: int = 2048,
                      chunk: int = 4096):
    """Long prefill: fp8 E4M3FN q/k with per-token scale, run in causal chunks of 4096 queries."""
    return _structured_prefill("long_prefill_128k", 3, seed, L, H, d, topk, "fp8", "fp8", chunk)


def million_chunk(seed: int = 0, L: int = 1048576, q_len: int = 8192, H: int = 64, d: int = 128,
                  topk: int = 2048, iid: bool = False):
    """~1M cached keys, one chunk of q_len new queries at the end; fp8 q/k.

    iid=True: the adversarial variant, q and k i.i.d. N(0,1), no sinks, mixed-sign w.
    """
    if not iid:
        return _structured_prefill("million_chunk", 5, seed, L, H, d, topk, "fp8", "fp8", 0, q_len=q_len)
    r = _streams(seed, 6, 3)
    k32 = _iid((L, d), r[0])
    q32 = _iid((q_len, H, d), r[1], 1024)
    w = _mixed_sign_weights(q_len, H, r[2])
    return _contig("million_chunk_iid", H, d, topk, "fp8", "fp8", q32, w, k32, [q_len], [L],
                   recipe="q,k iid N(0,1), no sinks, w 30% negative")


def decode_mtp(seed: int = 0, batch: int = 64, q_per_seq: int = 2, kv_min: int = 16384,
               kv_max: int = 262144, page_size: int = 64, H: int = 64, d: int = 128, topk: int = 2048,
               q_dtype: str = "bf16", k_dtype: str = "fp8"):
    """Batched decode with multi-token prediction over a paged key cache.

    kv_len ~ U[kv_min, kv_max] per sequence; each sequence's keys are drawn
    with the structured recipe (one low-rank basis shared by all sequences);
    the q_per_seq queries sit at the last positions.  Keys live in one global
    pool of pages whose order is a random permutation; page_table[b, i] is the
    pool page of sequence b's i-th page (-1 past the end).  Pool slots past a
    sequence's length hold large junk values so that any read beyond kv_len
    shows up in the result.
    """
    r = _streams(seed, 4, 6)
    U = _low_rank_basis(r[0], d)
    kv = r[1].integers(kv_min, kv_max + 1, size=batch).astype(np.int32)
    npg = (kv + page_size - 1) // page_size
    total_pages = int(npg.sum())
    max_pages = int((kv_max + page_size - 1) // page_size)
    perm = r[2].permutation(total_pages).astype(np.int32)
    table = np.full((batch, max_pages), -1, dtype=np.int32)
    seq_rngs = _child_streams(r[3], batch)
    q_rngs = _child_streams(r[4], batch)
    k_pool32 = np.full((total_pages, page_size, d), 300.0, dtype=np.float32)
    q32 = np.empty((batch * q_per_seq, H, d), dtype=np.float32)
    off = 0
    for b in range(batch):
        n = int(kv[b])
        kb = _structured_keys(n, d, U, seq_rngs[b])
        pages = perm[off: off + npg[b]]
        table[b, : npg[b]] = pages
        padded = np.full((npg[b] * page_size, d), 300.0, dtype=np.float32)
        padded[:n] = kb
        k_pool32[pages] = padded.reshape(npg[b], page_size, d)
        pos = np.arange(n - q_per_seq, n, dtype=np.int64)
        q32[b * q_per_seq:(b + 1) * q_per_seq] = _anchored_queries(pos, H, d, kb, q_rngs[b])
        off += npg[b]
    w = _mixed_sign_weights(batch * q_per_seq, H, r[5])
    q, qs = _encode(q32, q_dtype, 1)
    k, ks = _encode(k_pool32, k_dtype, 2)
    return Workload(name="decode_mtp", H=H, d=d, topk=topk, q_dtype=q_dtype, k_dtype=k_dtype, q=q,
                    q_scale=qs, w=w, k=k, k_scale=ks,
                    q_lens=np.full(batch, q_per_seq, np.int32), kv_lens=kv,
                    page_table=table, page_size=page_size,
                    recipe="per-sequence structured keys, permuted page pool, queries at the last positions")


def _correlated_tokens(rngs, L, H, d, pos, corr, head_noise, topic_window):
    """Keys of L tokens and queries at positions ``pos`` with cross-head structure.

    Keys drift slowly through topics: k_s = mu + U c_s + eps_s, where the
    rank-16 coordinates follow c_s = corr c_{s-1} + sqrt(1-corr^2) xi_s
    (correlation length ~1/(1-corr) tokens), mu is a common offset with
    ||mu|| = 0.6 sqrt(d), eps ~ N(0, 0.3^2), sinks 0..3 x4.
    Queries: every head of token t points along the current topic (the mean
    of U c over the previous ``topic_window`` keys, scaled to norm sqrt(d))
    plus ``head_noise`` sqrt(d) of its own random direction, times a per-head
    gain in [0.5, inf); a negative-weight head instead points mostly along mu
    (0.8 sqrt(d)) with 0.3 of the topic, so it fires on nearly every key.
    ``rngs``: seven generators.  Returns (k32 [L, d], q32 [m, H, d], w [m, H]).
    """
    from scipy.signal import lfilter

    m = len(pos)
    U = _low_rank_basis(rngs[0], d)
    mu = rngs[1].standard_normal(d).astype(np.float32)
    mu *= np.float32(0.6 * math.sqrt(d)) / np.linalg.norm(mu)
    xi = rngs[2].standard_normal((L, RANK)).astype(np.float64)
    xi[1:] *= math.sqrt(1.0 - corr * corr)
    c = lfilter([1.0], [1.0, -corr], xi, axis=0).astype(np.float32)
    z = c @ U.T                                                 # [L, d] topic part
    k32 = mu + z + rngs[3].standard_normal((L, d)).astype(np.float32) * np.float32(0.3)
    k32[:SINKS] *= np.float32(4.0)
    w = _mixed_sign_weights(m, H, rngs[4])
    cs = np.concatenate([np.zeros((1, d), np.float64), np.cumsum(z, axis=0, dtype=np.float64)])
    lo = np.maximum(pos - topic_window, 0)
    hi = np.maximum(pos, 1)
    topic = ((cs[hi] - cs[lo]) / (hi - lo)[:, None]).astype(np.float32)
    topic *= np.float32(math.sqrt(d)) / np.maximum(np.linalg.norm(topic, axis=1, keepdims=True), 1e-6)
    n = _iid((m, H, d), rngs[5], 1024)
    n *= np.float32(head_noise * math.sqrt(d)) / np.maximum(np.linalg.norm(n, axis=-1, keepdims=True), 1e-6)
    gain = np.abs(rngs[6].standard_normal((m, H))).astype(np.float32) * np.float32(0.5) + np.float32(0.5)
    mu_hat = mu / np.linalg.norm(mu)
    neg = (w < 0)[..., None]
    q32 = np.where(neg, np.float32(0.8 * math.sqrt(d)) * mu_hat + np.float32(0.3) * topic[:, None, :],
                   topic[:, None, :]) + n
    q32 *= gain[..., None]
    return k32, q32.astype(np.float32), w


def correlated_heads(seed: int = 0, L: int = 32768, H: int = 64, d: int = 128, topk: int = 2048,
                     dtype: str = "bf16", corr: float = 0.9995, head_noise: float = 0.05,
                     topic_window: int = 64, q_len: Optional[int] = None, chunk: int = 0):
    """Supplementary recipe with cross-head structure (not one of the headline workloads).

    One sequence of L tokens, the last q_len (default all) as queries, q and k
    in ``dtype`` (fp8: per-token scales), generated by _correlated_tokens.
    Heads are close to one another and the negative heads are active on broad
    support: the indexer shape the certificate is designed for, and one where
    the recent-window seed holds most of the true Top-K.
    """
    m = L if q_len is None else q_len
    r = _streams(seed, 7, 8)
    pos = np.arange(L - m, L, dtype=np.int64)
    k32, q32, w = _correlated_tokens(r, L, H, d, pos, corr, head_noise, topic_window)
    return _contig("correlated_heads", H, d, topk, dtype, dtype, q32, w, k32, [m], [L],
                   chunk=chunk,
                   recipe=f"supplementary: AR({corr}) topic-drift keys + common offset; heads along the "
                          f"topic of the last {topic_window} keys + {head_noise} noise; negative heads "
                          f"along the offset")


def correlated_decode(seed: int = 0, batch: int = 8, q_per_seq: int = 2, kv_min: int = 4096,
                      kv_max: int = 20000, page_size: int = 64, H: int = 64, d: int = 128, topk: int = 2048,
                      q_dtype: str = "bf16", k_dtype: str = "fp8", corr: float = 0.9995,
                      head_noise: float = 0.05, topic_window: int = 64):
    """Supplementary decode batch with the cross-head structure of correlated_heads.

    Like decode_mtp (paged key cache, one randomly permuted page pool, junk
    past each sequence's end, the q_per_seq queries at the last positions),
    but every sequence's keys and queries come from _correlated_tokens with
    streams of its own, so the certificate can prune.
    """
    r = _streams(seed, 9, 4)
    kv = r[0].integers(kv_min, kv_max + 1, size=batch).astype(np.int32)
    npg = (kv + page_size - 1) // page_size
    total_pages = int(npg.sum())
    max_pages = int((int(kv.max()) + page_size - 1) // page_size)
    perm = r[1].permutation(total_pages).astype(np.int32)
    table = np.full((batch, max_pages), -1, dtype=np.int32)
    seq_roots = _child_streams(r[2], batch)
    k_pool32 = np.full((total_pages, page_size, d), 300.0, dtype=np.float32)
    q32 = np.empty((batch * q_per_seq, H, d), dtype=np.float32)
    w = np.empty((batch * q_per_seq, H), dtype=np.float32)
    off = 0
    for b in range(batch):
        n = int(kv[b])
        pos = np.arange(n - q_per_seq, n, dtype=np.int64)
        kb, qb, wb = _correlated_tokens(_child_streams(seq_roots[b], 7), n, H, d, pos, corr, head_noise,
                                        topic_window)
        pages = perm[off: off + npg[b]]
        table[b, : npg[b]] = pages
        padded = np.full((npg[b] * page_size, d), 300.0, dtype=np.float32)
        padded[:n] = kb
        k_pool32[pages] = padded.reshape(npg[b], page_size, d)
        q32[b * q_per_seq:(b + 1) * q_per_seq] = qb
        w[b * q_per_seq:(b + 1) * q_per_seq] = wb
        off += npg[b]
    q, qs = _encode(q32, q_dtype, 1)
    k, ks = _encode(k_pool32, k_dtype, 2)
    return Workload(name="correlated_decode", H=H, d=d, topk=topk, q_dtype=q_dtype, k_dtype=k_dtype, q=q,
                    q_scale=qs, w=w, k=k, k_scale=ks,
                    q_lens=np.full(batch, q_per_seq, np.int32), kv_lens=kv,
                    page_table=table, page_size=page_size,
                    recipe="supplementary: correlated-heads sequences in a permuted page pool, queries at "
                           "the last positions")


def split_decode_steps(wl: Workload, q_per_step: int):
    """Two consecutive decode steps of a paged decode batch.

    ``wl`` holds 2 * q_per_step queries at the last positions of each
    sequence.  Returns (prev, cur): prev has each sequence's first q_per_step
    queries and a KV cache q_per_step keys shorter (the step before), cur the
    last q_per_step queries over the whole cache.  Pure slicing: the same keys,
    page table and query rows.
    """
    m = 2 * q_per_step
    assert wl.page_table is not None and np.all(wl.q_lens == m)
    rows = np.arange(wl.total_q).reshape(wl.batch, m)
    first, last = rows[:, :q_per_step].ravel(), rows[:, q_per_step:].ravel()

    def take(r, kv, tag):
        return Workload(name=f"{wl.name}_{tag}", H=wl.H, d=wl.d, topk=wl.topk, q_dtype=wl.q_dtype,
                        k_dtype=wl.k_dtype, q=wl.q[r], q_scale=None if wl.q_scale is None else wl.q_scale[r],
                        w=wl.w[r], k=wl.k, k_scale=wl.k_scale, q_lens=np.full(wl.batch, q_per_step, np.int32),
                        kv_lens=kv.astype(np.int32), page_table=wl.page_table, page_size=wl.page_size,
                        recipe=wl.recipe + f" ({tag} decode step)")

    return take(first, wl.kv_lens - q_per_step, "prev"), take(last, wl.kv_lens, "cur")


def custom(seed: int, lens, H: int, d: int, topk: int, q_dtype: str = "f32", k_dtype: str = "f32",
           structured: bool = False, page_size: int = 0, name: str = "custom"):
    """Small batched inputs for edge-case tests.

    ``lens`` is a list of (q_len, kv_len).  structured=False draws i.i.d.
    N(0,1) q, k and mixed-sign N(0,1) w.  page_size>0 stores the keys in a
    randomly permuted page pool with a page table (junk past each end).
    """
    r = _streams(seed, 8, 5)
    q_lens = np.array([a for a, _ in lens], np.int32)
    kv_lens = np.array([b for _, b in lens], np.int32)
    assert np.all(q_lens <= kv_lens)
    U = _low_rank_basis(r[0], d)
    krng = _child_streams(r[1], len(lens))
    qrng = _child_streams(r[2], len(lens))
    ks, qs = [], []
    for i, (m, n) in enumerate(lens):
        if structured:
            kb = _structured_keys(n, d, U, krng[i]) if n else np.zeros((0, d), np.float32)
            qb = (_anchored_queries(np.arange(n - m, n), H, d, kb, qrng[i]) if m
                  else np.zeros((0, H, d), np.float32))
        else:
            kb = krng[i].standard_normal((n, d), dtype=np.float32)
            qb = qrng[i].standard_normal((m, H, d), dtype=np.float32)
        ks.append(kb)
        qs.append(qb)
    k32 = np.concatenate(ks) if ks else np.zeros((0, d), np.float32)
    q32 = np.concatenate(qs) if qs else np.zeros((0, H, d), np.float32)
    tq = int(q_lens.sum())
    w = (_mixed_sign_weights(tq, H, r[3]) if structured
         else r[3].standard_normal((tq, H), dtype=np.float32))
    if page_size <= 0:
        return _contig(name, H, d, topk, q_dtype, k_dtype, q32, w, k32, q_lens, kv_lens,
                       recipe="custom")
    npg = (kv_lens + page_size - 1) // page_size
    total = int(npg.sum())
    max_pages = max(int(npg.max()) if len(npg) else 1, 1)
    perm = r[4].permutation(total).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, np.int32)
    pool = np.full((total, page_size, d), 300.0, np.float32)
    off = 0
    koff = 0
    for b in range(len(lens)):
        n = int(kv_lens[b])
        pages = perm[off: off + npg[b]]
        table[b, : npg[b]] = pages
        padded = np.full((npg[b] * page_size, d), 300.0, np.float32)
        padded[:n] = k32[koff: koff + n]
        pool[pages] = padded.reshape(npg[b], page_size, d)
        off += npg[b]
        koff += n
    q, qsc = _encode(q32, q_dtype, 1)
    k, ksc = _encode(pool, k_dtype, 2)
    return Workload(name=name, H=H, d=d, topk=topk, q_dtype=q_dtype, k_dtype=k_dtype, q=q,
                    q_scale=qsc, w=w, k=k, k_scale=ksc, q_lens=q_lens, kv_lens=kv_lens,
                    page_table=table, page_size=page_size, recipe="custom paged")


WORKLOADS = {
    "tiny_prefill": tiny_prefill,
    "dsa_prefill_32k": dsa_prefill_32k,
    "long_prefill_128k": long_prefill_128k,
    "decode_mtp": decode_mtp,
    "million_chunk": million_chunk,
    "million_chunk_iid": lambda seed=1, **kw: million_chunk(seed=seed, iid=True, **kw),
    "correlated_heads": correlated_heads,
    "correlated_decode": correlated_decode,
}


def make_workload(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)
