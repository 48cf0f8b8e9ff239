"""Checks that the seeded recipes have the stated shapes and value structure."""
import numpy as np

import synth
from oracle import formats, indexer


def test_tiny_shapes_and_determinism():
    a = synth.tiny_prefill()
    b = synth.tiny_prefill()
    assert a.q.shape == (2048, 8, 64) and a.k.shape == (2048, 64) and a.w.shape == (2048, 8)
    assert a.q.dtype == np.float32 and a.pairs() == 2048 * 2049 // 2
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.w, b.w)
    c = synth.tiny_prefill(seed=1)
    assert not np.array_equal(a.q, c.q)


def test_structured_recipe_properties():
    wl = synth.dsa_prefill_32k(L=2048)
    assert wl.q.dtype == np.uint16 and wl.k.dtype == np.uint16
    k = formats.decode(wl.k, "bf16")
    q = formats.decode(wl.q, "bf16")
    n = np.linalg.norm(k, axis=1)
    assert np.all(n[:4] > 3.0 * np.median(n[4:]))                        # sinks 4x norm
    assert abs(np.linalg.norm(q, axis=-1).mean() - np.sqrt(128)) < 0.1  # ||q|| = sqrt(d)
    # every query is cos ~0.5 with some key among the 512 before it
    for t in (5, 700, 2047):
        lo = max(0, t - 512)
        kk = k[lo: max(t, 1)]
        cos = (q[t] @ kk.T) / np.linalg.norm(q[t], axis=1)[:, None] / np.linalg.norm(kk, axis=1)[None]
        assert np.all(np.abs(cos.max(axis=1) - 0.5) < 0.02)
    w = wl.w
    assert 0.25 < np.mean(w < 0) < 0.35


def test_fp8_recipe_and_chunks():
    wl = synth.long_prefill_128k(L=8192, chunk=4096)
    assert wl.q.dtype == np.uint8 and wl.q_scale.shape == (8192,) and wl.k_scale.shape == (8192,)
    assert not np.any(np.isnan(formats.decode_fp8(wl.k)))
    calls = list(wl.chunk_calls())
    assert [(c["q0"], c["q_len"], c["kv_len"]) for c in calls] == [(0, 4096, 4096), (4096, 4096, 8192)]


def test_decode_recipe_page_table():
    wl = synth.decode_mtp(batch=4, kv_min=100, kv_max=700)
    P = wl.page_size
    used = wl.page_table[wl.page_table >= 0]
    assert used.size == len(set(used.tolist())) == wl.k.shape[0]        # a permutation of the pool
    for b in range(4):
        npg = (int(wl.kv_lens[b]) + P - 1) // P
        assert np.all(wl.page_table[b, :npg] >= 0) and np.all(wl.page_table[b, npg:] == -1)
    seq, pos = indexer.query_positions(wl)
    assert pos.tolist()[:2] == [int(wl.kv_lens[0]) - 2, int(wl.kv_lens[0]) - 1]


def test_iid_million_small():
    wl = synth.million_chunk(seed=1, L=4096, q_len=64, iid=True)
    assert wl.q.shape == (64, 64, 128) and wl.kv_lens.tolist() == [4096] and wl.q_lens.tolist() == [64]
