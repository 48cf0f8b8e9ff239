"""Extra seed keys (dosa_config::seed_idx): the previous decode step's Top-K, or
one candidate set per group of nearby queries, scored exactly and used only
for the seed threshold tau.  Whatever the seeds hold, the pruned path must
select exactly what the dense path selects; good seeds raise tau (never above
the true K-th score) and so cut the keys that survive the certificate."""
import numpy as np
import pytest

import synth
from parity_helpers import assert_same_selection, check_vs_oracle, sample_rows, score_tol

pytestmark = pytest.mark.gpu


def _call(wl, path, cfg=None, seeds=None, dumps=False):
    """One call; with dumps, also the per-key bounds and tau (debug arrays)."""
    import torch

    from exact_top_token_amd.runner import Runner, to_device

    print(f"[gpu] {wl.name} {path} q={wl.total_q} K={wl.topk} {wl.q_dtype}/{wl.k_dtype} "
          f"seeds={None if seeds is None else np.shape(seeds)} dumps={dumps}", flush=True)
    inp = to_device(wl)
    ub = tau = None
    if dumps:
        maxkv = int(max(wl.kv_lens))
        ub = torch.full((wl.total_q, maxkv), float("nan"), dtype=torch.float32, device="cuda")
        tau = torch.full((wl.total_q,), float("nan"), dtype=torch.float32, device="cuda")
        cfg.debug_ub = ub.data_ptr()
        cfg.debug_tau = tau.data_ptr()
    r = Runner(inp, path, cfg, seeds=seeds)
    idx, sc = r()
    torch.cuda.synchronize()
    if dumps:
        cfg.debug_ub = cfg.debug_tau = None
        ub, tau = ub.cpu().numpy(), tau.cpu().numpy()
    return idx.cpu().numpy(), sc.cpu().numpy(), r.stats_dict(), ub, tau


def _cfg(wl, no_probe=True):
    import exact_top_token_amd as E

    c = E.default_config(wl.topk)
    if no_probe:
        c.flags |= E.DOSA_NO_PROBE
    return c


def _check_tau(wl, rows, tau_plain, tau_seed, ub, seeds):
    """Per query: tau with seeds is at least tau without them and at least the K-th exact
    score over the query's own seed set (the keys without a bound plus its own listed keys
    that have one), and at most the true K-th score.  Returns the number of queries whose
    tau rose."""
    from oracle import certificate as cert
    from oracle import indexer

    seq, pos = indexer.query_positions(wl)
    _, _, theta = indexer.topk_rows(wl, rows)
    rose = 0
    for j, r in enumerate(rows):
        n = int(pos[r]) + 1
        kv = indexer.seq_keys(wl, int(seq[r]), n)
        q, w = indexer.query_rows(wl, [r]), indexer.weights(wl, [r])
        S = indexer.scores(q, w, kv)[0]
        A = indexer.abs_mass(q, w, kv)[0]
        tol = float(score_tol(max(abs(float(theta[j])), 1e-30) if np.isfinite(theta[j]) else 0.0, A.max()))
        tp, ts = float(tau_plain[r]), float(tau_seed[r])
        assert not np.isnan(ts), f"row {r}: tau not written"
        assert ts >= tp, f"row {r}: tau fell with seeds ({tp} -> {ts})"
        rose += int(ts > tp)
        if np.isfinite(theta[j]):
            assert ts <= theta[j] + tol, f"row {r}: tau {ts} above the true K-th score {theta[j]}"
        bounded = ~np.isnan(ub[r, :n])
        own = np.asarray(seeds[r])
        own = own[(own >= 0) & (own < n)]
        own = own[bounded[own]]
        keyset = np.union1d(np.nonzero(~bounded)[0], own)
        lo = cert.seed_threshold(S[keyset], wl.topk)
        if np.isfinite(lo):
            assert ts >= lo - tol, f"row {r}: tau {ts} below the K-th score of its own seeds {lo}"
    return rose


def test_decode_previous_step_topk():
    """Decode: the previous step's Top-K (the oracle's, for the queries two positions
    earlier over a cache two keys shorter) as each query's extra seeds."""
    from oracle import indexer

    base = synth.correlated_decode(seed=3, batch=8, q_per_seq=4, kv_min=6000, kv_max=20000)
    prev, cur = synth.split_decode_steps(base, 2)
    p_idx = indexer.topk_rows(prev, None, return_scores=False)
    seeds = p_idx.astype(np.int32)                                  # -1 padded rows
    di, ds, _, _, _ = _call(cur, "dsa")
    pi, ps, pst, ub0, tau0 = _call(cur, "dosa", _cfg(cur), dumps=True)
    si, ss, sst, ub1, tau1 = _call(cur, "dosa", _cfg(cur), seeds=seeds, dumps=True)
    assert_same_selection(pi, ps, di, ds)
    assert_same_selection(si, ss, di, ds)
    rows = np.arange(cur.total_q)
    check_vs_oracle(cur, si, ss, rows)
    rose = _check_tau(cur, rows, tau0, tau1, ub1, seeds)
    print(f"[seeds] decode: tau rose on {rose}/{rows.size} queries; survivors {pst['pairs_survived']} -> "
          f"{sst['pairs_survived']} of {sst['pairs_bounded']} bounded; seed pairs {pst['pairs_seed']} -> "
          f"{sst['pairs_seed']}", flush=True)
    assert rose > rows.size // 2
    assert sst["pairs_survived"] < pst["pairs_survived"]
    assert sst["pairs_bounded"] == pst["pairs_bounded"]


def test_group_candidate_sets_prefill():
    """Prefill with query tiles: every block of 16 consecutive queries shares the oracle
    Top-K of its first query as extra seeds (a candidate set per group of nearby queries)."""
    from oracle import indexer

    wl = synth.correlated_heads(seed=5, L=12288, q_len=2048, topk=256)
    blocks = np.arange(0, wl.total_q, 16)
    p_idx = indexer.topk_rows(wl, blocks, return_scores=False)
    seeds = np.repeat(p_idx.astype(np.int32), 16, axis=0)[: wl.total_q]
    cfg = _cfg(wl)
    cfg.seed_window = 512
    di, ds, _, _, _ = _call(wl, "dsa")
    pi, ps, pst, ub0, tau0 = _call(wl, "dosa", cfg, dumps=True)
    cfg = _cfg(wl)
    cfg.seed_window = 512
    si, ss, sst, ub1, tau1 = _call(wl, "dosa", cfg, seeds=seeds, dumps=True)
    assert_same_selection(pi, ps, di, ds)
    assert_same_selection(si, ss, di, ds)
    rows = sample_rows(wl, 48, seed=1)
    check_vs_oracle(wl, si, ss, rows)
    rose = _check_tau(wl, rows, tau0, tau1, ub1, seeds)
    print(f"[seeds] prefill: tau rose on {rose}/{rows.size} sampled queries; survivors "
          f"{pst['pairs_survived']} -> {sst['pairs_survived']} of {sst['pairs_bounded']} bounded", flush=True)
    assert rose > rows.size // 2
    assert sst["pairs_survived"] < pst["pairs_survived"]


@pytest.mark.parametrize("name", ["tiny_f32", "decode_bf16q_fp8k"])
def test_invalid_and_repeated_seeds(name):
    """Entries that are not bounded keys (negative, past the query, in the seed prefix or
    window, -1 padding) change nothing, bit for bit; repeats count once (the same tau as the
    list without them)."""
    rng = np.random.default_rng(7)
    if name == "tiny_f32":
        wl = synth.tiny_prefill(L=1024, topk=64)
    else:
        wl = synth.correlated_decode(seed=2, batch=4, q_per_seq=2, kv_min=3000, kv_max=6000, topk=128)
    from oracle import indexer

    _, pos = indexer.query_positions(wl)
    cfg0 = _cfg(wl)
    cfg0.seed_window = 256
    pi, ps, pst, _, tau0 = _call(wl, "dosa", cfg0, dumps=True)
    # invalid only: negative, past the query, far past the cache, prefix and window keys
    bad = np.stack([np.array([-7, -1, p + 1, p + 50, 10 ** 7, 0, 3, 63, p, max(p - 5, 0)], np.int32)
                    for p in pos])
    cfg1 = _cfg(wl)
    cfg1.seed_window = 256
    bi, bs, bst, _, tau1 = _call(wl, "dosa", cfg1, seeds=bad, dumps=True)
    assert_same_selection(bi, bs, pi, ps)
    assert np.array_equal(tau0.view(np.uint32), tau1.view(np.uint32)), "invalid seeds moved tau"
    assert bst["pairs_survived"] == pst["pairs_survived"]
    # valid keys, then the same keys repeated and shuffled with padding
    good = np.stack([rng.choice(np.arange(64, max(65, p - 300)), size=48, replace=True).astype(np.int32)
                     for p in pos])
    rep = np.concatenate([good, good[:, ::-1], np.full((good.shape[0], 8), -1, np.int32)], axis=1)
    rep = np.stack([rng.permutation(r) for r in rep])
    cfg2 = _cfg(wl)
    cfg2.seed_window = 256
    gi, gs, _, _, tau2 = _call(wl, "dosa", cfg2, seeds=good, dumps=True)
    cfg3 = _cfg(wl)
    cfg3.seed_window = 256
    ri, rs, _, _, tau3 = _call(wl, "dosa", cfg3, seeds=rep, dumps=True)
    assert_same_selection(gi, gs, pi, ps)
    assert_same_selection(ri, rs, pi, ps)
    assert np.array_equal(tau2.view(np.uint32), tau3.view(np.uint32)), "repeated seeds moved tau"
    assert np.all(tau2 >= tau0)


def test_seeds_with_the_probe_and_the_noalloc_entry_point():
    """Default flags (probe tile on) and the no-allocation entry point take the same seeds."""
    import torch

    import exact_top_token_amd as E
    from exact_top_token_amd.runner import to_device
    from oracle import indexer

    wl = synth.correlated_heads(seed=6, L=8192, q_len=1024, topk=128)
    blocks = np.arange(0, wl.total_q, 16)
    p_idx = indexer.topk_rows(wl, blocks, return_scores=False)
    seeds = np.repeat(p_idx.astype(np.int32), 16, axis=0)[: wl.total_q]
    di, ds, _, _, _ = _call(wl, "dsa")
    si, ss, _, _, _ = _call(wl, "dosa", _cfg(wl, no_probe=False), seeds=seeds)
    assert_same_selection(si, ss, di, ds)
    inp = to_device(wl)
    st = torch.from_numpy(seeds).cuda()
    cfg = E.default_config(wl.topk)
    cfg.seed_idx, cfg.seed_count = st.data_ptr(), int(st.shape[1])
    oi = torch.empty((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
    os_ = torch.empty((wl.total_q, wl.topk), dtype=torch.float32, device="cuda")
    print("[gpu] noalloc with seeds", flush=True)
    E.dosa_indexer_topk_noalloc(inp.q, inp.q_dtype, inp.q_scale, inp.w, inp.k, inp.k_dtype, inp.k_scale,
                                inp.q_lens, inp.kv_lens, None, 0, inp.H, inp.d, inp.topk, oi, os_, cfg=cfg)
    torch.cuda.synchronize()
    assert_same_selection(oi.cpu().numpy(), os_.cpu().numpy(), di, ds)
