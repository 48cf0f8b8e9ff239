"""GPU parity: both entry points against the oracle, and the pruned path
against the dense path (bit-identical selection), through the C-ABI."""
import sys

import numpy as np
import pytest

import synth
from parity_helpers import assert_same_selection, check_vs_oracle, sample_rows

pytestmark = pytest.mark.gpu


def _run(wl, path, **kw):
    from exact_top_token_amd.runner import run_once

    print(f"[gpu] {wl.name} {path} q={wl.total_q} H={wl.H} d={wl.d} K={wl.topk} {wl.q_dtype}/{wl.k_dtype} {kw}",
          flush=True)
    return run_once(wl, path, **kw)


def _both(wl, rows=None, cfg=None, **kw):
    di, ds, dst = _run(wl, "dsa", **kw)
    pi, ps, pst = _run(wl, "dosa", cfg=cfg, **kw)
    assert_same_selection(pi, ps, di, ds)
    if rows is not None:
        check_vs_oracle(wl, di, ds, rows)
    return (di, ds, dst), (pi, ps, pst)


def test_tiny_prefill_all_rows():
    import exact_top_token_amd as E

    wl = synth.tiny_prefill()
    cfg = E.default_config(wl.topk)
    cfg.flags |= E.DOSA_NO_PROBE
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=np.arange(wl.total_q), cfg=cfg)
    assert dst["pairs_total"] == wl.pairs() == dst["pairs_scored"]
    assert pst["pairs_seed"] + pst["pairs_bounded"] == wl.pairs()
    pi2, ps2, _ = _run(wl, "dosa")   # with the probe tile (default)
    assert_same_selection(pi2, ps2, di, ds)


def test_structured_bf16_4k():
    import exact_top_token_amd as E

    wl = synth.dsa_prefill_32k(L=4096)
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 40))
    # the certificate cannot prune this recipe: the probe tile sends the call to dense scoring
    assert pst["calls_unpruned"] == 1 and pst["pairs_bounded"] == 0 and pst["pairs_scored"] == wl.pairs()
    # without the probe the whole certificate pipeline runs, with the same result
    cfg = E.default_config(wl.topk)
    cfg.flags |= E.DOSA_NO_PROBE
    pi2, ps2, pst2 = _run(wl, "dosa", cfg=cfg)
    assert_same_selection(pi2, ps2, di, ds)
    assert pst2["calls_unpruned"] == 0 and pst2["pairs_seed"] + pst2["pairs_bounded"] == wl.pairs()


def test_fp8_chunked_prefill():
    import torch

    from exact_top_token_amd.runner import Runner, slice_chunk, to_device

    import exact_top_token_amd as E

    wl = synth.long_prefill_128k(L=8192, chunk=4096)
    inp = to_device(wl)
    outs = {}
    for path in ("dsa", "dosa", "dosa_no_probe"):
        idx = np.zeros((wl.total_q, wl.topk), np.int32)
        sc = np.zeros((wl.total_q, wl.topk), np.float32)
        cfg = E.default_config(wl.topk)
        if path == "dosa_no_probe":
            cfg.flags |= E.DOSA_NO_PROBE
        for c in wl.chunk_calls():
            print(f"[gpu] fp8 chunk {c} {path}", flush=True)
            r = Runner(slice_chunk(inp, c["q0"], c["q_len"], c["kv_len"]), path[:4], cfg)
            a, b = r()
            torch.cuda.synchronize()
            idx[c["q0"]:c["q0"] + c["q_len"]] = a.cpu().numpy()
            sc[c["q0"]:c["q0"] + c["q_len"]] = b.cpu().numpy()
        outs[path] = (idx, sc)
    assert_same_selection(*outs["dosa"], *outs["dsa"])
    assert_same_selection(*outs["dosa_no_probe"], *outs["dsa"])
    check_vs_oracle(wl, *outs["dsa"], sample_rows(wl, 24))


def test_decode_paged_bf16q_fp8k():
    wl = synth.decode_mtp(batch=6, kv_min=3000, kv_max=20000)
    _both(wl, rows=np.arange(wl.total_q))


@pytest.mark.parametrize("qd,kd", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "fp8"), ("bf16", "fp8")])
@pytest.mark.parametrize("page", [0, 16])
@pytest.mark.parametrize("K", [16, 300])
def test_edge_shapes(qd, kd, page, K):
    lens = [(1, 1), (3, 5), (0, 7), (17, 17), (5, 300), (2, 129), (33, 1000)]
    wl = synth.custom(3, lens, H=8, d=64, topk=K, q_dtype=qd, k_dtype=kd, page_size=page)
    _both(wl, rows=np.arange(wl.total_q))


def test_h64_d64_and_h32_d128():
    for H, d in ((64, 64), (32, 128), (16, 128)):
        wl = synth.custom(4, [(9, 700), (4, 4)], H=H, d=d, topk=64, q_dtype="bf16", k_dtype="bf16")
        _both(wl, rows=np.arange(wl.total_q))


def test_correlated_heads_prunes_and_matches():
    import exact_top_token_amd as E

    wl = synth.correlated_heads(L=8192)
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 2048
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 24), cfg=cfg)
    assert pst["pairs_bounded"] > 0 and pst["calls_unpruned"] == 0, "the probe tile should keep the pipeline"
    print("correlated stats", pst, flush=True)
    assert pst["pairs_survived"] < pst["pairs_bounded"], "certificate pruned nothing on the correlated recipe"


def test_survivor_shares_ragged_launch_order():
    """Union shares launched in the device-side order (longest first, a tile's shares on one XCD):
    a ragged tile count gives a share count that is not a multiple of the 32-item permutation
    runs, so the tail of the order is exercised too."""
    import exact_top_token_amd as E

    wl = synth.correlated_heads(L=5000, topk=256)
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 512
    cfg.flags |= E.DOSA_NO_PROBE
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 16), cfg=cfg)
    print("ragged shares stats", pst, flush=True)
    assert pst["pairs_bounded"] > 0 and pst["pairs_survived"] < pst["pairs_bounded"]


@pytest.mark.parametrize("knob", ["p0", "p1", "p2", "w64", "w512", "cap", "noprune", "separable", "noneg",
                                  "splits3", "frac0", "frac1", "probe", "blocks", "tworounds", "tworounds_probe",
                                  "grouplists"])
def test_knob_invariance(knob):
    import exact_top_token_amd as E
    from exact_top_token_amd.runner import run_once

    wl = synth.correlated_heads(L=3000, topk=128)
    di, ds, _ = run_once(wl, "dsa")
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 512
    cfg.flags |= E.DOSA_NO_PROBE     # every knob exercises the certificate pipeline itself
    ks = 0
    if knob == "probe":
        cfg.flags &= ~E.DOSA_NO_PROBE
    elif knob.startswith("p"):
        cfg.num_proxies = int(knob[1])
    elif knob == "w64":
        cfg.seed_window = 64
    elif knob == "w512":
        cfg.seed_window = 512
    elif knob == "cap":
        cfg.buffer_cap = wl.topk + 64
    elif knob == "noprune":
        cfg.flags |= E.DOSA_NO_PRUNE
    elif knob == "separable":
        cfg.flags |= E.DOSA_SEPARABLE_RHO
    elif knob == "noneg":
        cfg.flags |= E.DOSA_NO_NEGATIVE
    elif knob == "splits3":
        ks = 3
    elif knob == "frac0":
        cfg.neg_support_frac = 0.0
    elif knob == "frac1":
        cfg.neg_support_frac = 1.0
    elif knob == "blocks":
        cfg.flags |= E.DOSA_KEY_BLOCKS
    elif knob == "tworounds":
        cfg.flags |= E.DOSA_TWO_ROUNDS
    elif knob == "tworounds_probe":
        cfg.flags = (cfg.flags | E.DOSA_TWO_ROUNDS) & ~E.DOSA_NO_PROBE
    elif knob == "grouplists":
        cfg.flags |= E.DOSA_GROUP_LISTS | E.DOSA_TWO_ROUNDS
    print(f"[gpu] knob {knob}", flush=True)
    pi, ps, _ = run_once(wl, "dosa", cfg=cfg, key_splits=ks)
    assert_same_selection(pi, ps, di, ds)


def test_dense_small_buffer_and_splits():
    import torch

    from exact_top_token_amd.runner import Runner, to_device

    wl = synth.dsa_prefill_32k(L=3000, topk=256)
    base = _run(wl, "dsa")
    inp = to_device(wl)
    for ks in (1, 2, 5):
        # 3000 keys per query against a 2K+1024 buffer: every split re-selects in-kernel
        r = Runner(inp, "dsa", key_splits=ks)
        a, b = r()
        torch.cuda.synchronize()
        assert_same_selection(a.cpu().numpy(), b.cpu().numpy(), base[0], base[1])


def test_determinism_and_sorted_rows():
    import exact_top_token_amd as E

    wl = synth.dsa_prefill_32k(L=2500, topk=256)
    cfg = E.default_config(wl.topk)
    cfg.flags |= E.DOSA_NO_PROBE
    a = _run(wl, "dosa", cfg=cfg)
    b = _run(wl, "dosa", cfg=cfg)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    c = _run(wl, "dsa", sorted_rows=True)
    assert_same_selection(c[0], c[1], a[0], a[1])
    for r in range(wl.total_q):
        v = c[0][r] >= 0
        s, i = c[1][r][v], c[0][r][v]
        assert np.all((s[:-1] > s[1:]) | ((s[:-1] == s[1:]) & (i[:-1] < i[1:]))), r


def _debug_run(wl, cfg):
    """One pruned-path call with every debug dump attached; returns (idx, scores, stats, ub, tau, mask)."""
    import torch

    from exact_top_token_amd.runner import Runner, to_device

    inp = to_device(wl)
    maxkv = int(max(wl.kv_lens))
    dbg = torch.full((wl.total_q, maxkv), float("nan"), dtype=torch.float32, device="cuda")
    tau = torch.full((wl.total_q,), float("nan"), dtype=torch.float32, device="cuda")
    mask = torch.zeros((wl.total_q, (maxkv + 63) // 64), dtype=torch.int64, device="cuda")
    cfg.debug_ub = dbg.data_ptr()
    cfg.debug_tau = tau.data_ptr()
    cfg.debug_mask = mask.data_ptr()
    print(f"[gpu] debug dumps {wl.name} q={wl.total_q} {wl.q_dtype}/{wl.k_dtype}", flush=True)
    r = Runner(inp, "dosa", cfg)
    idx, sc = r()
    torch.cuda.synchronize()
    cfg.debug_ub = cfg.debug_tau = cfg.debug_mask = None
    return (idx.cpu().numpy(), sc.cpu().numpy(), r.stats_dict(), dbg.cpu().numpy(), tau.cpu().numpy(),
            mask.cpu().numpy().view(np.uint64))


def check_debug_dumps(wl, ub, tau, mask, rows):
    """The certificate as the GPU evaluated it, against the oracle, on the given rows:
    * every bound the GPU dumped dominates the oracle's exact score of that pair;
    * tau is the K-th largest oracle score over the query's seed keys (the visible keys
      that got no bound), within the score tolerance, hence a lower bound on the K-th score;
    * the survivor bits are exactly the bounded keys whose bound reached tau, or every
      bounded key (a query whose plan found nothing to prune);
    * no key of the oracle's Top-K (clear of boundary ties) was pruned.
    Returns the number of (query, key) bounds checked."""
    from oracle import certificate as cert
    from oracle import indexer
    from parity_helpers import score_tol

    seq, pos = indexer.query_positions(wl)
    o_idx, _, theta = indexer.topk_rows(wl, rows)
    n_checked = 0
    for j, r in enumerate(rows):
        n = int(pos[r]) + 1
        kv = indexer.seq_keys(wl, int(seq[r]), n)
        q = indexer.query_rows(wl, [r])
        w = indexer.weights(wl, [r])
        S = indexer.scores(q, w, kv)[0]
        A = indexer.abs_mass(q, w, kv)[0]
        bounded = ~np.isnan(ub[r, :n])
        keys = np.nonzero(bounded)[0]
        n_checked += keys.size
        assert np.all(ub[r, keys] >= S[keys] - 1e-6 * A[keys]), f"row {r}: bound below the exact score"
        seeds = np.nonzero(~bounded)[0]
        t_or = cert.seed_threshold(S[seeds], wl.topk)
        if np.isinf(t_or):
            assert np.isneginf(tau[r]), (r, tau[r])
        else:
            kth = seeds[np.argsort(-S[seeds], kind="stable")[wl.topk - 1]]
            assert abs(float(tau[r]) - t_or) <= score_tol(t_or, A[kth]), (r, tau[r], t_or)
            assert float(tau[r]) <= theta[j] + score_tol(theta[j], A[kth]), (r, tau[r], theta[j])
        bits = np.unpackbits(mask[r].view(np.uint8), bitorder="little")[:n].astype(bool)
        assert not np.any(bits & ~bounded), f"row {r}: survivor bit on a key without a bound"
        reach = bounded & (ub[r, :n] >= tau[r])
        assert np.array_equal(bits, reach) or np.array_equal(bits, bounded), f"row {r}: survivor bits"
        top = o_idx[j][o_idx[j] >= 0]
        if np.isneginf(theta[j]):
            clear = top                   # fewer than K visible keys: every one is selected
        else:
            clear = top[S[top] > theta[j] + score_tol(np.full(top.size, theta[j]), A[top])]
        assert np.all(~bounded[clear] | bits[clear]), f"row {r}: a Top-K key was pruned"
    return n_checked


@pytest.mark.parametrize("name", ["tiny", "correlated_bf16"])
def test_bound_dump_dominates_oracle_scores(name):
    import exact_top_token_amd as E

    wl = synth.tiny_prefill(L=1024, topk=64) if name == "tiny" else synth.correlated_heads(L=3000, topk=128)
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 256
    cfg.flags |= E.DOSA_NO_PROBE
    idx, sc, st, ub, tau, mask = _debug_run(wl, cfg)
    di, ds, _ = _run(wl, "dsa")
    assert_same_selection(idx, sc, di, ds)
    n = check_debug_dumps(wl, ub, tau, mask, sample_rows(wl, 16))
    assert n > 0, "no bound was dumped"


def test_correlated_fp8_chunked_prunes():
    """fp8 q and k with per-token scales (the headline operand type) on the correlated recipe:
    the certificate prunes, every chunk call matches the dense path bit for bit, and the
    fp8 certificate rows, aggregate terms and margin keep every bound above the exact score."""
    import torch

    import exact_top_token_amd as E
    from exact_top_token_amd.runner import Runner, slice_chunk, to_device

    wl = synth.correlated_heads(L=16384, dtype="fp8", chunk=4096)
    inp = to_device(wl)
    outs = {}
    stats = {}
    for path in ("dsa", "dosa"):
        idx = np.zeros((wl.total_q, wl.topk), np.int32)
        sc = np.zeros((wl.total_q, wl.topk), np.float32)
        cfg = E.default_config(wl.topk)
        cfg.flags |= E.DOSA_NO_PROBE
        cfg.seed_window = 2048
        tot = {}
        for c in wl.chunk_calls():
            print(f"[gpu] correlated fp8 chunk {c} {path}", flush=True)
            r = Runner(slice_chunk(inp, c["q0"], c["q_len"], c["kv_len"]), path, cfg)
            a, b = r()
            torch.cuda.synchronize()
            idx[c["q0"]:c["q0"] + c["q_len"]] = a.cpu().numpy()
            sc[c["q0"]:c["q0"] + c["q_len"]] = b.cpu().numpy()
            for k, v in r.stats_dict().items():
                tot[k] = tot.get(k, 0) + v
        outs[path] = (idx, sc)
        stats[path] = tot
    pst = stats["dosa"]
    print("correlated fp8 stats", pst, flush=True)
    print(f"[gpu] key blocks skipped by the bound pass: {pst['key_blocks_skipped']}", flush=True)
    assert pst["pairs_bounded"] > 0 and pst["pairs_survived"] < pst["pairs_bounded"]
    assert pst["groups_skipped"] < wl.total_q // 4, "every fp8 group was skipped"
    assert_same_selection(*outs["dosa"], *outs["dsa"])
    check_vs_oracle(wl, *outs["dsa"], sample_rows(wl, 192), verbose=True)
    # the last chunk again with the debug dumps: bounds, tau and survivor bits against the oracle
    c = list(wl.chunk_calls())[-1]
    sub = synth.Workload(name="correlated_fp8_last_chunk", H=wl.H, d=wl.d, topk=wl.topk, q_dtype="fp8",
                         k_dtype="fp8", q=wl.q[c["q0"]:], q_scale=wl.q_scale[c["q0"]:], w=wl.w[c["q0"]:],
                         k=wl.k[:c["kv_len"]], k_scale=wl.k_scale[:c["kv_len"]],
                         q_lens=np.array([c["q_len"]], np.int32), kv_lens=np.array([c["kv_len"]], np.int32))
    cfg = E.default_config(wl.topk)
    cfg.flags |= E.DOSA_NO_PROBE
    cfg.seed_window = 2048
    idx, sc, st, ub, tau, mask = _debug_run(sub, cfg)
    assert_same_selection(idx, sc, outs["dsa"][0][c["q0"]:], outs["dsa"][1][c["q0"]:])
    assert check_debug_dumps(sub, ub, tau, mask, sample_rows(sub, 12)) > 0


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_group_lists_match_the_union_route(dtype):
    """DOSA_GROUP_LISTS sends every tile's survivors to per-group streams (4 queries per group
    for fp8, 2 for bf16, 1 for fp32 at H = 64, d = 128) instead of the tile's shared union
    list: both routes return the dense path's selection bit for bit, the forced route scores
    its survivors from the group lists, and it never scores more pairs than the union does."""
    import exact_top_token_amd as E
    from exact_top_token_amd.runner import run_once

    wl = synth.correlated_heads(L=6144, topk=256, dtype=dtype)
    di, ds, _ = run_once(wl, "dsa")
    out = {}
    for name, extra in (("union", 0), ("lists", E.DOSA_GROUP_LISTS)):
        cfg = E.default_config(wl.topk)
        cfg.seed_window = 1024
        cfg.flags |= E.DOSA_NO_PROBE | extra
        print(f"[gpu] group lists {dtype} {name}", flush=True)
        pi, ps, pst = run_once(wl, "dosa", cfg=cfg)
        assert_same_selection(pi, ps, di, ds)
        out[name] = pst
    print("union route", out["union"], "\nlist route", out["lists"], flush=True)
    u, g = out["union"], out["lists"]
    assert u["pairs_survived"] == g["pairs_survived"] and u["pairs_bounded"] == g["pairs_bounded"]
    assert g["pairs_survived"] < g["pairs_bounded"], "the certificate should prune"
    assert g["pairs_scored_list"] == g["pairs_scored"] > 0
    assert g["pairs_scored"] <= u["pairs_scored"]
    check_vs_oracle(wl, di, ds, sample_rows(wl, 16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_two_rounds_raise_the_threshold_and_match(dtype):
    """DOSA_TWO_ROUNDS: the newer half of each tile's bounded keys is bounded and scored first,
    the K-th largest exact score so far bounds the older half.  Every chunk call equals the dense
    path bit for bit, the same pairs are bounded as with one round and no more survive (the
    older half is bounded against a threshold at least as high), and the oracle agrees."""
    import torch

    import exact_top_token_amd as E
    from exact_top_token_amd.runner import Runner, slice_chunk, to_device

    wl = synth.correlated_heads(L=16384, dtype=dtype, chunk=4096)
    inp = to_device(wl)
    outs, stats = {}, {}
    for name, path, flags in (("dense", "dsa", 0), ("one", "dosa", 0), ("two", "dosa", E.DOSA_TWO_ROUNDS)):
        idx = np.zeros((wl.total_q, wl.topk), np.int32)
        sc = np.zeros((wl.total_q, wl.topk), np.float32)
        cfg = E.default_config(wl.topk)
        cfg.flags |= E.DOSA_NO_PROBE | flags
        cfg.seed_window = 2048
        tot = {}
        for c in wl.chunk_calls():
            print(f"[gpu] two rounds {dtype} chunk {c} {name}", flush=True)
            r = Runner(slice_chunk(inp, c["q0"], c["q_len"], c["kv_len"]), path, cfg)
            a, b = r()
            torch.cuda.synchronize()
            idx[c["q0"]:c["q0"] + c["q_len"]] = a.cpu().numpy()
            sc[c["q0"]:c["q0"] + c["q_len"]] = b.cpu().numpy()
            for k, v in r.stats_dict().items():
                tot[k] = tot.get(k, 0) + v
        outs[name] = (idx, sc)
        stats[name] = tot
    one, two = stats["one"], stats["two"]
    print(f"two rounds {dtype}: one round {one}", flush=True)
    print(f"two rounds {dtype}: two rounds {two}", flush=True)
    assert_same_selection(*outs["one"], *outs["dense"])
    assert_same_selection(*outs["two"], *outs["dense"])
    assert two["pairs_bounded"] == one["pairs_bounded"] > 0
    assert two["pairs_survived"] <= one["pairs_survived"]
    check_vs_oracle(wl, *outs["two"], sample_rows(wl, 96), verbose=True)


def test_correlated_decode_bf16q_fp8k_prunes():
    """bf16 queries against a paged fp8 key cache (the decode operand types), correlated keys:
    groups are planned, bounded and pruned; the pruned path equals the dense path and the
    oracle on every row; the debug dumps check out against the oracle."""
    import exact_top_token_amd as E

    wl = synth.correlated_decode(batch=6, kv_min=3000, kv_max=20000, topk=256)
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 256
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=np.arange(wl.total_q), cfg=cfg)
    print("correlated decode stats", pst, flush=True)
    assert pst["pairs_bounded"] > 0 and pst["pairs_survived"] < pst["pairs_bounded"]
    assert pst["groups_skipped"] < wl.total_q // 2, "every decode group was skipped"
    idx, sc, st, ub, tau, mask = _debug_run(wl, cfg)
    assert_same_selection(idx, sc, di, ds)
    assert check_debug_dumps(wl, ub, tau, mask, np.arange(wl.total_q)) > 0


def test_decode_probe_decisions():
    """Decode-like batches of at least 8 sequences are probed by planning every group with an
    estimated threshold: the structured recipe (no query can prune) goes to the dense split items,
    the correlated one keeps the certificate pipeline; both equal the dense path on every row."""
    import exact_top_token_amd as E

    wl = synth.decode_mtp(batch=10, kv_min=3000, kv_max=20000)
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 8))
    assert pst["calls_unpruned"] == 1 and pst["pairs_bounded"] == 0 and pst["pairs_scored"] == wl.pairs()
    cfg = E.default_config(wl.topk)
    cfg.flags |= E.DOSA_NO_PROBE
    pi2, ps2, pst2 = _run(wl, "dosa", cfg=cfg)
    assert_same_selection(pi2, ps2, di, ds)
    assert pst2["calls_unpruned"] == 0 and pst2["pairs_seed"] + pst2["pairs_bounded"] == wl.pairs()

    wl = synth.correlated_decode(batch=10, kv_min=3000, kv_max=20000, topk=256)
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 256
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 8), cfg=cfg)
    assert pst["calls_unpruned"] == 0, "the probe sent a prunable decode batch to dense scoring"
    assert pst["pairs_bounded"] > 0 and pst["pairs_survived"] < pst["pairs_bounded"]

    # more groups than the probe plans (it takes a sample of the last ones)
    wl = synth.decode_mtp(batch=300, kv_min=5000, kv_max=9000)
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 8))
    assert pst["calls_unpruned"] == 1 and pst["pairs_bounded"] == 0


@pytest.mark.parametrize("H", [24, 40, 48, 56])
@pytest.mark.parametrize("qd,kd", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "fp8"), ("bf16", "fp8")])
def test_head_counts_padded(H, qd, kd):
    """Head counts between the kernels' 8/16/32/64 head slots: the stored rows are read with
    their own stride and the extra slots stay zero."""
    import exact_top_token_amd as E

    wl = synth.custom(6, [(37, 900), (3, 3), (9, 80)], H=H, d=128 if H != 24 else 64, topk=96, q_dtype=qd,
                      k_dtype=kd, page_size=16 if kd == "fp8" else 0)
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 128
    cfg.flags |= E.DOSA_NO_PROBE
    _both(wl, rows=np.arange(wl.total_q), cfg=cfg)


def test_correlated_heads_h32_prunes():
    """The GLM-5.2 head count (32 indexer heads) on the correlated recipe."""
    import exact_top_token_amd as E

    wl = synth.correlated_heads(L=6000, H=32, topk=512)
    cfg = E.default_config(wl.topk)
    cfg.seed_window = 1024
    cfg.flags |= E.DOSA_NO_PROBE
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 64), cfg=cfg)
    assert pst["pairs_survived"] < pst["pairs_bounded"]


@pytest.mark.parametrize("case", ["all_negative_w", "zero_queries", "huge_scale"])
def test_degenerate_score_distributions(case):
    """Massive exact ties and extreme magnitudes: the answer is still the oracle's."""
    wl = synth.custom(11, [(37, 3000), (5, 700)], H=8, d=64, topk=128, q_dtype="f32", k_dtype="f32")
    if case == "all_negative_w":
        wl.w = -np.abs(wl.w)                 # every score <= 0, most keys exactly 0
    elif case == "zero_queries":
        wl.q = np.zeros_like(wl.q)           # every score is 0: Top-K = the lowest positions
    else:
        wl.k = wl.k * np.float32(1e15)       # scores ~1e16..1e17
    (di, ds, _), _ = _both(wl, rows=np.arange(wl.total_q))
    if case == "zero_queries":
        for r in range(wl.total_q):
            v = np.sort(di[r][di[r] >= 0])
            assert np.array_equal(v, np.arange(v.size)), r


def test_key_block_test_skips_blocks_and_matches():
    """The key-block test of the bound pass (DOSA_KEY_BLOCKS): on the last queries of a long
    correlated context whole 64-key blocks fall below tau and are never loaded; the selection
    still equals the dense path's, and the dumped bounds -- the block bound for every key of a
    skipped block -- dominate the oracle's scores."""
    import exact_top_token_amd as E

    wl = synth.correlated_heads(L=32768, q_len=128)
    cfg = E.default_config(wl.topk)
    cfg.flags |= E.DOSA_NO_PROBE | E.DOSA_KEY_BLOCKS
    (di, ds, dst), (pi, ps, pst) = _both(wl, rows=sample_rows(wl, 8), cfg=cfg)
    print("key-block stats", pst, flush=True)
    assert pst["key_blocks_skipped"] > 0, "no key block was skipped"
    idx, sc, st, ub, tau, mask = _debug_run(wl, cfg)
    assert_same_selection(idx, sc, di, ds)
    assert check_debug_dumps(wl, ub, tau, mask, sample_rows(wl, 6)) > 0
