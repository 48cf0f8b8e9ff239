"""Pins for the CPU oracle: checks against things other than the oracle itself.

* hand-worked examples (tests/golden/hand_examples.json)
* exact rational arithmetic by brute force on tiny inputs
* closed forms (single head, collinear keys, all-negative weights, K >= visible)
* independent library routines (torch casts for the format tables, scipy NNLS)
* invariants (causality, scaling, permutation)
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import certificate as cert
from oracle import formats, indexer

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------
def test_fp8_hand_values():
    for code, val in GOLD["fp8_e4m3fn"].items():
        if code.startswith("_"):
            continue
        got = formats.decode_fp8(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == val, (code, got, val)


def test_fp8_table_matches_torch_cast():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.decode_fp8(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.nanmax(got) == 448.0 and np.sum(np.isnan(got)) == 2


def test_bf16_hand_and_torch():
    torch = pytest.importorskip("torch")
    for bits, val in GOLD["bf16"].items():
        if bits.startswith("_"):
            continue
        assert formats.decode_bf16(np.array([int(bits, 16)], np.uint16))[0] == val
    x = np.random.default_rng(3).standard_normal(1000).astype(np.float32) * 100
    b = synth.to_bf16_bits(x)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(formats.decode_bf16(b), ref)


def test_fp8_per_token_dequant_scale():
    x = np.random.default_rng(5).standard_normal((7, 3, 16)).astype(np.float32)
    codes, scale = synth.quantize_fp8_per_token(x, 1)
    dq = formats.decode(codes, "fp8", scale)
    # E4M3 keeps 4 significant bits: relative error <= 2^-4 for normal values
    amax = np.abs(x).reshape(7, -1).max(1)
    err = np.abs(dq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, (amax / 448.0 * 2.0 ** -10)[:, None, None])
    assert np.all(err <= bound * 1.0000001)
    assert np.allclose(np.abs(dq).reshape(7, -1).max(1), amax, rtol=2 ** -4)


# ----------------------------------------------------------------------------
# scores and selection: hand examples, brute force with exact rationals
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("ex", GOLD["scores"], ids=lambda e: e["name"])
def test_scores_hand_examples(ex):
    q = np.array(ex["q"], float)
    w = np.array(ex["w"], float)
    k = np.array(ex["k"], float)
    S = indexer.scores(q, w, k)
    assert np.array_equal(S, np.array(ex["S"], float))
    idx, _ = indexer.select_topk(S, len(S))
    assert idx.tolist() == ex["order"]
    idx, _ = indexer.select_topk(S, ex["K"])
    assert idx.tolist() == ex["topk"]


def _wl_from_lists(q, w, k, K, q_lens, kv_lens):
    q = np.array(q, np.float32)
    k = np.array(k, np.float32)
    return synth.Workload(name="hand", H=q.shape[1], d=q.shape[2], topk=K, q_dtype="f32", k_dtype="f32",
                          q=q, q_scale=None, w=np.array(w, np.float32), k=k, k_scale=None,
                          q_lens=np.array(q_lens, np.int32), kv_lens=np.array(kv_lens, np.int32))


def test_causal_hand_example():
    ex = GOLD["causal_prefill"]
    wl = _wl_from_lists(ex["q"], ex["w"], ex["k"], ex["K"], [2], [2])
    idx = indexer.topk_rows(wl, return_scores=False)
    assert idx.tolist() == ex["topk"]


def _fraction_scores(q, w, k):
    H, d = q.shape
    out = []
    for s in range(k.shape[0]):
        tot = Fraction(0)
        for h in range(H):
            x = sum(Fraction(q[h, i]) * Fraction(k[s, i]) for i in range(d))
            tot += Fraction(w[h]) * (x if x > 0 else Fraction(0))
        out.append(tot)
    return out


def _argmax_select(vals, K):
    """Repeated arg-max with the lower index winning ties."""
    remaining = list(range(len(vals)))
    picked = []
    for _ in range(min(K, len(vals))):
        best = remaining[0]
        for s in remaining[1:]:
            if vals[s] > vals[best]:
                best = s
        picked.append(best)
        remaining.remove(best)
    return picked + [-1] * (K - len(picked))


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_rational(seed):
    rng = np.random.default_rng(100 + seed)
    H, d, n, m, K = 3, 5, 14, 5, 4
    # dyadic inputs with few bits: every float64 product and sum is exact
    q = rng.integers(-8, 9, size=(m, H, d)) / 4.0
    w = rng.integers(-8, 9, size=(m, H)) / 8.0
    k = rng.integers(-8, 9, size=(n, d)) / 2.0
    k[3] = k[7]                     # duplicate keys -> exact ties
    wl = _wl_from_lists(q, w, k, K, [m], [n])
    idx, sc, _ = indexer.topk_rows(wl)
    for i in range(m):
        pos = n - m + i
        fr = _fraction_scores(q[i], w[i], k[: pos + 1])
        assert [float(v) for v in fr] == indexer.scores(q[i][None], w[i][None], k[: pos + 1])[0].tolist()
        assert idx[i].tolist() == _argmax_select(fr, K)


def test_select_bruteforce_random_ties():
    rng = np.random.default_rng(7)
    for _ in range(50):
        n = int(rng.integers(1, 30))
        K = int(rng.integers(1, 35))
        S = rng.integers(-3, 4, size=n).astype(float)     # many ties
        idx, sc = indexer.select_topk(S, K)
        assert idx.tolist() == _argmax_select(list(S), K)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_single_head_is_relu_mips():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((200, 16))
    w = np.array([[0.7]])
    S = indexer.scores(q, w, k)[0]
    dots = k @ q[0, 0]
    order = np.lexsort((np.arange(200), -np.maximum(dots, 0)))
    idx, _ = indexer.select_topk(S, 150)
    assert idx.tolist() == order[:150].tolist()
    # every key with a negative dot product scores exactly 0, ordered by index
    zeros = np.nonzero(dots <= 0)[0]
    npos = int(np.sum(dots > 0))
    assert idx[npos: npos + 10].tolist() == zeros[:10].tolist()


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_collinear_keys_monotone(sign):
    rng = np.random.default_rng(12)
    u = rng.standard_normal(8)
    c = rng.uniform(0.1, 5.0, size=60)
    k = c[:, None] * u[None, :]
    q = rng.standard_normal((1, 6, 8))
    w = rng.standard_normal((1, 6))
    C = float(np.sum(w[0] * np.maximum(q[0] @ u, 0)))
    w = w * sign * np.sign(C)            # make the common factor sign-controlled
    S = indexer.scores(q, w, k)[0]
    idx, _ = indexer.select_topk(S, 20)
    want = np.argsort(-c)[:20] if sign > 0 else np.argsort(c)[:20]
    assert idx.tolist() == want.tolist()


def test_all_negative_weights_nonpositive():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((2, 4, 8))
    w = -np.abs(rng.standard_normal((2, 4)))
    k = rng.standard_normal((100, 8))
    S = indexer.scores(q, w, k)
    assert np.all(S <= 0)
    x = np.einsum("thd,sd->ths", q, k)
    silent = np.all(x <= 0, axis=1)               # keys where no head fires score exactly 0
    assert np.all(S[silent] == 0) and np.all(S[~silent] < 0)


def test_k_at_least_visible_returns_all_then_pad():
    wl = synth.custom(0, [(3, 5)], H=4, d=8, topk=9)
    idx = indexer.topk_rows(wl, return_scores=False)
    for i in range(3):
        vis = 5 - 3 + i + 1
        assert sorted(idx[i, :vis].tolist()) == list(range(vis))
        assert np.all(idx[i, vis:] == -1)


def test_causality_and_positions():
    wl = synth.custom(1, [(4, 40), (2, 2), (5, 9)], H=4, d=8, topk=6)
    idx = indexer.topk_rows(wl, return_scores=False)
    seq, pos = indexer.query_positions(wl)
    assert pos.tolist() == [36, 37, 38, 39, 0, 1, 4, 5, 6, 7, 8]
    for r in range(wl.total_q):
        v = idx[r][idx[r] >= 0]
        assert np.all(v <= pos[r])
        assert v.size == min(6, pos[r] + 1)


def test_power_of_two_scaling_invariance():
    wl = synth.custom(2, [(6, 50)], H=4, d=8, topk=7)
    a = indexer.topk_rows(wl)
    wl.k = wl.k * np.float32(2.0)
    b = indexer.topk_rows(wl)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1] * 2, b[1])


def test_paged_equals_contiguous():
    lens = [(3, 70), (2, 130), (1, 1)]
    c = synth.custom(4, lens, H=4, d=8, topk=16)
    p = synth.custom(4, lens, H=4, d=8, topk=16, page_size=16)
    assert p.page_table is not None
    a = indexer.topk_rows(c)
    b = indexer.topk_rows(p)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_logical_permutation_maps_set():
    """Permuting the keys of a query that sees all of them permutes its Top-K (no ties in random data)."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 4, 8))
    w = rng.standard_normal((1, 4))
    k = rng.standard_normal((80, 8))
    perm = rng.permutation(80)
    i1, _ = indexer.select_topk(indexer.scores(q, w, k)[0], 10)
    i2, _ = indexer.select_topk(indexer.scores(q, w, k[perm])[0], 10)
    assert sorted(perm[i2].tolist()) == sorted(i1.tolist())


# ----------------------------------------------------------------------------
# certificate
# ----------------------------------------------------------------------------
def test_certificate_hand_example():
    ex = GOLD["certificate"]
    q = np.array(ex["q"], float)
    w = np.array(ex["w"], float)
    k = np.array(ex["k"], float)
    x_seed = q @ k.T
    pl = cert.plan(q, w, x_seed, num_proxies=ex["num_proxies"], support_frac=0.0)
    assert pl["P"].tolist() == ex["P"]
    assert np.allclose(pl["c"], ex["c"]) and math.isclose(pl["rho"], ex["rho"])
    assert np.allclose(pl["a"], ex["a"])
    assert np.allclose(indexer.scores(q[None], w[None], k)[0], ex["S"])
    assert np.allclose(cert.upper_bound(pl, k), ex["UB"], rtol=1e-14)


def test_nnls_matches_scipy():
    so = pytest.importorskip("scipy.optimize")
    rng = np.random.default_rng(21)
    for _ in range(40):
        p = int(rng.integers(1, 5))
        Q = rng.standard_normal((12, p))
        v = rng.standard_normal(12)
        a = cert.nnls(Q, v)
        b, _ = so.nnls(Q, v)
        assert np.all(a >= 0)
        assert np.allclose(np.linalg.norm(v - Q @ a), np.linalg.norm(v - Q @ b), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("p,rho_kind,frac", [(0, "joint", 0.5), (1, "joint", 0.5), (3, "joint", 0.5),
                                             (3, "separable", 0.5), (7, "joint", 0.0), (3, "joint", 1.0)])
def test_bound_dominates_scores_exhaustive(p, rho_kind, frac):
    """UB >= S for every (query, key) pair of a small i.i.d. problem, every knob setting."""
    rng = np.random.default_rng(31 + p)
    H, d, n = 8, 16, 300
    for t in range(6):
        q = rng.standard_normal((H, d))
        w = rng.standard_normal(H)
        k = rng.standard_normal((n, d)) * rng.uniform(0.2, 3.0, size=(n, 1))
        S = indexer.scores(q[None], w[None], k)[0]
        pl = cert.plan(q, w, q @ k[:50].T, num_proxies=p, support_frac=frac, rho_kind=rho_kind)
        UB = cert.upper_bound(pl, k)
        scale = indexer.abs_mass(q[None], w[None], k)[0] + 1.0
        assert np.all(UB - S >= -1e-12 * scale)


def test_bound_equality_case():
    """All positive heads as proxies and a single negative head in the support: UB == S."""
    rng = np.random.default_rng(41)
    H, d = 6, 10
    q = rng.standard_normal((H, d))
    w = np.abs(rng.standard_normal(H))
    w[2] = -w[2]
    k = rng.standard_normal((200, d))
    pl = cert.plan(q, w, q @ k.T, num_proxies=H, support_frac=0.0)
    assert pl["rho"] == 0.0 and pl["A"].tolist() == [2]
    assert np.allclose(cert.upper_bound(pl, k), indexer.scores(q[None], w[None], k)[0], rtol=1e-12, atol=1e-12)


def test_joint_rho_not_above_separable():
    rng = np.random.default_rng(43)
    for _ in range(20):
        q = rng.standard_normal((12, 8))
        w = rng.standard_normal(12)
        a = cert.plan(q, w, None, 2, rho_kind="joint")["rho"]
        b = cert.plan(q, w, None, 2, rho_kind="separable")["rho"]
        assert a <= b + 1e-12


def test_dropping_residual_term_is_caught():
    """A plausible mistake (no residual term) must break UB >= S somewhere."""
    rng = np.random.default_rng(44)
    q = rng.standard_normal((8, 16))
    w = np.abs(rng.standard_normal(8))
    k = rng.standard_normal((400, 16))
    pl = cert.plan(q, w, None, 2)
    pl_bad = dict(pl, rho=0.0)
    S = indexer.scores(q[None], w[None], k)[0]
    assert np.all(cert.upper_bound(pl, k) >= S - 1e-9)
    assert np.any(cert.upper_bound(pl_bad, k) < S - 1e-6)


def test_pruning_never_drops_topk_tiny_prefill():
    """Every pruned key of the tiny prefill scores strictly below the oracle's K-th score."""
    wl = synth.tiny_prefill(L=512, topk=32)
    rows = np.arange(40, 512, 37)
    idx, sc, theta = indexer.topk_rows(wl, rows)
    seq, pos = indexer.query_positions(wl)
    for j, r in enumerate(rows):
        kv = indexer.seq_keys(wl, 0, pos[r] + 1)
        c = cert.query_certificate(indexer.query_rows(wl, [r])[0], indexer.weights(wl, [r])[0], kv,
                                   int(pos[r]), wl.topk, num_proxies=3, prefix=4, window=48)
        assert np.all(c["UB"] >= c["S"] - 1e-9 * (1 + np.abs(c["S"])))
        pr = np.nonzero(c["pruned"])[0]
        assert not np.any(np.isin(pr, idx[j]))
        assert np.all(c["S"][pr] < theta[j])


@pytest.mark.parametrize("recipe", ["tiny", "correlated"])
def test_two_round_threshold_is_valid_and_prunes_more(recipe):
    """Two rounds (threshold raised by round-1 survivors): tau <= tau2 <= the K-th score of a
    full sort, every key one round prunes is pruned again, and no Top-K key is pruned."""
    if recipe == "tiny":
        wl = synth.tiny_prefill(L=600, topk=32)
        rows, kw = np.arange(300, 600, 41), dict(num_proxies=3, prefix=4, window=64)
    else:
        wl = synth.correlated_heads(L=2048, topk=64)
        rows, kw = np.array([1500, 1800, 2047]), dict(num_proxies=3, prefix=64, window=256)
    idx, sc, theta = indexer.topk_rows(wl, rows)
    seq, pos = indexer.query_positions(wl)
    gained = 0
    for j, r in enumerate(rows):
        kv = indexer.seq_keys(wl, 0, pos[r] + 1)
        c = cert.query_certificate(indexer.query_rows(wl, [r])[0], indexer.weights(wl, [r])[0], kv,
                                   int(pos[r]), wl.topk, **kw)
        pr2, tau2, mid = cert.two_round_pruned(c, wl.topk)
        kth = np.sort(c["S"])[::-1][wl.topk - 1]
        assert c["tau"] <= tau2 <= kth
        assert np.all(pr2[c["pruned"]])                    # round 2 only adds pruned keys
        assert not np.any(np.isin(np.nonzero(pr2)[0], idx[j]))
        assert np.all(c["S"][pr2] < theta[j])
        gained += int(pr2.sum() - c["pruned"].sum())
    assert gained >= 0


def test_seed_threshold_is_lower_bound():
    rng = np.random.default_rng(50)
    for _ in range(30):
        S = rng.standard_normal(int(rng.integers(5, 200)))
        K = int(rng.integers(1, 10))
        seeds = rng.choice(S.size, size=min(S.size, int(rng.integers(1, 60))), replace=False)
        tau = cert.seed_threshold(S[seeds], K)
        kth = np.sort(S)[::-1][K - 1] if S.size >= K else -np.inf
        assert tau <= kth


# ----------------------------------------------------------------------------
# helpers the parity checks lean on: score_pairs, abs_mass, seed_keys, filter_rate
# ----------------------------------------------------------------------------
def _dyadic_paged_workload(seed):
    """Small paged multi-sequence f32 workload with dyadic values (every float64 product and
    sum of the definition is exact)."""
    rng = np.random.default_rng(seed)
    lens = [(3, 40), (2, 17), (4, 33)]
    wl = synth.custom(seed, lens, H=3, d=5, topk=6, page_size=16)
    wl.q = (rng.integers(-8, 9, size=wl.q.shape) / 4.0).astype(np.float32)
    wl.w = (rng.integers(-8, 9, size=wl.w.shape) / 8.0).astype(np.float32)
    kvals = (rng.integers(-8, 9, size=wl.k.shape) / 2.0).astype(np.float32)
    wl.k = np.where(wl.k == 300.0, wl.k, kvals).astype(np.float32)   # keep the junk past each end
    return wl


def _logical_key(wl, b, s):
    pg = wl.page_table[b, s // wl.page_size]
    return wl.k[pg, s % wl.page_size].astype(np.float64)


@pytest.mark.parametrize("seed", range(3))
def test_score_pairs_and_abs_mass_exact_fractions(seed):
    """S and A of explicit (row, key) pairs across sequences of a paged cache, against exact
    rational arithmetic over the logical keys read through the page table by hand."""
    wl = _dyadic_paged_workload(seed)
    seq, pos = indexer.query_positions(wl)
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, wl.total_q, size=60)
    keys = np.array([int(rng.integers(0, pos[r] + 1)) for r in rows])
    S, A = indexer.score_pairs(wl, rows, keys)
    for i, (r, s) in enumerate(zip(rows, keys)):
        k = _logical_key(wl, int(seq[r]), int(s))
        tot_s, tot_a = Fraction(0), Fraction(0)
        for h in range(wl.H):
            x = sum(Fraction(float(wl.q[r, h, j])) * Fraction(float(k[j])) for j in range(wl.d))
            wf = Fraction(float(wl.w[r, h]))
            tot_s += wf * (x if x > 0 else Fraction(0))
            tot_a += abs(wf) * abs(x)
        assert S[i] == float(tot_s) and A[i] == float(tot_a), (r, s)
    # the same pairs through the dense scorer of whole rows
    for r in np.unique(rows):
        kv = indexer.seq_keys(wl, int(seq[r]), int(pos[r]) + 1)
        full = indexer.scores(indexer.query_rows(wl, [r]), indexer.weights(wl, [r]), kv)[0]
        sel = rows == r
        assert np.array_equal(full[keys[sel]], S[sel])


def test_abs_mass_hand_values():
    q = np.array([[[1.0, -2.0], [0.5, 0.5]]])          # 2 heads, d = 2
    w = np.array([[-3.0, 2.0]])
    k = np.array([[1.0, 1.0], [2.0, -1.0]])
    # key 0: x = (-1, 1) -> A = 3*1 + 2*1 = 5 ; key 1: x = (4, 0.5) -> A = 12 + 1 = 13
    assert indexer.abs_mass(q, w, k)[0].tolist() == [5.0, 13.0]
    # and S: key 0 -> 0 + 2*1 = 2 ; key 1 -> -12 + 1 = -11
    assert indexer.scores(q, w, k)[0].tolist() == [2.0, -11.0]


def test_seed_keys_hand_values():
    assert cert.seed_keys(10, 3, prefix=2, window=4).tolist() == [0, 1, 7, 8, 9, 10]
    assert cert.seed_keys(3, 3, prefix=8, window=4).tolist() == [0, 1, 2, 3]        # everything visible
    assert cert.seed_keys(5, 3, prefix=2, window=5).tolist() == [0, 1, 2, 3, 4, 5]  # prefix meets window
    assert cert.seed_keys(100, 4, prefix=0).tolist() == [97, 98, 99, 100]          # window defaults to K
    assert cert.seed_keys(0, 4, prefix=64, window=16).tolist() == [0]


def test_filter_rate_equality_case_counts_from_the_definition():
    """With every positive head a proxy and one negative head in the support the bound equals
    the score, so the pruned pairs are exactly the non-seed keys scoring below the K-th seed
    score: counted here from the scores and a sort."""
    rng = np.random.default_rng(61)
    H, d, L, K = 5, 8, 300, 7
    q = rng.standard_normal((L, H, d)).astype(np.float32)
    w = np.abs(rng.standard_normal((L, H))).astype(np.float32)
    w[:, 1] = -w[:, 1]
    k = rng.standard_normal((L, d)).astype(np.float32)
    wl = synth.Workload(name="eq", H=H, d=d, topk=K, q_dtype="f32", k_dtype="f32", q=q, q_scale=None, w=w, k=k,
                        k_scale=None, q_lens=np.array([L], np.int32), kv_lens=np.array([L], np.int32))
    rows = [40, 151, 299]
    rate, bounded, pruned = cert.filter_rate(wl, rows, num_proxies=H, support_frac=0.0, prefix=3, window=12)
    want_b = want_p = 0
    for r in rows:
        S = indexer.scores(q[r][None].astype(np.float64), w[r][None].astype(np.float64),
                           k[: r + 1].astype(np.float64))[0]
        seeds = np.union1d(np.arange(3), np.arange(r + 1 - 12, r + 1))
        tau = np.sort(S[seeds])[::-1][K - 1]
        rest = np.setdiff1d(np.arange(r + 1), seeds)
        want_b += rest.size
        # equality up to the float64 rounding of UB: exclude keys within 1e-9 of tau
        want_p += int(np.sum(S[rest] < tau - 1e-9))
        assert not np.any(np.abs(S[rest] - tau) <= 1e-9)
    assert bounded == want_b and pruned == want_p
    assert rate == pruned / bounded


def _ub_dominates(wl, rows, **kw):
    seq, pos = indexer.query_positions(wl)
    worst = np.inf
    for r in rows:
        kv = indexer.seq_keys(wl, int(seq[r]), int(pos[r]) + 1)
        q = indexer.query_rows(wl, [r])[0]
        w = indexer.weights(wl, [r])[0]
        c = cert.query_certificate(q, w, kv, int(pos[r]), wl.topk, **kw)
        A = indexer.abs_mass(q[None], w[None], kv)[0]
        worst = min(worst, float(np.min((c["UB"] - c["S"]) / (A + 1.0))))
    return worst


def test_bound_dominates_every_pair_of_the_tiny_prefill():
    """UB >= S for all 2,098,176 causal pairs of the tiny prefill (L = 2048, H = 8, d = 64,
    K = 256), with the seed prefix and window the library uses by default (64 and 4K)."""
    from concurrent.futures import ThreadPoolExecutor

    wl = synth.tiny_prefill()
    blocks = np.array_split(np.arange(wl.total_q), 16)
    with ThreadPoolExecutor(8) as ex:
        worst = min(ex.map(lambda b: _ub_dominates(wl, b, num_proxies=3, prefix=64, window=1024), blocks))
    assert worst >= -1e-12


def test_bound_dominates_sampled_queries_of_the_32k_prefill():
    """UB >= S over all visible keys of sampled queries of the 32K bf16 prefill (H = 64,
    d = 128), for the joint and the separable residual constant."""
    wl = synth.dsa_prefill_32k()
    rows = [100, 5000, 20000, 32767]
    assert _ub_dominates(wl, rows, num_proxies=3, prefix=64, window=8192) >= -1e-12
    assert _ub_dominates(wl, rows[-1:], num_proxies=3, prefix=64, window=8192, rho_kind="separable") >= -1e-12


# ----------------------------------------------------------------------------
# key-block certificate
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("p,frac,block", [(3, 0.5, 64), (1, 0.0, 16), (0, 0.5, 7), (3, 1.0, 1)])
def test_block_bound_dominates_every_key_bound(p, frac, block):
    """BUB >= UB(t, s) for every key of every block (i.i.d. and drifting keys)."""
    rng = np.random.default_rng(71 + p + block)
    H, d, n = 8, 16, 400
    for t in range(4):
        q = rng.standard_normal((H, d))
        w = rng.standard_normal(H)
        if t % 2:
            k = rng.standard_normal((n, d)) * rng.uniform(0.2, 3.0, size=(n, 1))
        else:   # slowly drifting keys: tight blocks
            k = np.cumsum(rng.standard_normal((n, d)) * 0.1, axis=0) + rng.standard_normal((n, d)) * 0.05
        pl = cert.plan(q, w, q @ k[:40].T, num_proxies=p, support_frac=frac)
        UB = cert.upper_bound(pl, k)
        cen, rad, mx = cert.block_summaries(k, block)
        BUB = cert.block_upper_bound(pl, cen, rad, mx)
        scale = indexer.abs_mass(q[None], w[None], k)[0] + 1.0
        for b in range(BUB.size):
            sl = slice(b * block, (b + 1) * block)
            assert np.all(BUB[b] - UB[sl] >= -1e-12 * scale[sl].max()), (t, b)


def test_block_bound_of_one_key_is_the_key_bound():
    """A one-key block has centre k, radius 0 and largest norm ||k||: BUB = UB exactly."""
    rng = np.random.default_rng(72)
    q = rng.standard_normal((6, 12))
    w = rng.standard_normal(6)
    k = rng.standard_normal((50, 12))
    pl = cert.plan(q, w, q @ k.T, num_proxies=2, support_frac=0.3)
    cen, rad, mx = cert.block_summaries(k, 1)
    assert np.all(rad == 0) and np.allclose(mx, np.linalg.norm(k, axis=1))
    assert np.allclose(cert.block_upper_bound(pl, cen, rad, mx), cert.upper_bound(pl, k), rtol=1e-13, atol=1e-12)


def test_block_bound_without_radius_is_caught():
    """A plausible mistake -- the centre used as if it were every key (radius dropped) --
    breaks BUB >= UB on some block."""
    rng = np.random.default_rng(73)
    q = rng.standard_normal((8, 16))
    w = np.abs(rng.standard_normal(8))
    k = rng.standard_normal((512, 16))
    pl = cert.plan(q, w, None, 3)
    cen, rad, mx = cert.block_summaries(k, 64)
    UB = cert.upper_bound(pl, k).reshape(8, 64).max(axis=1)
    assert np.all(cert.block_upper_bound(pl, cen, rad, mx) >= UB - 1e-9)
    assert np.any(cert.block_upper_bound(pl, cen, np.zeros_like(rad), mx) < UB - 1e-6)


def test_block_pruning_is_within_key_pruning_on_the_correlated_recipe():
    """Blocks the block bound prunes hold only keys the per-key certificate prunes, and the
    block bound does prune on the correlated recipe (a late query of a 12K context)."""
    wl = synth.correlated_heads(L=12288, topk=512)
    r = wl.total_q - 1
    kv = indexer.seq_keys(wl, 0, r + 1)
    c = cert.query_certificate(indexer.query_rows(wl, [r])[0], indexer.weights(wl, [r])[0], kv, r, wl.topk,
                               prefix=64, window=2048)
    cen, rad, mx = cert.block_summaries(kv, 64)
    BUB = cert.block_upper_bound(c["plan"], cen, rad, mx)
    seeds = np.zeros(r + 1, bool)
    seeds[c["seeds"]] = True
    pruned_blocks = [b for b in range(BUB.size) if BUB[b] < c["tau"] and not seeds[b * 64:(b + 1) * 64].any()]
    assert len(pruned_blocks) > 0
    for b in pruned_blocks:
        assert np.all(c["pruned"][b * 64:(b + 1) * 64])
