"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (chunked prefill as one call per chunk on shared device inputs).

Every row: the pruned path returns exactly the dense path's keys with
bit-identical scores (compared on the device).  Against the oracle, which
scores each checked row over all its visible keys: every row of the 32K
prefill and of the decode batch; 1024 rows of the 128K chunked prefill (the
first and last query of every chunk, the rest at random); 128 rows of each 1M
chunk (its first and last query, the rest at random).
"""
import numpy as np
import pytest

import synth
from parity_helpers import check_vs_oracle

pytestmark = pytest.mark.gpu


def _run_calls(wl, inp, path, flags=0):
    import torch

    import exact_top_token_amd as E
    from exact_top_token_amd.runner import slice_chunk

    calls = ([(c["q0"], slice_chunk(inp, c["q0"], c["q_len"], c["kv_len"])) for c in wl.chunk_calls()]
             if wl.chunk else [(0, inp)])
    K = wl.topk
    cfg = E.default_config(K)
    cfg.flags |= flags
    ws = torch.empty(max(E.workspace_size(c.q_lens, c.kv_lens, c.H, c.d, K, c.q_dtype, c.k_dtype,
                                          c.page_table is not None, path == "dsa", cfg) for _, c in calls),
                     dtype=torch.uint8, device="cuda")
    idx = torch.empty((wl.total_q, K), dtype=torch.int32, device="cuda")
    sc = torch.empty((wl.total_q, K), dtype=torch.float32, device="cuda")
    st = torch.zeros(len(E.STAT_FIELDS), dtype=torch.int64, device="cuda")
    f = E.dsa_indexer_topk if path == "dsa" else E.dosa_indexer_topk
    for q0, c in calls:
        f(c.q, c.q_dtype, c.q_scale, c.w, c.k, c.k_dtype, c.k_scale, c.q_lens, c.kv_lens, c.page_table,
          c.page_size, c.H, c.d, K, idx[q0:q0 + c.total_q], sc[q0:q0 + c.total_q], ws, cfg=cfg, stats=st)
    torch.cuda.synchronize()
    return idx, sc, {k: int(v) for k, v in zip(E.STAT_FIELDS, st.cpu().numpy().tolist())}


def _same_on_device(ia, sa, ib, sb, block=8192):
    import torch

    for r0 in range(0, ia.shape[0], block):
        xa, oa = torch.sort(ia[r0:r0 + block], dim=1)
        xb, ob = torch.sort(ib[r0:r0 + block], dim=1)
        assert torch.equal(xa, xb), f"key sets differ in rows {r0}..{r0 + block}"
        va = torch.gather(sa[r0:r0 + block], 1, oa).view(torch.int32)
        vb = torch.gather(sb[r0:r0 + block], 1, ob).view(torch.int32)
        assert torch.equal(va, vb), f"scores of the same keys differ in rows {r0}..{r0 + block}"


def _rows(wl, n_target, seed=0):
    """Stratified rows: the first and last query of every chunk call (or sequence), then random
    rows up to n_target (all rows if n_target >= total_q)."""
    if n_target >= wl.total_q:
        return np.arange(wl.total_q, dtype=np.int64)
    picks = set()
    if wl.chunk:
        for c in wl.chunk_calls():
            picks.update([c["q0"], c["q0"] + c["q_len"] - 1])
    else:
        cu = wl.cu_q()
        for b in range(wl.batch):
            if cu[b + 1] > cu[b]:
                picks.update([int(cu[b]), int(cu[b + 1] - 1)])
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(wl.total_q), np.array(sorted(picks), dtype=np.int64))
    need = max(0, n_target - len(picks))
    picks.update(rng.choice(rest, size=min(need, rest.size), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)


def _check(wl, n_rows):
    from exact_top_token_amd.runner import to_device

    print(f"[gpu] full size {wl.name}: q={wl.total_q} H={wl.H} d={wl.d} K={wl.topk} "
          f"{wl.q_dtype}/{wl.k_dtype} pairs={wl.pairs()}", flush=True)
    inp = to_device(wl)
    import exact_top_token_amd as E

    di, ds, dst = _run_calls(wl, inp, "dsa")
    # the certificate pipeline on every call
    pi, ps, pst = _run_calls(wl, inp, "dosa", E.DOSA_NO_PROBE)
    assert dst["pairs_total"] == wl.pairs() == pst["pairs_total"]
    assert pst["pairs_seed"] + pst["pairs_bounded"] == wl.pairs() and pst["calls_unpruned"] == 0
    _same_on_device(pi, ps, di, ds)
    del pi, ps
    # the default: calls whose probe tile cannot prune score densely
    pi, ps, pst2 = _run_calls(wl, inp, "dosa")
    _same_on_device(pi, ps, di, ds)
    del pi, ps
    print(f"[gpu] {wl.name}: calls scored densely after the probe: {pst2['calls_unpruned']}", flush=True)
    rows = _rows(wl, n_rows)
    print(f"[gpu] oracle on {rows.size} rows of {wl.total_q}", flush=True)
    ri = di[rows].cpu().numpy()
    rs = ds[rows].cpu().numpy()
    del di, ds, inp
    st = check_vs_oracle(wl, {int(r): ri[j] for j, r in enumerate(rows)},
                         {int(r): rs[j] for j, r in enumerate(rows)}, rows, verbose=True)
    assert st["rows"] == rows.size
    print(f"[gpu] {wl.name}: filtered {1 - pst['pairs_survived'] / max(pst['pairs_bounded'], 1):.3f}", flush=True)


def test_full_long_prefill_128k_fp8_chunked():
    _check(synth.long_prefill_128k(), 1024)


def test_full_dsa_prefill_32k_bf16():
    _check(synth.dsa_prefill_32k(), 1 << 30)       # every row


def test_full_decode_mtp_paged():
    _check(synth.decode_mtp(), 1 << 30)            # every row


@pytest.mark.parametrize("iid", [False, True])
def test_full_million_chunk(iid):
    _check(synth.make_workload("million_chunk_iid") if iid else synth.million_chunk(), 128)


@pytest.mark.parametrize("q_len", [16384, 32768])
def test_full_million_chunk_long_chunks(q_len):
    """The 1M-key context with 16K- and 32K-query chunks (the pages' larger prefill chunk sizes)."""
    _check(synth.million_chunk(q_len=q_len), 128)


def test_full_long_prefill_128k_h32():
    """The 128K fp8 chunked prefill with 32 indexer heads (the GLM-5.2 indexer's head count)."""
    _check(synth.long_prefill_128k(H=32), 512)
