"""The no-allocation entry point against the workspace entry point, through the C-ABI.

dosa_indexer_topk_noalloc runs the pruned path in the library's own scratch
array; its result must equal dosa_indexer_topk's on the same inputs (same keys,
bit-identical scores), on two calls in a row with the second smaller, so the
second call runs on whatever the first left in the scratch.  A call larger than
the scratch is rejected on the host.
"""
import numpy as np
import pytest

import synth
from parity_helpers import assert_same_selection

pytestmark = pytest.mark.gpu


def _noalloc(wl, cfg):
    import torch

    import exact_top_token_amd as E
    from exact_top_token_amd.runner import to_device

    inp = to_device(wl)
    idx = torch.full((inp.total_q, wl.topk), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((inp.total_q, wl.topk), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.zeros(len(E.STAT_FIELDS), dtype=torch.int64, device="cuda")
    print(f"[gpu] noalloc {wl.name} q={wl.total_q} H={wl.H} d={wl.d} K={wl.topk} {wl.q_dtype}/{wl.k_dtype}",
          flush=True)
    E.dosa_indexer_topk_noalloc(inp.q, inp.q_dtype, inp.q_scale, inp.w, inp.k, inp.k_dtype, inp.k_scale,
                                inp.q_lens, inp.kv_lens, inp.page_table, inp.page_size, inp.H, inp.d, wl.topk,
                                idx, sc, cfg=cfg, stats=st)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _workspace(wl, cfg):
    from exact_top_token_amd.runner import run_once

    print(f"[gpu] workspace entry point {wl.name}", flush=True)
    i, s, _ = run_once(wl, "dosa", cfg=cfg)
    return i, s


def test_noalloc_matches_workspace_entry_point_two_calls():
    import exact_top_token_amd as E

    big = synth.correlated_heads(L=3000, topk=128)               # ~60 MiB of workspace
    small = synth.custom(5, [(37, 900), (3, 3), (9, 80)], H=64, d=128, topk=96, q_dtype="fp8", k_dtype="fp8")
    for wl, no_probe in ((big, True), (small, False)):
        cfg = E.default_config(wl.topk)
        cfg.seed_window = 512
        if no_probe:
            cfg.flags |= E.DOSA_NO_PROBE
        need = E.workspace_size(wl.q_lens, wl.kv_lens, wl.H, wl.d, wl.topk, wl.q_dtype, wl.k_dtype,
                                wl.page_table is not None, False, cfg)
        assert 0 < need <= E.NOALLOC_SCRATCH_BYTES
        ri, rs = _workspace(wl, cfg)
        ni, ns = _noalloc(wl, cfg)
        assert_same_selection(ni, ns, ri, rs)


def test_noalloc_paged_decode_then_tiny_prefill():
    import exact_top_token_amd as E

    dec = synth.correlated_decode(batch=4, kv_min=3000, kv_max=12000, topk=256)
    tiny = synth.tiny_prefill(L=1024, topk=64)                     # probe tile on (>= 8 query tiles)
    for wl in (dec, tiny):
        cfg = E.default_config(wl.topk)
        cfg.seed_window = 256
        ri, rs = _workspace(wl, cfg)
        ni, ns = _noalloc(wl, cfg)
        assert_same_selection(ni, ns, ri, rs)


def test_noalloc_rejects_calls_beyond_the_scratch():
    import exact_top_token_amd as E

    q_lens, kv_lens = [4096], [131072]
    need = E.workspace_size(q_lens, kv_lens, 64, 128, 2048, "fp8", "fp8", False, False)
    assert need > E.NOALLOC_SCRATCH_BYTES

    class _Fake:
        shape = (1, 1)

        def data_ptr(self):
            return 0x1000

    f = _Fake()
    with pytest.raises(E.DosaError) as ei:
        E.dosa_indexer_topk_noalloc(f, "fp8", f, f, f, "fp8", f, q_lens, kv_lens, None, 0, 64, 128, 2048, f, None)
    assert ei.value.status == -2 and "workspace" in str(ei.value)
