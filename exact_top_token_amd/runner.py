"""Device plumbing around the C-ABI: move a workload's buffers to the GPU and
call either entry point with PyTorch-allocated outputs and workspace.

No arithmetic of the method happens here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import (DOSA_SORTED, STAT_FIELDS, DosaConfig, default_config, dosa_indexer_topk, dsa_indexer_topk,
               workspace_size)


@dataclass
class DeviceInputs:
    q: object
    q_scale: object
    w: object
    k: object
    k_scale: object
    page_table: object
    page_size: int
    q_lens: list
    kv_lens: list
    H: int
    d: int
    topk: int
    q_dtype: str
    k_dtype: str

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))


def _t(a, device):
    import torch

    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def to_device(wl, device="cuda") -> DeviceInputs:
    return DeviceInputs(q=_t(wl.q, device), q_scale=_t(wl.q_scale, device), w=_t(wl.w, device),
                        k=_t(wl.k, device), k_scale=_t(wl.k_scale, device),
                        page_table=_t(wl.page_table, device), page_size=int(wl.page_size or 0),
                        q_lens=[int(x) for x in wl.q_lens], kv_lens=[int(x) for x in wl.kv_lens],
                        H=wl.H, d=wl.d, topk=wl.topk, q_dtype=wl.q_dtype, k_dtype=wl.k_dtype)


class Runner:
    """Holds outputs, workspace and stats for repeated calls on one input set."""

    def __init__(self, inp: DeviceInputs, path: str = "dosa", cfg: Optional[DosaConfig] = None,
                 sorted_rows: bool = False, key_splits: int = 0, want_scores: bool = True,
                 device="cuda", seeds=None):
        import torch

        self.inp = inp
        self.path = path
        self.cfg = cfg if cfg is not None else default_config(inp.topk)
        self.seeds = None
        if seeds is not None:   # extra seed keys per query row: [total_q, S] int32, -1 padding
            self.seeds = (seeds if isinstance(seeds, torch.Tensor) else _t(np.asarray(seeds, np.int32), device))
            self.seeds = self.seeds.to(device=device, dtype=torch.int32).contiguous()
            assert self.seeds.dim() == 2 and self.seeds.shape[0] == inp.total_q
            self.cfg.seed_idx = self.seeds.data_ptr()
            self.cfg.seed_count = int(self.seeds.shape[1])
        if key_splits:
            self.cfg.key_splits = key_splits
        if sorted_rows:
            self.cfg.flags |= DOSA_SORTED
        self.flags = DOSA_SORTED if sorted_rows else 0
        self.key_splits = key_splits
        paged = inp.page_table is not None
        nbytes = workspace_size(inp.q_lens, inp.kv_lens, inp.H, inp.d, inp.topk, inp.q_dtype, inp.k_dtype,
                                paged, path == "dsa", self.cfg)
        if nbytes == 0:
            raise ValueError("invalid shapes for the library")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.out_idx = torch.empty((inp.total_q, inp.topk), dtype=torch.int32, device=device)
        self.out_score = (torch.empty((inp.total_q, inp.topk), dtype=torch.float32, device=device)
                          if want_scores else None)
        self.stats = torch.zeros(len(STAT_FIELDS), dtype=torch.int64, device=device)

    def __call__(self, stream=None):
        i = self.inp
        if self.path == "dsa":
            dsa_indexer_topk(i.q, i.q_dtype, i.q_scale, i.w, i.k, i.k_dtype, i.k_scale, i.q_lens, i.kv_lens,
                             i.page_table, i.page_size, i.H, i.d, i.topk, self.out_idx, self.out_score,
                             self.workspace, cfg=self.cfg, stats=self.stats, stream=stream)
        else:
            dosa_indexer_topk(i.q, i.q_dtype, i.q_scale, i.w, i.k, i.k_dtype, i.k_scale, i.q_lens, i.kv_lens,
                              i.page_table, i.page_size, i.H, i.d, i.topk, self.out_idx, self.out_score,
                              self.workspace, cfg=self.cfg, stats=self.stats, stream=stream)
        return self.out_idx, self.out_score

    def stats_dict(self) -> dict:
        v = self.stats.cpu().numpy().astype(np.uint64)
        return {k: int(x) for k, x in zip(STAT_FIELDS, v)}

    def reset_stats(self):
        self.stats.zero_()


def slice_chunk(inp: DeviceInputs, q0: int, q_len: int, kv_len: int) -> DeviceInputs:
    """View of a single-sequence contiguous input as one chunked-prefill call."""
    assert len(inp.q_lens) == 1 and inp.page_table is None
    return DeviceInputs(q=inp.q[q0:q0 + q_len], q_scale=None if inp.q_scale is None else inp.q_scale[q0:q0 + q_len],
                        w=inp.w[q0:q0 + q_len], k=inp.k[:kv_len],
                        k_scale=None if inp.k_scale is None else inp.k_scale[:kv_len], page_table=None,
                        page_size=0, q_lens=[q_len], kv_lens=[kv_len], H=inp.H, d=inp.d, topk=inp.topk,
                        q_dtype=inp.q_dtype, k_dtype=inp.k_dtype)


def run_once(wl, path="dosa", cfg=None, sorted_rows=False, key_splits=0, device="cuda", seeds=None):
    """Convenience: inputs to device, one call, results to host numpy."""
    import torch

    inp = to_device(wl, device)
    r = Runner(inp, path, cfg, sorted_rows, key_splits, device=device, seeds=seeds)
    idx, sc = r()
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy(), r.stats_dict()
