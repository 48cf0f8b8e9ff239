#!/usr/bin/env python3
"""Benchmark of the DSA-indexer exact Top-K on one MI355X.

Workload (default): long prefill, one sequence of 131072 tokens, H=64 indexer
heads, d=128, Top-K 2048, fp8 E4M3FN q/k with per-token fp32 scales, fp32 w,
run as 32 causal chunks of 4096 queries (chunk c sees the first 4096*(c+1)
keys).  One step = the 32 chunk calls = the indexer of the whole prefill.

Reported: dense-equivalent query-key scores per second of the pruned path
(dosa_indexer_topk) -- causal pairs / wall time, inputs resident in HBM --
next to the dense path (dsa_indexer_topk) on the same inputs, the filter rate,
per-pass kernel times from HIP events recorded around every launch, the
roofline fraction of the dominant kernel, and the CPU oracle timed on a
bounded sample on the host cores.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--workload long_prefill_128k]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
COMBO_ID = {("f32", "f32"): 0, ("bf16", "bf16"): 1, ("fp8", "fp8"): 2, ("bf16", "fp8"): 3}
ROLE_ID = {"score_dense": 0, "score_seed": 1, "score_survivor_tiles": 2, "score_survivor_lists": 2}
# HBM traffic per launch measured with rocprofv3 counters, valid while the
# kernel's sources are unchanged (sha256 over KERNEL_SOURCES)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["exact_top_token_amd/csrc/score_kernels.h", "exact_top_token_amd/csrc/dosa_device.h",
                  "exact_top_token_amd/csrc/dosa_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def padded_heads(H):
    """Head slots of the kernel instantiation that serves H heads."""
    return 8 if H <= 8 else (16 if H <= 16 else (32 if H <= 32 else 64))


def queries_per_group(wl):
    """Queries of one MFMA row group (4, 2 or 1, as the library plans them)."""
    qb = {"fp8": 1, "bf16": 2, "f32": 4}[wl.q_dtype]
    per = padded_heads(wl.H) * wl.d * qb
    return 4 if (4 * per <= 32768 and wl.H % 4 == 0) else (2 if (2 * per <= 32768 and wl.H % 8 == 0) else 1)


def uses_tiles(wl):
    """Whether the library scores this batch with the tiled kernel (8 query
    groups of 4/2/1 queries per workgroup) or, when tiles would hold fewer than
    4 groups on average (decode-like batches), the split kernel (a workgroup's
    8 wavefronts on one group's keys)."""
    qb = {"fp8": 1, "bf16": 2, "f32": 4}[wl.q_dtype]
    per = padded_heads(wl.H) * wl.d * qb
    qw = 4 if (4 * per <= 32768 and wl.H % 4 == 0) else (2 if (2 * per <= 32768 and wl.H % 8 == 0) else 1)
    lens = [wl.chunk] * (wl.total_q // wl.chunk) if wl.chunk else [int(m) for m in wl.q_lens]
    groups = sum((m + qw - 1) // qw for m in lens)
    tiles = sum(((m + qw - 1) // qw + 7) // 8 for m in lens if m > 0)
    return tiles > 0 and 2 * groups >= 8 * tiles


def kernel_name(pass_name, wl):
    """Name of the kernel instantiation a pass launches, as profilers print it."""
    c = COMBO_ID[(wl.q_dtype, wl.k_dtype)]
    H = padded_heads(wl.H)
    if pass_name in ROLE_ID:
        if not uses_tiles(wl):
            return f"score_split_kernel<{c}, {H}, {wl.d}, {ROLE_ID[pass_name]}>"
        if pass_name == "score_survivor_lists":
            return f"score_list_kernel<{c}, {H}, {wl.d}, {ROLE_ID[pass_name]}>"
        paged = "true" if wl.page_table is not None else "false"
        return f"score_tiled_kernel<{c}, {H}, {wl.d}, {ROLE_ID[pass_name]}, {paged}>"
    return {"plan": "plan_kernel", "bound": "bound_kernel", "compact": "compact_kernel",
            "key_norms": "key_norm_kernel", "select_seed": "select_kernel", "select_final": "select_kernel",
            "prep": "qbar_kernel", "seed_extra": "seed_union_kernel"}.get(pass_name, pass_name)


def bound_bytes(wl, keys_streamed):
    """Algorithmic HBM bytes of the bound pass: each key row it streams (once
    per query tile that shares an LDS key tile, or once per query group in the
    one-wavefront-per-group kernel) plus that key's scale and norm (8 B).
    Groups the plan marks hopeless stream nothing and count nothing."""
    kb = {"fp8": 1, "bf16": 2, "f32": 4}[wl.k_dtype] * wl.d + 8
    return keys_streamed * kb


def sources_digest():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kname, workload):
    """HBM bytes per launch of `kname` from the committed counter summary, or
    None if there is none for this kernel and workload or the sources changed."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    for rec in (t if isinstance(t, list) else [t]):
        if rec.get("kernel") == kname and rec.get("workload") == workload and rec.get("sources_sha256") == sources_digest():
            return rec.get("bytes_per_launch")
    return None


def build_calls(wl, inp):
    from exact_top_token_amd.runner import slice_chunk

    if wl.chunk > 0:
        return [(c["q0"], slice_chunk(inp, c["q0"], c["q_len"], c["kv_len"])) for c in wl.chunk_calls()]
    return [(0, inp)]


def cpu_baseline(wl, budget_s: float = 20.0):
    """The oracle (float64 dense scores + full sort) on a bounded sample of queries."""
    import numpy as np

    from oracle import indexer

    blas = []
    try:
        from threadpoolctl import threadpool_info

        pools = threadpool_info()
        cores = max([int(i.get("num_threads", 1)) for i in pools] or [os.cpu_count() or 1])
        blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('user_api')}, {i.get('num_threads')} threads)"
                for i in pools]
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    _, pos = indexer.query_positions(wl)
    order = np.argsort(-pos, kind="stable")        # the longest queries: the last chunk
    done, pairs, t0 = 0, 0, time.perf_counter()
    rows = []
    while time.perf_counter() - t0 < budget_s and done < len(order):
        r = int(order[done])
        indexer.topk_rows(wl, [r], return_scores=False)
        pairs += int(pos[r]) + 1
        rows.append(r)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": pairs / dt, "unit": "scores/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model, "cpus_visible": os.cpu_count(), "blas": blas,
            "sample": f"{done} queries of the last chunk (positions {int(pos[rows[-1]])}..{int(pos[rows[0]])}), "
                      f"{pairs} causal pairs, float64 dense scores + full sort, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long_prefill_128k")
    ap.add_argument("--L", type=int, default=0, help="override the context length (exploration only)")
    ap.add_argument("--chunk", type=int, default=0, help="query chunk per call, where the recipe takes one")
    ap.add_argument("--q-len", type=int, default=0, help="new queries of a chunk recipe (million_chunk)")
    ap.add_argument("--H", type=int, default=0, help="indexer heads (default: the recipe's)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--paths", default="dosa,dsa")
    ap.add_argument("--buffer-cap", type=int, default=0, help="candidate buffer entries per query (0 = default)")
    ap.add_argument("--key-splits", type=int, default=0)
    ap.add_argument("--flags", type=lambda x: int(x, 0), default=0, help="DOSA_* flags OR-ed into the config")
    ap.add_argument("--batch", type=int, default=0, help="sequences of a decode recipe (default: the recipe's)")
    ap.add_argument("--kv-min", type=int, default=0, help="shortest cache of a decode recipe")
    ap.add_argument("--kv-max", type=int, default=0, help="longest cache of a decode recipe")
    ap.add_argument("--seeds", choices=["none", "prev"], default="none",
                    help="decode recipes: 'prev' passes each query the previous decode step's Top-K (the dense "
                         "path's, for the queries q_per_seq positions earlier) as extra seed keys")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain copy of this size first (calibrates HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (queries shard across GPUs "
              "with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_top_token_amd as E
    import synth
    from exact_top_token_amd.runner import to_device

    E.lib()
    kw = {"L": a.L} if a.L else {}
    if a.chunk:
        kw["chunk"] = a.chunk
    if a.q_len:
        kw["q_len"] = a.q_len
    if a.H:
        kw["H"] = a.H
    for k_, v_ in (("batch", a.batch), ("kv_min", a.kv_min), ("kv_max", a.kv_max)):
        if v_:
            kw[k_] = v_
    t0 = time.perf_counter()
    prev = None
    if a.seeds == "prev":
        # two consecutive decode steps: the batch's sequences with twice the queries, split
        if a.workload not in ("decode_mtp", "correlated_decode"):
            sys.exit("--seeds prev needs a decode recipe (decode_mtp or correlated_decode)")
        kw["q_per_seq"] = 4
        prev, wl = synth.split_decode_steps(synth.make_workload(a.workload, **kw), 2)
    else:
        wl = synth.make_workload(a.workload, **kw)
    log(f"generated {wl.name}: q {wl.q.shape} {wl.q_dtype}, k {wl.k.shape} {wl.k_dtype}, "
        f"{wl.pairs()} pairs in {time.perf_counter() - t0:.1f}s")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = to_device(wl, dev)
    calls = build_calls(wl, inp)
    if a.calib_copy_mib:
        # a plain copy kernel of known size: reads and writes calib_copy_mib MiB
        x = torch.ones(a.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.neg(x, out=y)
        torch.cuda.synchronize()
        del x, y
    K = wl.topk
    pairs = wl.pairs()
    results = {}
    outs = {}
    seed_t = None
    if prev is not None:
        from exact_top_token_amd.runner import Runner

        rp = Runner(to_device(prev, dev), "dsa", want_scores=False, device=dev)
        seed_t = rp()[0].clone()
        torch.cuda.synchronize()
        del rp
        log(f"previous decode step's Top-K as extra seeds: {tuple(seed_t.shape)}")
    for path in a.paths.split(","):
        cfg = E.default_config(K)
        if a.buffer_cap:
            cfg.buffer_cap = a.buffer_cap
        if a.key_splits:
            cfg.key_splits = a.key_splits
        cfg.flags |= a.flags
        if seed_t is not None and path == "dosa":
            cfg.seed_idx, cfg.seed_count = seed_t.data_ptr(), int(seed_t.shape[1])
        ws_bytes = max(E.workspace_size(c.q_lens, c.kv_lens, c.H, c.d, K, c.q_dtype, c.k_dtype,
                                        c.page_table is not None, path == "dsa", cfg) for _, c in calls)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        out_idx = torch.empty((wl.total_q, K), dtype=torch.int32, device=dev)
        stats = torch.zeros(len(E.STAT_FIELDS), dtype=torch.int64, device=dev)

        def step():
            for q0, c in calls:
                oi = out_idx[q0:q0 + c.total_q]
                if path == "dsa":
                    E.dsa_indexer_topk(c.q, c.q_dtype, c.q_scale, c.w, c.k, c.k_dtype, c.k_scale, c.q_lens,
                                       c.kv_lens, c.page_table, c.page_size, c.H, c.d, K, oi, None, ws,
                                       cfg=cfg, stats=stats)
                else:
                    E.dosa_indexer_topk(c.q, c.q_dtype, c.q_scale, c.w, c.k, c.k_dtype, c.k_scale, c.q_lens,
                                        c.kv_lens, c.page_table, c.page_size, c.H, c.d, K, oi, None, ws,
                                        cfg=cfg, stats=stats)

        for _ in range(a.warmup):
            step()
        torch.cuda.synchronize()
        stats.zero_()
        # Timed steps: HIP events on the stream around the K steps only.
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record()
        for _ in range(a.steps):
            step()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms = ev0.elapsed_time(ev1) / a.steps
        st = {k: int(v) // a.steps for k, v in zip(E.STAT_FIELDS, stats.cpu().numpy().tolist())}
        # The same K steps again with the library's per-launch HIP events (two
        # per pass and call, recorded on the launch stream), for the per-kernel
        # durations; the events themselves cost a few microseconds per launch,
        # so the step time above is taken without them.
        E.profile_begin()
        pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pe0.record()
        for _ in range(a.steps):
            step()
        pe1.record()
        torch.cuda.synchronize()
        kern = E.profile_end()
        ms_prof = pe0.elapsed_time(pe1) / a.steps
        results[path] = {"ms_per_step": ms, "ms_per_step_with_launch_events": ms_prof,
                         "wall_ms_per_step": 1e3 * wall / a.steps,
                         "scores_per_s": pairs / (ms / 1e3), "stats": st,
                         "kernel_ms_per_step": {k: v[1] / a.steps for k, v in kern.items()},
                         "launches_per_step": {k: v[0] // a.steps for k, v in kern.items()}}
        outs[path] = out_idx
        log(f"{path}: {ms:.2f} ms/step, {pairs / (ms / 1e3):.3e} scores/s, kernels "
            + ", ".join(f"{k} {v[1] / a.steps:.2f}" for k, v in kern.items()))
        del ws
    same = None
    if "dosa" in outs and "dsa" in outs:
        a_, b_ = outs["dosa"], outs["dsa"]
        same = True
        for r0 in range(0, wl.total_q, 8192):
            x = torch.sort(a_[r0:r0 + 8192], dim=1).values
            y = torch.sort(b_[r0:r0 + 8192], dim=1).values
            same = same and bool(torch.equal(x, y))
        log(f"pruned path selection identical to dense path: {same}")

    main_path = "dosa" if "dosa" in results else "dsa"
    R = results[main_path]
    st = R["stats"]
    flop_pair = 2 * wl.H * wl.d
    # dominant kernel of the main path, by time
    kern = R["kernel_ms_per_step"]
    dom = max(kern, key=kern.get)
    launches = max(R["launches_per_step"].get(dom, 1), 1)
    avg_ms = kern[dom] / launches
    kname = kernel_name(dom, wl)
    if dom in ROLE_ID:
        units = {"score_seed": st["pairs_seed"],
                 "score_survivor_tiles": st["pairs_scored"] - st["pairs_scored_list"],
                 "score_survivor_lists": st["pairs_scored_list"], "score_dense": st["pairs_scored"]}[dom]
        per_launch = units * flop_pair / launches
        mpeak = PEAK_TFLOPS[wl.q_dtype if wl.q_dtype == wl.k_dtype else "bf16"]
        roof = {"kernel": kname, "bound": "mfma", "achieved": per_launch / (avg_ms / 1e3) / 1e12,
                "peak": mpeak, "unit": "TFLOP/s", "flop_per_launch": per_launch}
        if not uses_tiles(wl):
            # decode-like batches: a key row read from HBM serves one query group
            # (flop per byte below the MFMA ridge), so the key stream is the roof:
            # bytes = (query, key) pairs / queries per group x (row + scale bytes)
            kb = {"fp8": 1, "bf16": 2, "f32": 4}[wl.k_dtype]
            qpg = max(1.0, wl.total_q / max(1, sum((int(m) + queries_per_group(wl) - 1) // queries_per_group(wl)
                                                   for m in wl.q_lens)))
            row = wl.d * kb + (4 if wl.k_dtype == "fp8" else 0)
            bytes_launch = units / qpg * row / launches
            roof = {"kernel": kname, "bound": "hbm", "achieved": bytes_launch / (avg_ms / 1e3) / 1e9,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "bytes_per_launch": bytes_launch,
                    "mfma_frac": per_launch / (avg_ms / 1e3) / 1e12 / mpeak}
    elif dom == "bound":
        per_launch = bound_bytes(wl, st["keys_streamed"]) / launches
        roof = {"kernel": kname, "bound": "hbm", "achieved": per_launch / (avg_ms / 1e3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "bytes_per_launch": per_launch}
    else:
        roof = {"kernel": kname, "bound": "alu", "achieved": None, "peak": None, "unit": None}
    if roof.get("achieved") is not None:
        roof["frac"] = roof["achieved"] / roof["peak"]
    roof["launches_per_step"] = launches
    roof["avg_launch_ms"] = avg_ms
    roof["traffic"] = measured_traffic(kname, wl.name)
    bound_ms = kern.get("bound", 0.0)
    bound_line = None
    if bound_ms > 0 and st["pairs_bounded"] > 0 and st["keys_streamed"] == 0:
        bound_line = {"note": "the plan skipped every group: no keys were streamed"}
    elif bound_ms > 0 and st["keys_streamed"] > 0:
        bb = bound_bytes(wl, st["keys_streamed"])
        bound_line = {"kernel": "bound_tiled_kernel or bound_kernel", "bound": "hbm",
                      "achieved": bb / (bound_ms / 1e3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": bb / (bound_ms / 1e3) / 1e9 / PEAK_HBM_GBS, "bytes_per_step": bb,
                      "note": "bytes = key rows streamed (+8 B scale and norm each); the time is the whole pass, "
                              "including launches whose groups the plan skipped"}
    bounded = max(st["pairs_bounded"], 1)
    extra = {
        "dense_path_scores_per_s": results.get("dsa", {}).get("scores_per_s"),
        "dense_path_ms_per_step": results.get("dsa", {}).get("ms_per_step"),
        "speedup_vs_dense": (results["dsa"]["ms_per_step"] / results["dosa"]["ms_per_step"]
                             if "dsa" in results and "dosa" in results else None),
        "pct_filtered": 100.0 * (1.0 - st["pairs_survived"] / bounded) if st["pairs_bounded"] else 0.0,
        "pct_pairs_exactly_scored": 100.0 * (st["pairs_seed"] + st["pairs_scored"]) / max(pairs, 1),
        "selection_identical_to_dense": same,
        "bound_pass_roofline": bound_line,
        "ms_per_step_with_launch_events": {p: r["ms_per_step_with_launch_events"] for p, r in results.items()},
        "kernel_ms_per_step": {p: r["kernel_ms_per_step"] for p, r in results.items()},
        "stats_per_step": {p: r["stats"] for p, r in results.items()},
    }
    line = {
        "metric": "indexer dense-equiv query-key scores/s at 128K ctx; % filtered; HBM/MFMA roofline",
        "value": R["scores_per_s"],
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": R["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.q_dtype if wl.q_dtype == wl.k_dtype else f"{wl.q_dtype}x{wl.k_dtype}",
        "data": "synthetic",
        "config": {"workload": wl.name, "seq_len": int(max(wl.kv_lens)), "queries": wl.total_q,
                   "chunk": wl.chunk, "heads": wl.H, "head_dim": wl.d, "topk": K,
                   "pairs_per_step": pairs, "path": f"{main_path}_indexer_topk",
                   "recipe": wl.recipe, "extra_seeds": a.seeds},
        "roofline": roof,
        "cpu_baseline": None if a.no_cpu else cpu_baseline(wl, a.cpu_budget),
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
