#!/usr/bin/env python3
"""Benchmark of RIPE verification attention on one MI355X.

One step = one verification round: ripe_verify_attn for every recurrent
layer of the workload (the D x R grid, or the WaveFront diagonal), with the
committed prefix already resident in HBM.  Steps rotate over several copies
of the cache so that consecutive reads of one copy are separated by more
than the 256 MB Infinity Cache.  Each copy's round is captured once in a HIP
graph; the timed loop replays the graphs between two events.

Prints one JSON line: unique-KV GB/s (value), verified tokens/s, the roofline
fraction of the verify kernel, and the fp64 oracle timed on the host cores
on a bounded sample (one layer) of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RIPE verify-attn unique-KV GB/s (% HBM peak) + verified tokens/s, L=1K–32K"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="huginn",
                    choices=["tiny", "huginn", "gqa", "ragged", "wave"])
    ap.add_argument("--window", type=int, default=None, help="W (default: the workload's)")
    ap.add_argument("--full", action="store_true", help="full per-loop cache (W = all)")
    ap.add_argument("--anchor", type=int, default=None)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of graphs")
    return ap.parse_args()


def unique_kv_bytes(wl, window, anchor, rows, lens):
    """Distinct (position, loop) key and value vectors one layer's call reads."""
    R, H, d = wl.n_loops, wl.n_heads_kv, wl.head_dim
    total = 0
    for L in lens:
        e_min = {}      # loop r < R -> smallest first committed position read at r
        e_max_R = 0     # committed positions [0, e_max_R) read at loop R
        blk = {}        # loop -> largest block offset read at that loop
        for i, r in rows:
            t = L + i
            beta = t - window if anchor == 0 else L - window
            e = L if r == R else min(max(beta, 0), L)
            e_max_R = max(e_max_R, e)
            if r < R and e < L:
                e_min[r] = min(e_min.get(r, L), e)
            blk[r] = max(blk.get(r, -1), i)
        n = e_max_R + sum(L - e for e in e_min.values()) + sum(i + 1 for i in blk.values())
        total += n
    return total * 2 * H * d * 2


def cpu_baseline(wl, window, anchor, rows):
    """The fp64 oracle on one layer of the workload (the same rows, every head)."""
    import numpy as np
    import oracle
    w = wl.replace(n_layers=1)
    oc = oracle.prefix_cache(w, layers=[0], anchor=anchor, window=window)
    q = w.queries(0)
    bk, bv = w.block(0)
    t0 = time.perf_counter()
    oc.verify(0, rows, q, bk, bv, w.n_blk)
    dt = time.perf_counter() - t0
    u = unique_kv_bytes(w, window, anchor, rows, w.lens)
    del np
    return {"value": round(u / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"one of {wl.n_layers} layers: all {len(rows)} rows x {wl.n_heads_q} heads x "
                      f"{wl.batch} sequences ({dt:.1f} s)",
            "tokens_per_s": round(wl.batch * len({i for i, _ in rows}) / (dt * wl.n_layers), 3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verification path is data-parallel over sequences and KV heads and "
              "needs no collective; run one process per GPU).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import ripe_harness as H
    from synth import WINDOW_FULL, named_workload

    wl = named_workload(args.workload)
    window = WINDOW_FULL if args.full else (wl.window if args.window is None else args.window)
    anchor = wl.anchor if args.anchor is None else args.anchor
    rows = wl.rows
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    u_layer = [unique_kv_bytes(wl, window, anchor, rows, wl.lens) for _ in range(wl.n_layers)]
    u_round = sum(u_layer)
    copies = args.copies or max(2, 1 + math.ceil(2 * MALL_BYTES / max(u_round, 1)))

    # build the caches (same contents in every copy; host data generated once)
    memo = {}
    orig_prefix = wl.prefix

    def prefix(layer, b, n_win=None):
        key = (layer, b, n_win)
        if key not in memo:
            memo[key] = orig_prefix(layer, b, n_win=n_win)
        return memo[key]
    wl.prefix = prefix
    setups = []
    for c in range(copies):
        cache = H.make_cache(wl, device=dev, window=window, anchor=anchor)
        H.load_prefix(cache, wl, device=dev)
        ins = [H.verify_inputs(wl, layer, device=dev) for layer in range(wl.n_layers)]
        outs = [(torch.empty((wl.batch, len(rows), wl.n_heads_q, wl.head_dim), device=dev),
                 torch.empty((wl.batch, len(rows), wl.n_heads_q), device=dev))
                for _ in range(wl.n_layers)]
        setups.append((cache, ins, outs))
    torch.cuda.synchronize()

    def run_round(setup):
        cache, ins, outs = setup
        for layer in range(wl.n_layers):
            q, bk, bv = ins[layer]
            cache.verify(layer, rows, q, bk, bv, wl.n_blk, out=outs[layer][0], lse=outs[layer][1])

    for s in setups:            # eager warm-up (allocates workspaces outside capture)
        run_round(s)
    torch.cuda.synchronize()
    graphs = []
    if not args.eager:
        for s in setups:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_round(s)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(k):
        if args.eager:
            run_round(setups[k % copies])
        else:
            graphs[k % copies].replay()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        step(k)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / max(args.steps, 1)
    t = ms / 1e3
    n_verified = wl.batch * len({i for i, _ in rows})   # draft positions verified per step
    gbs = u_round / t / 1e9
    launch_s = t / wl.n_layers        # one verify launch per layer per step
    achieved = (u_round / wl.n_layers) / launch_s / 1e9

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, window, anchor, rows)

    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.n_layers, "loops": wl.n_loops,
                   "heads_q": wl.n_heads_q, "heads_kv": wl.n_heads_kv, "head_dim": wl.head_dim,
                   "window": "full" if window == WINDOW_FULL else window, "block": wl.n_blk,
                   "batch": wl.batch, "lens": wl.lens if wl.batch <= 8 else "ragged",
                   "rows_per_call": len(rows), "anchor": "query" if anchor == 0 else "cache",
                   "cache_copies": copies, "timing": "eager" if args.eager else "hip-graph"},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(n_verified / t, 1),
        "unique_kv_bytes_per_step": u_round,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    del np
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
