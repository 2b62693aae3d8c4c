#!/usr/bin/env python3
"""Benchmark of RIPE verification attention on one MI355X.

One step = one verification round: ripe_verify_attn for every recurrent
layer of the workload (the D x R grid, or the WaveFront diagonal), with the
committed prefix already resident in HBM.  The default workload is the
long-context ragged batch (L = 1K-32K, 8 sequences, 32/8 heads, d = 128,
W = 64, D = 8, R = 32, 4 layers).  Steps rotate over several copies of the
cache so that consecutive reads of one copy are separated by more than the
256 MB Infinity Cache.  Each copy's round is captured once in a HIP graph;
the timed loop replays the graphs between two events.  Caches hold N(0, 1)
bf16 values drawn on the device (the parity tests use the seeded recipe).

Prints one JSON line: unique-KV GB/s (value), verified tokens/s, the roofline
of the verify launch (HBM bytes or matrix-core flops, whichever bounds the
workload), the comparison rounds the workloads are quoted with (the
Huginn-scale shape at W = 0, 8, 64, 1024; the GQA shape with the deepest
plane alone and with the full per-loop cache; the small shape in both
layouts), and the fp64 oracle timed on the host cores on a bounded sample
(whole layers) of the same workload, plus one layer of the Huginn-scale
workload on a single thread.

``--mode per-loop`` times the same step as a forward pass runs it, R calls of
the D rows of one loop per layer; ``--mode draft`` times the draft pass,
D x r_draft calls of one row each (block keys 0..j).  Their value is the sum
of every call's unique-KV bytes over the step time; ``bytes_vs_batched`` says
how many more bytes that is than the batched call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RIPE verify-attn unique-KV GB/s (% HBM peak) + verified tokens/s, L=1K–32K"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0     # MI355X dense bf16 matrix peak
MALL_BYTES = 256 << 20
CPU_SAMPLE_S = 10.0             # oracle layers are timed until this much CPU time is spent
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_traffic_counters.txt")
SPIN_CYCLES = 20_000_000        # a spinning kernel that covers the host's enqueue of timed launches
SPIN_CYCLES_PER_CALL = 300_000  # ... of one call (~60 us of host work, more under a profiler)
MAX_SEQUENCE_CALLS = 160        # calls timed back to back behind one spin
MAX_WARM_CALLS = 64             # untimed calls before them ...
WARM_MS = 25.0                  # ... worth this much GPU time where they are long


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ragged",
                    choices=["tiny", "huginn", "gqa", "ragged", "wave"])
    ap.add_argument("--window", type=int, default=None, help="W (default: the workload's)")
    ap.add_argument("--full", action="store_true", help="full per-loop cache (W = all)")
    ap.add_argument("--anchor", type=int, default=None)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--tuning", default=None, metavar="JSON",
                    help="fixed launch choices for every cache (fields of ripe_tuning), e.g. "
                         "'{\"keys_waves\": 8}'")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the comparison rounds (Huginn-scale windows, GQA deepest-only "
                         "and full cache, the small shape in both layouts)")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of graphs")
    ap.add_argument("--mode", default="batched", choices=["batched", "per-loop", "draft", "wavefront"],
                    help="call schedule: the D x R grid in one call per layer (batched), "
                         "R calls of D rows (per-loop), or the draft pass of D x r_draft "
                         "single-row calls (draft)")
    ap.add_argument("--draft-loops", type=int, default=4, help="r_draft of the draft pass")
    ap.add_argument("--draft-window", type=int, default=-1, metavar="W_D",
                    help="draft mode: windowed draft attention keeping the W_D committed "
                         "positions before each query and --sinks sink positions (-1: full)")
    ap.add_argument("--sinks", type=int, default=4, help="sink positions of a windowed draft")
    ap.add_argument("--accept", type=float, default=0.8,
                    help="wavefront: probability that a draft token is accepted (seeded)")
    ap.add_argument("--shared-kv", action="store_true",
                    help="wavefront: one KV plane shared by all loops")
    ap.add_argument("--capacity-gib", type=float, default=0.0, metavar="GIB",
                    help="fixed-memory mode: for a cache budget of GIB GiB, the batch each "
                         "layout holds (full, RIPE, deepest plane) and the verify throughput "
                         "measured at that batch")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


def key_range(L, i, r, R, window, anchor):
    """e_row: committed positions [0, e) are read at loop R, [e, L) at loop r."""
    t = L + i
    beta = t - window if anchor == 0 else L - window
    return L if r == R else min(max(beta, 0), L)


def unique_kv_bytes(wl, window, anchor, rows, lens, sink_window=None):
    """Distinct (position, loop) key and value vectors one layer's call reads
    (sink_window = (n_sink, w): a windowed draft's committed keys only)."""
    if sink_window is not None:
        return _unique_windowed(wl, window, anchor, rows, lens, *sink_window)
    R, H, d = wl.n_loops, wl.n_heads_kv, wl.head_dim
    total = 0
    for L in lens:
        e_min = {}      # loop r < R -> smallest first committed position read at r
        e_max_R = 0     # committed positions [0, e_max_R) read at loop R
        blk = {}        # loop -> largest block offset read at that loop
        for i, r in rows:
            e = key_range(L, i, r, R, window, anchor)
            e_max_R = max(e_max_R, e)
            if r < R and e < L:
                e_min[r] = min(e_min.get(r, L), e)
            blk[r] = max(blk.get(r, -1), i)
        total += e_max_R + sum(L - e for e in e_min.values()) + sum(i + 1 for i in blk.values())
    return total * 2 * H * d * 2


def _unique_windowed(wl, window, anchor, rows, lens, n_sink, w):
    import numpy as np
    R, H, d = wl.n_loops, wl.n_heads_kv, wl.head_dim
    total = 0
    for L in lens:
        planes = {}                      # loop -> positions read at that loop
        blk = {}
        for i, r in rows:
            e = key_range(L, i, r, R, window, anchor)
            keep = np.zeros(L, dtype=bool)
            keep[:min(n_sink, L)] = True
            keep[max(L + i - w, 0):] = True
            deep = planes.setdefault(R, np.zeros(L, dtype=bool))
            deep[:e] |= keep[:e]
            if e < L:
                mine = planes.setdefault(r, np.zeros(L, dtype=bool))
                mine[e:] |= keep[e:]
            blk[r] = max(blk.get(r, -1), i)
        total += sum(int(m.sum()) for m in planes.values()) + sum(i + 1 for i in blk.values())
    return total * 2 * H * d * 2


def flops(wl, rows, lens):
    """Q.K^T plus P.V: 4*d per (row, query head, attended key)."""
    keys = sum(L + i + 1 for L in lens for i, _ in rows)
    return 4 * wl.head_dim * wl.n_heads_q * keys


def src_digest():
    """Digest of the kernel sources (ties stored counter readings to a build)."""
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "self_speculative_verify_amd", "csrc")
    for name in sorted(os.listdir(cdir)):
        with open(os.path.join(cdir, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, digest):
    """HBM bytes per verify launch from the committed counter summary, or None
    when it is absent or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for ln in lines:
        parts = ln.split()
        if len(parts) >= 4 and parts[0] == "traffic" and parts[1] == workload and parts[2] == digest:
            return int(parts[3])
    return None


def time_append(wl, window, anchor, dev, n_rep):
    """ripe_append of the n_blk accepted tokens of every sequence (loop R to the
    deep rows, loops 1..R-1 to the rings, evicting the oldest window positions),
    one layer, n_rep appends in a row on a cache with room for them."""
    import torch
    import ripe_harness as H
    w = wl.replace(n_layers=1, capacity=max(wl.lens) + wl.n_blk * (n_rep + 1))
    cache = H.make_cache(w, device=dev, window=window, anchor=anchor)
    fill_random(cache, w, window, dev, seed=4321)
    D, R, B = w.n_blk, w.n_loops, w.batch
    blk = (B, R, w.n_heads_kv, D, w.head_dim)
    tbk = torch.randn(blk, device=dev).to(torch.bfloat16)
    tbv = torch.randn(blk, device=dev).to(torch.bfloat16)
    args = (tbk[:, R - 1, :, :D], tbv[:, R - 1, :, :D],
            tbk[:, :R - 1, :, :D] if R > 1 else None, tbv[:, :R - 1, :, :D] if R > 1 else None)
    torch.cuda.synchronize()
    torch.cuda._sleep(SPIN_CYCLES)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
    evs[0].record()
    for k in range(n_rep):
        cache.append(0, [D] * B, *args)
        evs[k + 1].record()
    torch.cuda.synchronize()
    us = sum(evs[k].elapsed_time(evs[k + 1]) for k in range(n_rep)) / n_rep * 1e3
    n_win = min(D, cache.cfg.window, w.capacity) if R > 1 else 0
    moved = B * w.n_heads_kv * w.head_dim * 2 * 2 * (D + (R - 1) * n_win)   # K and V, bf16
    del cache
    return {"us_per_layer": round(us, 3), "bytes_read": moved, "bytes_written": moved,
            "GB/s": round(2 * moved / (us * 1e-6) / 1e9, 2), "tokens_per_seq": D}


def cpu_baseline(wl, window, anchor, calls, sw=None, max_layers=None):
    """The fp64 oracle on whole layers of the workload (the same calls, every
    head, the seeded inputs of ``synth``), layer after layer until
    CPU_SAMPLE_S seconds are spent (or max_layers layers)."""
    import numpy as np
    import oracle
    spent, u, n_layers = 0.0, 0, 0
    rows = [x for c in calls for x in c.rows]
    for layer in range(wl.n_layers):
        oc = oracle.prefix_cache(wl, layers=[layer], anchor=anchor, window=window)
        q = wl.queries(layer)
        bk, bv = wl.block(layer)
        for c in calls:
            qc = np.ascontiguousarray(q[:, [wl.rows.index(x) for x in c.rows]])
            t0 = time.perf_counter()
            if sw is None:
                oc.verify(layer, c.rows, qc, bk, bv, c.n_blk)
            else:
                oc.draft(layer, c.rows, qc, bk, bv, c.n_blk, sw[0], sw[1])
            spent += time.perf_counter() - t0
            u += unique_kv_bytes(wl, window, anchor, c.rows, wl.lens, sw)
        n_layers += 1
        del oc
        if spent >= CPU_SAMPLE_S or (max_layers and n_layers >= max_layers):
            break
    rounds = n_layers / wl.n_layers
    return {"value": round(u / spent / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{n_layers} of {wl.n_layers} layers: {len(calls)} call(s), {len(rows)} rows x {wl.n_heads_q} "
                      f"heads x {wl.batch} sequences, {spent:.1f} s",
            "tokens_per_s": round(wl.batch * len({i for i, _ in rows}) * rounds / spent, 3)}


def capacity_bench(args):
    """Batch capacity at fixed memory, fed with measured verify times.

    For a cache budget, each layout (the full per-loop cache, RIPE with window
    W, the deepest plane alone) holds ripe_max_batch sequences of the
    workload's shape; the verify call of one layer is timed at that batch
    (layers are alike, so a step of n_layers calls takes n_layers times as
    long) and the verified tokens per second of the attention alone are
    reported per layout.  Every sequence holds the same synthetic prefix
    (timing does not depend on the values; parity is covered by the tests).
    """
    import torch
    import ripe_harness as H
    from self_speculative_verify_amd import RipeCache, ripe
    from synth import WINDOW_FULL, named_workload

    wl = named_workload(args.workload)
    if args.workload == "wave" or len(set(wl.lens)) != 1:
        print("--capacity-gib needs a workload with one length and the D x R grid", file=sys.stderr)
        sys.exit(2)
    L, D, R = wl.lens[0], wl.n_blk, wl.n_loops
    w_ripe = args.window if args.window is not None else (wl.window if wl.window not in (0, WINDOW_FULL) else 64)
    budget = int(args.capacity_gib * (1 << 30))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows = wl.rows
    out = {}
    for name, W in (("full", WINDOW_FULL), ("ripe", w_ripe), ("deepest", 0)):
        cfg = ripe.config(wl.n_layers, R, wl.n_heads_q, wl.n_heads_kv, wl.head_dim, W, 1,
                          wl.capacity, wl.max_block, wl.anchor)
        B = ripe.ripe_max_batch(cfg, budget)
        if B < 1:
            out[name] = {"window": "full" if W == WINDOW_FULL else W, "batch": 0}
            continue
        print(f"capacity: {name} W={W} batch {B}", file=sys.stderr, flush=True)
        cfg.batch = B
        per_seq = (ripe.ripe_cache_bytes(cfg) - ripe.ripe_cache_bytes(
            ripe.config(wl.n_layers, R, wl.n_heads_q, wl.n_heads_kv, wl.head_dim, W, 1,
                        wl.capacity, wl.max_block, wl.anchor))) / max(B - 1, 1)
        cache = RipeCache(1, R, wl.n_heads_q, wl.n_heads_kv, wl.head_dim, W, B, wl.capacity,
                          wl.max_block, wl.anchor, device=dev)
        nw = 0 if R == 1 else min(L, cache.cfg.window, wl.capacity)
        dk, dv, wk, wv = wl.prefix(0, 0, n_win=nw)
        Hk, d = wl.n_heads_kv, wl.head_dim
        tk = H.to_dev(dk, dev).view(1, Hk, L, d).expand(B, Hk, L, d)
        tv = H.to_dev(dv, dev).view(1, Hk, L, d).expand(B, Hk, L, d)
        twk = twv = None
        if nw > 0:
            twk = H.to_dev(wk, dev).view(1, R - 1, Hk, nw, d).expand(B, R - 1, Hk, nw, d)
            twv = H.to_dev(wv, dev).view(1, R - 1, Hk, nw, d).expand(B, R - 1, Hk, nw, d)
        cache.append(0, [L] * B, tk, tv, twk, twv)
        del tk, tv, twk, twv
        q = torch.randn((B, len(rows), wl.n_heads_q, d), device=dev).to(torch.bfloat16)
        bk1, bv1 = wl.block(0)
        bk = H.to_dev(bk1[:1], dev).expand(B, *bk1.shape[1:])
        bv = H.to_dev(bv1[:1], dev).expand(B, *bv1.shape[1:])
        o = torch.empty((B, len(rows), wl.n_heads_q, d), device=dev)
        lse = torch.empty((B, len(rows), wl.n_heads_q), device=dev)
        for _ in range(max(2, args.warmup // 2)):
            cache.verify(0, rows, q, bk, bv, D, out=o, lse=lse)
        torch.cuda.synchronize()
        n = max(3, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            cache.verify(0, rows, q, bk, bv, D, out=o, lse=lse)
        e1.record()
        torch.cuda.synchronize()
        t_layer = e0.elapsed_time(e1) / n / 1e3
        u = unique_kv_bytes(wl, W, wl.anchor, rows, [L] * B)
        out[name] = {"window": "full" if W == WINDOW_FULL else W, "batch": B,
                     "cache_bytes": int(ripe.ripe_cache_bytes(cfg)),
                     "bytes_per_sequence": int(per_seq),
                     "us_per_layer": round(t_layer * 1e6, 2),
                     "GB/s": round(u / t_layer / 1e9, 1),
                     "tokens_per_s": round(B * D / (wl.n_layers * t_layer), 1)}
        del cache, q, o, lse, bk, bv
        torch.cuda.empty_cache()
    full_tps = out["full"].get("tokens_per_s") or None
    res = {
        "metric": "verified tokens/s of the attention at fixed cache memory (batch = what fits)",
        "value": out["ripe"].get("tokens_per_s", 0.0), "unit": "tokens/s", "n_gpus": 1,
        "steps": max(3, args.steps // 2), "warmup": max(2, args.warmup // 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "budget_gib": args.capacity_gib, "layers": wl.n_layers,
                   "loops": R, "heads_q": wl.n_heads_q, "heads_kv": wl.n_heads_kv,
                   "head_dim": wl.head_dim, "context": L, "block": D, "timed_layers": 1},
        "layouts": out,
        "ripe_vs_full": round(out["ripe"]["tokens_per_s"] / full_tps, 3) if full_tps and "tokens_per_s" in out["ripe"] else None,
        "deepest_vs_full": round(out["deepest"]["tokens_per_s"] / full_tps, 3) if full_tps and "tokens_per_s" in out["deepest"] else None,
    }
    print(json.dumps(res), flush=True)


def wavefront_bench(args):
    """WaveFront decoding of one sequence: every call verifies the positions in
    flight (one row each, at its own loop) in each layer; a position that
    reaches full depth is appended to every layer's cache; drafts are accepted
    with a seeded probability.  Timed: `steps` calls (at least 16R) after
    `warmup` calls, attention and commit appends only (the model's planes are
    not written; values do not change the timing).  The autoregressive
    baseline runs R single-row calls per token."""
    import numpy as np
    import torch
    import ripe_harness as H
    from self_speculative_verify_amd import RipeCache
    from self_speculative_verify_amd.wavefront import (WaveBuffer, WaveScheduler,
                                                       expected_calls_per_token, kernel_rows)
    from synth import named_workload

    wl = named_workload(args.workload)
    if wl.batch != 1:
        print("--mode wavefront runs one sequence; pick a workload with batch 1", file=sys.stderr)
        sys.exit(2)
    R, L = wl.n_loops, wl.lens[0]
    rd = min(args.draft_loops, R - 1)
    width = -(-R // rd)
    shared = args.shared_kv
    R_store = 1 if shared else R
    window = wl.window if args.window is None else args.window
    n_calls = max(args.steps, 16 * R)
    n_warm = max(args.warmup, 0)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.replace(n_loops=R_store, capacity=L + n_calls + n_warm + 2 * R + width, max_block=width)
    cache = RipeCache(w.n_layers, R_store, w.n_heads_q, w.n_heads_kv, w.head_dim, window, 1,
                      w.capacity, width, w.anchor, device=dev)
    H.load_prefix(cache, w, device=dev)
    buf = WaveBuffer(1, R_store, w.n_heads_kv, w.head_dim, slots=4 * width, device=dev)
    buf.k.normal_()
    buf.v.normal_()
    q = torch.randn((1, width, w.n_heads_q, w.head_dim), device=dev).to(torch.bfloat16)
    o = torch.empty((1, width, w.n_heads_q, w.head_dim), device=dev)
    lse = torch.empty((1, width, w.n_heads_q), device=dev)
    sched = WaveScheduler(R, rd, L)
    buf.push()
    rng = np.random.default_rng(np.random.SeedSequence([2024, int(args.accept * 1000)]))
    u_total = 0

    def call():
        nonlocal u_total
        rows = sched.rows()
        krows = kernel_rows(rows, shared)
        n = len(rows)
        bk, bv = buf.block()
        for layer in range(w.n_layers):
            cache.verify(layer, krows, q[:, :n], bk, bv, n, out=o[:, :n], lse=lse[:, :n])
        u_total += w.n_layers * unique_kv_bytes(w, window, w.anchor, krows, [sched.L])
        ev = sched.after_call(lambda: bool(rng.random() < args.accept))
        if ev.committed is not None:
            planes = buf.oldest_planes()
            for layer in range(w.n_layers):
                cache.append(layer, [1], *planes)
            buf.pop_oldest()
        if ev.rejected:
            buf.reset(0)
        while buf.count < sched.width:
            buf.push()

    for _ in range(n_warm):
        call()
    torch.cuda.synchronize()
    c0, k0 = sched.calls, sched.commits
    u_total = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_calls):
        call()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    commits = sched.commits - k0

    # autoregressive baseline: R single-row calls per token (every layer)
    n_tok = 2
    e0.record()
    for _ in range(n_tok):
        for r in range(1, R + 1):
            kr = kernel_rows([(0, r)], shared)
            for layer in range(w.n_layers):
                bk, bv = buf.block()
                cache.verify(layer, kr, q[:, :1], bk, bv, 1, out=o[:, :1], lse=lse[:, :1])
    e1.record()
    torch.cuda.synchronize()
    t_ar = e0.elapsed_time(e1) / 1e3 / n_tok
    tps = commits / t
    res = {
        "metric": "WaveFront decoding: committed tokens/s of the attention and commit appends",
        "value": round(tps, 1), "unit": "tokens/s", "n_gpus": 1, "steps": n_calls,
        "warmup": n_warm, "ms_per_step": round(t / n_calls * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "layers": w.n_layers, "loops": R, "draft_loops": rd,
                   "wave_width": width, "shared_kv": shared, "accept": args.accept,
                   "window": window, "heads_q": w.n_heads_q, "heads_kv": w.n_heads_kv,
                   "head_dim": w.head_dim, "context": L},
        "calls": n_calls, "commits": commits,
        "calls_per_token": round(n_calls / max(commits, 1), 3),
        "expected_calls_per_token": round(expected_calls_per_token(R, rd, args.accept), 3),
        "us_per_call": round(t / n_calls * 1e6, 2),
        "unique_kv_GB_per_s": round(u_total / t / 1e9, 1),
        "autoregressive_tokens_per_s": round(1 / t_ar, 1),
        "speedup_vs_autoregressive": round(tps * t_ar, 3),
    }
    print(json.dumps(res), flush=True)


def fill_random(cache, wl, window, dev, seed):
    """Append every sequence's committed prefix to every layer of `cache` with
    N(0, 1) bf16 keys and values drawn on the device (timing does not depend
    on the values; the parity tests use the seeded recipe of ``synth``)."""
    import torch
    R, H, d, B = wl.n_loops, wl.n_heads_kv, wl.head_dim, wl.batch
    wr = 0 if R == 1 else min(window, cache.cfg.capacity)
    T = max(wl.lens)
    U = min(T, wr)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    for layer in range(wl.n_layers):
        dk = torch.randn((B, H, T, d), generator=gen, device=dev).to(torch.bfloat16)
        dv = torch.randn((B, H, T, d), generator=gen, device=dev).to(torch.bfloat16)
        wk = wv = None
        if U > 0:
            wk = torch.randn((B, R - 1, H, U, d), generator=gen, device=dev).to(torch.bfloat16)
            wv = torch.randn((B, R - 1, H, U, d), generator=gen, device=dev).to(torch.bfloat16)
        cache.append(layer, wl.lens, dk, dv, wk, wv)
        del dk, dv, wk, wv


def build_setups(wl, window, anchor, calls, copies, dev):
    """`copies` caches of the workload (each with every layer), with the
    queries, draft-block planes and outputs of every call."""
    import torch
    import ripe_harness as H
    rows = wl.rows
    call_idx = [[rows.index(x) for x in c.rows] for c in calls]
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    setups = []
    for c in range(copies):
        cache = H.make_cache(wl, device=dev, window=window, anchor=anchor)
        fill_random(cache, wl, window, dev, seed=1000 + c)
        ins = []
        for layer in range(wl.n_layers):
            q = torch.randn((wl.batch, len(rows), wl.n_heads_q, wl.head_dim), generator=gen,
                            device=dev).to(torch.bfloat16)
            blk = (wl.batch, wl.n_loops, wl.n_heads_kv, wl.max_block, wl.head_dim)
            bk = torch.randn(blk, generator=gen, device=dev).to(torch.bfloat16)
            bv = torch.randn(blk, generator=gen, device=dev).to(torch.bfloat16)
            qs = [q if len(calls) == 1 else q[:, idx].contiguous() for idx in call_idx]
            ins.append((qs, bk, bv))
        outs = [[(torch.empty((wl.batch, len(c.rows), wl.n_heads_q, wl.head_dim), device=dev),
                  torch.empty((wl.batch, len(c.rows), wl.n_heads_q), device=dev)) for c in calls]
                for _ in range(wl.n_layers)]
        setups.append((cache, ins, outs))
    torch.cuda.synchronize()
    return setups


def round_runner(wl, calls, sw=None):
    """(run_call, run_round): one call of one layer on a cache copy, and a
    whole step's calls in the order a forward pass runs them."""
    def run_call(setup, k, layer):
        cache, ins, outs = setup
        qs, bk, bv = ins[layer]
        c = calls[k]
        if sw is not None:
            cache.draft(layer, c.rows, qs[k], bk, bv, c.n_blk, sw[0], sw[1], out=outs[layer][k][0],
                        lse=outs[layer][k][1])
        else:
            cache.verify(layer, c.rows, qs[k], bk, bv, c.n_blk, out=outs[layer][k][0],
                         lse=outs[layer][k][1])

    def run_round(setup):
        # the order a forward pass runs: call by call (loop by loop), each
        # through all layers
        for k in range(len(calls)):
            for layer in range(wl.n_layers):
                run_call(setup, k, layer)

    return run_call, run_round


def eager_step_ms(setups, wl, calls, steps, sw=None):
    """Mean step time (ms) with every call of the step issued from Python
    through the binding, no graph: the host work of the calls included.
    Rotates over the cache copies like the graph replays; a few untimed
    steps first."""
    import torch
    _, run_round = round_runner(wl, calls, sw)
    copies = len(setups)
    for k in range(min(steps, 3)):
        run_round(setups[k % copies])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        run_round(setups[k % copies])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / max(steps, 1)


def time_setups(setups, wl, calls, steps, warmup, eager=False, sw=None, n_rep=None):
    """Step time (ms; each copy's round replayed from a HIP graph, rotating
    over the copies), the time of each timed step, and the durations of
    single calls (ms), timed with events in one back-to-back sequence queued
    behind a spinning kernel so no host gap falls between them."""
    import torch
    copies = len(setups)
    run_call, run_round = round_runner(wl, calls, sw)

    for s in setups:            # eager warm-up (allocates workspaces outside capture)
        run_round(s)
    torch.cuda.synchronize()
    graphs = []
    if not eager:
        for s in setups:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_round(s)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(k):
        if eager:
            run_round(setups[k % copies])
        else:
            graphs[k % copies].replay()

    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record()
    for k in range(warmup):
        step(k)
    w1.record()
    torch.cuda.synchronize()
    # an event after every step, so the mean over the K steps and the spread
    # of single steps come from the same timed region; only where a step is
    # long enough that recording the events cannot make the host the bottleneck
    per_step = warmup > 0 and w0.elapsed_time(w1) / warmup >= 0.5
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step else 2)]
    marks[0].record()
    for k in range(steps):
        step(k)
        if per_step:
            marks[k + 1].record()
    if not per_step:
        marks[-1].record()
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[-1]) / max(steps, 1)
    step_ms = [marks[k].elapsed_time(marks[k + 1]) for k in range(steps)] if per_step else []
    del graphs

    if n_rep is None:
        n_rep = max(1, min(steps, 20 if len(calls) == 1 else 2))
    # n_rep rounds back to back in one sequence, as the timed steps run them,
    # after untimed calls worth WARM_MS of GPU time: the clock drops while the
    # GPU idles and takes ~20 ms of work to recover (a ragged call runs 720 us
    # right after an idle gap and 535 us once the clock has settled).  Calls
    # shorter than the host's enqueue of one (~0.2 ms) queue behind a spinning
    # kernel instead, so that no host gap falls between them.  Each call queues
    # two kernels and an event: the sequence stays well inside the hardware
    # queue, which would otherwise block the host and leave gaps.
    n_ev = len(calls) * wl.n_layers
    n_rep = max(1, min(n_rep, MAX_SEQUENCE_CALLS // n_ev))
    per_call = ms / n_ev
    n_warm = max(1, min(MAX_WARM_CALLS, math.ceil(WARM_MS / max(per_call, 1e-3))))
    total = n_rep * n_ev
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(total + 1)]
    if per_call < 0.2:
        torch.cuda._sleep(max(SPIN_CYCLES, SPIN_CYCLES_PER_CALL * (total + n_warm)))
    for j in range(n_warm):
        run_call(setups[-1], (j % n_ev) // wl.n_layers, j % wl.n_layers)
    evs[0].record()
    for k in range(n_rep):
        s = setups[k % copies]
        for j in range(n_ev):
            run_call(s, j // wl.n_layers, j % wl.n_layers)
            evs[k * n_ev + j + 1].record()
    if torch.cuda.current_stream().query():
        print("bench: the GPU ran out of queued work before the calls were enqueued; call times "
              "include host gaps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    launch_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(total)]
    return ms, launch_ms, step_ms


def spread(xs, digits=5):
    """Median, 10th and 90th percentile of a list of times."""
    v = sorted(xs)
    if not v:
        return None
    q = lambda f: v[min(len(v) - 1, max(0, int(round(f * (len(v) - 1)))))]
    return {"median": round(q(0.5), digits), "p10": round(q(0.1), digits), "p90": round(q(0.9), digits)}


def roofline_of(u_call, f_call, launch_s):
    """The binding roof of one call (HBM bytes or bf16 matrix flops) and the
    fraction of it the measured call duration reaches."""
    if u_call / (HBM_PEAK_GBS * 1e9) >= f_call / (MFMA_BF16_PEAK_TFS * 1e12):
        roof = {"bound": "hbm", "achieved": round(u_call / launch_s / 1e9, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(f_call / launch_s / 1e12, 2),
                "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    return roof


def copies_for(u_round):
    """Cache copies to rotate so that > 2x the Infinity Cache is read between
    two reads of one copy (at most 64: rounds that small are bound by launch
    latency, not by where their bytes come from)."""
    return min(64, max(2, 1 + math.ceil(2 * MALL_BYTES / max(u_round, 1))))


# The comparisons the metric's workloads are quoted with: the Huginn-scale
# shape at four windows, the GQA shape with the deepest plane alone and with
# the full per-loop cache, and the small shape in both layouts.
COMPARISONS = [("huginn", 0), ("huginn", 8), ("huginn", 64), ("huginn", 1024),
               ("gqa", 0), ("gqa", "full"), ("tiny", 16), ("tiny", "full")]


def comparisons(dev, steps, warmup):
    """One batched verify round of each comparison workload: per-call time,
    unique-KV GB/s, fraction of HBM and of the binding roof, tokens/s."""
    import torch
    from synth import WINDOW_FULL, named_workload
    from self_speculative_verify_amd import schedule
    out = {}
    for name, w in COMPARISONS:
        wl = named_workload(name)
        window = WINDOW_FULL if w == "full" else w
        calls = [schedule.Call(list(wl.rows), wl.n_blk)]
        u_call = unique_kv_bytes(wl, window, wl.anchor, wl.rows, wl.lens)
        f_call = flops(wl, wl.rows, wl.lens)
        copies = copies_for(u_call * wl.n_layers)
        print(f"bench: comparison {name} W={w} copies={copies}", file=sys.stderr, flush=True)
        setups = build_setups(wl, window, wl.anchor, calls, copies, dev)
        ms, launch_ms, _ = time_setups(setups, wl, calls, steps, warmup, n_rep=max(4, min(steps, 10)))
        del setups
        torch.cuda.empty_cache()
        launch_s = sum(launch_ms) / len(launch_ms) / 1e3
        roof = roofline_of(u_call, f_call, launch_s)
        out[f"{name}:W={w}"] = {
            "window": w, "us_per_call": round(launch_s * 1e6, 2), "ms_per_round": round(ms, 5),
            "unique_kv_bytes_per_call": u_call, "GB/s": round(u_call / launch_s / 1e9, 1),
            "hbm_frac": round(u_call / launch_s / 1e9 / HBM_PEAK_GBS, 4),
            "bound": roof["bound"], "frac_of_bound": roof["frac"],
            "tokens_per_s": round(wl.batch * wl.n_blk / (ms / 1e3), 1)}
    return out


def host_cpu():
    """CPU model and logical CPU count of the host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def single_thread_baseline():
    """The oracle on one thread: one layer of the Huginn-scale workload (the
    D x R grid, every head)."""
    import oracle
    from synth import named_workload
    from self_speculative_verify_amd import schedule
    wl = named_workload("huginn")
    n0 = oracle.threads()
    oracle.set_threads(1)
    try:
        r = cpu_baseline(wl, wl.window, wl.anchor, [schedule.Call(list(wl.rows), wl.n_blk)],
                         max_layers=1)
    finally:
        oracle.set_threads(n0)
    r["workload"] = "huginn"
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verification path is data-parallel over sequences and KV heads and "
              "needs no collective; run one process per GPU).", file=sys.stderr)
        sys.exit(2)
    if args.capacity_gib > 0:
        capacity_bench(args)
        return
    if args.mode == "wavefront":
        wavefront_bench(args)
        return
    import torch
    from synth import WINDOW_FULL, named_workload

    from self_speculative_verify_amd import schedule

    wl = named_workload(args.workload)
    window = WINDOW_FULL if args.full else (wl.window if args.window is None else args.window)
    anchor = wl.anchor if args.anchor is None else args.anchor
    rows = wl.rows
    if args.mode == "batched":
        calls = [schedule.Call(list(rows), wl.n_blk)]
    elif rows != schedule.batched_verify(wl.n_blk, wl.n_loops)[0].rows:
        print(f"--mode {args.mode} needs a workload that verifies the whole D x R grid",
              file=sys.stderr)
        sys.exit(2)
    elif args.mode == "per-loop":
        calls = schedule.per_loop_verify(wl.n_blk, wl.n_loops)
    else:
        calls = schedule.draft_pass(wl.n_blk, min(args.draft_loops, wl.n_loops))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.tuning:
        from self_speculative_verify_amd import cache as cache_mod
        cache_mod.DEFAULT_TUNING = json.loads(args.tuning)

    # algorithmic bytes and flops of one layer (all its calls)
    sw = (args.sinks, args.draft_window) if args.mode == "draft" and args.draft_window >= 0 else None
    u_calls = [unique_kv_bytes(wl, window, anchor, c.rows, wl.lens, sw) for c in calls]
    f_calls = [flops(wl, c.rows, wl.lens) for c in calls]
    u_layer, f_layer = sum(u_calls), sum(f_calls)
    u_round = u_layer * wl.n_layers
    copies = args.copies or copies_for(u_round)
    print(f"bench: {wl.name} W={window} anchor={anchor} copies={copies}", file=sys.stderr, flush=True)

    setups = build_setups(wl, window, anchor, calls, copies, dev)
    print("bench: caches built", file=sys.stderr, flush=True)
    ms, launch_ms, step_ms = time_setups(setups, wl, calls, args.steps, args.warmup, args.eager, sw)
    # the same steps issued eagerly (host work included), next to the graphs
    ms_eager = None if args.eager else eager_step_ms(setups, wl, calls, args.steps, sw)
    t = ms / 1e3
    launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    u_call, f_call = u_layer / len(calls), f_layer / len(calls)
    del setups
    torch.cuda.empty_cache()
    n_rep = max(1, min(args.steps, 20 if len(calls) == 1 else 2))
    append = time_append(wl, window, anchor, dev, n_rep)
    print("bench: timed", file=sys.stderr, flush=True)

    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # block positions verified (or, for the draft pass, drafted) per step
    n_tokens = wl.batch * len({i for i, _ in rows})
    gbs = u_round / t / 1e9
    digest = src_digest()
    traffic_key = args.workload if args.mode == "batched" else f"{args.workload}:{args.mode}"
    traffic = (stored_traffic(traffic_key, digest)
               if window == wl.window and anchor == wl.anchor else None)
    roof = roofline_of(u_call, f_call, launch_s)
    roof["traffic"] = traffic
    roof["launch_us"] = round(launch_s * 1e6, 3)
    roof["launch_us_spread"] = spread([x * 1e3 for x in launch_ms], 3)
    roof["algorithmic_bytes"] = round(u_call)
    roof["algorithmic_flops"] = round(f_call)

    comp = None
    if args.mode == "batched" and not args.no_compare and window == wl.window and anchor == wl.anchor:
        comp = comparisons(dev, max(5, min(args.steps, 20)), max(2, min(args.warmup, 5)))

    cpu = None
    if not args.no_cpu:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, window, anchor, calls, sw)
        model, ncpu = host_cpu()
        cpu["cpu_model"] = model
        cpu["host_cpus"] = ncpu
        if args.mode == "batched":
            cpu["single_thread"] = single_thread_baseline()
    u_batched = unique_kv_bytes(wl, window, anchor, rows, wl.lens)

    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "step_ms_spread": spread(step_ms),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.n_layers, "loops": wl.n_loops,
                   "heads_q": wl.n_heads_q, "heads_kv": wl.n_heads_kv, "head_dim": wl.head_dim,
                   "window": "full" if window == WINDOW_FULL else window, "block": wl.n_blk,
                   "batch": wl.batch, "lens": wl.lens if wl.batch <= 8 else "ragged",
                   "mode": args.mode, "calls_per_layer": len(calls),
                   **({"draft_loops": min(args.draft_loops, wl.n_loops)} if args.mode == "draft" else {}),
                   **({"draft_window": sw[1], "sinks": sw[0]} if sw is not None else {}),
                   "rows_per_call": len(rows) // len(calls),
                   "anchor": "query" if anchor == 0 else "cache",
                   "cache_copies": copies, "timing": "eager" if args.eager else "hip-graph",
                   "values": "N(0,1) bf16 drawn on the device",
                   **({"tuning": json.loads(args.tuning)} if args.tuning else {})},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(n_tokens / t, 1),
        "bytes_vs_batched": round(u_layer / u_batched, 4),
        "unique_kv_bytes_per_step": u_round,
        "flops_per_step": f_layer * wl.n_layers,
        "kernel_sources": digest,
        "roofline": roof,
        "host_inclusive": None if ms_eager is None else {
            "ms_per_step": round(ms_eager, 5), "GB/s": round(u_round / ms_eager / 1e6, 2),
            "tokens_per_s": round(n_tokens / ms_eager * 1e3, 1),
            "timing": "the step's calls issued from Python through the binding, no graph"},
        "append": append,
        "comparisons": comp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
