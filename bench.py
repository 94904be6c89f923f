#!/usr/bin/env python3
"""Benchmark of the STA forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p]

One step is one pass of the whole hot path over one batch of synthetic
input: the STA forward over Q, K, V in natural [B, heads, T, H, W, D] order
(the tile-major permutation is applied inside the kernel through its row
tables) producing O in the same order.  Inputs are resident in HBM before
the timed region.  Printed: one JSON line with the achieved TFLOP/s
(FLOPs of the attended tile pairs only), the forward kernel's roofline
position, and the CPU oracle timed on a bounded sample of the same workload.
Context lines (not the metric): the explicit reorder -> tile-major forward ->
unreorder path, and the same kernel with a full window (dense attention).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

METRIC = "STA fwd ms + achieved TFLOP/s (MFMA util) at 30×48×80 tok, 24h, d128 bf16"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) MFMA, published
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed calls (default 50, more for calls under 5 ms: at least 0.25 s of them; "
                         "3 for the window search, whose sweep takes seconds)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed calls first (default 10, more for calls under 10 ms: at least 0.1 s "
                         "of them, so that the clock has settled; 1 for search)")
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--pass", dest="which", choices=["forward", "backward", "search", "swa"],
                    default="forward",
                    help="forward (the metric line), backward (delta + dQ + dK/dV kernels), "
                         "search (per-head window search over the default candidates) or swa "
                         "(token-wise sliding window attention with the same keys per query, "
                         "against STA on the same inputs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (4 times); "
                         "used to calibrate HBM traffic counters")
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "profiles", "traffic.json"))
    args = ap.parse_args()
    search = args.which == "search"
    args.auto_steps, args.auto_warmup = args.steps is None, args.warmup is None
    if args.steps is None:
        args.steps = 3 if search else 50
    if args.warmup is None:
        args.warmup = 1 if search else 10
    return args


def fit_counts(args, fn, stream):
    """Default call counts for short calls: warm up for at least 0.1 s and
    time at least 0.25 s of calls (10 and 50 at least; flags given on the
    command line are kept)."""
    import math
    import torch
    if not (args.auto_steps or args.auto_warmup):
        return
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = max(e0.elapsed_time(e1), 1e-3)
    if args.auto_warmup:
        args.warmup = min(20000, max(args.warmup, math.ceil(100.0 / ms)))
    if args.auto_steps:
        args.steps = min(20000, max(args.steps, math.ceil(250.0 / ms)))


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call_ms(fn, calls, stream):
    """Each call bracketed by its own pair of events (after the timed
    region): median, min and max milliseconds per call."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return {"calls": calls, "median": round(t[len(t) // 2], 4), "min": round(t[0], 4), "max": round(t[-1], 4)}


def sdpa_dense(q, k, v, scale, stream, ms_sta):
    """torch's scaled_dot_product_attention on the whole sequence (dense),
    restricted to its flash backend so that it never takes the math path;
    a library kernel, reported for context."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    B, Hh = q.shape[0], q.shape[1]
    qs, ks, vs = (x.reshape(B, Hh, -1, x.shape[-1]) for x in (q, k, v))
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            f = lambda: torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=scale)
            ms = timed(f, 3, 1, stream)
    except RuntimeError as e:
        return {"skipped": str(e).splitlines()[0][:160]}
    n = qs.shape[2]
    flops = 4.0 * B * Hh * n * n * qs.shape[-1]
    return {"backend": "torch SDPA, flash backend (library kernel)", "ms": round(ms, 3),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "sta_speedup": round(ms / ms_sta, 2)}


def cpu_baseline(w, q, k, v, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample: query tiles of head 0
    (then 1, ...) until about budget_s seconds of CPU work."""
    import numpy as np
    from oracle import sta_oracle as O
    from sliding_tile_attention_sta_amd.synthetic import sample_query_tiles
    threads = _threads()
    grid = O.tile_grid(w.video, w.tile)
    V = w.tile[0] * w.tile[1] * w.tile[2]
    done_tiles, flops, t_used = 0, 0.0, 0.0
    h = 0
    while t_used < budget_s and h < w.heads:
        qh, kh, vh = (x[:, h:h + 1].float().cpu().numpy() for x in (q, k, v))
        we = O.effective_window(w.windows[h], grid)
        for c in sample_query_tiles(w, h):
            t0 = time.perf_counter()
            O.sta_forward_query_tiles(qh, kh, vh, w.tile, w.windows[h], 0, [c], scale=w.scale)
            t_used += time.perf_counter() - t0
            done_tiles += 1
            flops += 4.0 * V * V * w.head_dim * we[0] * we[1] * we[2]
            if t_used >= budget_s:
                break
        h += 1
    full_s = t_used * O.sta_flops(w.video, w.tile, w.windows, w.head_dim, w.batch) / flops
    if done_tiles == w.heads * sum(1 for _ in sample_query_tiles(w, 0)) and \
            all(len(list(sample_query_tiles(w, x))) == grid[0] * grid[1] * grid[2] for x in range(w.heads)):
        sample = (f"every query tile of every head of the {w.name} workload ({done_tiles}: the whole "
                  f"call), float64 numpy, {t_used:.2f} s")
    else:
        sample = (f"{done_tiles} query tiles (heads 0..{h - 1}) of the {w.name} workload, "
                  f"float64 numpy, {t_used:.1f} s; a full call extrapolates to {full_s:.0f} s")
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": sample,
        "seconds": t_used,
        "cpu_model": _cpu_model(),
    }


def _affinity():
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _threads():
    """Host threads the oracle's numpy products can use: the BLAS thread
    pool, bounded by the CPUs this process may run on."""
    try:
        import numpy  # noqa: F401  (loads the BLAS whose pool is read)
        from threadpoolctl import threadpool_info
        blas = int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        blas = _affinity()
    return min(blas, _affinity())


def _timed_tiles(w, heads_tiles, fn, flops_per_tile, budget_s):
    """Run fn(head, tile) over (head, tile) pairs until budget_s seconds of
    CPU work; returns (tiles done, FLOPs, seconds, last head)."""
    done, flops, t_used, last = 0, 0.0, 0.0, 0
    for h, c in heads_tiles:
        t0 = time.perf_counter()
        fn(h, c)
        t_used += time.perf_counter() - t0
        done += 1
        flops += flops_per_tile(h)
        last = h
        if t_used >= budget_s:
            break
    return done, flops, t_used, last


def cpu_baseline_bwd(w, q, k, v, g, budget_s=10.0):
    """The backward oracle on a bounded sample: dq and lse of query tiles of
    head 0, 1, ... (each call forms every gradient product of its tile's
    window pairs: 2.5x the forward's FLOPs per pair, counted as such)."""
    from oracle import sta_oracle as O
    from oracle import sta_oracle_bwd as OB
    from sliding_tile_attention_sta_amd.synthetic import sample_query_tiles
    grid = O.tile_grid(w.video, w.tile)
    V = w.tile[0] * w.tile[1] * w.tile[2]
    cache = {}

    def heads_tiles():
        for h in range(w.heads):
            for c in sample_query_tiles(w, h):
                yield h, c

    def fn(h, c):
        if h not in cache:
            cache.clear()
            cache[h] = [x[:, h:h + 1].float().cpu().numpy() for x in (q, k, v, g)]
        OB.sta_backward_query_tiles(*cache[h], w.tile, w.windows[h], 0, [c], scale=w.scale)

    def fl(h):
        we = O.effective_window(w.windows[h], grid)
        return 2.5 * 4.0 * V * V * w.head_dim * we[0] * we[1] * we[2]

    done, flops, t_used, last = _timed_tiles(w, heads_tiles(), fn, fl, budget_s)
    full_s = t_used * 2.5 * O.sta_flops(w.video, w.tile, w.windows, w.head_dim, w.batch) / flops
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{done} query tiles (heads 0..{last}) of the {w.name} workload through the "
                      f"backward oracle, float64 numpy, {t_used:.1f} s; a full backward extrapolates "
                      f"to {full_s:.0f} s",
            "seconds": t_used, "cpu_model": _cpu_model()}


def cpu_baseline_swa(w, q, k, v, toks, budget_s=10.0):
    """The token-wise SWA oracle on a bounded sample of query tiles."""
    from oracle import sta_oracle_swa as OS
    from sliding_tile_attention_sta_amd.synthetic import sample_query_tiles
    V = w.tile[0] * w.tile[1] * w.tile[2]
    cache = {}

    def heads_tiles():
        for h in range(w.heads):
            for c in sample_query_tiles(w, h):
                yield h, c

    def fn(h, c):
        if h not in cache:
            cache.clear()
            cache[h] = [x[:, h:h + 1].float().cpu().numpy() for x in (q, k, v)]
        OS.swa_forward_query_tiles(*cache[h], w.tile, toks[h], 0, [c], scale=w.scale)

    def fl(h):
        keys = 1
        for a, e in zip(toks[h], w.video):
            keys *= min(a, e)
        return 4.0 * V * keys * w.head_dim

    done, flops, t_used, last = _timed_tiles(w, heads_tiles(), fn, fl, budget_s)
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s (permitted pairs)", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{done} query tiles (heads 0..{last}) of the {w.name} workload through the "
                      f"token-wise SWA oracle, float64 numpy, {t_used:.1f} s",
            "seconds": t_used, "cpu_model": _cpu_model()}


def _cpu_model():
    """Model name, family / model / stepping and the CPUs this process may
    use, from /proc/cpuinfo and the scheduler's affinity mask."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if fields:
                        break      # the first processor's block is enough
                    continue
                key, val = (x.strip() for x in line.split(":", 1))
                fields.setdefault(key, val)
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{name} ({ids}; {_affinity()} CPUs in this process's affinity mask)" if ids else \
        f"{name} ({_affinity()} CPUs in this process's affinity mask)"


def _build_flags(source):
    """The compiler flags of one HIP source (include paths left out: they
    name the checkout's location)."""
    from sliding_tile_attention_sta_amd import build as B
    flags = [f for i, f in enumerate(B.HIP_FLAGS) if f != "-I" and (i == 0 or B.HIP_FLAGS[i - 1] != "-I")]
    return flags + list(B.HIP_EXTRA.get(source, []))


def _measured_traffic(path, source, workload, key):
    """HBM bytes from a committed rocprofv3 counter summary, used only while
    the kernel source hashes to the one measured and is built with the same
    flags (else None)."""
    try:
        with open(path) as f:
            t = json.load(f)
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sliding_tile_attention_sta_amd", "csrc", source)
        with open(src, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if t.get("workload") == workload and t.get("kernel_source_sha256") == digest \
            and t.get("kernel_build_flags") == _build_flags(source):
        return t.get(key)
    return None


def backward(args, w, plan, q, k, v, stream):
    """One step = the STA backward call (delta, dQ and dK/dV kernels) for
    the forward's output and row log-sum-exp, computed once beforehand."""
    import torch
    from sliding_tile_attention_sta_amd import api
    from sliding_tile_attention_sta_amd.synthetic import make_grad_out

    g = make_grad_out(w, q.device)
    out, lse = api.sta_forward_plan(plan, q, k, v, scale=w.scale, out_dtype=torch.float32, lse=True)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    delta = torch.empty_like(lse)

    def step():
        api.sta_backward_plan(plan, q, k, v, out, g, lse, scale=w.scale, dq=dq, dk=dk, dv=dv,
                              delta=delta, stream=stream)

    fit_counts(args, step, stream)
    ms = timed(step, args.steps, args.warmup, stream)
    fwd_flops = plan.flops
    # Algorithmic backward FLOPs: five products per attended tile pair
    # (Q K^T recomputed, dO V^T, P^T dO, dS K, dS^T Q), 2.5x the forward's.
    # The two kernels execute seven (dQ recomputes Q K^T and dO V^T).
    flops = 2.5 * fwd_flops
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None if args.no_cpu_baseline else cpu_baseline_bwd(w, q, k, v, g)
    traffic = _measured_traffic(os.path.join(os.path.dirname(args.traffic_json), "traffic_bwd.json"),
                                "sta_backward.hip", w.name, "bytes_per_call")
    return {
        "cpu_baseline": cpu,
        "metric": "STA bwd ms + achieved TFLOP/s (algorithmic, 2.5x forward FLOPs)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.name, "video": list(w.video), "tile": list(w.tile),
                   "windows": sorted({tuple(x) for x in w.windows}), "heads": w.heads,
                   "head_dim": w.head_dim, "batch": w.batch, "layout": "natural",
                   "in_dtype": "bf16", "grad_dtype": "f32",
                   "products": "fp16 MFMA (bf16 for the dQ kernel's dO V^T), fp32 accumulate", "flops_per_step": flops,
                   "executed_flops_per_step": 3.5 * fwd_flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per call (HBM, FETCH_SIZE + WRITE_SIZE of the three kernels, copy-calibrated)",
                     "kernel": "whole backward call (delta + dQ + dK/dV)"},
    }


def search(args, w, stream):
    """One step = one sweep of the per-head window search over the default
    candidates of the workload's grid, on a locality calibration input of
    the workload's shape: head h has length scale l_h = 4 * 2^(h mod 6)
    tokens, i.e. attends to a Gaussian neighbourhood about l_h / 4 = 1 to 32
    tokens wide.  The sweep runs the forward once with
    the full window and once per candidate, plus the error reduction, and
    synchronises once per candidate."""
    import torch
    from sliding_tile_attention_sta_amd import api
    from sliding_tile_attention_sta_amd.synthetic import make_local_qkv

    lengths = [4.0 * 2 ** (h % 6) for h in range(w.heads)]
    q, k, v = make_local_qkv(w.video, lengths, w.head_dim, batch=w.batch, sharpness=16.0,
                             seed=w.seed + 900, dtype=torch.bfloat16, device="cuda:0")
    grid = tuple(e // t for e, t in zip(w.video, w.tile))
    cands = api.window_candidates(grid)
    for _ in range(args.warmup):
        api.window_errors(q, k, v, w.tile, cands[:2], stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        err = api.window_errors(q, k, v, w.tile, cands, stream=stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    V = w.tile[0] * w.tile[1] * w.tile[2]
    n_tiles = grid[0] * grid[1] * grid[2]
    per_pair = 4.0 * V * V * w.head_dim * w.heads * w.batch
    pairs = n_tiles * (n_tiles + sum(min(a, grid[0]) * min(b, grid[1]) * min(c, grid[2]) for a, b, c in cands))
    flops = per_pair * pairs
    tau = 0.1
    windows = api.window_select(err, cands, grid, tau)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's per-query-tile STA forward over the candidates for
        # sampled tiles of head 0, then 1, ..., until ~10 s; its FLOP rate
        # extrapolates the oracle's time for the whole sweep
        from oracle import sta_oracle as O
        from sliding_tile_attention_sta_amd.synthetic import sample_query_tiles
        qs, ks, vs = None, None, None
        done, fl, t_used, hh = 0, 0.0, 0.0, 0
        while t_used < 10.0 and hh < w.heads:
            qs, ks, vs = (x[:, hh:hh + 1].float().cpu().numpy() for x in (q, k, v))
            for c in sample_query_tiles(w, hh, count=4)[:4]:
                for win in cands:
                    t0 = time.perf_counter()
                    O.sta_forward_query_tiles(qs, ks, vs, w.tile, win, 0, [c], scale=w.scale)
                    t_used += time.perf_counter() - t0
                    fl += 4.0 * V * V * w.head_dim * (min(win[0], grid[0]) * min(win[1], grid[1]) *
                                                     min(win[2], grid[2]))
                    done += 1
                if t_used >= 10.0:
                    break
            hh += 1
        rate = fl / t_used
        cpu = {"value": round(flops / rate, 1), "unit": "s per sweep (extrapolated)", "cores": _threads(),
               "kind": "oracle",
               "sample": f"{done} (query tile, candidate) forwards of heads 0..{hh - 1} through the "
                         f"oracle, float64 numpy, {t_used:.1f} s, {rate / 1e12:.3f} TFLOP/s",
               "seconds": t_used, "cpu_model": _cpu_model()}
    kept = sum(a * b * c for a, b, c in windows) / (len(windows) * n_tiles)
    return {
        "metric": "STA per-head window search: seconds per candidate sweep",
        "value": round(sec, 3), "unit": "s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 1), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (locality calibration inputs)",
        "config": {"workload": w.name + "-locality", "video": list(w.video), "tile": list(w.tile),
                   "heads": w.heads, "head_dim": w.head_dim, "lengths": lengths,
                   "candidates": len(cands), "threshold": tau},
        "cpu_baseline": cpu,
        "forward_tflops": round(flops / sec / 1e12, 1),
        "chosen_windows": windows,
        "attended_fraction_of_dense": round(kept, 4),
    }


def swa(args, w, plan, q, k, v, stream):
    """Token-wise 3D sliding window attention on the workload's inputs, each
    query's window sized so that it holds as many keys as STA's window
    (wT * tT x wH * tH x wW * tW tokens), timed beside STA on the same
    inputs.  Both compute the same algorithmic FLOPs; SWA walks the union of
    a query tile's windows with per-score masks."""
    import torch
    from sliding_tile_attention_sta_amd import api

    toks = [tuple(a * t for a, t in zip(win, w.tile)) for win in w.windows]
    splan = api.Plan(w.batch, w.heads, w.video, w.tile, toks, w.head_dim, token_windows=True)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ms_swa = timed(lambda: api.sta_forward_plan(splan, q, k, v, out=out, scale=w.scale, stream=stream),
                   args.steps, args.warmup, stream)
    ms_sta = timed(lambda: api.sta_forward_plan(plan, q, k, v, out=out, scale=w.scale, stream=stream),
                   args.steps, args.warmup, stream)
    # executed key blocks of the SWA walk: rows of the union box x 32-key runs
    def start(x, wd, e):
        return min(max(x - (wd - 1) // 2, 0), e - wd)
    grid = [e // t for e, t in zip(w.video, w.tile)]
    V = w.tile[0] * w.tile[1] * w.tile[2]
    blocks = 0
    for win in toks:
        wc = [min(a, e) for a, e in zip(win, w.video)]
        span = []
        for d in range(3):
            per = []
            for c in range(grid[d]):
                lo = start(c * w.tile[d], wc[d], w.video[d])
                hi = start(c * w.tile[d] + w.tile[d] - 1, wc[d], w.video[d]) + wc[d]
                per.append(hi - lo)
            span.append(per)
        for a in span[0]:
            for b in span[1]:
                for c in span[2]:
                    blocks += a * b * ((c + 31) // 32)
    executed = 4.0 * blocks * 32 * V * w.head_dim * w.batch
    fl_swa = splan.flops
    cpu = None if args.no_cpu_baseline else cpu_baseline_swa(w, q, k, v, toks)
    return {
        "cpu_baseline": cpu,
        "metric": "token-wise SWA fwd ms vs STA fwd ms, same keys per query",
        "value": round(ms_swa / ms_sta, 3), "unit": "SWA time / STA time", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_swa, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "video": list(w.video), "tile": list(w.tile),
                   "sta_windows_tiles": sorted({tuple(x) for x in w.windows}),
                   "swa_windows_tokens": sorted(set(toks)), "heads": w.heads, "head_dim": w.head_dim},
        "swa": {"ms": round(ms_swa, 4), "tflops_algorithmic": round(fl_swa / (ms_swa * 1e-3) / 1e12, 1),
                "executed_over_algorithmic": round(executed / fl_swa, 3),
                "tflops_executed": round(executed / (ms_swa * 1e-3) / 1e12, 1)},
        "sta": {"ms": round(ms_sta, 4), "tflops": round(plan.flops / (ms_sta * 1e-3) / 1e12, 1)},
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this STA build runs on a single MI355X; "
              "multi-GPU sharding is a design note only (heads shard with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sliding_tile_attention_sta_amd import api
    from sliding_tile_attention_sta_amd.synthetic import WORKLOADS, make_qkv

    if args.copy_bytes:
        n = args.copy_bytes // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(4):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 4}))
        return

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    q, k, v = make_qkv(w, dev)
    # extents that are not multiples of the tile: partial tiles at the far edges
    partial = any(e % t for e, t in zip(w.video, w.tile))
    plan = api.Plan(w.batch, w.heads, w.video, w.tile, w.windows, w.head_dim, partial_tiles=partial)
    if args.which == "backward":
        print(json.dumps(backward(args, w, plan, q, k, v, stream)), flush=True)
        return
    if args.which == "search":
        del q, k, v
        print(json.dumps(search(args, w, stream)), flush=True)
        return
    if args.which == "swa":
        print(json.dumps(swa(args, w, plan, q, k, v, stream)), flush=True)
        return
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    flops = plan.flops

    def step():
        api.sta_forward_plan(plan, q, k, v, out=out, scale=w.scale, layout="natural", stream=stream)

    fit_counts(args, step, stream)
    ms = timed(step, args.steps, args.warmup, stream)
    tflops = flops / (ms * 1e-3) / 1e12

    # The step is a single launch of the forward kernel on `stream`, so the
    # per-launch kernel duration is the event time per step.
    # HBM traffic per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    # measurement, used only while the kernel source is the one measured.
    traffic = _measured_traffic(args.traffic_json, "sta_forward.hip", w.name, "bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (HBM, FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_flops_per_launch": flops,
                "kernel": "sta_fwd_kernel<128,3,8,bf16 in,f32 out>"}

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "video": list(w.video), "tile": list(w.tile),
                   "windows": sorted({tuple(x) for x in w.windows}), "heads": w.heads,
                   "head_dim": w.head_dim, "batch": w.batch, "layout": "natural",
                   "out_dtype": "f32", "products": "QK^T bf16 MFMA, PV fp16 MFMA, fp32 accumulate",
                   "flops_per_step": flops},
        "roofline": roofline,
    }

    result["per_call_ms"] = per_call_ms(step, args.steps, stream)
    if not args.no_context:
        out_b = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        ms_b = timed(lambda: api.sta_forward_plan(plan, q, k, v, out=out_b, scale=w.scale, layout="natural",
                                                  stream=stream), max(3, args.steps // 2), 1, stream)
        result["bf16_out"] = {"ms": round(ms_b, 4), "tflops": round(flops / (ms_b * 1e-3) / 1e12, 2)}
        del out_b

    if not args.no_context and not partial:
        # explicit reorder -> tile-major forward -> unreorder
        qt, kt, vt = (api.sta_tile_reorder(plan, x) for x in (q, k, v))
        out_t = torch.empty(qt.shape, dtype=torch.float32, device=dev)
        out_n = torch.empty_like(out)

        def reorder_in():
            for x, y in ((q, qt), (k, kt), (v, vt)):
                api.sta_tile_reorder(plan, x, out=y, stream=stream)

        def fwd_tm():
            api.sta_forward_plan(plan, qt, kt, vt, out=out_t, scale=w.scale, layout="tile_major",
                                 stream=stream)

        def unreorder_out():
            api.sta_tile_unreorder(plan, out_t, out=out_n, stream=stream)

        ms_r = timed(reorder_in, max(3, args.steps // 2), 1, stream)
        ms_f = timed(fwd_tm, max(3, args.steps // 2), 1, stream)
        ms_u = timed(unreorder_out, max(3, args.steps // 2), 1, stream)
        bytes_r = 3 * 2 * q.numel() * q.element_size()
        bytes_u = 2 * out_t.numel() * 4
        result["reorder_path"] = {
            "reorder_qkv_ms": round(ms_r, 4), "reorder_GBps": round(bytes_r / ms_r / 1e6, 1),
            "forward_tile_major_ms": round(ms_f, 4),
            "unreorder_o_ms": round(ms_u, 4), "unreorder_GBps": round(bytes_u / ms_u / 1e6, 1),
            "total_ms": round(ms_r + ms_f + ms_u, 4),
        }
        del qt, kt, vt, out_t, out_n
        # dense context: the same kernel with the window covering the whole grid
        grid = tuple(e // t for e, t in zip(w.video, w.tile))
        dplan = api.Plan(w.batch, w.heads, w.video, w.tile, [grid] * w.heads, w.head_dim)
        ms_d = timed(lambda: api.sta_forward_plan(dplan, q, k, v, out=out, scale=w.scale,
                                                  stream=stream), 3, 1, stream)
        result["dense_context"] = {"ms": round(ms_d, 3),
                                   "tflops": round(dplan.flops / (ms_d * 1e-3) / 1e12, 2),
                                   "sta_speedup": round(ms_d / ms, 2)}
        if w.dtype == "bf16":
            result["sdpa_dense_context"] = sdpa_dense(q, k, v, w.scale, stream, ms)
        if w.name == "720p":
            # the exact 720p latent (720 / 16 = 45 rows): partial tiles on H,
            # the same number of tiles and the same work as the padded 48 rows
            we = WORKLOADS["720p-exact"]
            del dplan
            qe, ke, ve = make_qkv(we, dev)
            eplan = api.Plan(we.batch, we.heads, we.video, we.tile, we.windows, we.head_dim, partial_tiles=True)
            oute = torch.empty(qe.shape, dtype=torch.float32, device=dev)
            ms_e = timed(lambda: api.sta_forward_plan(eplan, qe, ke, ve, out=oute, scale=we.scale,
                                                      stream=stream), max(3, args.steps // 2), 3, stream)
            result["exact_latent"] = {"video": list(we.video), "ms": round(ms_e, 4),
                                      "tflops_whole_tiles": round(eplan.flops / (ms_e * 1e-3) / 1e12, 2),
                                      "vs_padded": round(ms_e / ms, 3)}
            del qe, ke, ve, oute, eplan

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
