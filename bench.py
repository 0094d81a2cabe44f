#!/usr/bin/env python3
"""Benchmark of the TBE training hot path on one MI355X.

One step = forward gather-and-pool with the transpose (sort + run-length
encoding + routing) hoisted into the forward, then the backward with
row-wise Adagrad. The headline workload: T=32 tables of 2M rows, D=128 bf16,
B=131072 bags per table, Poisson(20) bag lengths (about 84M lookups),
Zipf-Mandelbrot skewed rows (about 3M unique, hottest about 125K), per-sample
weights. Inputs are resident in HBM before timing starts.

Prints one JSON line:
- `value`: wall-clock ms per step over K back-to-back steps (bracketed by
  device synchronisation), the metric;
- per-stage ms from HIP events recorded on the library's stream, and the
  same step timed after a 1 GiB scratch write that evicts L2 and the MALL
  (median and min over the steps);
- `gates`: the forward gather and the backward accumulate+apply, each as
  compulsory HBM bytes (every input byte the step must read at least once,
  every output byte it must write) over its time, as a fraction of the 8 TB/s
  peak. This is the fraction the memory can be held to: it cannot exceed 1.
  Beside it, `effective_GBps` counts one row read per lookup (the
  per-lookup model; L2 and MALL hits included, so it can exceed the peak);
- `roofline`: the same compulsory-byte model for the dominant single kernel,
  with its gathered bytes over the L2 row-gather ceiling measured in the
  same run by the library's own probe (include/tbe_probe.h);
- `configs`: every workload of the build (the tiny one, the three demo tables,
  the 16-table f16 one, the headline and the small-table one), each with
  fwd / pre / bwd / combined ms and its bytes;
- `cpu_baseline`: the CPU oracle (one thread, f64) on a bounded sample of the
  headline batch, per phase, scaled to the whole batch.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak, 8 TB/s
PEAK_F16_TFLOPS = 2500.0        # MI355X dense f16 matrix-core peak, 2.5 PFLOP/s
HOT_K = 256                     # hot rows per table in the backward's contraction
HOT_WGS = 512                   # workgroups the contraction runs over all tables (at most)
HOT_TILE = 16                   # bags per tile of the contraction
GATE = 0.6                      # target fraction of the HBM roofline
FLUSH_BYTES = 1 << 30           # scratch written before each flushed step


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


# --- byte models ---------------------------------------------------------------
def effective_bytes(cfg, N, U, n_chunks, long_lookups, weighted, n_long=0):
    """Per-lookup model: one weight row per lookup in the forward, one f32
    upstream-gradient row per lookup in the backward (every row a gather
    reads, including those L2 or the MALL serve)."""
    w = 2 if cfg.dtype in ("f16", "bf16") else 4
    a = 8 if cfg.dtype == "f32" else 4
    D, nb = cfg.D, cfg.T * cfg.B
    psw = 4 if weighted else 0
    fwd = N * (D * w + 4 + psw) + 4 * (nb + 1) + 4 * nb * D
    bwd = N * (4 * D + 4 + psw) + U * (2 * D * w + 16) + 2 * n_chunks * D * a
    long_kernel = long_lookups * (4 * D + 4 + psw) + n_chunks * (D * a + 12)
    fused = long_kernel + n_chunks * D * a + n_long * (2 * D * w + 8)
    return dict(fwd=fwd, bwd=bwd, bwd_long=long_kernel, bwd_long_fused=fused)


def compulsory_bytes(cfg, st, weighted):
    """Bytes the step must move across HBM at least once: each touched weight
    row read (and, in the backward, written) once, each upstream-gradient row
    of a bag with lookups read once, the index/metadata streams once, each
    output row written once, chunk partials written and read once."""
    w = 2 if cfg.dtype in ("f16", "bf16") else 4
    a = 8 if cfg.dtype == "f32" else 4
    D, nb, N, U = cfg.D, cfg.T * cfg.B, st["N"], st["U"]
    psw = 4 if weighted else 0
    fwd = U * D * w + N * (4 + psw) + 4 * (nb + 1) + 4 * nb * D
    hot = st.get("hot_runs", 0) > 0
    # with the hot rows' contraction, the chunk kernel takes only the other long runs
    chunk_lookups = st["long_lookups"] - st.get("hot_lookups", 0)
    chunks = st.get("chunk_chunks", st["n_chunks"]) if hot else st["n_chunks"]
    bags_chunk = st.get("bags_chunk", st["bags_long"]) if hot else st["bags_long"]
    hot_parts = 4 * cfg.T * st.get("hot_nseg", 0) * HOT_K * D if hot else 0
    bwd = (st["bags_touched"] * 4 * D + N * (4 + psw) + U * (2 * D * w + 8 + 8 + 4)
           + 2 * chunks * D * a + 2 * hot_parts)
    long_k = bags_chunk * 4 * D + chunk_lookups * (4 + psw) + chunks * (D * a + 12)
    short_k = (st["bags_short"] * 4 * D + (N - st["long_lookups"]) * (4 + psw)
               + st["n_short"] * (2 * D * w + 8 + 12))
    out = dict(fwd=fwd, bwd=bwd, fwd_pool=fwd, bwd_long=long_k, bwd_short=short_k)
    if hot:
        # every gradient row and every lookup's index and weight once, the
        # offsets, the segment partials written
        out["bwd_hot"] = nb * 4 * D + N * (4 + psw) + 4 * (nb + 1) + hot_parts
    return out


def hot_flops(cfg, st, weighted):
    """Matrix-core flops of the hot rows' contraction: per table and 16-bag
    tile, 256 slots x 16 bags x D columns, two products (hi, lo), three when
    weighted (the weight sums' residual too)."""
    tiles = -(-cfg.B // HOT_TILE)
    return 2 * cfg.T * tiles * HOT_TILE * HOT_K * cfg.D * (3 if weighted else 2)


def small_table_bytes(cfg, N):
    """Small-table path (counts kept as uint8, 64 per bag). Its kernels stream
    their inputs once, so the compulsory and the algorithmic bytes coincide.
    Counting reads indices and offsets and writes the counts; pooling reads
    the counts and the tables and writes the output; the backward contraction
    reads counts and gradients; the apply updates each table's 64 rows."""
    T, B, D, E = cfg.T, cfg.B, cfg.D, 64
    hist = T * B * E
    fwd = 4 * N + 4 * (T * B + 1) + 4 * T * B * D + hist + 2 * T * E * D
    bwd = hist + 4 * T * B * D + T * E * (2 * 2 * D + 8)
    return dict(fwd=fwd, bwd=bwd,
                small_count=4 * N + 4 * (T * B + 1) + hist,
                small_fwd=hist + 4 * T * B * D + 2 * T * E * D,
                small_bwd=hist + 4 * T * B * D,
                fwd_flop=2 * T * B * E * D,
                bwd_flop=2 * 2 * T * B * E * D)          # hi and lo products


def run_structure(torch, meta, cfg, N, S=256, C=256, hot=False):
    """Counts of the transpose's output, read back from the metadata the
    library wrote: runs, routing, long-run lookups, and how many distinct
    upstream-gradient rows the short and the long runs read; with the hot
    rows' contraction, which long runs it takes and what is left to chunks."""
    counts = meta["counts"][:4].cpu().numpy()
    U, n_short, n_long, n_chunks = (int(x) for x in counts)
    nb = cfg.T * cfg.B
    st = dict(N=N, U=U, n_short=n_short, n_long=n_long, n_chunks=n_chunks, long_lookups=0,
              bags_touched=0, bags_long=0, bags_short=0)
    if U == 0:
        return st
    ro = meta["run_offsets"][:U + 1].long()
    sl = ro[1:] - ro[:-1]
    is_long = torch.repeat_interleave(sl >= S, sl)
    sb = meta["sorted_bag"][:N].long()
    bl = torch.bincount(sb[is_long], minlength=nb) > 0
    bs = torch.bincount(sb[~is_long], minlength=nb) > 0
    st.update(long_lookups=int(is_long.sum().item()), bags_long=int(bl.sum().item()),
              bags_short=int(bs.sum().item()), bags_touched=int((bl | bs).sum().item()),
              max_sl=int(sl.max().item()))
    if hot:
        # the hot-row plan's choice: per table, the long runs of the longest
        # lengths while at most HOT_K of them reach that length (a tie at the
        # cut leaves the tied runs out)
        keys = meta["run_keys"][:U].long()
        toff = torch.tensor(np.concatenate([[0], np.cumsum(cfg.rows)]), device=keys.device)
        tab = torch.searchsorted(toff, keys, right=True) - 1
        hot_run = torch.zeros(U, dtype=torch.bool, device=keys.device)
        lr = torch.nonzero(sl >= S).flatten()
        for t in range(cfg.T):
            mine = lr[tab[lr] == t]
            if mine.numel() == 0:
                continue
            lens = sl[mine]
            if mine.numel() <= HOT_K:
                hot_run[mine] = True
                continue
            srt = torch.sort(lens, descending=True).values
            v = int(srt[HOT_K].item()) + 1      # the (K+1)-th longest is left out, with its ties
            hot_run[mine[lens >= v]] = True
        is_hot = torch.repeat_interleave(hot_run, sl)
        chunk_run = (sl >= S) & ~hot_run
        bc = torch.bincount(sb[is_long & ~is_hot], minlength=nb) > 0
        tiles = -(-cfg.B // HOT_TILE)
        st.update(hot_runs=int(hot_run.sum().item()), hot_lookups=int(is_hot.sum().item()),
                  chunk_chunks=int(((sl[chunk_run] + C - 1) // C).sum().item()),
                  bags_chunk=int(bc.sum().item()),
                  hot_nseg=max(1, min(HOT_WGS // cfg.T, -(-tiles // 32))))
        del is_hot, bc
    del is_long, sb, bl, bs
    return st


# --- committed counter readings ------------------------------------------------
def counters_for(name, stage):
    """Counter bytes per launch of `stage` from profiles/hbm_counters_<name>.json,
    if they were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(stage)
    if not rec:
        return None
    src = os.path.join(ROOT, "bwd_tbe_pooled_amd", "csrc", rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec


# --- device helpers ------------------------------------------------------------
def profile_copy(torch, dev):
    """One plain 1 GiB device-to-device copy: the known-size reference that
    scales the byte counters."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def stream_copy_gbps(torch, dev, reps=5):
    """Context: a plain 1 GiB device copy (bytes read + written over its best time)."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    return round(2 * (1 << 30) / (best * 1e6), 1)


def l2_gather_ceiling(torch, tbe, dev, row_floats, n=64 << 20, reps=5):
    """Rows per second the device gathers from a working set its L2 holds
    (1 MiB of float32 rows, random row ids), with the library's load shape:
    row bytes x rows / best time, in GB/s."""
    R = (1 << 20) // (4 * row_floats)
    src = torch.randn((R, row_floats), device=dev, dtype=torch.float32)
    g = torch.Generator(device=dev).manual_seed(77)
    rows = torch.randint(0, R, (n,), device=dev, dtype=torch.int32, generator=g)
    sink = torch.empty(tbe.TBE_PROBE_SINK_FLOATS, device=dev, dtype=torch.float32)
    tbe.tbe_probe_row_gather(src, rows, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        e0.record()
        tbe.tbe_probe_row_gather(src, rows, sink)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, rows, sink
    return round(n * row_floats * 4 / (best * 1e6), 1)


def graph_ms(torch, step, steps):
    """Milliseconds per step when the step is captured once in a HIP graph and
    replayed (no per-launch host cost); None if capture is not possible."""
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        return round((time.perf_counter() - t0) * 1000.0 / steps, 4)
    except Exception as e:  # report, never fail the benchmark over it
        log(f"graph capture unavailable: {e}")
        return None


def time_steps(torch, tbe, desc, step, steps, scratch):
    """K back-to-back steps (wall clock between synchronisations, and the
    library's per-stage HIP events), then K steps each preceded by a 1 GiB
    scratch write outside its timed window (HIP events around the step only)."""
    timer = tbe.Timer(capacity=steps + 1)
    desc.set_timer(timer)
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / steps
    desc.set_timer(None)
    st = timer.read()
    avg = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in st.items()}
    stages = {k: round(v, 4) for k, v in avg.items() if st[k][1]}
    flushed = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(steps):
        scratch.fill_(i & 0xff)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        flushed.append(e0.elapsed_time(e1))
    return wall_ms, avg, stages, {"median": round(statistics.median(flushed), 4),
                                  "min": round(min(flushed), 4)}


def frac(bytes_, ms):
    gbps = bytes_ / (ms * 1e6) if ms > 0 else 0.0
    return round(gbps, 1), round(gbps / PEAK_HBM_GBPS, 4)


# --- one workload on the generic path ----------------------------------------------
def measure_generic(torch, tbe, cfg, batch, args, scratch, *, headline=False):
    dev = torch.device("cuda")
    N = batch.indices.size
    weighted = batch.psw is not None
    idx = torch.from_numpy(batch.indices).to(dev)
    off = torch.from_numpy(batch.offsets).to(dev)
    psw = torch.from_numpy(batch.psw).to(dev) if weighted else None
    grad = torch.from_numpy(batch.grad).to(dev)
    from workloads import init_state, init_weights
    W = init_weights(cfg, dev)
    m = init_state(cfg, dev)
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    # the long-run path applies to every generic workload (the library takes
    # the hot rows' contraction only where it is eligible); the rest of the
    # diagnostics only to the headline
    flags = {"two_launch": 0, "fused": tbe.TBE_FLAG_FUSED_LONG,
             "hot": tbe.TBE_FLAG_HOT_BACKWARD}[args.long]
    if headline:
        flags |= {"none": 0, "fused": tbe.TBE_FLAG_CHECK, "validate": tbe.TBE_FLAG_VALIDATE}[args.check]
        if args.hot_rows == "off":
            flags |= tbe.TBE_FLAG_NO_HOT_ROWS
    desc = tbe.Desc(cfg.T, cfg.D, cfg.B, cfg.rows, cfg.dtype, flags=flags, error_flags=err)
    assert tbe.tbe_select_path(desc, N, weighted) == tbe.TBE_PATH_GENERIC
    meta = tbe.Meta(desc, N, weighted, with_pos=False)   # the backward needs no positions
    wide = headline and args.index == "int64"
    in_fwd = not (headline and (args.preprocess == "backward" or wide))
    if wide:
        idx64, off64 = idx.long(), off.long()
        ws_f = tbe.workspace_i64(desc, N, weighted, tbe.TBE_OP_FORWARD)
        ws_b = tbe.workspace_i64(desc, N, weighted, tbe.TBE_OP_BACKWARD_SELF)
    else:
        ws_f = tbe.workspace(desc, N, weighted,
                             tbe.TBE_OP_FORWARD_PREPROCESS if in_fwd else tbe.TBE_OP_FORWARD)
        ws_b = tbe.workspace(desc, N, weighted,
                             tbe.TBE_OP_BACKWARD if in_fwd else tbe.TBE_OP_BACKWARD_SELF)
    if headline and args.profile_copy:
        profile_copy(torch, dev)
    torch.cuda.synchronize()

    def step():
        if wide:
            tbe.tbe_forward_i64(desc, W, idx64, off64, psw, out, ws_f)
            tbe.tbe_backward_adagrad_i64(desc, W, m, grad, idx64, off64, psw, cfg.lr, cfg.eps, ws_b)
        elif in_fwd:
            tbe.tbe_forward(desc, W, idx, off, psw, out, meta, ws_f)
            tbe.tbe_backward_adagrad(desc, W, m, grad, idx, off, psw, meta, cfg.lr, cfg.eps, ws_b)
        else:   # the backward preprocesses into its own workspace
            tbe.tbe_forward(desc, W, idx, off, psw, out, None, ws_f)
            tbe.tbe_backward_adagrad(desc, W, m, grad, idx, off, psw, None, cfg.lr, cfg.eps, ws_b)

    for _ in range(args.warmup):
        step()
    if not in_fwd:   # the run structure for the byte counts
        tbe.tbe_preprocess(desc, idx, off, psw, meta,
                           tbe.workspace(desc, N, weighted, tbe.TBE_OP_PREPROCESS))
    torch.cuda.synchronize()
    steps = args.steps if headline else max(3, args.steps // 2)
    wall_ms, avg, stages, flushed = time_steps(torch, tbe, desc, step, steps, scratch)
    st = run_structure(torch, meta, cfg, N, hot="bwd_hot" in stages)
    g_ms = None
    if headline and not wide and args.check != "validate":
        g_ms = graph_ms(torch, step, steps)

    fwd_ms = avg["fwd_pool"] + avg.get("hot_plan", 0.0)   # the gather, and its hot-row plan
    pre_ms = avg["linearize"] + avg["sort"] + avg["rle_route"]
    bwd_ms = (avg["bwd_short"] + avg.get("bwd_hot_plan", 0.0) + avg.get("bwd_hot", 0.0)
              + avg["long_schedule"] + avg["bwd_long"] + avg["bwd_apply"])
    eff = effective_bytes(cfg, N, st["U"], st["n_chunks"], st["long_lookups"], weighted, st["n_long"])
    comp = compulsory_bytes(cfg, st, weighted)
    res = {
        "workload": cfg.name, "path": "generic",
        "shape": {"T": cfg.T, "E": list(sorted(set(cfg.rows))), "D": cfg.D, "B": cfg.B, "N": N,
                  "dtype": cfg.dtype, "weighted": weighted},
        "structure": st,
        "ms_per_step": round(wall_ms, 4),
        "flushed_ms_per_step": flushed,
        "graph_ms_per_step": g_ms,
        "stages_ms": stages,
        "fwd_ms": round(fwd_ms, 4), "pre_ms": round(pre_ms, 4),
        "fwd_total_ms": round(fwd_ms + pre_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "combined_ms": round(fwd_ms + pre_ms + bwd_ms, 4),
        "bytes": {"fwd": {"compulsory": comp["fwd"], "effective": eff["fwd"]},
                  "bwd": {"compulsory": comp["bwd"], "effective": eff["bwd"]}},
    }
    gates = {}
    for part, ms in (("fwd_gather", fwd_ms), ("bwd_accumulate_apply", bwd_ms)):
        key = "fwd" if part == "fwd_gather" else "bwd"
        gb, fr = frac(comp[key], ms)
        egb, efr = frac(eff[key], ms)
        gates[part] = {"ms": round(ms, 4), "compulsory_bytes": comp[key], "GBps": gb,
                       "frac_of_peak": fr, "target": GATE, "met": fr >= GATE,
                       "effective_bytes": eff[key], "effective_GBps": egb}
    res["gates"] = gates
    kernels = {}
    gathered = {"fwd_pool": N * cfg.D * (2 if cfg.dtype != "f32" else 4),
                "bwd_long": st["long_lookups"] * 4 * cfg.D,
                "bwd_short": (N - st["long_lookups"]) * 4 * cfg.D}
    if st.get("hot_runs", 0):
        gathered["bwd_long"] = (st["long_lookups"] - st["hot_lookups"]) * 4 * cfg.D
        gathered["bwd_short"] = (N - st["long_lookups"]) * 4 * cfg.D
    for k in ("fwd_pool", "bwd_short", "bwd_long"):
        ms = avg[k]
        if ms <= 0:
            continue
        gb, fr = frac(comp[k], ms)
        kernels[k] = {"ms": round(ms, 4), "compulsory_bytes": comp[k], "GBps": gb,
                      "frac_of_peak": fr, "gathered_bytes": gathered[k],
                      "gathered_GBps": round(gathered[k] / (ms * 1e6), 1)}
    if avg.get("bwd_hot", 0.0) > 0 and "bwd_hot" in comp:
        # the contraction alone (its plan is the bwd_hot_plan stage)
        ms = avg["bwd_hot"]
        fl = hot_flops(cfg, st, weighted)
        gb, fr = frac(comp["bwd_hot"], ms)
        tf = fl / (ms * 1e9)
        kernels["bwd_hot"] = {"ms": round(ms, 4), "bound": "mfma", "flops": fl,
                              "TFLOPs": round(tf, 1), "peak_TFLOPs": PEAK_F16_TFLOPS,
                              "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4),
                              "compulsory_bytes": comp["bwd_hot"], "GBps": gb,
                              "frac_of_hbm_peak": fr}
    res["kernels"] = kernels
    del W, m, out, grad, idx, off, psw, ws_f, ws_b, meta
    if wide:
        del idx64, off64
    torch.cuda.empty_cache()
    return res


# --- the small-table workload --------------------------------------------------------
def measure_small(torch, tbe, cfg, batch, args, scratch, *, headline=False):
    from workloads import init_state, init_weights
    dev = torch.device("cuda")
    N = batch.indices.size
    idx = torch.from_numpy(batch.indices).to(dev)
    off = torch.from_numpy(batch.offsets).to(dev)
    grad = torch.from_numpy(batch.grad).to(dev)
    W = init_weights(cfg, dev)
    m = init_state(cfg, dev)
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device=dev)
    desc = tbe.Desc(cfg.T, cfg.D, cfg.B, cfg.rows, cfg.dtype)
    assert tbe.tbe_select_path(desc, N, False) == tbe.TBE_PATH_SMALL_TABLE
    meta = tbe.Meta(desc, N, False)
    ws_f = tbe.workspace(desc, N, False, tbe.TBE_OP_FORWARD_PREPROCESS)
    ws_b = tbe.workspace(desc, N, False, tbe.TBE_OP_BACKWARD)
    if headline and args.profile_copy:
        profile_copy(torch, dev)
    torch.cuda.synchronize()

    def step():
        tbe.tbe_forward(desc, W, idx, off, None, out, meta, ws_f)
        tbe.tbe_backward_adagrad(desc, W, m, grad, idx, off, None, meta, cfg.lr, cfg.eps, ws_b)

    for _ in range(args.warmup):
        step()
    steps = args.steps if headline else max(3, args.steps // 2)
    wall_ms, avg, stages, flushed = time_steps(torch, tbe, desc, step, steps, scratch)
    g_ms = graph_ms(torch, step, steps) if headline else None
    by = small_table_bytes(cfg, N)
    fwd_ms = avg["small_count"] + avg["small_fwd"]
    bwd_ms = avg["small_bwd"] + avg["small_apply"]
    res = {
        "workload": cfg.name, "path": "small_table",
        "shape": {"T": cfg.T, "E": list(sorted(set(cfg.rows))), "D": cfg.D, "B": cfg.B, "N": N,
                  "dtype": cfg.dtype, "weighted": False},
        "ms_per_step": round(wall_ms, 4), "flushed_ms_per_step": flushed,
        "graph_ms_per_step": g_ms, "stages_ms": stages,
        "fwd_ms": round(fwd_ms, 4), "pre_ms": 0.0, "fwd_total_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4), "combined_ms": round(fwd_ms + bwd_ms, 4),
        "bytes": {"fwd": {"compulsory": by["fwd"], "effective": by["fwd"]},
                  "bwd": {"compulsory": by["bwd"], "effective": by["bwd"]}},
    }
    gates = {}
    for part, ms, key in (("fwd_gather", fwd_ms, "fwd"), ("bwd_accumulate_apply", bwd_ms, "bwd")):
        gb, fr = frac(by[key], ms)
        gates[part] = {"ms": round(ms, 4), "compulsory_bytes": by[key], "GBps": gb,
                       "frac_of_peak": fr, "target": GATE, "met": fr >= GATE}
    res["gates"] = gates
    kernels = {}
    for k in ("small_count", "small_fwd", "small_bwd"):
        ms = avg[k]
        if ms <= 0:
            continue
        gb, fr = frac(by[k], ms)
        kernels[k] = {"ms": round(ms, 4), "compulsory_bytes": by[k], "GBps": gb, "frac_of_peak": fr}
    kernels["small_fwd"]["mfma_TFLOPs"] = round(by["fwd_flop"] / (avg["small_fwd"] * 1e9), 2)
    kernels["small_bwd"]["mfma_TFLOPs"] = round(by["bwd_flop"] / (avg["small_bwd"] * 1e9), 2)
    res["kernels"] = kernels
    del W, m, out, grad, idx, off, ws_f, ws_b, meta
    torch.cuda.empty_cache()
    return res


def all_hot_forward_ms(torch, tbe, cfg, batch, steps=5, transpose=True):
    """The forward gather on the headline batch's bags with every lookup
    redirected to one of its table's first 64 rows (512 KiB of weights in
    all): the same gather count, every row an L2 hit. With `transpose` it is
    the headline's forward (the transpose, then the gather that reads each
    table's hot rows from LDS; those 64 rows are then all hot), and its gather
    stage is that kernel's time with no row read from memory; without, the
    plain gather, whose time is then its own L2-hit ceiling."""
    from workloads import init_weights
    dev = torch.device("cuda")
    idx = torch.from_numpy(batch.indices).to(dev) & 63
    off = torch.from_numpy(batch.offsets).to(dev)
    psw = torch.from_numpy(batch.psw).to(dev) if batch.psw is not None else None
    W = init_weights(cfg, dev)
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device=dev)
    desc = tbe.Desc(cfg.T, cfg.D, cfg.B, cfg.rows, cfg.dtype)
    N, weighted = idx.numel(), psw is not None
    meta = tbe.Meta(desc, N, weighted, with_pos=False) if transpose else None
    ws = tbe.workspace(desc, N, weighted,
                       tbe.TBE_OP_FORWARD_PREPROCESS if transpose else tbe.TBE_OP_FORWARD)
    tbe.tbe_forward(desc, W, idx, off, psw, out, meta, ws)
    timer = tbe.Timer(capacity=steps + 1)
    desc.set_timer(timer)
    for _ in range(steps):
        tbe.tbe_forward(desc, W, idx, off, psw, out, meta, ws)
    torch.cuda.synchronize()
    desc.set_timer(None)
    t = timer.read()
    ms, n = t["fwd_pool"]
    if transpose and t["hot_plan"][1] == 0:
        log("all-hot probe: the forward after the transpose did not take the hot rows")
    del idx, off, psw, W, out, ws, meta
    torch.cuda.empty_cache()
    return round(ms / n, 4)


# --- CPU baseline ----------------------------------------------------------------
def cpu_baseline(cfg, batch, W0, B_sample):
    """The oracle (single thread, fp64) on the first B_sample bags of every
    table, timed per phase; each phase's time is scaled by lookups to the
    whole batch."""
    import torch
    import oracle
    T, B = cfg.T, cfg.B
    offs = batch.offsets
    w16 = W0.dtype != torch.float32
    parts_idx, parts_psw, lengths = [], [], []
    for t in range(T):
        a, e = int(offs[t * B]), int(offs[t * B + B_sample])
        parts_idx.append(batch.indices[a:e])
        parts_psw.append(batch.psw[a:e] if batch.psw is not None else None)
        lengths.append(np.diff(offs[t * B:t * B + B_sample + 1]))
    idx = np.concatenate(parts_idx)
    psw = np.concatenate(parts_psw) if batch.psw is not None else None
    off = np.concatenate([[0], np.cumsum(np.concatenate(lengths))]).astype(np.int32)
    grad = np.ascontiguousarray(batch.grad[:B_sample])
    keys, bags = oracle.linearize(T, B_sample, cfg.rows, idx, off)
    uk = np.unique(keys)
    kt = torch.from_numpy(uk.astype(np.int64)).to(W0.device)
    Wrows = W0.index_select(0, kt).cpu()
    Wrows = Wrows.view(torch.int16).numpy().view(np.uint16) if w16 else Wrows.numpy()
    m = np.zeros(uk.size, dtype=np.float32)
    ph = {}
    t0 = time.perf_counter()
    keys, bags = oracle.linearize(T, B_sample, cfg.rows, idx, off)
    oracle.forward(T, B_sample, cfg.D, cfg.dtype, off, keys, psw, Wrows, wkeys=uk)
    t1 = time.perf_counter()
    pos = oracle.sort(keys)
    r = oracle.rle(keys, pos, bags, psw)
    oracle.route(r["run_offsets"])
    t2 = time.perf_counter()
    oracle.backward_adagrad(T, B_sample, cfg.D, cfg.dtype, r["run_keys"], r["run_offsets"],
                            r["sorted_bag"], r["sorted_psw"], grad, Wrows, m, cfg.lr, cfg.eps,
                            wkeys=uk)
    t3 = time.perf_counter()
    scale = batch.indices.size / max(1, idx.size)
    ph = {"fwd": (t1 - t0) * 1000.0 * scale, "sort_rle_route": (t2 - t1) * 1000.0 * scale,
          "bwd_adagrad": (t3 - t2) * 1000.0 * scale}
    secs = t3 - t0
    return {"value": round(secs * 1000.0 * scale, 1), "unit": "ms", "cores": 1, "kind": "oracle",
            "phases_ms": {k: round(v, 1) for k, v in ph.items()},
            "sample": f"first {B_sample} of {B} bags of each table ({idx.size} of "
                      f"{batch.indices.size} lookups): linearize + forward, sort/RLE/route, "
                      f"backward + Adagrad, in fp64 on one thread; {secs:.2f} s measured, "
                      f"each phase scaled by lookups to the whole batch",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "host_cpu_model": cpu_model()}


# --- main ----------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only (profiling runs)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the L2 row-gather ceilings and the plain copy")
    ap.add_argument("--cpu-sample-bags", type=int, default=65536)
    ap.add_argument("--workload", choices=["large", "small"], default="large",
                    help="headline workload: large (T=32 E=2M D=128 bf16 B=131072, the metric's) "
                         "or small (the small-table histogram path, T=64 E=64 D=128 f16 B=32768 "
                         "L=64; for its profiles)")
    ap.add_argument("--check", choices=["none", "fused", "validate"], default="none",
                    help="index checking: none (default), fused into the kernels "
                         "(TBE_FLAG_CHECK), or the separate synchronous pass (TBE_FLAG_VALIDATE)")
    ap.add_argument("--preprocess", choices=["forward", "backward"], default="forward",
                    help="where the transpose (sort, RLE, routing) runs: in the forward "
                         "(default; the pages' hoisting) or inside the backward (their baseline)")
    ap.add_argument("--hot-rows", choices=["on", "off"], default="on",
                    help="the forward after the transpose reads each table's hottest rows from "
                         "LDS (on, default) or gathers every row (off: TBE_FLAG_NO_HOT_ROWS)")
    ap.add_argument("--long", choices=["two_launch", "fused", "hot"], default="hot",
                    help="long runs: each table's hottest rows' gradients as one matrix-core "
                         "contraction and the rest as chunk partials then a separate apply "
                         "(hot, default: TBE_FLAG_HOT_BACKWARD), every long run as chunks "
                         "(two_launch: the library's default), or one launch whose last "
                         "chunk per run reduces and applies (fused: TBE_FLAG_FUSED_LONG)")
    ap.add_argument("--rows", choices=["zipf", "uniform"], default="zipf",
                    help="row distribution of the large workload: Zipf-Mandelbrot (default) or "
                         "uniform (a diagnostic without reuse)")
    ap.add_argument("--tables", type=int, default=32,
                    help="tables of the large workload (diagnostic: other values keep every "
                         "table's shape and distribution; 32 is the headline)")
    ap.add_argument("--index", choices=["int32", "int64"], default="int32",
                    help="index arrays: int32 (default) or int64 through the _i64 entry points "
                         "(which preprocess inside the backward)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (calibrates the byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library "
              "is the single-GPU hot path (a table-wise shard of a multi-GPU run is the same "
              "call on fewer tables).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import dataclasses
    import bwd_tbe_pooled_amd as tbe
    from workloads import WORKLOADS, LARGE, SMALL_TABLE, init_weights, make_batch

    dev = torch.device("cuda")
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    diagnostic = (args.check != "none" or args.preprocess != "forward" or args.long != "hot"
                  or args.rows != "zipf" or args.index != "int32" or args.tables != 32
                  or args.hot_rows != "on")

    if args.workload == "small":
        cfg = SMALL_TABLE
        log("generating the small-table batch")
        batch = make_batch(cfg)
        head = measure_small(torch, tbe, cfg, batch, args, scratch, headline=True)
        dom_candidates = ("small_count", "small_fwd", "small_bwd")
        metric = ("TBE small-table path fwd+bwd(Adagrad) ms and achieved HBM GB/s % peak, "
                  "T=64 E=64 B=32K D=128")
        dtype = "f16"
    else:
        cfg = LARGE if args.rows == "zipf" else dataclasses.replace(LARGE, index=("uniform",))
        if args.tables != 32:
            cfg = dataclasses.replace(cfg, T=args.tables, rows=(cfg.rows[0],) * args.tables)
        log("generating the headline batch")
        batch = make_batch(cfg)
        head = measure_generic(torch, tbe, cfg, batch, args, scratch, headline=True)
        dom_candidates = ("fwd_pool", "bwd_short", "bwd_long", "bwd_hot")
        metric = "TBE fwd+bwd(Adagrad) ms and achieved HBM GB/s % peak, T=32 B=128K D=128"
        dtype = "bf16"
    log(f"headline {head['ms_per_step']} ms per step")

    probes = {}
    if not args.no_probes:
        log("probes: L2 row-gather ceilings, plain copy")
        probes["l2_gather_GBps_256B_rows"] = l2_gather_ceiling(torch, tbe, dev, 64)
        probes["l2_gather_GBps_512B_rows"] = l2_gather_ceiling(torch, tbe, dev, 128)
        probes["stream_copy_GBps"] = stream_copy_gbps(torch, dev)
        if args.workload == "large" and not diagnostic:
            probes["fwd_pool_all_hot_ms"] = all_hot_forward_ms(torch, tbe, cfg, batch)
            probes["fwd_plain_all_l2_hits_ms"] = all_hot_forward_ms(torch, tbe, cfg, batch,
                                                                    transpose=False)

    # dominant single kernel, on the compulsory-byte model
    ks = head["kernels"]
    dom = max((k for k in dom_candidates if k in ks), key=lambda k: ks[k]["ms"])
    dk = ks[dom]
    name_for_counters = cfg.name if not diagnostic else None
    rec = counters_for(name_for_counters, dom) if name_for_counters else None
    traffic = rec["hbm_bytes_per_launch"] if rec else None
    if dk.get("bound") == "mfma":
        # a dense contraction: its flops against the f16 matrix-core peak
        roofline = {"kernel": dom, "bound": "mfma", "achieved": dk["TFLOPs"],
                    "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": dk["frac_of_peak"],
                    "traffic": traffic, "flops_per_launch": dk["flops"],
                    "avg_launch_ms": dk["ms"], "bytes_per_launch": dk["compulsory_bytes"],
                    "hbm_GBps": dk["GBps"], "hbm_frac": dk["frac_of_hbm_peak"]}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "bytes_model": "compulsory",
                    "achieved": dk["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": dk["frac_of_peak"], "traffic": traffic,
                    "bytes_per_launch": dk["compulsory_bytes"], "avg_launch_ms": dk["ms"]}
    if traffic:
        roofline["traffic_GBps"] = round(traffic / (dk["ms"] * 1e6), 1)
        roofline["traffic_counters"] = rec.get("counters", "FETCH_SIZE + WRITE_SIZE")
    if "gathered_bytes" in dk:
        roofline["gathered_bytes"] = dk["gathered_bytes"]
        roofline["gathered_GBps"] = dk["gathered_GBps"]
        row_bytes = 4 * cfg.D if dom != "fwd_pool" else cfg.D * (2 if cfg.dtype != "f32" else 4)
        ceil = probes.get(f"l2_gather_GBps_{row_bytes}B_rows")
        if ceil:
            roofline["l2_gather_ceiling_GBps"] = ceil
            roofline["frac_of_l2_gather_ceiling"] = round(dk["gathered_GBps"] / ceil, 4)
    if "fwd_pool_all_hot_ms" in probes and "fwd_pool" in ks:
        # the same gather with every row hot: its own time with no row from memory
        ks["fwd_pool"]["all_hot_ms"] = probes["fwd_pool_all_hot_ms"]
        ks["fwd_pool"]["frac_of_all_hot_speed"] = round(
            probes["fwd_pool_all_hot_ms"] / ks["fwd_pool"]["ms"], 4)
    for k, v in ks.items():
        if "gathered_GBps" in v:
            row_bytes = 4 * cfg.D if k != "fwd_pool" else cfg.D * (2 if cfg.dtype != "f32" else 4)
            ceil = probes.get(f"l2_gather_GBps_{row_bytes}B_rows")
            if ceil:
                v["frac_of_l2_gather_ceiling"] = round(v["gathered_GBps"] / ceil, 4)

    configs = None
    if not args.no_configs and not diagnostic:
        configs = {}
        for name, c in WORKLOADS.items():
            if name == cfg.name:
                configs[name] = {k: head[k] for k in ("workload", "path", "shape", "ms_per_step",
                                                       "flushed_ms_per_step", "fwd_ms", "pre_ms",
                                                       "fwd_total_ms", "bwd_ms", "combined_ms",
                                                       "bytes", "gates")}
                configs[name]["headline"] = True
                continue
            log(f"config {name}")
            b = make_batch(c)
            if c is SMALL_TABLE:
                r = measure_small(torch, tbe, c, b, args, scratch)
            else:
                r = measure_generic(torch, tbe, c, b, args, scratch)
            r.pop("kernels", None)
            r.pop("graph_ms_per_step", None)
            configs[name] = r
            del b

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        W0 = init_weights(cfg, dev)
        bags = args.cpu_sample_bags if args.workload == "large" else args.cpu_sample_bags // 8
        cpu = cpu_baseline(cfg, batch, W0, min(bags, cfg.B))
        del W0

    result = {
        "metric": metric,
        "value": head["ms_per_step"],
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name + (f" ({args.rows} rows)" if args.rows != "zipf" else "")
                   + ("" if args.preprocess == "forward" else ", preprocessing in the backward")
                   + ("" if args.check == "none" else f", index check {args.check}")
                   + {"two_launch": ", every long run on the chunk path",
                      "fused": ", long runs in one launch",
                      "hot": ""}[args.long]
                   + ("" if args.hot_rows == "on" else ", no hot rows in the forward")
                   + ("" if args.index == "int32" else ", int64 indices")
                   + ("" if args.tables == 32 else f", {args.tables} tables"),
                   **head["shape"], "parallelism": "single GPU"},
        "flushed_ms_per_step": head["flushed_ms_per_step"],
        "graph_ms_per_step": head["graph_ms_per_step"],
        "stages_ms": head["stages_ms"],
        "fwd_ms": head["fwd_ms"], "pre_ms": head["pre_ms"], "fwd_total_ms": head["fwd_total_ms"],
        "bwd_ms": head["bwd_ms"], "combined_ms": head["combined_ms"],
        "gates": head["gates"],
        "kernels": head["kernels"],
        "roofline": roofline,
        "structure": head.get("structure"),
        "probes": probes,
        "configs": configs,
        "cpu_baseline": cpu,
        "context": "B200 figures on the pages (another machine, unstated shape): combined "
                   "79.537 ms -> 66.183 ms with forward-side preprocessing",
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
