#!/usr/bin/env python3
"""Benchmark of the TBE training hot path on one MI355X.

One step = forward gather-and-pool with the transpose (sort + run-length
encoding + routing) hoisted into the forward, then the backward with
row-wise Adagrad, on the large skewed workload: T=32 tables of 2M rows,
D=128 bf16, B=131072 bags per table, Poisson(20) bag lengths (about 84M
lookups), Zipf-Mandelbrot skewed rows (about 3M unique, hottest about 125K),
per-sample weights. Inputs are resident in HBM before timing starts.

Prints one JSON line: combined forward+backward ms per step (the metric), the
per-stage split measured with HIP events on the library's stream, effective
HBM GB/s of the forward gather and of the backward accumulate+apply, the
roofline of the dominant kernel, and the CPU oracle timed on a bounded sample
of the same batch (its ms scaled to the whole batch).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak, 8 TB/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, N, U, n_chunks, long_lookups, weighted, n_long=0):
    """Bytes each part of the method must move at least once per step. The
    fused long kernel also re-reads the partials and updates the long rows."""
    w = 2 if cfg.dtype in ("f16", "bf16") else 4
    a = 8 if cfg.dtype == "f32" else 4
    D, nb = cfg.D, cfg.T * cfg.B
    psw = 4 if weighted else 0
    fwd = N * (D * w + 4 + psw) + 4 * (nb + 1) + 4 * nb * D
    bwd = N * (4 * D + 4 + psw) + U * (2 * D * w + 16) + 2 * n_chunks * D * a
    long_kernel = long_lookups * (4 * D + 4 + psw) + n_chunks * (D * a + 12)
    fused = long_kernel + n_chunks * D * a + n_long * (2 * D * w + 8)
    return dict(fwd=fwd, bwd=bwd, bwd_long=long_kernel, bwd_long_fused=fused)


def small_table_bytes(cfg, N):
    """Algorithmic bytes and MFMA flops of the small-table path (counts kept
    as uint8, 64 per bag): forward reads indices, offsets and the tables and
    writes the pooled rows and counts; backward reads counts and gradients,
    applies Adagrad to the 64 rows of every table. Per kernel: counting reads
    indices and offsets and writes the counts; pooling reads the counts and
    the tables and writes the output (the counts cross HBM once more than in
    the forward's own total); the backward contraction reads counts and
    gradients; apply updates the rows."""
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


def cpu_baseline(cfg, batch, W0, B_sample):
    """The oracle (single thread, fp64) on the first B_sample bags of every
    table; its time is scaled by lookups to the whole batch."""
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
    t0 = time.perf_counter()
    keys, bags = oracle.linearize(T, B_sample, cfg.rows, idx, off)
    oracle.forward(T, B_sample, cfg.D, cfg.dtype, off, keys, psw, Wrows, wkeys=uk)
    pos = oracle.sort(keys)
    r = oracle.rle(keys, pos, bags, psw)
    oracle.route(r["run_offsets"])
    oracle.backward_adagrad(T, B_sample, cfg.D, cfg.dtype, r["run_keys"], r["run_offsets"],
                            r["sorted_bag"], r["sorted_psw"], grad, Wrows, m, cfg.lr, cfg.eps,
                            wkeys=uk)
    secs = time.perf_counter() - t0
    scale = batch.indices.size / max(1, idx.size)
    return {"value": secs * 1000.0 * scale, "unit": "ms", "cores": 1, "kind": "oracle",
            "sample": f"first {B_sample} of {B} bags of each table ({idx.size} of "
                      f"{batch.indices.size} lookups), fwd + sort/RLE/route + bwd/Adagrad "
                      f"in fp64 on one thread, {secs:.2f} s measured, scaled by lookups",
            "host_cpus": os.cpu_count(), "host_cpu_model": platform.processor() or platform.machine()}


LARGE_COUNTERS = "hbm_counters_t32_b128k_bf16.json"
SMALL_COUNTERS = "hbm_counters_t64_e64_b32k_f16.json"


def counters_for(kernel_stage, name=LARGE_COUNTERS):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_stage)
    if not rec:
        return None
    src = os.path.join(ROOT, "bwd_tbe_pooled_amd", "csrc", rec["source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def traffic_rate(traffic, ms):
    """Measured HBM bytes per launch over the launch time. Algorithmic bytes
    count every row a gather reads, also the ones L2 serves, so `frac` can
    exceed 1; this is the rate the memory itself sees."""
    if not traffic:
        return {}
    gbps = traffic / (ms * 1e6)
    return {"traffic_GBps": round(gbps, 1), "traffic_frac": round(gbps / PEAK_HBM_GBPS, 4)}


def profile_copy(torch, dev):
    """One plain 1 GiB device-to-device copy: the known-size reference that
    scales the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def stream_copy_gbps(torch, dev, reps=5):
    """Context only: a plain 1 GiB device-to-device copy timed with events
    (bytes read + written over its time), outside the timed steps."""
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-bags", type=int, default=65536)
    ap.add_argument("--workload", choices=["large", "small"], default="large",
                    help="large: T=32 E=2M D=128 bf16 B=131072 (the headline); "
                         "small: the small-table histogram path, T=64 E=64 D=128 f16 B=32768 L=64")
    ap.add_argument("--check", choices=["none", "fused", "validate"], default="none",
                    help="index checking: none (default), fused into the kernels "
                         "(TBE_FLAG_CHECK), or the separate synchronous pass (TBE_FLAG_VALIDATE)")
    ap.add_argument("--preprocess", choices=["forward", "backward"], default="forward",
                    help="where the transpose (sort, RLE, routing) runs: in the forward "
                         "(default; the pages' hoisting) or inside the backward (their baseline)")
    ap.add_argument("--long", choices=["two_launch", "fused"], default="two_launch",
                    help="long runs: chunk partials then a separate apply (default), or one "
                         "launch whose last chunk per run reduces and applies (TBE_FLAG_FUSED_LONG)")
    ap.add_argument("--rows", choices=["zipf", "uniform"], default="zipf",
                    help="row distribution of the large workload: Zipf-Mandelbrot (default, "
                         "the headline) or uniform (a diagnostic without reuse, in which the "
                         "effective and the counter-measured rates should agree)")
    ap.add_argument("--index", choices=["int32", "int64"], default="int32",
                    help="index arrays: int32 (default) or int64 through the _i64 entry points "
                         "(which preprocess inside the backward, so --preprocess backward)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library is a single-GPU hot path).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import bwd_tbe_pooled_amd as tbe
    from workloads import WORKLOADS, TINY, DEMO3, MEDIUM, LARGE, SMALL_TABLE, init_state, init_weights, make_batch

    if args.workload == "small":
        return main_small(args, torch, tbe)
    cfg = LARGE
    if args.rows == "uniform":
        import dataclasses
        cfg = dataclasses.replace(LARGE, index=("uniform",))
    log("generating the batch")
    batch = make_batch(cfg)
    N = batch.indices.size
    dev = torch.device("cuda")
    idx = torch.from_numpy(batch.indices).to(dev)
    off = torch.from_numpy(batch.offsets).to(dev)
    psw = torch.from_numpy(batch.psw).to(dev)
    grad = torch.from_numpy(batch.grad).to(dev)
    W = init_weights(cfg, dev)
    W0 = W.clone() if not args.no_cpu_baseline else None
    m = init_state(cfg, dev)
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device=dev)
    timer = tbe.Timer(capacity=args.steps + 1)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    flags = {"none": 0, "fused": tbe.TBE_FLAG_CHECK, "validate": tbe.TBE_FLAG_VALIDATE}[args.check]
    fused_long = args.long == "fused"
    if fused_long:
        flags |= tbe.TBE_FLAG_FUSED_LONG
    desc = tbe.Desc(cfg.T, cfg.D, cfg.B, cfg.rows, cfg.dtype, flags=flags, error_flags=err)
    meta = tbe.Meta(desc, N, True, with_pos=False)   # the backward needs no positions
    wide = args.index == "int64"
    if wide and args.preprocess == "forward":
        args.preprocess = "backward"   # the int64 entry points keep no metadata
    in_fwd = args.preprocess == "forward"
    if wide:
        idx64, off64 = idx.long(), off.long()
        ws_f = tbe.workspace_i64(desc, N, True, tbe.TBE_OP_FORWARD)
        ws_b = tbe.workspace_i64(desc, N, True, tbe.TBE_OP_BACKWARD_SELF)
    else:
        ws_f = tbe.workspace(desc, N, True, tbe.TBE_OP_FORWARD_PREPROCESS if in_fwd else tbe.TBE_OP_FORWARD)
        ws_b = tbe.workspace(desc, N, True, tbe.TBE_OP_BACKWARD if in_fwd else tbe.TBE_OP_BACKWARD_SELF)
    if args.profile_copy:
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

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    if not in_fwd:   # run structure for the byte counts below
        tbe.tbe_preprocess(desc, idx, off, psw, meta, tbe.workspace(desc, N, True, tbe.TBE_OP_PREPROCESS))
    torch.cuda.synchronize()
    counts = meta["counts"][:4].cpu().numpy()
    U, n_short, n_long, n_chunks = (int(x) for x in counts)
    ro = meta["run_offsets"][:U + 1]
    lr_ = meta["long_runs"][:n_long].long()
    long_lookups = int((ro[lr_ + 1] - ro[lr_]).sum().item()) if n_long else 0

    log(f"timing {args.steps} steps")
    desc.set_timer(timer)
    timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    desc.set_timer(None)
    st = timer.read()
    avg = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in st.items()}
    # the int64 calls and the validation flag synchronise with the host
    g_ms = graph_ms(torch, step, args.steps) if not wide and args.check != "validate" else None

    fwd_ms = avg["fwd_pool"]
    pre_ms = avg["linearize"] + avg["sort"] + avg["rle_route"]
    bwd_ms = avg["bwd_short"] + avg["long_schedule"] + avg["bwd_long"] + avg["bwd_apply"]
    by = algorithmic_bytes(cfg, N, U, n_chunks, long_lookups, True, n_long)
    fwd_gbps = by["fwd"] / (fwd_ms * 1e6)
    bwd_gbps = by["bwd"] / (bwd_ms * 1e6)
    # dominant single kernel: the longest of the one-kernel stages
    long_name = "bwd_long_fused" if fused_long else "bwd_long"
    cand = {"fwd_pool": (avg["fwd_pool"], by["fwd"]), long_name: (avg["bwd_long"], by[long_name])}
    dom = max(cand, key=lambda k: cand[k][0])
    dom_ms, dom_bytes = cand[dom]
    achieved = dom_bytes / (dom_ms * 1e6)
    # the committed counters were taken on this workload as bench.py runs it
    # by default: other row distributions or int64 groups move other bytes
    traffic = counters_for(dom) if args.rows == "zipf" and not wide else None

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(cfg, batch, W0, min(args.cpu_sample_bags, cfg.B))

    result = {
        "metric": "TBE fwd+bwd(Adagrad) ms and achieved HBM GB/s % peak, T=32 B=128K D=128",
        "value": round(wall_ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "graph_ms_per_step": g_ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "T=32 E=2M D=128 bf16 B=131072 Poisson(20) "
                               + ("Zipf-Mandelbrot" if args.rows == "zipf" else "uniform")
                               + f" rows, weighted, preprocessing in {args.preprocess}"
                               + ("" if args.check == "none" else f", index check: {args.check}")
                               + (", long runs in one launch" if fused_long else "")
                               + (", int64 indices and offsets" if wide else ""),
                   "T": cfg.T, "E": cfg.rows[0], "D": cfg.D, "B": cfg.B, "N": N, "U": U,
                   "long_runs": n_long, "chunks": n_chunks, "long_lookups": long_lookups,
                   "parallelism": "single GPU"},
        "stages_ms": {k: round(v, 4) for k, v in avg.items() if st[k][1]},
        "fwd_ms": round(fwd_ms, 4),
        "pre_ms": round(pre_ms, 4),
        "fwd_total_ms": round(fwd_ms + pre_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "combined_ms": round(fwd_ms + pre_ms + bwd_ms, 4),
        "fwd_gather": {"bytes": by["fwd"], "GBps": round(fwd_gbps, 1),
                       "frac_peak": round(fwd_gbps / PEAK_HBM_GBPS, 4)},
        "bwd_accumulate_apply": {"bytes": by["bwd"], "GBps": round(bwd_gbps, 1),
                                 "frac_peak": round(bwd_gbps / PEAK_HBM_GBPS, 4)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": dom_bytes,
                     "avg_launch_ms": round(dom_ms, 4), **traffic_rate(traffic, dom_ms)},
        "cpu_baseline": cpu,
        "stream_copy_GBps": stream_copy_gbps(torch, torch.device("cuda")),
        "context": "B200 figures on the pages (not this workload's hardware): combined "
                   "79.537 ms -> 66.183 ms with forward-side preprocessing",
    }
    print(json.dumps(result), flush=True)


def main_small(args, torch, tbe):
    from workloads import WORKLOADS, TINY, DEMO3, MEDIUM, LARGE, SMALL_TABLE, init_state, init_weights, make_batch
    cfg = SMALL_TABLE
    log("generating the small-table batch")
    batch = make_batch(cfg)
    N = batch.indices.size
    dev = torch.device("cuda")
    idx = torch.from_numpy(batch.indices).to(dev)
    off = torch.from_numpy(batch.offsets).to(dev)
    grad = torch.from_numpy(batch.grad).to(dev)
    W = init_weights(cfg, dev)
    W0 = W.clone() if not args.no_cpu_baseline else None
    m = init_state(cfg, dev)
    out = torch.empty((cfg.B, cfg.T * cfg.D), dtype=torch.float32, device=dev)
    timer = tbe.Timer(capacity=args.steps + 1)
    desc = tbe.Desc(cfg.T, cfg.D, cfg.B, cfg.rows, cfg.dtype)
    assert tbe.tbe_select_path(desc, N, False) == tbe.TBE_PATH_SMALL_TABLE
    meta = tbe.Meta(desc, N, False)
    ws_f = tbe.workspace(desc, N, False, tbe.TBE_OP_FORWARD_PREPROCESS)
    ws_b = tbe.workspace(desc, N, False, tbe.TBE_OP_BACKWARD)
    if args.profile_copy:
        profile_copy(torch, dev)
    torch.cuda.synchronize()

    def step():
        tbe.tbe_forward(desc, W, idx, off, None, out, meta, ws_f)
        tbe.tbe_backward_adagrad(desc, W, m, grad, idx, off, None, meta, cfg.lr, cfg.eps, ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    desc.set_timer(timer)
    timer.reset()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    desc.set_timer(None)
    st = timer.read()
    g_ms = graph_ms(torch, step, args.steps)
    avg = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in st.items()}
    by = small_table_bytes(cfg, N)
    fwd_ms, bwd_ms = avg["small_count"] + avg["small_fwd"], avg["small_bwd"] + avg["small_apply"]
    # dominant single kernel: the longest of the one-kernel stages (small_fwd
    # also holds the recounting kernel's launch, which exits at once here)
    cand = {k: (avg[k], by[k]) for k in ("small_count", "small_fwd", "small_bwd")}
    dom = max(cand, key=lambda k: cand[k][0])
    achieved = cand[dom][1] / (cand[dom][0] * 1e6)
    traffic = counters_for(dom, SMALL_COUNTERS)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(cfg, batch, W0, min(args.cpu_sample_bags // 8, cfg.B))
    result = {
        "metric": "TBE small-table path fwd+bwd(Adagrad) ms and achieved HBM GB/s % peak, "
                  "T=64 E=64 B=32K D=128",
        "value": round(wall_ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall_ms, 4), "graph_ms_per_step": g_ms,
        "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "T=64 E=64 D=128 f16 B=32768 L=64 uniform rows, small-table "
                               "histogram path", "T": cfg.T, "E": 64, "D": cfg.D, "B": cfg.B, "N": N,
                   "parallelism": "single GPU"},
        "stages_ms": {k: round(v, 4) for k, v in avg.items() if st[k][1]},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "combined_ms": round(fwd_ms + bwd_ms, 4),
        "fwd": {"bytes": by["fwd"], "GBps": round(by["fwd"] / (fwd_ms * 1e6), 1),
                "frac_peak": round(by["fwd"] / (fwd_ms * 1e6) / PEAK_HBM_GBPS, 4),
                "mfma_TFLOPs": round(by["fwd_flop"] / (avg["small_fwd"] * 1e9), 2)},
        "bwd": {"bytes": by["bwd"], "GBps": round(by["bwd"] / (bwd_ms * 1e6), 1),
                "frac_peak": round(by["bwd"] / (bwd_ms * 1e6) / PEAK_HBM_GBPS, 4),
                "mfma_TFLOPs": round(by["bwd_flop"] / (avg["small_bwd"] * 1e9), 2)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": cand[dom][1],
                     "avg_launch_ms": round(cand[dom][0], 4), **traffic_rate(traffic, cand[dom][0])},
        "cpu_baseline": cpu,
        "stream_copy_GBps": stream_copy_gbps(torch, torch.device("cuda")),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
