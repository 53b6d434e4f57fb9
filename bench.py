"""Benchmark of the DLRM sparse hot path on one MI355X.

One step = the whole path over one synthetic batch of the multi-hot bf16
workload (26 tables, D=128, B=16384, bag lengths truncated-geometric on
[1,100] with mean 20, Zipf(1.05) rows):
    emb_bag_fwd -> dlrm_interact_fwd -> dlrm_interact_bwd -> emb_bag_bwd_adagrad
(sort / unique / segment-reduce / row-wise Adagrad in place on the bf16
tables, all integer outputs requested), every call in order on one stream.  The
step is also timed with the batch-only half of the embedding backward
(emb_bag_bwd_plan: keys, sort, segments) on a second stream beside the lookup
and the interaction, emb_bag_bwd_apply following the interaction backward (the
results are the same bits); --overlap-plan makes that form the headline.
Inputs are resident in HBM before the timed region; R pre-generated batches
rotate.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rotate R] [--no-cpu] [--overlap-plan]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_multihot_bf16.md")


def measured_traffic(kernel: str, workload: str, path: str = TRAFFIC_PROFILE, root: str = ROOT):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None when the summary is
    missing, covers another workload, or the kernel's sources changed since it was taken."""
    import hashlib
    try:
        line = next(l for l in open(path) if l.startswith("traffic-json: "))
    except (OSError, StopIteration):
        return None
    rec = json.loads(line[len("traffic-json: "):])
    e = rec.get("kernels", {}).get(kernel)
    if rec.get("workload") != workload or e is None:
        return None
    h = hashlib.sha256()
    for f in e["sources"]:
        h.update(f.encode())
        h.update(b"\0")
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != e["source_sha256"]:
        return None
    return {"bytes": e["read_bytes"] + e["write_bytes"], "read": e["read_bytes"],
            "write": e["write_bytes"]}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(wl, batches, n_samples: int, min_seconds: float = 10.0):
    """The oracle, as it stands, on a bounded sample of the same workload (host cores): the full
    step on the first n_samples samples of successive batches, until about min_seconds of work."""
    import oracle
    from recommendation_model_sparse_amd.synth import subset_tables

    cores = len(os.sched_getaffinity(0))
    S = np.arange(n_samples)
    done, lookups, dt = 0, 0, 0.0
    for batch in batches:
        sub_wl, sub, row_ids = batch.sample_subset(S)
        tabs = subset_tables(wl, row_ids)
        states = [np.zeros(len(r), np.float32) for r in row_ids]
        g = batch.grad_out()[S]
        t0 = time.perf_counter()
        pooled, _ = oracle.emb_bag_fwd(tabs, sub.indices, sub.offsets, sub.weights, len(S), threads=cores)
        p32 = pooled.astype(np.float32)
        oracle.interact_fwd(sub.dense, p32, threads=cores)
        _, gp, _, _ = oracle.interact_bwd(g, sub.dense, p32, threads=cores)
        oracle.emb_bag_bwd_adagrad(tabs, states, sub.indices, sub.offsets, sub.weights, len(S),
                                   gp.astype(np.float32), wl.lr, wl.eps)
        dt += time.perf_counter() - t0
        done += len(S)
        lookups += sub.nnz
        if dt >= min_seconds:
            break
    return {"value": done / dt, "unit": "samples/s", "cores": cores, "kind": "oracle",
            "sample": f"{done // len(S)} batch(es) x {len(S)} of {wl.B} samples ({lookups} lookups): the full "
                      f"step (pool, interaction fwd/bwd, sort/segment/Adagrad) in fp64, {dt:.1f} s"}


def time_inference(tabs, batches, steps, pooled, inter):
    """Mean ms of emb_bag_interact_fwd and of emb_bag_fwd + dlrm_interact_fwd (HIP events)."""
    import torch
    from recommendation_model_sparse_amd import dlrm_interact_fwd, emb_bag_fwd, emb_bag_interact_fwd

    def fused(b):
        emb_bag_interact_fwd(tabs, b["idx"], b["off"], None, b["dense"], out=inter)

    def two(b):
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)
        dlrm_interact_fwd(b["dense"], pooled, out=inter)

    res = {}
    for name, fn in (("fused", fused), ("two_call", two)):
        for i in range(3):
            fn(batches[i % len(batches)])
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            fn(batches[i % len(batches)])
        ev[1].record()
        torch.cuda.synchronize()
        res[name] = ev[0].elapsed_time(ev[1]) / steps
    return res


def time_variants(tabs, states, batches, steps, ws, outs, gpooled, wl):
    """Mean ms (HIP events) of the path variants on the same batches: bf16 pooled output, int32
    indices and offsets, the SGD backward (updates the tables in place), and the weighted lookup
    and Adagrad backward with per-sample weights U(0,1) (seeded, one array per batch)."""
    import torch
    from recommendation_model_sparse_amd import (DLRM_OPT_SGD, emb_bag_bwd_adagrad, emb_bag_bwd_update,
                                                 emb_bag_fwd, emb_bag_fwd_ex)

    dev = tabs[0].device
    b32 = [dict(idx=b["idx"].to(torch.int32), off=b["off"].to(torch.int32)) for b in batches]
    pooled_bf16 = torch.empty((wl.B, wl.T, wl.D), dtype=torch.bfloat16, device=dev)
    pooled = torch.empty((wl.B, wl.T, wl.D), dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(wl.seed + 7)
    wts = [torch.rand(b["idx"].numel(), generator=gen, device=dev) for b in batches]
    runs = {
        "fwd_weighted": lambda i: emb_bag_fwd(tabs, batches[i]["idx"], batches[i]["off"], wts[i], out=pooled),
        "bwd_adagrad_weighted": lambda i: emb_bag_bwd_adagrad(tabs, states, batches[i]["idx"], batches[i]["off"],
                                                              wts[i], gpooled, wl.lr, wl.eps, workspace=ws,
                                                              outputs=outs),
        "fwd_bf16_out": lambda i: emb_bag_fwd_ex(tabs, batches[i]["idx"], batches[i]["off"], None, out=pooled_bf16,
                                                 out_dtype=torch.bfloat16),
        "fwd_int32_indices": lambda i: emb_bag_fwd_ex(tabs, b32[i]["idx"], b32[i]["off"], None),
        "bwd_sgd": lambda i: emb_bag_bwd_update(tabs, None, batches[i]["idx"], batches[i]["off"], None, gpooled,
                                                DLRM_OPT_SGD, wl.lr, 0.0, workspace=ws, outputs=outs),
    }
    res = {}
    for name, fn in runs.items():
        for i in range(2):
            fn(i % len(batches))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            fn(i % len(batches))
        ev[1].record()
        torch.cuda.synchronize()
        res[name + "_ms"] = ev[0].elapsed_time(ev[1]) / steps
    return res


def time_full_step(tabs, states, batches, host_batches, steps, wl, max_nnz):
    """The full single-GPU DLRM training step around the sparse path: bottom MLP 13-512-256-128,
    the lookup, the interaction, top MLP 480-1024-1024-512-256 and the sigmoid + BCE head, the
    backward pass, SGD on the dense layers and row-wise Adagrad on the tables (HIP events)."""
    import torch
    from recommendation_model_sparse_amd.dlrm_step import DlrmStep

    from recommendation_model_sparse_amd import dlrm_synth_fill_table, synth

    dev = tabs[0].device
    # start from the initial tables: the timed regions before this one updated them with
    # synthetic upstream gradients, which are no training signal
    for t, (x, v) in enumerate(zip(tabs, wl.rows)):
        dlrm_synth_fill_table(x, t, wl.seed_tab(), float(synth.table_scale(v)))
    for st in states:
        st.zero_()
    m = DlrmStep(tabs, states, wl.B, 13, bottom=[512, 256, wl.D], top=[1024, 1024, 512, 256], lr_dense=0.01,
                 lr_emb=wl.lr, eps=wl.eps, seed=wl.seed + 99, max_nnz=max_nnz)
    extra = [(torch.from_numpy(hb.features(13)).to(dev), torch.from_numpy(hb.labels()).to(dev)) for hb in host_batches]

    def run(i):
        b = batches[i % len(batches)]
        x, y = extra[i % len(extra)]
        m.step(b["idx"], b["off"], x, y)

    def region(overlap):
        m.overlap = overlap
        for i in range(2):
            run(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            run(i)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    ms_one = region(False)
    ms = region(True)
    dims_b = [(16, 512), (512, 256), (256, wl.D)]
    dims_t = [(m.Ip, 1024), (1024, 1024), (1024, 512), (512, 256), (256, 1)]
    flops = 3 * 2 * wl.B * sum(k * n for k, n in dims_b + dims_t)  # forward + two backward GEMMs
    return {"ms_per_step": ms, "samples_per_s": wl.B / (ms / 1e3), "ms_per_step_one_stream": ms_one,
            "dense_gemm_tflop_per_step": flops / 1e12,
            "loss_after": float(m.head_out["loss"].item()),
            "layers": "bottom 13(16)-512-256-128, top 480-1024-1024-512-256-1, bf16 GEMMs (hipBLASLt), fp32 accumulation"}


def hbm_context(dev):
    """What plain streaming reaches on this GPU, as context for the kernels' figures: a 2 GiB
    device-to-device copy, far larger than the caches (read + write bytes; HIP events, median of 5)."""
    import torch
    n = 1 << 29  # 2 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def med(fn):
        ts = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts[1:])) / 1e3

    t_copy = med(lambda: dst.copy_(src))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_GBps": 2 * 4 * n / t_copy / 1e9, "bytes_copied": 4 * n,
            "how": "2 GiB fp32 device copy, read + write bytes over its time, median of 5"}


def inference_summary(inf, wl, nnz_avg):
    D, T, B, N, P = wl.D, wl.T, wl.B, wl.N, wl.P
    alg = nnz_avg * (D * wl.elem_size + 8) + (T * B + 1) * 8 + B * D * 4 + B * (P + D) * 4
    f = inf["fused"] / 1e3
    return {"fused_ms": inf["fused"], "two_call_ms": inf["two_call"],
            "fused_samples_per_s": B / f, "two_call_samples_per_s": B / (inf["two_call"] / 1e3),
            "speedup": inf["two_call"] / inf["fused"],
            "fused_algorithmic_bytes": alg, "fused_GBps": alg / f / 1e9,
            "fused_frac_hbm_peak": alg / f / 1e9 / HBM_PEAK_GBPS,
            "gathered_GBps": nnz_avg * D * wl.elem_size / f / 1e9}


def bench_inference_big(args, dev):
    """Inference on one GPU's share of 8 x 50M-row bf16 tables (102.4 GB), one-hot, B=65536."""
    import torch
    from recommendation_model_sparse_amd import dlrm_synth_fill_table, synth
    from recommendation_model_sparse_amd.configs import make_config

    wl = make_config(4)
    if args.dist == "zipf":
        wl = wl.with_(dist="zipf", alpha=1.2)
    log(f"[bench] workload {wl.name} ({args.dist})")
    tabs = []
    for t, v in enumerate(wl.rows):
        x = torch.empty((v, wl.D), dtype=torch.bfloat16, device=dev)
        dlrm_synth_fill_table(x, t, wl.seed_tab(), float(synth.table_scale(v)))
        tabs.append(x)
    batches = []
    for i in range(args.rotate):
        b = wl.batch(i)
        batches.append(dict(idx=torch.from_numpy(b.indices).to(dev), off=torch.from_numpy(b.offsets).to(dev),
                            dense=torch.from_numpy(b.dense).to(dev), nnz=b.nnz))
    pooled = torch.empty((wl.B, wl.T, wl.D), dtype=torch.float32, device=dev)
    inter = torch.empty((wl.B, wl.P + wl.D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    inf = time_inference(tabs, batches, args.steps, pooled, inter)
    hbm = hbm_context(dev)
    nnz_avg = float(np.mean([b["nnz"] for b in batches]))
    summ = inference_summary(inf, wl, nnz_avg)
    res = {
        "metric": "inference samples/sec (lookup fused with the interaction), 1 MI355X",
        "value": summ["fused_samples_per_s"], "unit": "samples/s", "n_gpus": 1, "steps": args.steps,
        "warmup": 3, "ms_per_step": inf["fused"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic (seeded; counter-hash tables, {'Zipf(1.2)' if args.dist == 'zipf' else 'uniform'} rows)",
        "config": {"workload": "one-hot inference: 8 bf16 tables of 50M x 128 (102.4 GB), B=65536, N=9",
                   "global_batch": wl.B, "tables": wl.T, "D": wl.D, "table_dtype": "bf16",
                   "table_GB": wl.table_bytes() / 1e9, "parallelism": "single GPU"},
        "inference": summ,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--cpu-samples", type=int, default=16384)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--overlap-plan", action="store_true",
                    help="headline the step form with the backward's sort on a second stream")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    ap.add_argument("--dist", choices=["zipf", "uniform"], default="zipf",
                    help="row distribution of the lookups (uniform: a cache-cold control)")
    ap.add_argument("--workload", choices=["multihot", "onehot-big"], default="multihot",
                    help="multihot: the training step (default); onehot-big: inference only "
                         "(fused lookup + interaction against the two calls) on 8 x 50M-row "
                         "bf16 tables, B=65536 one-hot, uniform or --dist zipf (Zipf 1.2)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path is "
              f"single-GPU: tables are not sharded and no collective runs).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy probe: 3 copies of 1 GiB")
        return
    from recommendation_model_sparse_amd import (DLRM_OPT_ADAGRAD, AdagradOutputs, dlrm_interact_bwd,
                                                 dlrm_interact_fwd, dlrm_synth_fill_table, dlrm_trace_enable,
                                                 dlrm_trace_read, emb_bag_bwd_adagrad, emb_bag_bwd_apply,
                                                 emb_bag_bwd_plan, emb_bag_bwd_workspace_size, emb_bag_fwd,
                                                 synth)
    from recommendation_model_sparse_amd.configs import make_config

    dev = torch.device("cuda:0")
    if args.workload == "onehot-big":
        return bench_inference_big(args, dev)
    wl = make_config(3)
    if args.dist == "uniform":
        wl = wl.with_(dist="uniform")
    log(f"[bench] workload {wl.name}: {wl.note}")
    t0 = time.time()
    tabs = []
    for t, v in enumerate(wl.rows):
        x = torch.empty((v, wl.D), dtype=torch.bfloat16, device=dev)
        dlrm_synth_fill_table(x, t, wl.seed_tab(), float(synth.table_scale(v)))
        tabs.append(x)
    states = [torch.zeros(v, dtype=torch.float32, device=dev) for v in wl.rows]
    torch.cuda.synchronize()
    log(f"[bench] tables {wl.table_bytes() / 1e9:.2f} GB filled in {time.time() - t0:.1f}s")

    batches, host_batches = [], []
    for i in range(args.rotate):
        b = wl.batch(i)
        host_batches.append(b)
        batches.append(dict(idx=torch.from_numpy(b.indices).to(dev),
                            off=torch.from_numpy(b.offsets).to(dev),
                            dense=torch.from_numpy(b.dense).to(dev),
                            g=torch.from_numpy(b.grad_out()).to(dev), nnz=b.nnz))
        log(f"[bench] batch {i}: nnz={b.nnz}")
    max_nnz = max(b["nnz"] for b in batches)
    ws = torch.empty(emb_bag_bwd_workspace_size(wl.rows, wl.D, wl.B, max_nnz), dtype=torch.uint8, device=dev)
    outs = AdagradOutputs(max_nnz, dev)
    pooled = torch.empty((wl.B, wl.T, wl.D), dtype=torch.float32, device=dev)
    inter = torch.empty((wl.B, wl.P + wl.D), dtype=torch.float32, device=dev)
    gdense = torch.empty((wl.B, wl.D), dtype=torch.float32, device=dev)
    gpooled = torch.empty_like(pooled)
    names = ["emb_bag_fwd", "dlrm_interact_fwd", "dlrm_interact_bwd", "emb_bag_bwd_adagrad"]

    def step(i, ev=None):
        b = batches[i % len(batches)]
        if ev is not None:
            ev[0].record()
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)
        if ev is not None:
            ev[1].record()
        dlrm_interact_fwd(b["dense"], pooled, out=inter)
        if ev is not None:
            ev[2].record()
        dlrm_interact_bwd(b["g"], b["dense"], pooled, grad_dense=gdense, grad_pooled=gpooled)
        if ev is not None:
            ev[3].record()
        emb_bag_bwd_adagrad(tabs, states, b["idx"], b["off"], None, gpooled, wl.lr, wl.eps,
                            workspace=ws, outputs=outs)
        if ev is not None:
            ev[4].record()

    side = torch.cuda.Stream(device=dev)  # default priority
    plan_done = torch.cuda.Event()

    def step_overlap(i):
        b = batches[i % len(batches)]
        main = torch.cuda.current_stream(dev)
        side.wait_stream(main)  # the previous step's update has read the workspace
        with torch.cuda.stream(side):
            emb_bag_bwd_plan(wl.rows, wl.D, b["idx"], b["off"], None, ws, outputs=outs)
            plan_done.record(side)
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)
        dlrm_interact_fwd(b["dense"], pooled, out=inter)
        dlrm_interact_bwd(b["g"], b["dense"], pooled, grad_dense=gdense, grad_pooled=gpooled)
        main.wait_event(plan_done)
        emb_bag_bwd_apply(tabs, states, wl.B, b["nnz"], False, gpooled, DLRM_OPT_ADAGRAD, wl.lr, wl.eps, ws,
                          outputs=outs)

    def timed(fn):
        """Whole-step wall clock over args.steps steps between two synchronisations (ms/step)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    for i in range(args.warmup):
        step(i)
        step_overlap(i)
    torch.cuda.synchronize()

    # timed region: the step as configured; the other form timed beside it for the record
    headline = step_overlap if args.overlap_plan else step
    ms = timed(headline)
    ms_other = timed(step if args.overlap_plan else step_overlap)
    ms_ovl, ms_one = (ms, ms_other) if args.overlap_plan else (ms_other, ms)
    log(f"[bench] ms/step: one stream {ms_one:.4f}, plan overlapped {ms_ovl:.4f}")

    # per-call HIP event times on the launching stream, over a second identical region
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_ms = {n: float(np.mean([evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(args.steps)]))
               for k, n in enumerate(names)}
    step_ev_ms = np.array([evs[i][0].elapsed_time(evs[i][4]) for i in range(args.steps)])
    step_pct = {f"p{q}": float(np.percentile(step_ev_ms, q)) for q in (10, 50, 90)}
    log("[bench] per call (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in call_ms.items()))

    # per-kernel HIP event times recorded by the library itself (dlrm_trace_*), third region
    dlrm_trace_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    trace = dlrm_trace_read()
    dlrm_trace_enable(False)
    kern_ms = {k: ms / args.steps for k, (n, ms) in trace.items()}  # per step
    kern_launch_ms = {k: ms / n for k, (n, ms) in trace.items()}    # per launch
    log("[bench] per kernel (ms/step): " + ", ".join(f"{k}={v:.4f}" for k, v in
                                                     sorted(kern_ms.items(), key=lambda x: -x[1])))

    # inference: the fused lookup + interaction against the two calls, same batches and tables
    inf = time_inference(tabs, batches, args.steps, pooled, inter)
    variants = time_variants(tabs, states, batches, args.steps, ws, outs, gpooled, wl)
    full = time_full_step(tabs, states, batches, host_batches, args.steps, wl, max_nnz)

    hbm = hbm_context(dev)
    nnz_avg = float(np.mean([b["nnz"] for b in batches]))
    U_last = int(outs.num_unique.item())
    es = wl.elem_size
    D, T, B, N, P = wl.D, wl.T, wl.B, wl.N, wl.P
    gathered = nnz_avg * D * es
    sort_passes = round(kern_ms.get("radix_scatter", 0.0) / kern_launch_ms["radix_scatter"]) \
        if kern_launch_ms.get("radix_scatter") else 0
    # algorithmic bytes per launch of the main kernels
    alg = {
        "pool_wave_per_bag": gathered + nnz_avg * 8 + (T * B + 1) * 8 + B * T * D * 4,
        # sorted key + grad-row index per lookup, each pooled-gradient row once (the kernel reads
        # it once per lookup: the re-reads are served by L2 / Infinity Cache or count in traffic),
        # each touched table row read and written, its state read and written
        "seg_reduce_adagrad": nnz_avg * 8 + B * T * D * 4 + U_last * (2 * D * es + 8),
        "interact_fwd_mfma": B * (N * D * 4 + (P + D) * 4),
        "interact_bwd": B * ((P + D) * 4 + 2 * N * D * 4),
        # key, grad row and position read and written per pass; the first pass makes the
        # positions instead of reading them (mean over the passes)
        "radix_scatter": nnz_avg * (3 * 4 * 2 - 4 / max(1, sort_passes)),
        "radix_hist": nnz_avg * 4,
        # index read, key and grad row written per lookup; offsets per bag
        "expand": nnz_avg * (8 + 4 * 2) + (T * B + 1) * 8,
    }
    # what the kernels load including re-reads (one gradient row per lookup in the backward)
    requested = {"seg_reduce_adagrad": nnz_avg * (4 * D + 8) + U_last * (2 * D * es + 8),
                 "pool_wave_per_bag": alg["pool_wave_per_bag"]}
    kernels = {}
    for k, b_alg in alg.items():
        if k in kern_launch_ms:
            gbps = b_alg / (kern_launch_ms[k] / 1e3) / 1e9
            kernels[k] = {"ms_per_launch": kern_launch_ms[k], "ms_per_step": kern_ms[k],
                          "algorithmic_bytes": b_alg, "GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS}
    dominant = max(kern_ms, key=lambda k: kern_ms[k])
    dom = kernels.get(dominant)
    k1_s = call_ms["emb_bag_fwd"] / 1e3
    gathered_gbps = gathered / k1_s / 1e9

    traffic = measured_traffic(dominant, "multihot-bf16-" + args.dist)
    res = {
        "metric": "samples/sec + gathered-embedding GB/s (fraction of HBM peak), 1 MI355X",
        "value": wl.B / (ms / 1e3),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_form": "plan on a second stream" if args.overlap_plan else "one stream",
        "ms_per_step_one_stream": ms_one,
        "ms_per_step_plan_overlapped": ms_ovl,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": f"synthetic (seeded; counter-hash tables U(+-1/sqrt(V)), {args.dist} rows)",
        "config": {"workload": "multi-hot bf16 training step: 26 tables, D=128, B=16384, "
                               "bag length truncated-geometric [1,100] mean 20, "
                               + ("Zipf(1.05)" if args.dist == "zipf" else "uniform") +
                               " rows, V log-uniform [1e3,1e7]",
                   "global_batch": wl.B, "tables": wl.T, "D": wl.D, "table_dtype": "bf16", "nnz_avg": nnz_avg,
                   "table_GB": wl.table_bytes() / 1e9, "parallelism": "single GPU"},
        "gathered_GBps": gathered_gbps,
        "gathered_frac_of_hbm_peak": gathered_gbps / HBM_PEAK_GBPS,
        "hbm_context": hbm,
        "step_ms_per_step_events": step_pct,
        "fwd_samples_per_s": wl.B / ((call_ms["emb_bag_fwd"] + call_ms["dlrm_interact_fwd"]) / 1e3),
        "unique_rows": U_last,
        "call_ms": call_ms,
        "kernel_ms_per_step": kern_ms,
        "roofline": {"bound": "hbm", "kernel": dominant,
                     "achieved": dom["GBps"] if dom else None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dom["frac_hbm_peak"] if dom else None,
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_read_write": [traffic["read"], traffic["write"]] if traffic else None,
                     # the bytes the counters saw per launch over the launch time: how hard the kernel
                     # drives HBM / the Infinity Cache, re-reads included
                     "traffic_GBps": traffic["bytes"] / (kern_launch_ms[dominant] / 1e3) / 1e9 if traffic else None,
                     "ms_per_launch": kern_launch_ms[dominant],
                     "requested_bytes_per_launch": requested.get(dominant),
                     "algorithmic_bytes_per_launch": dom["algorithmic_bytes"] if dom else None},
        "kernels": kernels,
        "inference": inference_summary(inf, wl, nnz_avg),
        "variants": variants,
        "full_step": full,
    }
    if not args.no_cpu:
        log(f"[bench] cpu baseline on {args.cpu_samples} samples ...")
        res["cpu_baseline"] = cpu_baseline(wl, host_batches, args.cpu_samples)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
