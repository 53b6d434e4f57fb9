"""Benchmark of the DLRM sparse hot path on one MI355X.

Headline step = the whole path over one synthetic batch of the multi-hot bf16 workload (26 tables,
D=128, B=16384, bag lengths truncated-geometric on [1,100] with mean 20, Zipf(1.05) rows):
    emb_bag_fwd -> dlrm_interact_fwd -> dlrm_interact_bwd -> emb_bag_bwd_adagrad
(sort / unique / segment-reduce / row-wise Adagrad in place on the bf16 tables, all integer outputs
requested), every call in order on one stream.  The step is also timed with the batch-only half of
the embedding backward (emb_bag_bwd_plan) on a second stream; --overlap-plan makes that the headline.
Inputs are resident in HBM before the timed region; R pre-generated batches rotate.

The same JSON line also carries:
  configs      every workload timed on its own: the tiny forward, the one-hot fp32 forward, the
               multi-hot step with uniform rows (cache-cold control), the big-table forward
               (8 x 50M bf16 rows) with uniform and Zipf(1.2) rows, and the fp32 training step on
               the one-hot shapes;
  gather       per workload, the lookup kernel's time, its logical gathered GB/s, and the HBM bytes
               the counters saw (FETCH_SIZE + WRITE_SIZE, profiles/hbm_traffic_<workload>.md) as
               GB/s and as a fraction of the 8 TB/s HBM peak;
  hbm_context  what plain streaming reaches here: a device copy, a read-only stream, and a gather of
               random 256-byte rows from 102 GB with no output (the cold lookup's read ceiling);
  cpu_baseline the oracle on the host cores (all, and one), samples/s and gathered GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rotate R] [--no-cpu] [--overlap-plan]
                    [--only SECTION]

--only runs one section and prints its object (for profiling runs): headline, tiny, onehot,
multihot-uniform, bigtables-uniform, bigtables-zipf, train-onehot, probes, interaction, inference,
full-step.
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
SECTIONS = ("headline", "tiny", "onehot", "multihot-uniform", "bigtables-uniform", "bigtables-zipf",
            "train-onehot", "probes", "interaction", "inference", "full-step")


def traffic_profile(workload: str) -> str:
    return os.path.join(ROOT, "profiles", "hbm_traffic_" + workload.replace("-", "_") + ".md")


TRAFFIC_PROFILE = traffic_profile("multihot-bf16-zipf")


def measured_traffic(kernel: str, workload: str, path: str = None, root: str = ROOT):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None when the summary is
    missing, covers another workload, or the kernel's sources changed since it was taken."""
    import hashlib
    path = path or traffic_profile(workload)
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
        try:
            with open(os.path.join(root, f), "rb") as fh:
                h.update(fh.read())
        except OSError:
            return None
    if h.hexdigest() != e["source_sha256"]:
        return None
    return {"bytes": e["read_bytes"] + e["write_bytes"], "read": e["read_bytes"],
            "write": e["write_bytes"]}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- timing helpers

def ev_ms(fn, nb: int, steps: int, warm: int = 2) -> float:
    """Mean ms per call of fn(i) over `steps` calls, HIP events on the current stream."""
    import torch
    for i in range(warm):
        fn(i % nb)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        fn(i % nb)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def traced(fn, nb: int, steps: int):
    """{kernel: {launches per call, ms per launch, ms per call}} from the library's own HIP events."""
    import torch
    from recommendation_model_sparse_amd import dlrm_trace_enable, dlrm_trace_read
    torch.cuda.synchronize()
    dlrm_trace_enable(True)
    for i in range(steps):
        fn(i % nb)
    torch.cuda.synchronize()
    tr = dlrm_trace_read()
    dlrm_trace_enable(False)
    return {k: {"launches_per_call": n / steps, "ms_per_launch": ms / n, "ms_per_call": ms / steps}
            for k, (n, ms) in tr.items()}


def dominant(kern: dict) -> str:
    return max(kern, key=lambda k: kern[k]["ms_per_call"])


def lookup_kernel(kern: dict) -> str:
    """The pooling kernel of an emb_bag_fwd trace (the one that ran longest)."""
    pools = {k: v for k, v in kern.items() if k.startswith("pool_")}
    return dominant(pools) if pools else dominant(kern)


def gpu_spinup(dev, seconds: float = 0.3) -> float:
    """Bring the GPU to its working clock before anything is timed: an idle MI355X starts near
    200 MHz and ramps up over the first ~0.1 s of load, so the first steps of a run take close to
    3 times longer.  Plain 256 MB device copies until `seconds` have passed; returns the time spent."""
    import torch
    src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
    del src, dst
    return time.perf_counter() - t0


# ---------------------------------------------------------------- inputs

def device_tables(wl, dev):
    import torch
    from recommendation_model_sparse_amd import dlrm_synth_fill_table, synth
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    if wl.init == "normal":
        tabs = []
        for t in wl.host_tables():
            x = torch.from_numpy(t.view(np.int16) if t.dtype == np.uint16 else t)
            tabs.append((x.view(torch.bfloat16) if t.dtype == np.uint16 else x).to(dev))
        return tabs
    tabs = []
    for t, v in enumerate(wl.rows):
        x = torch.empty((v, wl.D), dtype=dt, device=dev)
        dlrm_synth_fill_table(x, t, wl.seed_tab(), float(synth.table_scale(v)))
        tabs.append(x)
    return tabs


def device_batches(wl, dev, n: int, grads: bool = False):
    import torch
    out, host = [], []
    for i in range(n):
        b = wl.batch(i)
        host.append(b)
        d = dict(idx=torch.from_numpy(b.indices).to(dev), off=torch.from_numpy(b.offsets).to(dev),
                 dense=torch.from_numpy(b.dense).to(dev), nnz=b.nnz)
        if grads:
            d["g"] = torch.from_numpy(b.grad_out()).to(dev)
        out.append(d)
    return out, host


def lookup_bytes(wl, nnz: float):
    """(gathered bytes, all algorithmic bytes) of one lookup call: rows, indices, offsets, fp32 output."""
    gathered = nnz * wl.D * wl.elem_size
    return gathered, gathered + nnz * 8 + (wl.T * wl.B + 1) * 8 + wl.B * wl.T * wl.D * 4


def gather_entry(wl, workload: str, kernel: str, ms: float, nnz: float) -> dict:
    """Lookup bandwidth of one workload: logical (rows gathered / time) and counted (HBM bytes the
    FETCH_SIZE/WRITE_SIZE counters saw per launch / time), each against the 8 TB/s peak."""
    gathered, alg = lookup_bytes(wl, nnz)
    s = ms / 1e3
    tr = measured_traffic(kernel, workload)
    e = {"kernel": kernel, "ms_per_launch": ms, "lookups": nnz, "gathered_bytes": gathered,
         "logical_gathered_GBps": gathered / s / 1e9,
         "logical_gathered_frac_of_hbm_peak": gathered / s / 1e9 / HBM_PEAK_GBPS,
         "algorithmic_bytes": alg, "algorithmic_GBps": alg / s / 1e9,
         "hbm_read_bytes": None, "hbm_write_bytes": None, "hbm_GBps": None, "hbm_frac_of_peak": None,
         "counters": os.path.relpath(traffic_profile(workload), ROOT)}
    if tr:
        e.update(hbm_read_bytes=tr["read"], hbm_write_bytes=tr["write"], hbm_GBps=tr["bytes"] / s / 1e9,
                 hbm_frac_of_peak=tr["bytes"] / s / 1e9 / HBM_PEAK_GBPS)
    return e


# ---------------------------------------------------------------- forward-only workloads

def bench_forward(wl, workload: str, dev, steps: int, rotate: int, probe_gather: bool = False):
    """Lookup alone, the interaction alone, the two calls, and the fused call (HIP events)."""
    import torch
    from recommendation_model_sparse_amd import TableSet, dlrm_interact_fwd, emb_bag_fwd, emb_bag_interact_fwd
    t0 = time.time()
    tabs = TableSet(device_tables(wl, dev))
    batches, _ = device_batches(wl, dev, rotate)
    pooled = torch.empty((wl.B, wl.T, wl.D), dtype=torch.float32, device=dev)
    inter = torch.empty((wl.B, wl.P + wl.D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {workload}: {wl.table_bytes() / 1e9:.2f} GB of tables, inputs ready in {time.time() - t0:.1f}s")
    nb = len(batches)

    def look(i):
        b = batches[i]
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)

    def inter_only(i):
        dlrm_interact_fwd(batches[i]["dense"], pooled, out=inter)

    def two(i):
        look(i)
        inter_only(i)

    def fused(i):
        b = batches[i]
        emb_bag_interact_fwd(tabs, b["idx"], b["off"], None, b["dense"], out=inter)

    ms = {"lookup": ev_ms(look, nb, steps), "interaction": ev_ms(inter_only, nb, steps),
          "two_call": ev_ms(two, nb, steps), "fused": ev_ms(fused, nb, steps)}
    kern = traced(two, nb, steps)
    kern.update({("fused:" + k): v for k, v in traced(fused, nb, steps).items()})
    nnz = float(np.mean([b["nnz"] for b in batches]))
    lk = lookup_kernel({k: v for k, v in kern.items() if not k.startswith("fused:")})
    gathered, alg = lookup_bytes(wl, nnz)
    B = wl.B
    res = {"workload": wl.note, "B": B, "tables": wl.T, "D": wl.D, "table_dtype": wl.dtype,
           "table_GB": wl.table_bytes() / 1e9, "lookups_per_batch": nnz, "ms": ms,
           "fwd_samples_per_s": B / (min(ms["two_call"], ms["fused"]) / 1e3),
           "two_call_samples_per_s": B / (ms["two_call"] / 1e3), "fused_samples_per_s": B / (ms["fused"] / 1e3),
           "fused_speedup": ms["two_call"] / ms["fused"],
           "lookup_gathered_GBps": gathered / (ms["lookup"] / 1e3) / 1e9,
           "lookup_algorithmic_GBps": alg / (ms["lookup"] / 1e3) / 1e9,
           "kernels": kern}
    gat = gather_entry(wl, workload, lk, kern[lk]["ms_per_launch"], nnz)
    extra = {}
    if probe_gather:
        # the same number of random rows of the same tables, read with no output written: the
        # lookup's read ceiling on this GPU for this access pattern
        from recommendation_model_sparse_amd import dlrm_probe_gather
        sink = torch.empty(4096, dtype=torch.int32, device=dev)
        gen = torch.Generator(device=dev).manual_seed(wl.seed + 17)
        per_t = 1 << 20  # 256 MB of 256-byte rows per launch: far above launch overhead and the caches
        rows = [torch.randint(0, v, (per_t,), generator=gen, device=dev, dtype=torch.int64) for v in wl.rows]
        t_probe = ev_ms(lambda i: [dlrm_probe_gather(tabs[t], rows[t], sink) for t in range(wl.T)], 1, steps)
        nbytes = per_t * wl.T * wl.D * wl.elem_size
        extra = {"random_row_read_GBps": nbytes / (t_probe / 1e3) / 1e9, "random_rows": per_t * wl.T,
                 "row_bytes": wl.D * wl.elem_size,
                 "how": f"dlrm_probe_gather: {per_t} uniform random rows of each of the {wl.T} tables, "
                        f"no output; HIP events over {steps} passes"}
    del tabs
    torch.cuda.empty_cache()
    return res, gat, extra


# ---------------------------------------------------------------- the interaction's Gram paths

def bench_interaction_paths(dev, steps: int):
    """dlrm_interact_fwd_ex on each Gram path (the automatic choice, the fp32 matrix-core Gram, the
    LDS-staged VALU Gram) at the multi-hot shape (N=27, D=128, B=16384) and the big-table shape
    (N=9, D=128, B=65536), on seeded N(0,1) inputs resident in HBM; HIP events."""
    import torch
    from recommendation_model_sparse_amd import (DLRM_GRAM_AUTO, DLRM_GRAM_MFMA, DLRM_GRAM_VALU,
                                                 dlrm_interact_fwd_ex)
    res = {}
    gen = torch.Generator(device=dev).manual_seed(20261227)
    for name, N, D, B in (("multihot_N27", 27, 128, 16384), ("bigtables_N9", 9, 128, 65536)):
        dense = torch.randn((B, D), generator=gen, device=dev)
        pooled = torch.randn((B, N - 1, D), generator=gen, device=dev)
        P = N * (N - 1) // 2
        out = torch.empty((B, P + D), device=dev)
        alg = B * (N * D * 4 + (P + D) * 4)
        r = {"N": N, "D": D, "B": B, "algorithmic_bytes": alg, "gflop": 2.0 * D * P * B / 1e9}
        for pname, path in (("auto", DLRM_GRAM_AUTO), ("mfma", DLRM_GRAM_MFMA), ("valu_lds", DLRM_GRAM_VALU)):
            ms = ev_ms(lambda i: dlrm_interact_fwd_ex(dense, pooled, path, out=out), 1, steps, 3)
            r[pname] = {"ms": ms, "GBps": alg / (ms / 1e3) / 1e9, "TFLOPs": 2.0 * D * P * B / (ms / 1e3) / 1e12}
        res[name] = r
        log(f"[bench] interaction {name}: " + ", ".join(f"{k} {r[k]['ms'] * 1e3:.1f} us" for k in
                                                        ("auto", "mfma", "valu_lds")))
        del dense, pooled, out
    return res


# ---------------------------------------------------------------- the fp32 training step

def bench_train_onehot(wl, dev, steps: int, rotate: int):
    """The training step on the one-hot fp32 shapes: lookup, interaction forward and backward, and
    the embedding backward with row-wise Adagrad in place (no integer outputs requested)."""
    import torch
    from recommendation_model_sparse_amd import (TableSet, dlrm_interact_bwd, dlrm_interact_fwd, emb_bag_bwd_adagrad,
                                                 emb_bag_bwd_workspace_size, emb_bag_fwd)
    states = [torch.zeros(v, dtype=torch.float32, device=dev) for v in wl.rows]
    # checked once; each call then only re-reads the tensors' pointers and row counts
    tabs = TableSet(device_tables(wl, dev), states)
    batches, _ = device_batches(wl, dev, rotate, grads=True)
    nb = len(batches)
    max_nnz = max(b["nnz"] for b in batches)
    ws = torch.empty(emb_bag_bwd_workspace_size(wl.rows, wl.D, wl.B, max_nnz), dtype=torch.uint8, device=dev)
    pooled = torch.empty((wl.B, wl.T, wl.D), dtype=torch.float32, device=dev)
    inter = torch.empty((wl.B, wl.P + wl.D), dtype=torch.float32, device=dev)
    gd = torch.empty((wl.B, wl.D), dtype=torch.float32, device=dev)
    gp = torch.empty_like(pooled)

    def fwd(i):
        b = batches[i]
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)
        dlrm_interact_fwd(b["dense"], pooled, out=inter)

    def bwd(i):
        b = batches[i]
        dlrm_interact_bwd(b["g"], b["dense"], pooled, grad_dense=gd, grad_pooled=gp)
        emb_bag_bwd_adagrad(tabs, states, b["idx"], b["off"], None, gp, wl.lr, wl.eps, workspace=ws)

    def step(i):
        fwd(i)
        bwd(i)

    for i in range(3):
        step(i % nb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i % nb)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / steps * 1e3
    ms_bwd = ev_ms(bwd, nb, steps)
    kern = traced(step, nb, steps)
    launches = sum(v["launches_per_call"] for v in kern.values())
    # the same steps replayed as HIP graphs, one captured per batch: the library calls allocate
    # nothing and never synchronize, so a step records as is; a replay launches its kernels without
    # the host-side work of the four calls, which at this size is close to the kernels' own time
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    graphs = []
    for i in range(nb):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(3):
        graphs[i % nb].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % nb].replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) / steps * 1e3
    del graphs, tabs, states
    torch.cuda.empty_cache()
    return {"workload": wl.note, "B": wl.B, "tables": wl.T, "D": wl.D, "table_dtype": "f32",
            "ms_per_step": ms_step, "samples_per_s": wl.B / (ms_step / 1e3),
            "ms_per_step_graph": ms_graph, "samples_per_s_graph": wl.B / (ms_graph / 1e3),
            "ms_backward": ms_bwd, "backward_samples_per_s": wl.B / (ms_bwd / 1e3),
            "kernel_launches_per_step": launches,
            "kernel_ms_sum_per_step": sum(v["ms_per_call"] for v in kern.values()), "kernels": kern,
            "note": "wall clock over the timed steps; every call of the step on one stream; _graph: "
                    "the same steps replayed as HIP graphs (one per batch)"}


# ---------------------------------------------------------------- the multi-hot step (headline)

def cpu_baseline(wl, batches, n_samples: int, min_seconds: float = 10.0, one_core_samples: int = 1024,
                 one_core_seconds: float = 4.0):
    """The oracle, as it stands, on bounded samples of the same workload (host cores): the full step
    on the first n_samples samples of successive batches until about min_seconds of work, with every
    core in the affinity mask; the same on one core over one_core_samples samples; and the pooling
    alone on one full batch, as gathered GB/s."""
    import oracle
    from recommendation_model_sparse_amd.synth import subset_tables

    cores = len(os.sched_getaffinity(0))

    def run(samples, threads, budget):
        S = np.arange(samples)
        done, lookups, dt, dt_pool = 0, 0, 0.0, 0.0
        for batch in batches:
            sub_wl, sub, row_ids = batch.sample_subset(S)
            tabs = subset_tables(wl, row_ids)
            states = [np.zeros(len(r), np.float32) for r in row_ids]
            g = batch.grad_out()[S]
            t0 = time.perf_counter()
            pooled, _ = oracle.emb_bag_fwd(tabs, sub.indices, sub.offsets, sub.weights, len(S), threads=threads)
            dt_pool += time.perf_counter() - t0
            p32 = pooled.astype(np.float32)
            oracle.interact_fwd(sub.dense, p32, threads=threads)
            _, gp, _, _ = oracle.interact_bwd(g, sub.dense, p32, threads=threads)
            oracle.emb_bag_bwd_adagrad(tabs, states, sub.indices, sub.offsets, sub.weights, len(S),
                                       gp.astype(np.float32), wl.lr, wl.eps)
            dt += time.perf_counter() - t0
            done += len(S)
            lookups += sub.nnz
            if dt >= budget:
                break
        return done / dt, done, lookups, dt, dt_pool

    v_all, done, lookups, dt, dt_pool = run(n_samples, cores, min_seconds)
    v_one, done1, _, dt1, _ = run(one_core_samples, 1, one_core_seconds)
    return {"value": v_all, "unit": "samples/s", "cores": cores, "kind": "oracle",
            "sample": f"{done // n_samples} batch(es) x {n_samples} of {wl.B} samples ({lookups} lookups): the full "
                      f"step (pool, interaction fwd/bwd, sort/segment/Adagrad) in fp64, {dt:.1f} s",
            "value_1_core": v_one, "cores_1": 1,
            "sample_1_core": f"{done1 // one_core_samples} batch(es) x {one_core_samples} samples, the same step "
                             f"on one thread, {dt1:.1f} s",
            # the pooling step of the all-core run alone, by the GPU's formula (rows gathered / time)
            "gathered_GBps": lookups * wl.D * wl.elem_size / dt_pool / 1e9,
            "gathered_sample": f"the oracle's pooling in the all-core run ({lookups} lookups, {cores} threads), "
                               f"{dt_pool:.2f} s",
            "threads_note": "pooling and the interaction run on OpenMP threads; the sort, segments and "
                            "Adagrad step of the oracle are single-threaded"}


def bench_headline(args, dev):
    import torch
    from recommendation_model_sparse_amd import (DLRM_OPT_ADAGRAD, AdagradOutputs, TableSet, dlrm_interact_bwd,
                                                 dlrm_interact_fwd, emb_bag_bwd_adagrad, emb_bag_bwd_apply,
                                                 emb_bag_bwd_plan, emb_bag_bwd_workspace_size, emb_bag_fwd)
    from recommendation_model_sparse_amd.configs import make_config

    wl = make_config(3)
    log(f"[bench] workload {wl.name}: {wl.note}")
    t0 = time.time()
    states = [torch.zeros(v, dtype=torch.float32, device=dev) for v in wl.rows]
    # checked once; each call then only re-reads the tensors' pointers and row counts
    tabs = TableSet(device_tables(wl, dev), states)
    torch.cuda.synchronize()
    log(f"[bench] tables {wl.table_bytes() / 1e9:.2f} GB filled in {time.time() - t0:.1f}s")
    batches, host_batches = device_batches(wl, dev, 1 if args.only == "multihot-uniform" else args.rotate,
                                           grads=True)
    for i, b in enumerate(batches):
        log(f"[bench] batch {i}: nnz={b['nnz']}")
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

    if args.only == "multihot-uniform":
        # the uniform control alone (its counter profile must hold no Zipf launches)
        uni, gat_u = bench_multihot_uniform(wl, dev, args, tabs, states, ws, outs, pooled, inter, gdense, gpooled)
        return None, None, uni, gat_u, None
    if args.only == "full-step":
        # the full DLRM training step alone (for its kernel profile)
        gpu_spinup(dev)
        return time_full_step(tabs, states, batches, host_batches, args.steps, wl, max_nnz), None, None, None, None
    if args.only == "inference":
        # the fused lookup + interaction against the two calls alone (for its counter profiles)
        gpu_spinup(dev)
        inf = inference_summary(time_inference(tabs, batches, args.steps, pooled, inter), wl,
                                float(np.mean([b["nnz"] for b in batches])))
        return inf, None, None, None, None

    def timed(fn):
        """Whole-step wall clock over args.steps steps between two synchronisations (ms/step)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps * 1e3

    # before the W warm-up steps: the GPU brought to its working clock, and 50 untimed steps of each
    # step form, because once within a process's first few dozen steps the HIP runtime holds the
    # host for ~35 ms inside a launch (measured: the GPU then idles and one region of 20 steps reads
    # 2.8-3.6 ms/step instead of 1.15); neither is part of the step
    spin = {"seconds": gpu_spinup(dev), "untimed_steps_per_form": 50}
    for i in range(50):
        step(i)
        step_overlap(i)
    torch.cuda.synchronize()
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
    kern = traced(step, len(batches), args.steps)
    kern_ms = {k: v["ms_per_call"] for k, v in kern.items()}  # per step
    kern_launch_ms = {k: v["ms_per_launch"] for k, v in kern.items()}
    log("[bench] per kernel (ms/step): " + ", ".join(f"{k}={v:.4f}" for k, v in
                                                     sorted(kern_ms.items(), key=lambda x: -x[1])))
    extras = {}
    if args.only is None:
        # inference: the fused lookup + interaction against the two calls, same batches and tables
        extras["inference"] = inference_summary(time_inference(tabs, batches, args.steps, pooled, inter), wl,
                                                float(np.mean([b["nnz"] for b in batches])))
        extras["variants"] = time_variants(tabs, states, batches, args.steps, ws, outs, gpooled, wl)
        extras["full_step"] = time_full_step(tabs, states, batches, host_batches, args.steps, wl, max_nnz)

    nnz_avg = float(np.mean([b["nnz"] for b in batches]))
    U_last = int(outs.num_unique.item())
    es = wl.elem_size
    D, T, B, N, P = wl.D, wl.T, wl.B, wl.N, wl.P
    gathered, alg_lookup = lookup_bytes(wl, nnz_avg)
    sort_passes = round(kern_ms.get("radix_scatter", 0.0) / kern_launch_ms["radix_scatter"]) \
        if kern_launch_ms.get("radix_scatter") else 0
    # algorithmic bytes per launch of the main kernels
    alg = {
        "pool_wave_per_bag": alg_lookup,
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
    dom = max(kern_ms, key=lambda k: kern_ms[k])
    dk = kernels.get(dom)
    traffic = measured_traffic(dom, "multihot-bf16-zipf")
    floor = gradient_gather_floor(wl, batches[0], gpooled, args.steps) if dom == "seg_reduce_adagrad" else None
    lk = lookup_kernel(kern)
    res = {
        "metric": "samples/sec + gathered-embedding GB/s (fraction of HBM peak), 1 MI355X",
        "value": wl.B / (ms / 1e3),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_form": "plan on a second stream" if args.overlap_plan else "one stream",
        "spinup": spin,
        "ms_per_step_one_stream": ms_one,
        "ms_per_step_plan_overlapped": ms_ovl,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; counter-hash tables U(+-1/sqrt(V)), zipf rows)",
        "config": {"workload": "multi-hot bf16 training step: 26 tables, D=128, B=16384, "
                               "bag length truncated-geometric [1,100] mean 20, Zipf(1.05) rows, "
                               "V log-uniform [1e3,1e7]",
                   "global_batch": wl.B, "tables": wl.T, "D": wl.D, "table_dtype": "bf16", "nnz_avg": nnz_avg,
                   "table_GB": wl.table_bytes() / 1e9, "parallelism": "single GPU"},
        # rows gathered per second by the lookup: logical bytes, mostly served by L2 and the
        # Infinity Cache at Zipf(1.05); the HBM bytes the counters saw are in gather[...]
        "gathered_GBps": gathered / (call_ms["emb_bag_fwd"] / 1e3) / 1e9,
        "gathered_logical_frac_of_hbm_peak": gathered / (call_ms["emb_bag_fwd"] / 1e3) / 1e9 / HBM_PEAK_GBPS,
        "step_ms_per_step_events": step_pct,
        "fwd_samples_per_s": wl.B / ((call_ms["emb_bag_fwd"] + call_ms["dlrm_interact_fwd"]) / 1e3),
        "bwd_samples_per_s": wl.B / ((call_ms["dlrm_interact_bwd"] + call_ms["emb_bag_bwd_adagrad"]) / 1e3),
        "unique_rows": U_last,
        "call_ms": call_ms,
        "kernel_ms_per_step": kern_ms,
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": dk["GBps"] if dk else None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dk["frac_hbm_peak"] if dk else None,
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_read_write": [traffic["read"], traffic["write"]] if traffic else None,
                     # the bytes the counters saw per launch over the launch time: how hard the kernel
                     # drives HBM / the Infinity Cache, re-reads included
                     "traffic_GBps": traffic["bytes"] / (kern_launch_ms[dom] / 1e3) / 1e9 if traffic else None,
                     "ms_per_launch": kern_launch_ms[dom],
                     "requested_bytes_per_launch": requested.get(dom),
                     "algorithmic_bytes_per_launch": dk["algorithmic_bytes"] if dk else None,
                     # the kernel's own gradient-row loads alone, read with no other work in the
                     # same order (a probe gather): what this access pattern costs on the GPU
                     "gradient_gather_floor": floor,
                     "frac_of_gradient_gather_floor":
                         floor["sorted_order_ms"] / kern_launch_ms[dom] if floor else None},
        "kernels": kernels,
    }
    res.update(extras)
    gat = gather_entry(wl, "multihot-bf16-zipf", lk, kern_launch_ms[lk], nnz_avg)
    # the lookup's row reads alone, in its own order: what that access pattern costs on the GPU
    fl = row_gather_floor(wl, batches[0], args.steps)
    gat["row_gather_floor"] = fl
    gat["frac_of_row_gather_floor"] = fl["ms"] / kern_launch_ms[lk]

    # the same step with uniform rows: the cache-cold control of the lookup and the backward
    uni = gat_u = None
    if args.only is None:
        uni, gat_u = bench_multihot_uniform(wl, dev, args, tabs, states, ws, outs, pooled, inter, gdense, gpooled)
    cpu = None
    if args.only is None and not args.no_cpu:
        log(f"[bench] cpu baseline on {args.cpu_samples} samples ...")
        cpu = cpu_baseline(wl, host_batches, args.cpu_samples)
    del tabs, states, ws
    torch.cuda.empty_cache()
    return res, gat, uni, gat_u, cpu


def bench_multihot_uniform(wl3, dev, args, tabs, states, ws, outs, pooled, inter, gdense, gpooled):
    """The multi-hot step on the same tables with uniform rows (4 batches): lookup alone and the step."""
    import torch
    from recommendation_model_sparse_amd import (dlrm_interact_bwd, dlrm_interact_fwd, emb_bag_bwd_adagrad,
                                                 emb_bag_fwd)
    wl = wl3.with_(dist="uniform")
    batches, _ = device_batches(wl, dev, min(args.rotate, 4), grads=True)
    nb = len(batches)
    if max(b["nnz"] for b in batches) > outs.unique_keys.numel():
        from recommendation_model_sparse_amd import AdagradOutputs, emb_bag_bwd_workspace_size
        n = max(b["nnz"] for b in batches)
        outs = AdagradOutputs(n, dev)
        ws = torch.empty(emb_bag_bwd_workspace_size(wl.rows, wl.D, wl.B, n), dtype=torch.uint8, device=dev)

    def look(i):
        b = batches[i]
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)

    def step(i):
        b = batches[i]
        look(i)
        dlrm_interact_fwd(b["dense"], pooled, out=inter)
        dlrm_interact_bwd(b["g"], b["dense"], pooled, grad_dense=gdense, grad_pooled=gpooled)
        emb_bag_bwd_adagrad(tabs, states, b["idx"], b["off"], None, gpooled, wl.lr, wl.eps, workspace=ws,
                            outputs=outs)

    for i in range(2):
        step(i % nb)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % nb)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    ms_look = ev_ms(look, nb, args.steps)
    kern = traced(step, nb, args.steps)
    nnz = float(np.mean([b["nnz"] for b in batches]))
    lk = lookup_kernel(kern)
    gathered, _ = lookup_bytes(wl, nnz)
    res = {"workload": "multi-hot bf16 step (the headline's shapes and tables) with uniform rows",
           "ms_per_step": ms_step, "samples_per_s": wl.B / (ms_step / 1e3), "lookup_ms": ms_look,
           "lookup_gathered_GBps": gathered / (ms_look / 1e3) / 1e9, "unique_rows": int(outs.num_unique.item()),
           "kernels": kern}
    return res, gather_entry(wl, "multihot-bf16-uniform", lk, kern[lk]["ms_per_launch"], nnz)


# ---------------------------------------------------------------- headline extras (inference, variants, full step)

def gradient_gather_floor(wl, b, grad_pooled, steps):
    """How fast the GPU reads the segment reduce's gradient rows in its own order and nothing else:
    dlrm_probe_gather over the pooled gradient [B*T, D] (fp32) at the grad-row index of every
    lookup, (i) in stable key-sorted order, as the segment reduce walks them, and (ii) in lookup
    order, where a bag's row repeats for each of its lookups (cache hits: the request rate's
    floor).  The index sequences are built here with torch (measurement only)."""
    import torch
    from recommendation_model_sparse_amd import dlrm_probe_gather
    dev = grad_pooled.device
    T, B = wl.T, wl.B
    idx, off = b["idx"], b["off"]
    bag = torch.repeat_interleave(torch.arange(T * B, device=dev), off[1:] - off[:-1])
    t, s = bag // B, bag % B
    base = torch.tensor(np.concatenate([[0], np.cumsum(wl.rows)[:-1]]), dtype=torch.int64, device=dev)
    grow = (s * T + t).contiguous()
    sorted_grow = grow[torch.argsort(base[t] + idx, stable=True)].contiguous()
    table = grad_pooled.view(B * T, wl.D)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    out = {}
    for name, g in (("sorted_order_ms", sorted_grow), ("lookup_order_ms", grow)):
        out[name] = ev_ms(lambda i: dlrm_probe_gather(table, g, sink), 1, steps, warm=3)
    out["rows"] = int(grow.numel())
    out["row_bytes"] = wl.D * 4
    del bag, t, s, grow, sorted_grow
    return out


def row_gather_floor(wl, b, steps):
    """The lookup's row reads alone: dlrm_probe_gather over one buffer that holds all T tables one
    after another (its contents do not matter), at every lookup's global row (table base + index)
    in lookup order; it reads the indices and the rows and writes nothing (the lookup also writes
    the pooled output).  The index sequence is built here with torch (measurement only)."""
    import torch
    from recommendation_model_sparse_amd import dlrm_probe_gather
    idx, off = b["idx"], b["off"]
    dev = idx.device
    T, B = wl.T, wl.B
    big = torch.empty((int(sum(wl.rows)), wl.D), dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32,
                      device=dev)
    t = torch.repeat_interleave(torch.arange(T * B, device=dev) // B, off[1:] - off[:-1])
    base = torch.tensor(np.concatenate([[0], np.cumsum(wl.rows)[:-1]]), dtype=torch.int64, device=dev)
    gidx = (base[t] + idx).contiguous()
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    ms = ev_ms(lambda i: dlrm_probe_gather(big, gidx, sink), 1, steps, warm=3)
    out = {"ms": ms, "rows": int(gidx.numel()), "row_bytes": wl.D * wl.elem_size}
    del big, gidx, t
    torch.cuda.empty_cache()
    return out


def time_inference(tabs, batches, steps, pooled, inter):
    """Mean ms of emb_bag_interact_fwd and of emb_bag_fwd + dlrm_interact_fwd (HIP events)."""
    from recommendation_model_sparse_amd import dlrm_interact_fwd, emb_bag_fwd, emb_bag_interact_fwd

    def fused(i):
        b = batches[i]
        emb_bag_interact_fwd(tabs, b["idx"], b["off"], None, b["dense"], out=inter)

    def two(i):
        b = batches[i]
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)
        dlrm_interact_fwd(b["dense"], pooled, out=inter)

    return {"fused": ev_ms(fused, len(batches), steps, 3), "two_call": ev_ms(two, len(batches), steps, 3)}


def inference_summary(inf, wl, nnz_avg):
    """Fused call against the two calls; with the counters' bytes past L2 per call of each form
    (profiles/hbm_traffic_multihot_bf16_zipf_inference.md) while the kernels' sources match."""
    D, T, B, N, P = wl.D, wl.T, wl.B, wl.N, wl.P
    alg = nnz_avg * (D * wl.elem_size + 8) + (T * B + 1) * 8 + B * D * 4 + B * (P + D) * 4
    f = inf["fused"] / 1e3
    out = {"fused_ms": inf["fused"], "two_call_ms": inf["two_call"],
           "fused_samples_per_s": B / f, "two_call_samples_per_s": B / (inf["two_call"] / 1e3),
           "speedup": inf["two_call"] / inf["fused"],
           "fused_algorithmic_bytes": alg, "fused_GBps": alg / f / 1e9,
           "fused_frac_hbm_peak": alg / f / 1e9 / HBM_PEAK_GBPS,
           "gathered_GBps": nnz_avg * D * wl.elem_size / f / 1e9,
           "fused_hbm_bytes": None, "two_call_hbm_bytes": None}
    wkl = "multihot-bf16-zipf-inference"
    tf = measured_traffic("emb_interact_fwd", wkl)
    tp, ti = measured_traffic("pool_wave_per_bag", wkl), measured_traffic("interact_fwd_mfma_pipe", wkl)
    if tf:
        out["fused_hbm_bytes"] = tf["bytes"]
        out["fused_hbm_GBps"] = tf["bytes"] / f / 1e9
    if tp and ti:
        out["two_call_hbm_bytes"] = tp["bytes"] + ti["bytes"]
    out["counters"] = os.path.relpath(traffic_profile(wkl), ROOT)
    return out


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
        "fwd_int32_indices": lambda i: emb_bag_fwd_ex(tabs, b32[i]["idx"], b32[i]["off"], None, out=pooled),
        "bwd_sgd": lambda i: emb_bag_bwd_update(tabs, None, batches[i]["idx"], batches[i]["off"], None, gpooled,
                                                DLRM_OPT_SGD, wl.lr, 0.0, workspace=ws, outputs=outs),
    }
    return {name + "_ms": ev_ms(fn, len(batches), steps) for name, fn in runs.items()}


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
        return ev_ms(run, len(batches), steps)

    ms_one = region(False)
    ms = region(True)
    # the same steps (sort on the second stream) replayed as HIP graphs, one captured per batch
    # after the regions above have run every call once (hipBLASLt picks its algorithms on a
    # shape's first call, which must not happen inside a capture)
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    graphs = []
    for i in range(len(batches)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(3):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) / steps * 1e3
    del graphs
    dims_b = [(16, 512), (512, 256), (256, wl.D)]
    dims_t = [(m.Ip, 1024), (1024, 1024), (1024, 512), (512, 256), (256, 1)]
    flops = 3 * 2 * wl.B * sum(k * n for k, n in dims_b + dims_t)  # forward + two backward GEMMs
    return {"ms_per_step": ms, "samples_per_s": wl.B / (ms / 1e3), "ms_per_step_one_stream": ms_one,
            "ms_per_step_graph": ms_graph, "samples_per_s_graph": wl.B / (ms_graph / 1e3),
            "dense_gemm_tflop_per_step": flops / 1e12,
            "loss_after": float(m.head_out["loss"].item()),
            "layers": "bottom 13(16)-512-256-128, top 480-1024-1024-512-256-1, bf16 GEMMs (hipBLASLt), fp32 accumulation"}


# ---------------------------------------------------------------- streaming context

def hbm_context(dev, steps: int):
    """What plain streaming reaches on this GPU, as context for the kernels' figures: a 4 GiB
    device-to-device copy (read + write bytes), and a 4 GiB read-only stream (dlrm_probe_read),
    both far larger than the caches; HIP events, median of 5."""
    import torch
    from recommendation_model_sparse_amd import dlrm_probe_read
    n = 1 << 30  # 4 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)

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
    t_read = med(lambda: dlrm_probe_read(src, sink))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_GBps": 2 * 4 * n / t_copy / 1e9, "read_GBps": 4 * n / t_read / 1e9, "bytes": 4 * n,
            "how": "4 GiB fp32: device copy (read + write bytes over its time) and dlrm_probe_read "
                   "(read-only stream, 16-byte loads); HIP events, median of 5"}


# ---------------------------------------------------------------- main

def add_read_ceiling(gather: dict, ctx: dict):
    """Each lookup's counted HBM rate also as a fraction of what a gather of random 256-byte rows
    with no output reaches on the same GPU (the probe in hbm_context), when both were measured."""
    ceil = (ctx.get("random_row_gather") or {}).get("random_row_read_GBps")
    for e in gather.values():
        if ceil and e.get("hbm_GBps"):
            e["hbm_frac_of_random_row_read_ceiling"] = e["hbm_GBps"] / ceil


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--cpu-samples", type=int, default=16384)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--overlap-plan", action="store_true",
                    help="headline the step form with the backward's sort on a second stream")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM byte counters)")
    ap.add_argument("--only", choices=SECTIONS, default=None,
                    help="run one section and print its object (for profiling runs)")
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
    from recommendation_model_sparse_amd.configs import make_config

    dev = torch.device("cuda:0")
    only = args.only
    out = {}
    configs, gather = {}, {}
    if only in (None, "headline", "multihot-uniform", "inference", "full-step"):
        res, gat, uni, gat_u, cpu = bench_headline(args, dev)
        if only == "full-step":
            print(json.dumps({"full_step": res}), flush=True)
            return
        if only == "inference":
            print(json.dumps({"inference": res}), flush=True)
            return
        if only == "multihot-uniform":
            print(json.dumps({"multihot_uniform": uni, "gather": gat_u}), flush=True)
            return
        if only == "headline":
            print(json.dumps(dict(res, gather={"multihot-bf16-zipf": gat})), flush=True)
            return
        out = res
        gather["multihot-bf16-zipf"] = gat
        configs["multihot_bf16_uniform"] = uni
        gather["multihot-bf16-uniform"] = gat_u
    else:
        cpu = None
    ctx = {}
    if only in (None, "tiny"):
        r, g, _ = bench_forward(make_config(1), "tiny-f32", dev, args.steps, 1)
        configs["tiny_f32"] = r
    if only in (None, "onehot"):
        r, g, _ = bench_forward(make_config(2), "onehot-f32-zipf", dev, args.steps, min(args.rotate, 4))
        configs["onehot_f32"] = r
        gather["onehot-f32-zipf"] = g
    for dist in ("uniform", "zipf"):
        name = f"bigtables-{dist}"
        if only in (None, name):
            wl4 = make_config(4)
            if dist == "zipf":
                wl4 = wl4.with_(dist="zipf", alpha=1.2)
            r, g, probe = bench_forward(wl4, f"bigtables-bf16-{dist}", dev, args.steps, min(args.rotate, 4),
                                        probe_gather=dist == "uniform")
            configs[f"bigtables_bf16_{dist}"] = r
            gather[f"bigtables-bf16-{dist}"] = g
            if probe:
                ctx["random_row_gather"] = probe
    if only in (None, "train-onehot"):
        configs["train_onehot_f32"] = bench_train_onehot(make_config(5), dev, args.steps, min(args.rotate, 4))
    if only in (None, "probes"):
        ctx.update(hbm_context(dev, args.steps))
    if only in (None, "interaction"):
        configs["interaction_paths"] = bench_interaction_paths(dev, args.steps)
    if only is not None:
        add_read_ceiling(gather, ctx)
        print(json.dumps({"configs": configs, "gather": gather, "hbm_context": ctx}), flush=True)
        return
    out["configs"] = configs
    out["gather"] = gather
    out["hbm_context"] = ctx
    add_read_ceiling(gather, ctx)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
