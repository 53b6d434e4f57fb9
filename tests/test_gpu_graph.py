"""The sparse training step recorded in a HIP graph (needs an MI355X).

emb_bag_fwd -> dlrm_interact_fwd -> dlrm_interact_bwd -> emb_bag_bwd_adagrad (every integer output
requested) is captured once per batch on a side stream; nothing in those calls allocates, copies
to the host or synchronizes.  Each replay starts from the same tables and states as an eager run of
the same step and must leave bit-identical tables, states, interaction output, pooled gradient and
integer outputs.  The replays are interleaved with eager work and synchronizations, and each batch's
graph is replayed more than once.
"""
import numpy as np
import pytest
import torch

from recommendation_model_sparse_amd import (AdagradOutputs, dlrm_interact_bwd, dlrm_interact_fwd,
                                             emb_bag_bwd_adagrad, emb_bag_bwd_workspace_size, emb_bag_fwd)

from gpu_util import DEV, random_csr, random_tables, say, to_dev

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    rng = np.random.default_rng(2026)
    rows, D, B = [1000, 50, 3000, 7], 128, 300
    T = len(rows)
    tabs = [to_dev(t) for t in random_tables(rng, rows, D, "bf16")]
    states = [torch.from_numpy(rng.random(v).astype(np.float32)).to(DEV) for v in rows]
    batches = []
    for i in range(2):
        idx, off, _ = random_csr(rng, T, B, rows, "multi", 30, hot=i)
        P = (T + 1) * T // 2
        batches.append(dict(idx=to_dev(idx), off=to_dev(off), nnz=len(idx),
                            dense=to_dev(rng.standard_normal((B, D)).astype(np.float32)),
                            g=to_dev((rng.standard_normal((B, P + D)) * 1e-2).astype(np.float32))))
    max_nnz = max(b["nnz"] for b in batches)
    ws = torch.empty(emb_bag_bwd_workspace_size(rows, D, B, max_nnz), dtype=torch.uint8, device=DEV)
    outs = AdagradOutputs(max_nnz, DEV)
    pooled = torch.empty((B, T, D), device=DEV)
    inter = torch.empty((B, (T + 1) * T // 2 + D), device=DEV)
    gdense = torch.empty((B, D), device=DEV)
    gpooled = torch.empty_like(pooled)

    def step(i):
        b = batches[i]
        emb_bag_fwd(tabs, b["idx"], b["off"], None, out=pooled)
        dlrm_interact_fwd(b["dense"], pooled, out=inter)
        dlrm_interact_bwd(b["g"], b["dense"], pooled, grad_dense=gdense, grad_pooled=gpooled)
        emb_bag_bwd_adagrad(tabs, states, b["idx"], b["off"], None, gpooled, 0.01, 1e-8, workspace=ws, outputs=outs)

    def state(nnz):
        n = int(outs.num_unique.item())
        return ([t.clone() for t in tabs] + [s.clone() for s in states] +
                [inter.clone(), gdense.clone(), gpooled.clone(), outs.unique_keys[:n].clone(),
                 outs.segment_offsets[:n + 1].clone(), outs.sorted_pos[:nnz].clone(), outs.num_unique.clone()])

    step(0)
    step(1)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for rep, i in enumerate([0, 1, 0, 1]):
        say(f"[graph] replay {rep} of batch {i}")
        start = ([t.clone() for t in tabs], [s.clone() for s in states])
        step(i)
        torch.cuda.synchronize()
        ref = state(batches[i]["nnz"])
        for t, c in zip(tabs, start[0]):
            t.copy_(c)
        for s, c in zip(states, start[1]):
            s.copy_(c)
        torch.cuda.synchronize()
        graphs[i].replay()
        torch.cuda.synchronize()
        got = state(batches[i]["nnz"])
        for k, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: tensor {k} differs"


def test_full_step_graph_replays_match_eager():
    """The full DLRM step (bottom and top MLPs through hipBLASLt, the sparse path, the embedding
    backward's sort on a second stream, SGD and Adagrad) recorded as a HIP graph per batch, after
    every call has run once eagerly (hipBLASLt picks its algorithms on a shape's first call).  Each
    replay starts from the parameters, tables and states of an eager step of the same batch and
    must leave them, the loss and the predictions bit-identical."""
    from recommendation_model_sparse_amd.dlrm_step import DlrmStep
    from recommendation_model_sparse_amd.synth import Workload
    from gpu_util import device_tables

    wl = Workload(name="graph-step", seed=99, T=4, D=32, dtype="bf16", B=256, rows=[500, 7000, 40, 3000],
                  init="hash", bags="geom", bag_lo=1, bag_hi=12, bag_mean=4.0, dist="zipf", alpha=1.05)
    host = [wl.batch(i) for i in range(2)]
    tabs = device_tables(wl)
    states = [torch.zeros(v, dtype=torch.float32, device=DEV) for v in wl.rows]
    m = DlrmStep(tabs, states, wl.B, 13, bottom=[32, 32], top=[64, 16], lr_dense=0.05, lr_emb=0.01, eps=1e-8,
                 seed=3, max_nnz=max(b.nnz for b in host), overlap=True)
    inputs = [(to_dev(b.indices), to_dev(b.offsets), to_dev(b.features(13)), to_dev(b.labels())) for b in host]

    def tensors():
        layers = m.bottom + m.top + [m.head]
        return [t for l in layers for t in (l.W32, l.W16, l.b)] + m.tables + m.states

    def bits(t):
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)

    def snapshot():
        return [t.clone() for t in tensors()] + [m.head_out["loss"].clone(), m.head_out["p"].clone()]

    for i in range(2):
        m.step(*inputs[i])
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            m.step(*inputs[i])
        graphs.append(g)
    torch.cuda.synchronize()
    for rep, i in enumerate([0, 1, 1, 0]):
        say(f"[graph] full step replay {rep} of batch {i}")
        start = [t.clone() for t in tensors()]
        m.step(*inputs[i])
        torch.cuda.synchronize()
        ref = snapshot()
        for t, c in zip(tensors(), start):
            t.copy_(c)
        torch.cuda.synchronize()
        graphs[i].replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(bits(a), bits(b)), f"replay {rep}: tensor {k} differs from the eager step"
