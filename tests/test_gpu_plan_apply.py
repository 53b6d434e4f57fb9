"""The embedding backward split into emb_bag_bwd_plan (keys, sort, segments) and
emb_bag_bwd_apply (segment sums and the update), needs an MI355X.

Gates: plan + apply gives the bits of emb_bag_bwd_update (tables, states and the integer outputs),
on one stream and with the plan on a second stream ordered by an event; one plan applied twice
(to two copies of the tables, with and without the plan's segment-offset output) gives the same
bits both times, also when hot rows send segments through the finisher; without the integer
outputs (the sort then carries no position payload) the update gives the same bits; an empty batch
leaves the tables untouched.  emb_bag_bwd_update itself is checked against the oracle elsewhere; one
case here is checked against the oracle directly too (Adagrad rows: per-row relative error
<= 1e-4 for fp32).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from recommendation_model_sparse_amd import (
    DLRM_OPT_ADAGRAD,
    DLRM_OPT_SGD,
    AdagradOutputs,
    emb_bag_bwd_apply,
    emb_bag_bwd_plan,
    emb_bag_bwd_update,
    emb_bag_bwd_workspace_size,
    emb_bag_fwd,
)

from gpu_util import DEV, as_f64, random_csr, random_tables, row_inf_rel, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def case(seed, rows, D, dtype, B, weighted, lengths="multi", max_len=12, hot=None):
    rng = np.random.default_rng(seed)
    T = len(rows)
    tables = random_tables(rng, rows, D, dtype)
    states = [rng.random(v).astype(np.float32) for v in rows]
    idx, off, w = random_csr(rng, T, B, rows, lengths, max_len, weighted, hot)
    gp = (rng.standard_normal((B, T, D)) * 1e-3).astype(np.float32)
    return tables, states, idx, off, w, gp


def snapshot(tabs, sts, outs=None):
    t = [to_host(x) for x in tabs]
    s = None if sts is None else [x.cpu().numpy() for x in sts]
    o = None
    if outs is not None:
        U = int(outs.num_unique.item())
        n = outs.sorted_pos.numel()
        o = (U, outs.unique_keys[:U].cpu().numpy(), outs.segment_offsets[:U + 1].cpu().numpy(),
             outs.sorted_pos[:n].cpu().numpy())
    return t, s, o


def same(a, b):
    (ta, sa, oa), (tb, sb, ob) = a, b
    for x, y in zip(ta + (sa or []), tb + (sb or [])):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    if oa is not None and ob is not None:
        assert oa[0] == ob[0]
        for x, y in zip(oa[1:], ob[1:]):
            assert np.array_equal(x, y)


def run_update(tables, states, idx, off, w, gp, opt, index32=False):
    tabs = [to_dev(t) for t in tables]
    sts = [to_dev(s) for s in states] if opt == DLRM_OPT_ADAGRAD else None
    outs = AdagradOutputs(len(idx), DEV)
    di, do = dev_csr(idx, off, index32)
    emb_bag_bwd_update(tabs, sts, di, do, None if w is None else to_dev(w), to_dev(gp), opt, 0.01, 1e-8,
                       outputs=outs)
    torch.cuda.synchronize()
    return snapshot(tabs, sts, outs)


def dev_csr(idx, off, index32):
    if index32:
        return to_dev(idx.astype(np.int32)), to_dev(off.astype(np.int32))
    return to_dev(idx), to_dev(off)


@pytest.mark.parametrize("opt", [DLRM_OPT_ADAGRAD, DLRM_OPT_SGD])
@pytest.mark.parametrize("dtype,D", [("f32", 16), ("f32", 128), ("bf16", 64), ("bf16", 256)])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("side_stream", [False, True])
def test_plan_apply_equals_update(opt, dtype, D, weighted, side_stream):
    rows = [700, 2, 30000, 90]
    B = 211
    seed = zlib.crc32(f"pa-{opt}-{dtype}-{D}-{weighted}".encode())
    tables, states, idx, off, w, gp = case(seed, rows, D, dtype, B, weighted)
    index32 = weighted  # both index types, over the cases
    say(f"[plan/apply] opt={opt} {dtype} D={D} weighted={weighted} side={side_stream} nnz={len(idx)}")
    want = run_update(tables, states, idx, off, w, gp, opt, index32)

    tabs = [to_dev(t) for t in tables]
    sts = [to_dev(s) for s in states] if opt == DLRM_OPT_ADAGRAD else None
    di, do = dev_csr(idx, off, index32)
    dw = None if w is None else to_dev(w)
    dgp = to_dev(gp)
    ws = torch.empty(emb_bag_bwd_workspace_size(rows, D, B, len(idx)), dtype=torch.uint8, device=DEV)
    outs = AdagradOutputs(len(idx), DEV)
    main = torch.cuda.current_stream()
    if side_stream:
        side = torch.cuda.Stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            emb_bag_bwd_plan(rows, D, di, do, dw, ws, outputs=outs)
            done = torch.cuda.Event()
            done.record(side)
        # the main stream works meanwhile (a lookup that reads the same batch), then waits
        pooled = emb_bag_fwd(tabs, di.long(), do.long(), dw)
        main.wait_event(done)
    else:
        emb_bag_bwd_plan(rows, D, di, do, dw, ws, outputs=outs)
    emb_bag_bwd_apply(tabs, sts, B, len(idx), w is not None, dgp, opt, 0.01, 1e-8, ws, outputs=outs)
    torch.cuda.synchronize()
    same(snapshot(tabs, sts, outs), want)
    if side_stream:
        del pooled


@pytest.mark.parametrize("opt", [DLRM_OPT_ADAGRAD, DLRM_OPT_SGD])
@pytest.mark.parametrize("hot", [None, 3])
def test_one_plan_applied_twice(opt, hot):
    """Both applications start the finisher worklist empty: hot rows make segments that span many
    chunks and go through the finisher."""
    rows = [50, 5000, 77]
    B = 3000 if hot is not None else 400
    seed = zlib.crc32(f"twice-{opt}-{hot}".encode())
    tables, states, idx, off, w, gp = case(seed, rows, 128, "f32", B, True, max_len=40, hot=hot)
    say(f"[plan/apply] twice opt={opt} hot={hot} nnz={len(idx)}")
    want = run_update(tables, states, idx, off, w, gp, opt)
    di, do = to_dev(idx), to_dev(off)
    ws = torch.empty(emb_bag_bwd_workspace_size(rows, 128, B, len(idx)), dtype=torch.uint8, device=DEV)
    emb_bag_bwd_plan(rows, 128, di, do, to_dev(w), ws)
    got = []
    for rep in range(2):
        tabs = [to_dev(t) for t in tables]
        sts = [to_dev(s) for s in states] if opt == DLRM_OPT_ADAGRAD else None
        emb_bag_bwd_apply(tabs, sts, B, len(idx), True, to_dev(gp), opt, 0.01, 1e-8, ws)
        torch.cuda.synchronize()
        got.append(snapshot(tabs, sts))
    for g in got:
        same(g, (want[0], want[1], None))


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_update_without_outputs(weighted, dtype):
    """Without the integer outputs the sort carries no position payload; the update is the same."""
    rows = [700, 2, 30000, 90]
    B = 211
    tables, states, idx, off, w, gp = case(zlib.crc32(f"noout-{weighted}-{dtype}".encode()), rows, 64, dtype, B,
                                           weighted)
    say(f"[plan/apply] no outputs weighted={weighted} {dtype} nnz={len(idx)}")
    want = run_update(tables, states, idx, off, w, gp, DLRM_OPT_ADAGRAD)
    tabs = [to_dev(t) for t in tables]
    sts = [to_dev(s) for s in states]
    emb_bag_bwd_update(tabs, sts, to_dev(idx), to_dev(off), None if w is None else to_dev(w), to_dev(gp),
                       DLRM_OPT_ADAGRAD, 0.01, 1e-8)
    torch.cuda.synchronize()
    same(snapshot(tabs, sts), (want[0], want[1], None))


def test_plan_apply_vs_oracle():
    rows = [300, 1, 2000, 77]
    B = 130
    tables, states, idx, off, w, gp = case(5151, rows, 64, "f32", B, True)
    say(f"[plan/apply] oracle nnz={len(idx)}")
    tabs = [to_dev(t) for t in tables]
    sts = [to_dev(s) for s in states]
    ws = torch.empty(emb_bag_bwd_workspace_size(rows, 64, B, len(idx)), dtype=torch.uint8, device=DEV)
    outs = AdagradOutputs(len(idx), DEV)
    emb_bag_bwd_plan(rows, 64, to_dev(idx), to_dev(off), to_dev(w), ws, outputs=outs)
    emb_bag_bwd_apply(tabs, sts, B, len(idx), True, to_dev(gp), DLRM_OPT_ADAGRAD, 0.01, 1e-8, ws, outputs=outs)
    torch.cuda.synchronize()
    r = oracle.emb_bag_bwd_adagrad(tables, states, idx, off, w, B, gp, 0.01, 1e-8)
    U = int(outs.num_unique.item())
    assert U == r.U
    assert np.array_equal(outs.unique_keys.cpu().numpy()[:U], r.unique_keys)
    assert np.array_equal(outs.segment_offsets.cpu().numpy()[:U + 1], r.seg_offsets)
    assert np.array_equal(outs.sorted_pos.cpu().numpy()[:len(idx)], r.perm)
    tt, rr = r.table_and_row()
    for t in range(len(rows)):
        sel = tt == t
        if sel.any():
            assert row_inf_rel(as_f64(to_host(tabs[t])[rr[sel]]), r.new_rows[sel]) <= 1e-4


def test_plan_apply_empty_batch():
    rows = [10, 20]
    B = 5
    tables, states, idx, off, w, gp = case(77, rows, 32, "bf16", B, False, lengths="empty")
    assert len(idx) == 0
    say("[plan/apply] empty batch")
    tabs = [to_dev(t) for t in tables]
    sts = [to_dev(s) for s in states]
    ws = torch.empty(max(emb_bag_bwd_workspace_size(rows, 32, B, 0), 256), dtype=torch.uint8, device=DEV)
    outs = AdagradOutputs(0, DEV)
    emb_bag_bwd_plan(rows, 32, to_dev(idx), to_dev(off), None, ws, outputs=outs)
    emb_bag_bwd_apply(tabs, sts, B, 0, False, to_dev(gp), DLRM_OPT_ADAGRAD, 0.01, 1e-8, ws, outputs=outs)
    torch.cuda.synchronize()
    assert int(outs.num_unique.item()) == 0
    for a, b in zip([to_host(t) for t in tabs], tables):
        assert np.array_equal(a, b)
    for a, b in zip([s.cpu().numpy() for s in sts], states):
        assert np.array_equal(a, b)
