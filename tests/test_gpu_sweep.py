"""A seeded sweep over random shapes of the whole path against the oracle (needs an MI355X).

Each case draws T tables of random sizes (from 1 row, so that every lookup of a table hits one row,
up to thousands), a width D and table dtype, a batch size, a mix of bag lengths (empty bags,
one-hot bags, long bags past 64 lookups), optional weights, int32 or int64 indices, and a row
distribution that is uniform or concentrated on a few hot rows.  Per case:
  - emb_bag_fwd against the oracle (R19 error <= 1e-5: fp32 accumulation for both table dtypes);
  - dlrm_interact_fwd after emb_bag_fwd within 1e-5 of the oracle's lookup + interaction, and
    emb_bag_interact_fwd bit-identical to it (rows of 64 bytes or more, which the fused call takes);
  - emb_bag_bwd_update (Adagrad or SGD, alternating) on a seeded pooled gradient: unique keys,
    segment offsets, sorted positions and the unique count bit-exact; touched rows within the
    row gates (fp32: per-row relative 1e-4; bf16: half a bf16 ulp plus 1e-4 of the row), states
    within 1e-4, untouched rows and states bit-identical.
Every oracle input is generated on the host.
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
    dlrm_interact_fwd,
    emb_bag_bwd_update,
    emb_bag_fwd,
    emb_bag_interact_fwd,
)

from gpu_util import DEV, as_f64, bf16_half_ulp, random_tables, rel_err, row_inf_rel, say, to_dev, to_host

pytestmark = pytest.mark.gpu

N_CASES = 40


def draw_case(k):
    rng = np.random.default_rng(zlib.crc32(f"sweep-{k}".encode()))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    D = int(rng.choice([8, 16, 32, 64, 128, 256] if dtype == "bf16" else [4, 8, 16, 32, 64, 128, 256]))
    T = int(rng.integers(1, 13))
    rows = [int(v) for v in np.where(rng.random(T) < 0.2, rng.integers(1, 4, T), rng.integers(4, 5000, T))]
    B = int(rng.integers(1, 300))
    mode = rng.choice(["onehot", "short", "mixed", "long"])
    if mode == "onehot":
        L = np.ones(T * B, np.int64)
    elif mode == "short":
        L = rng.integers(0, 4, T * B)
    elif mode == "mixed":
        L = rng.integers(0, 30, T * B)
    else:
        L = np.where(rng.random(T * B) < 0.2, rng.integers(60, 150, T * B), rng.integers(0, 10, T * B))
    off = np.zeros(T * B + 1, np.int64)
    np.cumsum(L, out=off[1:])
    idx = np.empty(int(off[-1]), np.int64)
    hot = rng.random() < 0.5
    for t in range(T):
        a, b = off[t * B], off[(t + 1) * B]
        if hot:  # most lookups on a few rows
            few = rng.integers(0, rows[t], 3)
            idx[a:b] = np.where(rng.random(b - a) < 0.7, rng.choice(few, b - a), rng.integers(0, rows[t], b - a))
        else:
            idx[a:b] = rng.integers(0, rows[t], b - a)
    weighted = rng.random() < 0.4
    w = rng.random(len(idx)).astype(np.float32) if weighted else None
    tables = random_tables(rng, rows, D, dtype)
    dense = rng.standard_normal((B, D)).astype(np.float32)
    gp = (rng.standard_normal((B, T, D)) * 1e-3).astype(np.float32)
    states = [rng.random(v).astype(np.float32) for v in rows]
    index32 = rng.random() < 0.3
    opt = DLRM_OPT_ADAGRAD if k % 2 == 0 else DLRM_OPT_SGD
    return dict(dtype=dtype, D=D, T=T, rows=rows, B=B, mode=mode, hot=hot, idx=idx, off=off, w=w,
                tables=tables, dense=dense, gp=gp, states=states, index32=index32, opt=opt)


@pytest.mark.parametrize("k", range(N_CASES))
def test_sweep(k):
    c = draw_case(k)
    idx, off, w, tables, B, D, T = c["idx"], c["off"], c["w"], c["tables"], c["B"], c["D"], c["T"]
    say(f"[sweep {k}] {c['dtype']} D={D} T={T} rows={c['rows'][:4]}{'...' if T > 4 else ''} B={B} "
        f"{c['mode']} hot={c['hot']} nnz={len(idx)} weighted={w is not None} int32={c['index32']} "
        f"opt={'adagrad' if c['opt'] == DLRM_OPT_ADAGRAD else 'sgd'}")
    tabs = [to_dev(t) for t in tables]
    it = np.int32 if c["index32"] else np.int64
    di, do = to_dev(idx.astype(it)), to_dev(off.astype(it))
    dw = None if w is None else to_dev(w)

    # lookup; the fused path and the interaction take int64 indices
    pooled = emb_bag_fwd(tabs, to_dev(idx), to_dev(off), dw)
    torch.cuda.synchronize()
    ref, scale = oracle.emb_bag_fwd(tables, idx, off, w, B)
    assert rel_err(pooled.cpu().numpy(), ref, scale) <= 1e-5
    dd = to_dev(c["dense"])
    two = dlrm_interact_fwd(dd, pooled)
    torch.cuda.synchronize()
    fref, fscale = oracle.emb_interact_fwd(tables, idx, off, w, B, c["dense"])
    assert rel_err(two.cpu().numpy(), fref, fscale) <= 1e-5
    if D * (2 if c["dtype"] == "bf16" else 4) >= 64:  # rows the fused kernels take: 64 bytes or more
        fused = emb_bag_interact_fwd(tabs, to_dev(idx), to_dev(off), dw, dd)
        torch.cuda.synchronize()
        assert torch.equal(fused.view(torch.int32), two.view(torch.int32)), "fused != two-call path"

    # backward + update
    adagrad = c["opt"] == DLRM_OPT_ADAGRAD
    sts = [to_dev(s) for s in c["states"]] if adagrad else None
    outs = AdagradOutputs(len(idx), DEV)
    emb_bag_bwd_update(tabs, sts, di, do, dw, to_dev(c["gp"]), c["opt"], 0.01, 1e-8, outputs=outs)
    torch.cuda.synchronize()
    if adagrad:
        r = oracle.emb_bag_bwd_adagrad(tables, c["states"], idx, off, w, B, c["gp"], 0.01, 1e-8)
    else:
        r = oracle.emb_bag_bwd_sgd(tables, idx, off, w, B, c["gp"], 0.01)
    U = int(outs.num_unique.item())
    assert U == r.U
    assert np.array_equal(outs.unique_keys.cpu().numpy()[:U], r.unique_keys)
    assert np.array_equal(outs.segment_offsets.cpu().numpy()[:U + 1], r.seg_offsets)
    assert np.array_equal(outs.sorted_pos.cpu().numpy()[:len(idx)], r.perm)
    tt, rr = r.table_and_row()
    for t in range(T):
        sel = tt == t
        new = to_host(tabs[t])
        touched = np.zeros(c["rows"][t], dtype=bool)
        touched[rr[sel]] = True
        assert np.array_equal(new[~touched].view(np.uint8), tables[t][~touched].view(np.uint8))
        if adagrad:
            st = sts[t].cpu().numpy()
            assert np.array_equal(st[~touched], c["states"][t][~touched])
        if not sel.any():
            continue
        got, want = as_f64(new[rr[sel]]), r.new_rows[sel]
        if c["dtype"] == "f32":
            assert row_inf_rel(got, want) <= 1e-4, f"table {t}"
        else:
            tol = bf16_half_ulp(want) * 1.0001 + 1e-4 * np.max(np.abs(want), axis=1, keepdims=True)
            assert np.all(np.abs(got - want) <= tol), f"table {t}"
        if adagrad:
            gs, ws = st[rr[sel]].astype(np.float64), r.new_state[sel]
            assert np.all(np.abs(gs - ws) <= 1e-4 * np.abs(ws)), f"table {t} state"
