"""GPU parity on the five full-size workloads (needs an MI355X).

The GPU runs each workload at its full size, in the launch configuration the
benchmark times.  The oracle checks sampled batch rows one by one: the sampled
bags are restricted to the table rows they touch (a monotone renumbering, so
pooling, sort order and segments are unchanged), and those rows are
regenerated on the host from the same counter hash the device fill wrote.
Every oracle input is generated on the host: a call that consumes another
call's output (the interaction, its backward, the update) is checked on
host-made inputs of the same shape, the oracle's own upstream results or
seeded arrays, not on the GPU's.
"""
import numpy as np
import pytest
import torch

import oracle
from recommendation_model_sparse_amd import (
    DLRM_OPT_ADAGRAD,
    DLRM_OPT_SGD,
    AdagradOutputs,
    dlrm_interact_bwd,
    dlrm_interact_fwd,
    dlrm_synth_fill_table,
    emb_bag_bwd_adagrad,
    emb_bag_bwd_update,
    emb_bag_fwd,
    emb_bag_fwd_ex,
    emb_bag_interact_fwd,
    synth,
)
from recommendation_model_sparse_amd.configs import make_config
from recommendation_model_sparse_amd.synth import subset_tables

from gpu_util import DEV, as_f64, bf16_half_ulp, device_tables, rel_err, row_inf_rel, say, to_dev, to_host

pytestmark = pytest.mark.gpu

POOL_TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_device_fill_matches_host_hash(dtype):
    V, D, t = 5000, 128, 7
    seed = synth.table_seed(123)
    scale = synth.table_scale(V)
    x = torch.empty((V, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=DEV)
    say(f"[fill] {dtype} V={V}")
    dlrm_synth_fill_table(x, t, seed, float(scale))
    rows = np.array([0, 1, 2, 777, V - 1])
    got = to_host(x)[rows]
    ref = synth.hash_rows(t, rows, D, seed, scale, dtype)
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


def sample_rows(B, n, seed):
    if B <= n:
        return np.arange(B)
    rng = np.random.default_rng(seed)
    s = rng.choice(B, n, replace=False)
    return np.unique(np.concatenate([s, [0, B - 1]]))


def check_forward(wl, batch, tabs, n_samples=256):
    say(f"[workload] {wl.name} B={wl.B} nnz={batch.nnz} table bytes={wl.table_bytes() / 1e9:.2f} GB "
        f"weighted={batch.weights is not None}")
    di, do = to_dev(batch.indices), to_dev(batch.offsets)
    dw = None if batch.weights is None else to_dev(batch.weights)
    dense = to_dev(batch.dense)
    pooled = emb_bag_fwd(tabs, di, do, dw)
    inter = dlrm_interact_fwd(dense, pooled)
    fused = emb_bag_interact_fwd(tabs, di, do, dw, dense)
    torch.cuda.synchronize()
    # the fused inference call runs the same arithmetic without the pooled round trip
    assert torch.equal(fused.view(torch.int32), inter.view(torch.int32)), "fused != two-call path"
    # int32 indices and offsets: the same bits as int64
    pooled32 = emb_bag_fwd_ex(tabs, di.to(torch.int32), do.to(torch.int32), dw)
    torch.cuda.synchronize()
    assert torch.equal(pooled32.view(torch.int32), pooled.view(torch.int32)), "int32 indices != int64"
    # bf16 pooled output: the round-to-nearest-even of the fp32 output, bit for bit
    pooled16 = emb_bag_fwd_ex(tabs, di, do, dw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(pooled16.view(torch.int16), pooled.to(torch.bfloat16).view(torch.int16)), "bf16 output != RNE"
    S = sample_rows(wl.B, n_samples, wl.seed)
    sub_wl, sub, row_ids = batch.sample_subset(S)
    host_tabs = subset_tables(wl, row_ids)
    ref, scale = oracle.emb_bag_fwd(host_tabs, sub.indices, sub.offsets, sub.weights, len(S))
    got = pooled[torch.from_numpy(S).to(DEV)].cpu().numpy()
    err = rel_err(got, ref, scale)
    say(f"   pooled max rel err {err:.3e} over {len(S)} samples")
    assert err <= POOL_TOL[wl.dtype]
    if wl.bags == "onehot":
        assert np.array_equal(got, ref.astype(np.float32))
    # the interaction at full size on a seeded host-made pooled input
    pz = (np.random.default_rng(wl.seed + 17).standard_normal((wl.B, wl.T, wl.D)) * 0.1).astype(np.float32)
    inter_z = dlrm_interact_fwd(dense, to_dev(pz))
    iref, iscale = oracle.interact_fwd(batch.dense[S], pz[S])
    igot = inter_z[torch.from_numpy(S).to(DEV)].cpu().numpy()
    ierr = rel_err(igot, iref, iscale)
    say(f"   interaction max rel err {ierr:.3e}")
    assert ierr <= 1e-5
    # its backward at full size, on the same pooled input and a seeded gradient of the output
    g = (np.random.default_rng(wl.seed + 29).standard_normal((wl.B, wl.P + wl.D)) * 1e-3).astype(np.float32)
    gd, gp = dlrm_interact_bwd(to_dev(g), dense, to_dev(pz))
    torch.cuda.synchronize()
    rd, rp, md, mp = oracle.interact_bwd(g[S], batch.dense[S], pz[S])
    sel = torch.from_numpy(S).to(DEV)
    berr = max(rel_err(gd[sel].cpu().numpy(), rd, md), rel_err(gp[sel].cpu().numpy(), rp, mp))
    say(f"   interaction backward max rel err {berr:.3e}")
    assert berr <= 1e-5
    return pooled, inter


@pytest.mark.parametrize("k", [1, 2, 3])
def test_workload_forward(k):
    wl = make_config(k)
    tabs = device_tables(wl)
    check_forward(wl, wl.batch(0), tabs)
    if k == 3:  # the weighted variant
        check_forward(wl, wl.batch(1, weighted=True), tabs)
    del tabs
    torch.cuda.empty_cache()


def test_workload_big_tables():
    """One GPU's share of 8 x 50M-row bf16 tables (102.4 GB), uniform and Zipf(1.2) indices."""
    wl = make_config(4)
    tabs = device_tables(wl)
    try:
        check_forward(wl, wl.batch(0), tabs, n_samples=512)
        check_forward(wl.with_(dist="zipf", alpha=1.2), wl.with_(dist="zipf", alpha=1.2).batch(0), tabs,
                      n_samples=512)
    finally:
        del tabs
        torch.cuda.empty_cache()


def test_workload_training_step():
    """Interaction backward + sort/unique/segment-reduce + row-wise Adagrad on the one-hot fp32 shapes."""
    wl = make_config(5)
    b = wl.batch(0)
    tabs = device_tables(wl)
    states = [torch.zeros(v, dtype=torch.float32, device=DEV) for v in wl.rows]
    say(f"[workload] {wl.name} training step B={wl.B} nnz={b.nnz}")
    di, do = to_dev(b.indices), to_dev(b.offsets)
    dense = to_dev(b.dense)
    # every bag over the rows it touches (monotone renumbering), regenerated on the host
    sub_wl, sub, row_ids = b.sample_subset(np.arange(wl.B))
    host_tabs = subset_tables(wl, row_ids)
    pref, _ = oracle.emb_bag_fwd(host_tabs, sub.indices, sub.offsets, None, wl.B)
    pooled_h = pref.astype(np.float32)  # one-hot: the rows themselves, exact
    pooled = emb_bag_fwd(tabs, di, do)
    # the backward calls take the oracle's upstream results: its pooled rows, then its gradient
    gd, gp = dlrm_interact_bwd(to_dev(b.grad_out()), dense, to_dev(pooled_h))
    rd, rp, md, mp = oracle.interact_bwd(b.grad_out(), b.dense, pooled_h)
    gin = rp.astype(np.float32)
    outs = AdagradOutputs(b.nnz, DEV)
    emb_bag_bwd_adagrad(tabs, states, di, do, None, to_dev(gin), wl.lr, wl.eps, outputs=outs)
    torch.cuda.synchronize()
    assert np.array_equal(pooled.cpu().numpy(), pooled_h)

    e1 = rel_err(gd.cpu().numpy(), rd, md)
    e2 = rel_err(gp.cpu().numpy(), rp, mp)
    say(f"   interact_bwd max rel err {e1:.3e} / {e2:.3e}")
    assert e1 <= 1e-5 and e2 <= 1e-5

    # Adagrad on every lookup, over the touched rows only
    host_states = [np.zeros(len(r), np.float32) for r in row_ids]
    r = oracle.emb_bag_bwd_adagrad(host_tabs, host_states, sub.indices, sub.offsets, None, wl.B,
                                   gin, wl.lr, wl.eps)
    U = int(outs.num_unique.item())
    assert U == r.U
    assert np.array_equal(outs.sorted_pos.cpu().numpy(), r.perm)
    assert np.array_equal(outs.segment_offsets.cpu().numpy()[:U + 1], r.seg_offsets)
    rowbase = np.zeros(wl.T + 1, dtype=np.int64)
    np.cumsum(wl.rows, out=rowbase[1:])
    tt, rr = r.table_and_row()
    full_keys = rowbase[tt] + np.array([row_ids[t][x] for t, x in zip(tt, rr)], dtype=np.int64)
    assert np.array_equal(outs.unique_keys.cpu().numpy()[:U], full_keys)
    rng = np.random.default_rng(3)
    worst = 0.0
    for t in range(wl.T):
        sel = tt == t
        rows_t = row_ids[t][rr[sel]]
        if len(rows_t):
            got = tabs[t][torch.from_numpy(rows_t).to(DEV)].cpu().numpy().astype(np.float64)
            e = row_inf_rel(got, r.new_rows[sel])
            worst = max(worst, e)
            assert e <= 1e-4
            gs = states[t][torch.from_numpy(rows_t).to(DEV)].cpu().numpy().astype(np.float64)
            assert np.all(np.abs(gs - r.new_state[sel]) <= 1e-4 * np.abs(r.new_state[sel]))
        # untouched rows: unchanged (bit-exact against the hash), state still zero
        cand = rng.integers(0, wl.rows[t], 512)
        cand = np.setdiff1d(cand, row_ids[t])
        if len(cand):
            got = tabs[t][torch.from_numpy(cand).to(DEV)].cpu().numpy()
            assert np.array_equal(got.view(np.uint8), wl.table_rows(t, cand).view(np.uint8))
            assert torch.all(states[t][torch.from_numpy(cand).to(DEV)] == 0)
    say(f"   Adagrad U={U} worst row rel err {worst:.3e}")
    del tabs, states
    torch.cuda.empty_cache()


@pytest.mark.parametrize("weighted,opt", [(False, DLRM_OPT_ADAGRAD), (True, DLRM_OPT_ADAGRAD), (False, DLRM_OPT_SGD)])
def test_workload_multihot_backward(weighted, opt):
    """The timed backward at its full size: 26 bf16 tables (D = 128), B = 16384 multi-hot bags
    (~8.5M lookups, Zipf rows, so hot rows make segments over hundreds of chunks), row-wise Adagrad
    in place with every integer output requested; also with the workload's per-sample weights (the
    weighted segment reduce), and the SGD update.  The gradient is a seeded stand-alone one (not the
    GPU's interaction backward), so the oracle's inputs are all host-generated.  Integer outputs are
    compared whole and bit-exactly; every touched row (and Adagrad state) against the oracle."""
    adagrad = opt == DLRM_OPT_ADAGRAD
    wl = make_config(3)
    b = wl.batch(1, weighted=True) if weighted else wl.batch(0)
    gp = b.grad_pooled()
    tabs = device_tables(wl)
    states = [torch.zeros(v, dtype=torch.float32, device=DEV) for v in wl.rows]
    say(f"[workload] {wl.name} multi-hot backward B={wl.B} nnz={b.nnz} weighted={weighted} opt={opt}")
    outs = AdagradOutputs(b.nnz, DEV)
    emb_bag_bwd_update(tabs, states if adagrad else None, to_dev(b.indices), to_dev(b.offsets),
                       to_dev(b.weights) if weighted else None, to_dev(gp), opt, wl.lr, wl.eps if adagrad else 0.0,
                       outputs=outs)
    torch.cuda.synchronize()
    if not weighted and adagrad:
        # the same update from int32 indices and offsets, on fresh tables: the same bits
        tabs32 = device_tables(wl)
        states32 = [torch.zeros(v, dtype=torch.float32, device=DEV) for v in wl.rows]
        emb_bag_bwd_update(tabs32, states32, to_dev(b.indices.astype(np.int32)), to_dev(b.offsets.astype(np.int32)),
                           None, to_dev(gp), opt, wl.lr, wl.eps)
        torch.cuda.synchronize()
        for x, y in zip(tabs + states, tabs32 + states32):
            assert torch.equal(x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
                               y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)), "int32 != int64"
        del tabs32, states32

    sub_wl, sub, row_ids = b.sample_subset(np.arange(wl.B))
    host_tabs = subset_tables(wl, row_ids)
    if adagrad:
        r = oracle.emb_bag_bwd_adagrad(host_tabs, [np.zeros(len(x), np.float32) for x in row_ids], sub.indices,
                                       sub.offsets, sub.weights, wl.B, gp, wl.lr, wl.eps)
    else:
        r = oracle.emb_bag_bwd_sgd(host_tabs, sub.indices, sub.offsets, sub.weights, wl.B, gp, wl.lr)
    U = int(outs.num_unique.item())
    assert U == r.U
    assert np.array_equal(outs.sorted_pos.cpu().numpy(), r.perm)
    assert np.array_equal(outs.segment_offsets.cpu().numpy()[:U + 1], r.seg_offsets)
    rowbase = np.zeros(wl.T + 1, dtype=np.int64)
    np.cumsum(wl.rows, out=rowbase[1:])
    tt, rr = r.table_and_row()
    full_keys = rowbase[tt] + np.concatenate([row_ids[t][rr[tt == t]] for t in range(wl.T)])
    assert np.array_equal(outs.unique_keys.cpu().numpy()[:U], full_keys)
    longest = int(np.max(np.diff(r.seg_offsets)))
    rng = np.random.default_rng(11)
    for t in range(wl.T):
        sel = tt == t
        rows_t = torch.from_numpy(row_ids[t][rr[sel]]).to(DEV)
        ref = r.new_rows[sel]
        got = as_f64(to_host(tabs[t][rows_t]))
        tol = bf16_half_ulp(ref) * 1.0001 + 1e-4 * np.max(np.abs(ref), axis=1, keepdims=True)
        assert np.all(np.abs(got - ref) <= tol), f"table {t}"
        if adagrad:
            gs = states[t][rows_t].cpu().numpy().astype(np.float64)
            rs = r.new_state[sel]
            assert np.all(np.abs(gs - rs) <= 1e-4 * np.abs(rs)), f"table {t} state"
        cand = np.setdiff1d(rng.integers(0, wl.rows[t], 512), row_ids[t])
        if len(cand):
            dc = torch.from_numpy(cand).to(DEV)
            assert np.array_equal(to_host(tabs[t][dc]).view(np.uint8), wl.table_rows(t, cand).view(np.uint8))
            assert torch.all(states[t][dc] == 0)
    say(f"   U={U} longest segment {longest} lookups: rows and states within the gates")
    del tabs, states
    torch.cuda.empty_cache()


def test_adagrad_wide_keys():
    """30-bit keys (2^29 + 12345 rows): three sort passes of 10-bit digits, checked on every lookup."""
    from recommendation_model_sparse_amd.synth import Workload
    V = (1 << 29) + 12345
    wl = Workload(name="wide-keys", seed=777, T=1, D=4, dtype="f32", B=4096, rows=[V], init="hash",
                  bags="geom", bag_lo=1, bag_hi=8, bag_mean=3.0, dist="uniform")
    b = wl.batch(0, weighted=True)
    say(f"[adagrad] wide keys V={V} nnz={b.nnz}")
    tabs = device_tables(wl)
    states = [torch.zeros(V, dtype=torch.float32, device=DEV)]
    gp = (np.random.default_rng(5).standard_normal((wl.B, 1, wl.D)) * 1e-3).astype(np.float32)
    outs = AdagradOutputs(b.nnz, DEV)
    emb_bag_bwd_adagrad(tabs, states, to_dev(b.indices), to_dev(b.offsets), to_dev(b.weights),
                        to_dev(gp), wl.lr, wl.eps, outputs=outs)
    torch.cuda.synchronize()
    sub_wl, sub, row_ids = b.sample_subset(np.arange(wl.B))
    r = oracle.emb_bag_bwd_adagrad(subset_tables(wl, row_ids), [np.zeros(len(row_ids[0]), np.float32)],
                                   sub.indices, sub.offsets, sub.weights, wl.B, gp, wl.lr, wl.eps)
    U = int(outs.num_unique.item())
    assert U == r.U
    assert np.array_equal(outs.sorted_pos.cpu().numpy(), r.perm)
    assert np.array_equal(outs.segment_offsets.cpu().numpy()[:U + 1], r.seg_offsets)
    assert np.array_equal(outs.unique_keys.cpu().numpy()[:U], row_ids[0][r.unique_keys])
    got = tabs[0][torch.from_numpy(row_ids[0][r.unique_keys]).to(DEV)].cpu().numpy().astype(np.float64)
    assert row_inf_rel(got, r.new_rows) <= 1e-4
    del tabs, states
    torch.cuda.empty_cache()
