"""The allocation-free embedding backward against the workspace entry point (GPU).

emb_bag_bwd_update_noalloc runs the same kernels as emb_bag_bwd_update with the library's fixed
per-GPU scratch as the workspace, so tables, states and every integer output must match bit for
bit.  Two calls in a row, the second on a smaller batch (the scratch keeps the first call's
contents), for both optimisers, weighted and unweighted, int64 and int32 indices; a batch larger
than the scratch is refused on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

from recommendation_model_sparse_amd import (DLRM_OPT_ADAGRAD, DLRM_OPT_SGD, AdagradOutputs, DlrmError,
                                             emb_bag_bwd_noalloc_max_bytes, emb_bag_bwd_update,
                                             emb_bag_bwd_update_noalloc, emb_bag_bwd_workspace_size)
from recommendation_model_sparse_amd import binding

from gpu_util import DEV, random_csr, random_tables, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_pair(tables, rows, idx, off, w, gp, opt, itype):
    """Both entry points on copies of the same tables and states; returns both results."""
    res = []
    for noalloc in (False, True):
        tabs = [to_dev(t) for t in tables]
        sts = [torch.full((v,), 0.25, device=DEV) for v in rows] if opt == DLRM_OPT_ADAGRAD else None
        di, do = to_dev(idx.astype(itype)), to_dev(off.astype(itype))
        dw = None if w is None else to_dev(w)
        outs = AdagradOutputs(len(idx), DEV)
        if noalloc:
            emb_bag_bwd_update_noalloc(tabs, sts, di, do, dw, to_dev(gp), opt, 0.01, 1e-8, outputs=outs)
        else:
            ws = torch.empty(emb_bag_bwd_workspace_size(rows, tables[0].shape[1], gp.shape[0], len(idx)),
                             dtype=torch.uint8, device=DEV)
            emb_bag_bwd_update(tabs, sts, di, do, dw, to_dev(gp), opt, 0.01, 1e-8, workspace=ws, outputs=outs)
        torch.cuda.synchronize()
        U = int(outs.num_unique.item())
        res.append(([to_host(t) for t in tabs], None if sts is None else [s.cpu().numpy() for s in sts],
                    outs.unique_keys.cpu().numpy()[:U], outs.segment_offsets.cpu().numpy()[:U + 1],
                    outs.sorted_pos.cpu().numpy()[:len(idx)], U))
    return res


def same(a, b):
    ta, sa, ka, oa, pa, ua = a
    tb, sb, kb, ob, pb, ub = b
    assert ua == ub
    assert np.array_equal(ka, kb) and np.array_equal(oa, ob) and np.array_equal(pa, pb)
    for x, y in zip(ta, tb):
        assert np.array_equal(x, y)
    if sa is not None:
        for x, y in zip(sa, sb):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("opt", [DLRM_OPT_ADAGRAD, DLRM_OPT_SGD])
@pytest.mark.parametrize("dtype,D", [("f32", 128), ("bf16", 64)])
def test_noalloc_matches_workspace_entry_point(opt, dtype, D):
    rng = np.random.default_rng(900 + D + opt)
    rows = [700, 3, 20000, 90]
    T = len(rows)
    tables = random_tables(rng, rows, D, dtype)
    # first a larger batch, then a smaller one: the scratch holds the first call's contents
    for B, max_len, weighted, itype in ((96, 30, True, np.int64), (17, 5, False, np.int32)):
        idx, off, w = random_csr(rng, T, B, rows, "multi", max_len, weighted)
        gp = (rng.standard_normal((B, T, D)) * 1e-2).astype(np.float32)
        say(f"[noalloc] opt={opt} {dtype} D={D} B={B} nnz={len(idx)} weighted={weighted} {itype.__name__}")
        a, b = run_pair(tables, rows, idx, off, w, gp, opt, itype)
        same(a, b)


def test_noalloc_onehot_training_batch_and_limit():
    """The one-hot training batch (26 tables x 2048 samples) fits; a batch over the limit is refused."""
    rng = np.random.default_rng(77)
    rows = [int(v) for v in rng.integers(1000, 50000, 26)]
    D, B = 128, 2048
    tables = random_tables(rng, rows, D, "f32")
    idx, off, _ = random_csr(rng, 26, B, rows, "onehot")
    gp = (rng.standard_normal((B, 26, D)) * 1e-3).astype(np.float32)
    say("[noalloc] one-hot 26 x 2048")
    a, b = run_pair(tables, rows, idx, off, None, gp, DLRM_OPT_ADAGRAD, np.int64)
    same(a, b)
    assert emb_bag_bwd_workspace_size(rows, D, B, len(idx)) <= emb_bag_bwd_noalloc_max_bytes()
    # too large for the scratch: refused on the host with DLRM_ERR_WORKSPACE, nothing enqueued
    big = 4 << 20
    assert emb_bag_bwd_workspace_size([1000], D, 1, big) > emb_bag_bwd_noalloc_max_bytes()
    L = binding.lib()
    tab = torch.zeros((1000, D), device=DEV)
    st = torch.zeros(1000, device=DEV)
    p = lambda *v: (ctypes.c_void_p * len(v))(*v)
    rc = L.emb_bag_bwd_update_noalloc(p(tab.data_ptr()), p(st.data_ptr()), (ctypes.c_int64 * 1)(1000), 1, D, 0,
                                      ctypes.c_void_p(tab.data_ptr()), ctypes.c_void_p(tab.data_ptr()), 0, None, 1,
                                      big, ctypes.c_void_p(tab.data_ptr()), 0, 0.01, 1e-8, None, None, None, None, 0,
                                      None)
    assert rc == -5
    torch.cuda.synchronize()
    assert bool((tab == 0).all()) and bool((st == 0).all())
