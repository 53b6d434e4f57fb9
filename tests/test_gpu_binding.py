"""Bad device tensors are refused by the binding before anything is enqueued (GPU)."""
import pytest
import torch

from recommendation_model_sparse_amd import dlrm_interact_bwd, dlrm_interact_fwd, emb_bag_bwd_adagrad, emb_bag_fwd

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def test_wrong_shapes_on_the_device_are_refused():
    T, V, D, B = 3, 20, 16, 5
    tabs = [torch.ones(V, D, device=DEV) for _ in range(T)]
    idx = torch.zeros(T * B * 2, dtype=torch.int64, device=DEV)
    off = torch.arange(0, T * B * 2 + 1, 2, dtype=torch.int64, device=DEV)
    sentinel = torch.full((B, T, D + 1), 7.0, device=DEV)
    say("[binding] refused: out of the wrong shape")
    with pytest.raises(ValueError, match="out must have shape"):
        emb_bag_fwd(tabs, idx, off, out=sentinel)
    with pytest.raises(ValueError, match="per_sample_weights"):
        emb_bag_fwd(tabs, idx, off, torch.ones(3, device=DEV))
    with pytest.raises(ValueError, match="CUDA|must be on"):
        emb_bag_fwd(tabs, idx.cpu(), off)
    dense, pooled = torch.ones(B, D, device=DEV), torch.ones(B, T, D, device=DEV)
    with pytest.raises(ValueError, match="out must have shape"):
        dlrm_interact_fwd(dense, pooled, out=sentinel.view(B, -1)[:, :7].contiguous())
    with pytest.raises(ValueError, match="grad_out must have shape"):
        dlrm_interact_bwd(torch.ones(B, 3, device=DEV), dense, pooled)
    states = [torch.zeros(V, device=DEV) for _ in range(T)]
    with pytest.raises(ValueError, match="grad_pooled must have shape"):
        emb_bag_bwd_adagrad(tabs, states, idx, off, None, torch.ones(B, T, D // 2, device=DEV), 0.01, 1e-8)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())
    assert all(bool((t == 1.0).all()) for t in tabs) and all(bool((s == 0).all()) for s in states)
    say("[binding] a good call still runs")
    out = emb_bag_fwd(tabs, idx, off)
    torch.cuda.synchronize()
    assert bool((out == 2.0).all())


def test_table_set_matches_the_list_form():
    """The same lookup, fused call and Adagrad step through a TableSet and through plain lists give
    bit-identical results, also after one of the set's tables is re-allocated."""
    import numpy as np
    from recommendation_model_sparse_amd import TableSet, emb_bag_interact_fwd
    from gpu_util import random_csr, random_tables, to_dev

    rng = np.random.default_rng(5)
    rows, D, B = [300, 40, 2000], 32, 64
    T = len(rows)
    host = random_tables(rng, rows, D, "f32")
    idx, off, _ = random_csr(rng, T, B, rows, "multi", 9)
    idx, off = to_dev(idx), to_dev(off)
    dense = to_dev(rng.standard_normal((B, D)).astype(np.float32))
    gp = to_dev((rng.standard_normal((B, T, D)) * 1e-2).astype(np.float32))

    def run(use_set):
        tabs = [to_dev(t) for t in host]
        states = [torch.zeros(v, device=DEV) for v in rows]
        ts = TableSet(tabs, states) if use_set else tabs
        out = [emb_bag_fwd(ts, idx, off), emb_bag_interact_fwd(ts, idx, off, None, dense)]
        emb_bag_bwd_adagrad(ts, states, idx, off, None, gp, 0.01, 1e-8)
        tabs[1] = tabs[1].clone()  # a new allocation swapped into the list the set holds
        emb_bag_bwd_adagrad(ts, states, idx, off, None, gp, 0.01, 1e-8)
        out.append(emb_bag_fwd(ts, idx, off))
        torch.cuda.synchronize()
        return out + tabs + states

    say("[binding] table set against lists")
    for a, b in zip(run(False), run(True)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
