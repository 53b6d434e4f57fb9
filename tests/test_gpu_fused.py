"""GPU parity of the lookup fused with the interaction (emb_bag_interact_fwd; needs an MI355X).

Two references for every case: the oracle (fp64, pooled rows unrounded), gate 1e-5 relative
to the sum of absolute product terms behind each dot; and the two-call path
dlrm_interact_fwd(emb_bag_fwd(...)), which the fused kernel must match bit for bit (it runs
the same pooling and matrix-core arithmetic without the HBM round trip).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from recommendation_model_sparse_amd import (
    DLRM_FLAG_CHECK_INDICES,
    DlrmError,
    dlrm_interact_fwd,
    emb_bag_fwd,
    emb_bag_interact_fwd,
)

from gpu_util import DEV, random_csr, random_tables, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def run_fused(tables, idx, off, w, B, dense, label, check_oracle=True):
    T, D = len(tables), tables[0].shape[1]
    say(f"[fused] {label} T={T} D={D} {tables[0].dtype} B={B} nnz={len(idx)} weighted={w is not None}")
    tabs = [to_dev(t) for t in tables]
    di, do, dd = to_dev(idx), to_dev(off), to_dev(dense)
    dw = None if w is None else to_dev(w)
    out = emb_bag_interact_fwd(tabs, di, do, dw, dd)
    two = dlrm_interact_fwd(dd, emb_bag_fwd(tabs, di, do, dw))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), two.view(torch.int32)), "fused != two-call path"
    got = out.cpu().numpy()
    if check_oracle:
        ref, scale = oracle.emb_interact_fwd(tables, idx, off, w, B, dense)
        err = rel_err(got, ref, scale)
        say(f"   max rel err {err:.3e}")
        assert err <= 1e-5
    return got


@pytest.mark.parametrize("dtype,D", [("f32", 16), ("f32", 32), ("f32", 64), ("f32", 128), ("f32", 256),
                                     ("bf16", 32), ("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512)])
@pytest.mark.parametrize("mode", ["onehot", "multi", "long"])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("T", [3, 10, 26])
def test_fused_random(dtype, D, mode, weighted, T):
    rng = np.random.default_rng(zlib.crc32(f"fused-{dtype}-{D}-{mode}-{weighted}-{T}".encode()))
    B = 37  # not a multiple of the samples per block
    rows = [int(v) for v in rng.integers(1, 300, T)]
    tables = random_tables(rng, rows, D, dtype)
    max_len = 150 if mode == "long" else 12
    idx, off, w = random_csr(rng, T, B, rows, "onehot" if mode == "onehot" else "multi", max_len, weighted)
    dense = rng.standard_normal((B, D)).astype(np.float32)
    got = run_fused(tables, idx, off, w, B, dense, mode)
    P = (T + 1) * T // 2
    assert np.array_equal(got[:, P:], dense)


def test_fused_empty_batch_with_weights():
    """nnz = 0 with a weights tensor: every pooled row is zero, the weights are never read."""
    rng = np.random.default_rng(34)
    for T, D in [(3, 128), (10, 64), (26, 128)]:
        tables = random_tables(rng, [7] * T, D, "bf16")
        idx, off, _ = random_csr(rng, T, 5, [7] * T, "empty")
        w = np.zeros(0, np.float32)
        dense = rng.standard_normal((5, D)).astype(np.float32)
        got = run_fused(tables, idx, off, w, 5, dense, "empty-weighted")
        assert np.all(got[:, :(T + 1) * T // 2] == 0)


def test_fused_short_bags_group_mode():
    """Bags of 0-2 lookups (fewer than 4 per bag on average): one lane group per bag, several
    samples per block, ragged last block."""
    rng = np.random.default_rng(31)
    for T, B, D, dtype in [(8, 4099, 128, "bf16"), (1, 9, 32, "f32"), (26, 513, 64, "f32")]:
        rows = [int(v) for v in rng.integers(1, 5000, T)]
        tables = random_tables(rng, rows, D, dtype)
        idx, off, w = random_csr(rng, T, B, rows, "multi", 2, weighted=True)
        dense = rng.standard_normal((B, D)).astype(np.float32)
        run_fused(tables, idx, off, w, B, dense, "short-bags")


def test_fused_edge_cases():
    rng = np.random.default_rng(32)
    # all bags empty: every dot that involves a pooled row is 0
    T, B, D = 4, 6, 32
    tables = random_tables(rng, [10] * T, D, "f32")
    idx, off, _ = random_csr(rng, T, B, [10] * T, "empty")
    dense = rng.standard_normal((B, D)).astype(np.float32)
    got = run_fused(tables, idx, off, None, B, dense, "all-empty")
    assert np.all(got[:, :(T + 1) * T // 2] == 0)
    # B = 1, one table with one row, a bag longer than two wavefronts of indices
    tables = random_tables(rng, [1], 64, "bf16")
    idx, off = np.zeros(150, dtype=np.int64), np.array([0, 150], dtype=np.int64)
    run_fused(tables, idx, off, None, 1, rng.standard_normal((1, 64)).astype(np.float32), "B1")
    # 64 tables (N = 65: five 16-row blocks, 15 upper blocks), short and long bags
    rows = [int(x) for x in rng.integers(1, 100, 64)]
    tables = random_tables(rng, rows, 32, "bf16")
    for max_len in (2, 6, 12):
        idx, off, w = random_csr(rng, 64, 5, rows, "multi", max_len, weighted=True)
        run_fused(tables, idx, off, w, 5, rng.standard_normal((5, 32)).astype(np.float32), f"T64-len{max_len}")
    # N = 33 (three row blocks) with short bags at the smallest row width
    rows = [int(x) for x in rng.integers(1, 100, 32)]
    tables = random_tables(rng, rows, 16, "f32")
    idx, off, w = random_csr(rng, 32, 7, rows, "onehot")
    run_fused(tables, idx, off, None, 7, rng.standard_normal((7, 16)).astype(np.float32), "T32-onehot")
    # every lookup hits one row
    tables = random_tables(rng, [40, 40], 128, "f32")
    idx, off, _ = random_csr(rng, 2, 300, [40, 40], "multi", 20, hot=7)
    run_fused(tables, idx, off, None, 300, rng.standard_normal((300, 128)).astype(np.float32), "hot-row")


def test_fused_unsupported_shapes_and_check_flag():
    rng = np.random.default_rng(33)
    # D = 48 fp32 (192-byte rows) and N*(D+4)*4 over 64 KiB are refused, not computed
    for rows, D, T in [([10] * 2, 48, 2), ([10] * 64, 256, 64)]:
        tables = random_tables(rng, rows, D, "f32")
        idx, off, _ = random_csr(rng, T, 3, rows, "multi", 3)
        say(f"[fused] unsupported T={T} D={D}")
        with pytest.raises(DlrmError) as e:
            emb_bag_interact_fwd([to_dev(t) for t in tables], to_dev(idx), to_dev(off), None,
                                 to_dev(np.zeros((3, D), np.float32)))
        assert e.value.status == -2
    tables = random_tables(rng, [20, 30], 16, "f32")
    idx, off, _ = random_csr(rng, 2, 8, [20, 30], "multi", 5)
    tabs = [to_dev(t) for t in tables]
    dense = rng.standard_normal((8, 16)).astype(np.float32)
    say("[fused] check-indices: valid batch")
    out = emb_bag_interact_fwd(tabs, to_dev(idx), to_dev(off), None, to_dev(dense), flags=DLRM_FLAG_CHECK_INDICES)
    ref, scale = oracle.emb_interact_fwd(tables, idx, off, None, 8, dense)
    assert rel_err(out.cpu().numpy(), ref, scale) <= 1e-5
    bad = idx.copy()
    bad[0] = -1
    say("[fused] check-indices: negative index")
    with pytest.raises(DlrmError) as e:
        emb_bag_interact_fwd(tabs, to_dev(bad), to_dev(off), None, to_dev(dense), flags=DLRM_FLAG_CHECK_INDICES)
    assert e.value.status == -4
