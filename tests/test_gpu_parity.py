"""GPU parity: every C-ABI call against the CPU oracle on seeded inputs (needs an MI355X).

Sizes span several tiles / wavefronts with ragged tails.  Gates (relative to the
sum of absolute terms behind each output): 1e-5 for fp32 tables, 1e-2 for bf16
tables (both accumulate in fp32, so both are in fact far below 1e-5);
Adagrad-updated rows 1e-4 in the per-row infinity norm (bf16 rows: half a bf16
ulp on top); integer outputs bit-exact; one-hot pooling bit-exact.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from recommendation_model_sparse_amd import (
    DLRM_FLAG_CHECK_INDICES,
    DLRM_GRAM_MFMA,
    DLRM_GRAM_VALU,
    AdagradOutputs,
    DlrmError,
    dlrm_interact_bwd,
    dlrm_interact_fwd,
    dlrm_interact_fwd_ex,
    emb_bag_bwd_adagrad,
    emb_bag_fwd,
)

from gpu_util import (DEV, as_f64, bf16_half_ulp, random_csr, random_tables, rel_err, row_inf_rel,
                      say, to_dev, to_host)

pytestmark = pytest.mark.gpu

POOL_TOL = {"f32": 1e-5, "bf16": 1e-2}


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32), b.view(torch.int32)) if a.dtype == torch.float32 else torch.equal(a, b)


# ---------------------------------------------------------------- emb_bag_fwd

def run_pool(tables, idx, off, w, B, dtype, label):
    say(f"[pool] {label} T={len(tables)} D={tables[0].shape[1]} {dtype} B={B} nnz={len(idx)} "
        f"weighted={w is not None}")
    tabs = [to_dev(t) for t in tables]
    di, do = to_dev(idx), to_dev(off)
    dw = None if w is None else to_dev(w)
    out = emb_bag_fwd(tabs, di, do, dw)
    out2 = emb_bag_fwd(tabs, di, do, dw)
    torch.cuda.synchronize()
    assert bits_equal(out, out2), "emb_bag_fwd is not bitwise reproducible"
    got = out.cpu().numpy()
    ref, scale = oracle.emb_bag_fwd(tables, idx, off, w, B)
    err = rel_err(got, ref, scale)
    say(f"   max rel err {err:.3e}")
    assert err <= POOL_TOL[dtype]
    assert err <= 1e-5  # fp32 accumulation either way
    return got, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [4, 8, 16, 24, 32, 64, 128, 256, 512])
@pytest.mark.parametrize("mode", ["onehot", "multi", "long"])
@pytest.mark.parametrize("weighted", [False, True])
def test_emb_bag_fwd_random(dtype, D, mode, weighted):
    if dtype == "bf16" and D % 8:
        pytest.skip("bf16 rows must be a multiple of 16 bytes")
    rng = np.random.default_rng(zlib.crc32(f"{dtype}-{D}-{mode}-{weighted}".encode()))
    T, B = 3, 37
    rows = [50, 1, 129]
    tables = random_tables(rng, rows, D, dtype)
    lengths = "onehot" if mode == "onehot" else "multi"
    max_len = 150 if mode == "long" else 12
    idx, off, w = random_csr(rng, T, B, rows, lengths, max_len, weighted)
    if w is not None:
        w[::7] = 0.0
    got, ref = run_pool(tables, idx, off, w, B, dtype, f"{mode}")
    if mode == "onehot":
        # a one-row bag returns the row (times its weight) exactly: fp32 rounding of the exact value
        assert np.array_equal(got, ref.astype(np.float32))


def test_emb_bag_fwd_many_bags_ragged():
    """Enough bags for many workgroups (and an XCD remap with idle tail blocks)."""
    rng = np.random.default_rng(5)
    T, B, D = 5, 1001, 128
    rows = [1000, 3, 70000, 17, 256]
    for dtype in ("f32", "bf16"):
        tables = random_tables(rng, rows, D, dtype)
        for lengths in ("onehot", "multi"):
            idx, off, w = random_csr(rng, T, B, rows, lengths, 30, weighted=True)
            run_pool(tables, idx, off, w, B, dtype, f"ragged-{lengths}")


def test_emb_bag_fwd_edge_cases():
    rng = np.random.default_rng(6)
    D = 16
    # all bags empty (nnz = 0): zeros
    tables = random_tables(rng, [10, 10], D, "f32")
    idx, off, w = random_csr(rng, 2, 9, [10, 10], "empty")
    got, _ = run_pool(tables, idx, off, None, 9, "f32", "all-empty")
    assert np.all(got == 0)
    # B = 1, T = 1, V = 1
    tables = random_tables(rng, [1], D, "bf16")
    idx, off, w = random_csr(rng, 1, 1, [1], "multi", 70)
    run_pool(tables, idx, off, None, 1, "bf16", "B1-T1-V1")
    # every bag hits one row
    tables = random_tables(rng, [40], 64, "f32")
    idx, off, w = random_csr(rng, 1, 300, [40], "multi", 20, hot=7)
    run_pool(tables, idx, off, None, 300, "f32", "hot-row")
    # 64 tables (the limit)
    rows = [int(x) for x in rng.integers(1, 100, 64)]
    tables = random_tables(rng, rows, 8, "bf16")
    idx, off, w = random_csr(rng, 64, 5, rows, "multi", 6)
    run_pool(tables, idx, off, None, 5, "bf16", "T64")


def test_emb_bag_fwd_check_indices_flag():
    rng = np.random.default_rng(7)
    tables = random_tables(rng, [20, 30], 16, "f32")
    idx, off, _ = random_csr(rng, 2, 8, [20, 30], "multi", 5)
    tabs = [to_dev(t) for t in tables]
    say("[pool] check-indices: valid batch")
    out = emb_bag_fwd(tabs, to_dev(idx), to_dev(off), flags=DLRM_FLAG_CHECK_INDICES)
    ref, _ = oracle.emb_bag_fwd(tables, idx, off, None, 8)
    assert np.allclose(out.cpu().numpy(), ref, rtol=1e-5, atol=1e-6)
    bad = idx.copy()
    bad[-1] = 30  # one past the end of table 1
    say("[pool] check-indices: out-of-range index")
    with pytest.raises(DlrmError) as e:
        emb_bag_fwd(tabs, to_dev(bad), to_dev(off), flags=DLRM_FLAG_CHECK_INDICES)
    assert e.value.status == -4
    bad_off = off.copy()
    bad_off[2] = bad_off[3] + 1  # offsets[2] > offsets[3]
    say("[pool] check-indices: decreasing offsets")
    with pytest.raises(DlrmError) as e:
        emb_bag_fwd(tabs, to_dev(idx), to_dev(bad_off), flags=DLRM_FLAG_CHECK_INDICES)
    assert e.value.status == -4


# ---------------------------------------------------------------- interaction

@pytest.mark.parametrize("N", [1, 2, 4, 9, 16, 17, 27, 33, 48, 65])
@pytest.mark.parametrize("D", [4, 12, 16, 32, 64, 128, 256, 512])
def test_interact_fwd_random(N, D):
    rng = np.random.default_rng(N * 1000 + D)
    B = 13
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    say(f"[interact_fwd] B={B} N={N} D={D}")
    out = dlrm_interact_fwd(to_dev(dense), to_dev(pooled))
    out2 = dlrm_interact_fwd(to_dev(dense), to_dev(pooled))
    torch.cuda.synchronize()
    assert bits_equal(out, out2)
    got = out.cpu().numpy()
    ref, scale = oracle.interact_fwd(dense, pooled)
    P = N * (N - 1) // 2
    assert got.shape == (B, P + D)
    err = rel_err(got, ref, scale)
    say(f"   max rel err {err:.3e}")
    assert err <= 1e-5
    assert np.array_equal(got[:, P:], dense)


# each Gram path on its own (the matrix-core Gram at every N, the LDS-staged VALU Gram), against the
# oracle; the batch leaves the VALU kernel's last block with fewer samples than the others
@pytest.mark.parametrize("N", [2, 3, 9, 11, 17, 27, 32, 33, 65])
@pytest.mark.parametrize("D", [16, 64, 128, 256])
@pytest.mark.parametrize("path", [DLRM_GRAM_MFMA, DLRM_GRAM_VALU])
def test_interact_fwd_paths(N, D, path):
    rng = np.random.default_rng(N * 31 + D + path)
    B = 37
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    if path == DLRM_GRAM_VALU and N * (D + 4) * 4 > 64 * 1024:
        with pytest.raises(DlrmError) as e:
            dlrm_interact_fwd_ex(to_dev(dense), to_dev(pooled), path)
        assert e.value.status == -2
        return
    say(f"[interact_fwd path={path}] B={B} N={N} D={D}")
    out = dlrm_interact_fwd_ex(to_dev(dense), to_dev(pooled), path)
    out2 = dlrm_interact_fwd_ex(to_dev(dense), to_dev(pooled), path)
    torch.cuda.synchronize()
    assert bits_equal(out, out2)
    got = out.cpu().numpy()
    ref, scale = oracle.interact_fwd(dense, pooled)
    err = rel_err(got, ref, scale)
    say(f"   max rel err {err:.3e}")
    assert err <= 1e-5
    assert np.array_equal(got[:, N * (N - 1) // 2:], dense)


# D = 128 with N <= 32 takes 1, 2 or 4 samples per wavefront by batch size (thresholds 3072 and
# 12288): each choice, with batches that leave the last wavefront short
@pytest.mark.parametrize("B", [3071, 3072, 4099, 12287, 12289, 16387])
@pytest.mark.parametrize("N", [17, 27, 32])
def test_interact_fwd_samples_per_wave(B, N):
    rng = np.random.default_rng(B * 100 + N)
    D = 128
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    say(f"[interact_fwd] B={B} N={N} D={D}")
    out = dlrm_interact_fwd(to_dev(dense), to_dev(pooled))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref, scale = oracle.interact_fwd(dense, pooled)
    err = rel_err(got, ref, scale)
    say(f"   max rel err {err:.3e}")
    assert err <= 1e-5
    assert np.array_equal(got[:, N * (N - 1) // 2:], dense)


@pytest.mark.parametrize("N", [1, 2, 4, 9, 16, 27, 33, 65])
@pytest.mark.parametrize("D", [4, 16, 32, 64, 128, 256, 512])
def test_interact_bwd_random(N, D):
    rng = np.random.default_rng(N * 7 + D)
    B = 11
    P = N * (N - 1) // 2
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    g = rng.standard_normal((B, P + D)).astype(np.float32)
    say(f"[interact_bwd] B={B} N={N} D={D}")
    gd, gp = dlrm_interact_bwd(to_dev(g), to_dev(dense), to_dev(pooled))
    torch.cuda.synchronize()
    rd, rp, md, mp = oracle.interact_bwd(g, dense, pooled)
    e1 = rel_err(gd.cpu().numpy(), rd, md)
    e2 = rel_err(gp.cpu().numpy(), rp, mp) if N > 1 else 0.0
    say(f"   max rel err dense {e1:.3e} pooled {e2:.3e}")
    assert e1 <= 1e-5 and e2 <= 1e-5


def test_interact_many_samples():
    rng = np.random.default_rng(9)
    B, N, D = 4099, 27, 128
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    say(f"[interact] many samples B={B}")
    out = dlrm_interact_fwd(to_dev(dense), to_dev(pooled))
    ref, scale = oracle.interact_fwd(dense, pooled)
    assert rel_err(out.cpu().numpy(), ref, scale) <= 1e-5
    g = rng.standard_normal(out.shape).astype(np.float32)
    gd, gp = dlrm_interact_bwd(to_dev(g), to_dev(dense), to_dev(pooled))
    rd, rp, md, mp = oracle.interact_bwd(g, dense, pooled)
    assert rel_err(gd.cpu().numpy(), rd, md) <= 1e-5
    assert rel_err(gp.cpu().numpy(), rp, mp) <= 1e-5


# ---------------------------------------------------------------- backward + Adagrad

def run_adagrad(rows, D, dtype, B, lengths, weighted, seed, max_len=12, hot=None, lr=0.01,
                eps=1e-8, random_state=False, label=""):
    rng = np.random.default_rng(seed)
    T = len(rows)
    tables = random_tables(rng, rows, D, dtype)
    states = [(rng.random(v).astype(np.float32) if random_state else np.zeros(v, np.float32)) for v in rows]
    idx, off, w = random_csr(rng, T, B, rows, lengths, max_len, weighted, hot)
    if w is not None:
        w[::5] = 0.0
    gp = (rng.standard_normal((B, T, D)) * 1e-3).astype(np.float32)
    nnz = len(idx)
    say(f"[adagrad] {label} rows={rows[:4]}{'...' if T > 4 else ''} D={D} {dtype} B={B} nnz={nnz} "
        f"weighted={weighted}")
    results = []
    for rep in range(2):
        tabs = [to_dev(t) for t in tables]
        sts = [to_dev(s) for s in states]
        outs = AdagradOutputs(nnz, DEV)
        emb_bag_bwd_adagrad(tabs, sts, to_dev(idx), to_dev(off), None if w is None else to_dev(w),
                            to_dev(gp), lr, eps, outputs=outs)
        torch.cuda.synchronize()
        results.append(([to_host(t) for t in tabs], [s.cpu().numpy() for s in sts], outs))
    (tabs_a, sts_a, outs), (tabs_b, sts_b, _) = results
    for x, y in zip(tabs_a + sts_a, tabs_b + sts_b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), "update is not bitwise reproducible"

    r = oracle.emb_bag_bwd_adagrad(tables, states, idx, off, w, B, gp, lr, eps)
    U = int(outs.num_unique.item())
    assert U == r.U
    assert np.array_equal(outs.unique_keys.cpu().numpy()[:U], r.unique_keys)
    assert np.array_equal(outs.segment_offsets.cpu().numpy()[:U + 1], r.seg_offsets)
    assert np.array_equal(outs.sorted_pos.cpu().numpy()[:nnz], r.perm)
    tt, rr = r.table_and_row()
    worst = 0.0
    for t in range(T):
        sel = tt == t
        urows = rr[sel]
        touched = np.zeros(rows[t], dtype=bool)
        touched[urows] = True
        new = tabs_a[t]
        # untouched rows and states: bit-identical
        assert np.array_equal(new[~touched].view(np.uint8), tables[t][~touched].view(np.uint8))
        assert np.array_equal(sts_a[t][~touched], states[t][~touched])
        if not len(urows):
            continue
        ref_rows = r.new_rows[sel]
        got_rows = as_f64(new[urows])
        if dtype == "f32":
            e = row_inf_rel(got_rows, ref_rows)
            assert e <= 1e-4, e
            worst = max(worst, e)
        else:
            tol = bf16_half_ulp(ref_rows) * 1.0001 + 1e-4 * np.max(np.abs(ref_rows), axis=1, keepdims=True)
            assert np.all(np.abs(got_rows - ref_rows) <= tol)
        ref_s = r.new_state[sel]
        got_s = sts_a[t][urows].astype(np.float64)
        srel = np.abs(got_s - ref_s) / np.where(ref_s == 0, 1.0, ref_s)
        assert np.all(srel <= 1e-4)
    say(f"   U={U} worst row rel err {worst:.3e}")
    return r


# powers of two fill their lane groups; the others leave lanes past the row (12: 3 of 4 lanes,
# 200: 50 of 64, 384: 48 of 64 lanes of 8 columns, 504: 63 of 64)
@pytest.mark.parametrize("D", [4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 136, 200, 256, 264, 384, 504, 512])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("weighted", [False, True])
def test_adagrad_random(D, dtype, weighted):
    if dtype == "bf16" and D % 8:
        pytest.skip("bf16 rows must be a multiple of 16 bytes")
    run_adagrad([300, 7, 1000], D, dtype, 257, "multi", weighted, seed=D * 3 + weighted,
                label="random")


@pytest.mark.parametrize("rows,label", [([200], "8-bit keys: 1 pass of 8"),
                                        ([300, 300], "10-bit keys: 1 pass of 10"),
                                        ([70000, 5], "17-bit keys: 2 passes, 9 + 8 bits"),
                                        ([(1 << 18) + 3], "19-bit keys: 2 passes, 10 + 9 bits"),
                                        ([(1 << 20) + 7], "21-bit keys: 3 passes of 8"),
                                        ([(1 << 24) + 5], "25-bit keys: 3 passes, 9 + 8 + 8 bits"),
                                        ([1], "one row: no pass")])
def test_adagrad_sort_passes(rows, label):
    run_adagrad(rows, 4, "f32", 1500, "multi", True, seed=len(rows) + rows[0] % 97, max_len=10,
                random_state=True, label=label)


@pytest.mark.parametrize("B", [4096 * 16, 4096 * 16 + 1])
def test_adagrad_sort_tiles_around_inline_scan(B):
    """16 sort tiles (each scatter block adds up the raw tile counts itself) and 17 (a scan launch
    per pass), with 17-bit keys (two passes)."""
    run_adagrad([70000], 4, "f32", B, "onehot", True, seed=B % 1000, random_state=True,
                label=f"{B} lookups: {(B + 4095) // 4096} sort tiles")


def test_adagrad_long_segments_cross_chunks():
    """One row hit by every lookup: one segment over ~150 chunks (finisher path)."""
    run_adagrad([50], 128, "f32", 2000, "multi", True, seed=11, max_len=10, hot=3, label="hot-f32")
    run_adagrad([50, 9], 64, "bf16", 1200, "multi", False, seed=12, max_len=10, hot=0, label="hot-bf16")


def test_adagrad_long_segments_partial_lane_groups():
    """Segments over many chunks (partials and the finisher) at widths whose lane groups hold
    lanes past the row."""
    run_adagrad([50], 96, "f32", 2000, "multi", True, seed=15, max_len=10, hot=3, label="hot-f32-D96")
    run_adagrad([40, 9], 200, "bf16", 1200, "multi", False, seed=16, max_len=10, hot=0, label="hot-bf16-D200")
    run_adagrad([30], 384, "f32", 1500, "multi", True, seed=17, max_len=10, hot=1, label="hot-f32-D384")


def test_adagrad_batches_on_both_chunk_lengths():
    """Batches of 2^18 lookups or more walk 64-position chunks at D = 128 (16 per lane group of 4
    lanes at D = 16), smaller ones chunks of half that; both against the oracle, with segments of
    thousands of lookups (a 50-row table) beside mostly single ones (200000 rows)."""
    run_adagrad([50, 200000], 128, "f32", 8000, "multi", True, seed=21, max_len=60, label="long chunks f32")
    run_adagrad([50, 200000], 200, "bf16", 8000, "multi", False, seed=22, max_len=60, label="long chunks bf16 D200")
    run_adagrad([30, 100000], 16, "f32", 131072, "onehot", False, seed=23, label="2^18 lookups: long chunks")
    run_adagrad([30, 100000], 16, "f32", 131071, "onehot", True, seed=24, label="2^18 - 2 lookups: short chunks")


def test_adagrad_64_tables():
    """64 tables (the limit), from one row to a few thousand each, with empty bags: every table's
    row base in the keys, and tables whose keys are all one value."""
    rng = np.random.default_rng(31)
    rows = [int(x) for x in rng.integers(1, 3000, 64)]
    rows[5] = rows[40] = 1
    run_adagrad(rows, 16, "f32", 300, "multi", True, seed=31, max_len=8, label="T64 f32")
    run_adagrad(rows, 64, "bf16", 300, "multi", False, seed=32, max_len=8, label="T64 bf16")


def test_adagrad_onehot_and_zipf_like():
    run_adagrad([100000, 20, 3000], 128, "f32", 4000, "onehot", False, seed=13, label="onehot")
    run_adagrad([5, 6, 7], 16, "f32", 3000, "multi", True, seed=14, max_len=40, label="few rows")


def test_adagrad_edge_cases():
    # nnz = 0: nothing changes, U = 0
    rng = np.random.default_rng(15)
    tables = random_tables(rng, [10], 16, "f32")
    tabs = [to_dev(tables[0])]
    sts = [torch.zeros(10, device=DEV)]
    off = np.zeros(5, dtype=np.int64)
    outs = AdagradOutputs(0, DEV)
    say("[adagrad] nnz=0")
    emb_bag_bwd_adagrad(tabs, sts, to_dev(np.zeros(0, dtype=np.int64)), to_dev(off), None,
                        torch.zeros((4, 1, 16), device=DEV), 0.01, 1e-8, outputs=outs)
    torch.cuda.synchronize()
    assert outs.num_unique.item() == 0 and outs.segment_offsets[0].item() == 0
    assert np.array_equal(to_host(tabs[0]), tables[0])
    # B = 1, T = 1, V = 1
    run_adagrad([1], 8, "bf16", 1, "multi", True, seed=16, max_len=100, label="B1-T1-V1")
    # without the optional outputs
    tables = random_tables(rng, [64], 32, "f32")
    idx, off, w = random_csr(rng, 1, 100, [64], "multi", 9)
    gp = (rng.standard_normal((100, 1, 32)) * 1e-3).astype(np.float32)
    tabs = [to_dev(tables[0])]
    sts = [torch.zeros(64, device=DEV)]
    say("[adagrad] no optional outputs")
    emb_bag_bwd_adagrad(tabs, sts, to_dev(idx), to_dev(off), None, to_dev(gp), 0.01, 1e-8)
    torch.cuda.synchronize()
    r = oracle.emb_bag_bwd_adagrad(tables, [np.zeros(64, np.float32)], idx, off, None, 100, gp,
                                   0.01, 1e-8)
    got = to_host(tabs[0])[r.unique_keys]
    assert row_inf_rel(got, r.new_rows) <= 1e-4


def test_adagrad_check_indices_flag():
    rng = np.random.default_rng(17)
    tables = random_tables(rng, [30], 16, "f32")
    idx, off, _ = random_csr(rng, 1, 20, [30], "multi", 5)
    idx[3] = -1
    tabs = [to_dev(tables[0])]
    sts = [torch.zeros(30, device=DEV)]
    gp = torch.zeros((20, 1, 16), device=DEV)
    say("[adagrad] check-indices: negative index")
    with pytest.raises(DlrmError) as e:
        emb_bag_bwd_adagrad(tabs, sts, to_dev(idx), to_dev(off), None, gp, 0.01, 1e-8,
                            flags=DLRM_FLAG_CHECK_INDICES)
    assert e.value.status == -4
    assert np.array_equal(to_host(tabs[0]), tables[0])
