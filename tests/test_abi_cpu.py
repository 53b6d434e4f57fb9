"""The C-ABI library on a machine without a GPU: it loads, exports what the headers declare,
and rejects invalid arguments on the host before anything touches a device.

No call here reaches a kernel launch: every case fails host validation (fake device pointers
are never dereferenced).
"""
import ctypes
import os
import re
import subprocess

import pytest

from recommendation_model_sparse_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

OK, INVALID, UNSUPPORTED, HIP, INDEX, WORKSPACE = 0, -1, -2, -3, -4, -5
FAKE = 0x7F0000000000  # a 256-byte aligned address that is never dereferenced


def declared_functions():
    names = set()
    for h in os.listdir(INCLUDE):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"emb_bag_fwd", "emb_bag_fwd_ex", "emb_bag_bwd_update", "emb_bag_bwd_plan", "emb_bag_bwd_apply", "emb_bag_interact_fwd", "dlrm_interact_fwd", "dlrm_interact_bwd", "emb_bag_bwd_workspace_size",
            "emb_bag_bwd_adagrad", "dlrm_status_string", "dlrm_synth_fill_table",
            "dlrm_trace_enable", "dlrm_trace_read"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_status_strings(L):
    for s in (OK, INVALID, UNSUPPORTED, HIP, INDEX, WORKSPACE):
        assert binding.status_string(s)
    assert "unknown" in binding.status_string(17)


def ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def i64s(*vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def fwd(L, tables=None, rows=None, T=1, D=16, dtype=0, idx=FAKE, off=FAKE, w=None, B=4, nnz=4,
        out=FAKE, flags=0):
    tables = ptrs(FAKE) if tables is None else tables
    rows = i64s(10) if rows is None else rows
    return L.emb_bag_fwd(tables, rows, T, D, dtype, idx, off, w, B, nnz, out, flags, None)


def test_emb_bag_fwd_rejects(L):
    assert fwd(L, T=0) == INVALID
    assert fwd(L, T=65, tables=ptrs(*[FAKE] * 65), rows=i64s(*[1] * 65)) == INVALID
    assert fwd(L, D=0) == INVALID
    assert fwd(L, D=6) == UNSUPPORTED          # fp32 rows must be a multiple of 16 bytes
    assert fwd(L, D=12, dtype=1) == UNSUPPORTED  # bf16 rows likewise
    assert fwd(L, D=1024) == UNSUPPORTED
    assert fwd(L, dtype=7) == INVALID
    assert fwd(L, B=-1) == INVALID
    assert fwd(L, nnz=-1) == INVALID
    assert fwd(L, tables=ptrs(0)) == INVALID
    assert fwd(L, tables=ptrs(FAKE + 4)) == INVALID   # misaligned table
    assert fwd(L, rows=i64s(0)) == INVALID
    assert fwd(L, off=0) == INVALID
    assert fwd(L, idx=0) == INVALID
    assert fwd(L, idx=FAKE + 4) == INVALID
    assert fwd(L, out=0) == INVALID
    assert fwd(L, out=FAKE + 4) == INVALID
    assert fwd(L, flags=8) == INVALID
    assert fwd(L, B=0, nnz=3) == INVALID
    assert fwd(L, B=0, nnz=0) == OK            # nothing to do, nothing launched
    assert fwd(L, B=1 << 30, T=2, tables=ptrs(FAKE, FAKE), rows=i64s(1, 1)) == UNSUPPORTED


def fwd_ex(L, index_type=0, out_dtype=0, idx=FAKE, off=FAKE, out=FAKE, D=16, dtype=0):
    return L.emb_bag_fwd_ex(ptrs(FAKE), i64s(10), 1, D, dtype, idx, off, index_type, None, 4, 4, out,
                            out_dtype, 0, None)


def test_emb_bag_fwd_ex_rejects(L):
    assert fwd_ex(L, index_type=2) == INVALID
    assert fwd_ex(L, out_dtype=3) == INVALID
    assert fwd_ex(L, index_type=0, idx=FAKE + 4) == INVALID   # int64 indices need 8-byte alignment
    assert fwd_ex(L, index_type=1, idx=FAKE + 2) == INVALID   # int32 indices need 4-byte alignment
    assert fwd_ex(L, index_type=1, off=FAKE + 6) == INVALID
    assert fwd_ex(L, out=FAKE + 8) == INVALID                 # output 16-byte aligned
    assert fwd_ex(L, D=6) == UNSUPPORTED


def upd(L, optimizer=0, index_type=0, state=True, T=1, D=16, wsz=None, idx=FAKE):
    rows = [10] * T
    st = ptrs(*[FAKE] * T) if state else None
    if wsz is None:
        wsz = binding.emb_bag_bwd_workspace_size(rows, D, 4, 4)
    return L.emb_bag_bwd_update(ptrs(*[FAKE] * T), st, i64s(*rows), T, D, 0, idx, FAKE, index_type, None, 4,
                                4, FAKE, optimizer, 0.01, 1e-8, FAKE, wsz, None, None, None, None, 0, None)


def test_emb_bag_bwd_update_rejects(L):
    assert upd(L, optimizer=2) == INVALID
    assert upd(L, index_type=5) == INVALID
    assert upd(L, optimizer=0, state=False) == INVALID       # Adagrad needs its state
    assert upd(L, optimizer=1, state=False, wsz=1) == WORKSPACE  # SGD takes no state; reaches the workspace check
    assert upd(L, index_type=1, idx=FAKE + 2) == INVALID
    assert upd(L, D=20, wsz=1) == WORKSPACE        # any multiple of 4 passes the width check
    assert upd(L, D=260) == UNSUPPORTED


def plan(L, T=1, D=16, index_type=0, wsz=None, flags=0, rows=None, idx=FAKE):
    rows = [10] * T if rows is None else rows
    if wsz is None:
        wsz = binding.emb_bag_bwd_workspace_size(rows, D, 4, 4)
    return L.emb_bag_bwd_plan(i64s(*rows), T, D, idx, FAKE, index_type, None, 4, 4, FAKE, wsz, None, None,
                              None, None, flags, None)


def test_emb_bag_bwd_plan_rejects(L):
    assert plan(L, index_type=5) == INVALID
    assert plan(L, T=0, rows=[]) == INVALID
    assert plan(L, D=260) == UNSUPPORTED
    assert plan(L, D=24, wsz=1) == WORKSPACE       # any multiple of 4 passes the width check
    assert plan(L, flags=4) == INVALID
    assert plan(L, wsz=1) == WORKSPACE
    assert plan(L, index_type=1, idx=FAKE + 2) == INVALID
    assert plan(L, T=2, rows=[2 ** 31, 2 ** 31 + 1], wsz=1 << 20) == UNSUPPORTED  # keys over 32 bits


def apply(L, optimizer=0, state=True, T=1, D=16, dtype=0, grad=FAKE, wsz=None, tables=None):
    rows = [10] * T
    st = ptrs(*[FAKE] * T) if state else None
    if wsz is None:
        wsz = binding.emb_bag_bwd_workspace_size(rows, D, 4, 4)
    tabs = ptrs(*[FAKE] * T) if tables is None else tables
    return L.emb_bag_bwd_apply(tabs, st, i64s(*rows), T, D, dtype, 4, 4, 0, grad, optimizer, 0.01, 1e-8, FAKE,
                               wsz, None, None)


def test_emb_bag_bwd_apply_rejects(L):
    assert apply(L, optimizer=2) == INVALID
    assert apply(L, state=False) == INVALID                 # Adagrad needs its state
    assert apply(L, optimizer=1, state=False, wsz=1) == WORKSPACE
    assert apply(L, D=260) == UNSUPPORTED
    assert apply(L, D=12, dtype=1) == UNSUPPORTED   # 24-byte bf16 rows
    assert apply(L, D=24, wsz=1) == WORKSPACE       # any multiple of 4 passes the width check
    assert apply(L, D=4, dtype=1) == UNSUPPORTED            # bf16 rows under 16 bytes
    assert apply(L, dtype=3) == INVALID
    assert apply(L, grad=FAKE + 4) == INVALID               # grad_pooled 16-byte aligned
    assert apply(L, tables=ptrs(FAKE + 8)) == INVALID
    assert apply(L, wsz=1) == WORKSPACE


def fused(L, T=2, D=32, dtype=0, rows=None, tables=None, dense=FAKE, out=FAKE, B=4, nnz=4, flags=0):
    tables = ptrs(*[FAKE] * T) if tables is None else tables
    rows = i64s(*([10] * T)) if rows is None else rows
    return L.emb_bag_interact_fwd(tables, rows, T, D, dtype, FAKE, FAKE, None, B, nnz, dense, out, flags, None)


def test_emb_bag_interact_fwd_rejects(L):
    assert fused(L, T=0) == INVALID
    assert fused(L, D=48) == UNSUPPORTED            # 192-byte rows: not a power-of-two chunk count
    assert fused(L, D=8) == UNSUPPORTED             # D % 16
    assert fused(L, D=16, dtype=1) == UNSUPPORTED   # 32-byte bf16 rows
    assert fused(L, D=512) == UNSUPPORTED           # 2 KiB fp32 rows
    assert fused(L, T=64, D=256) == UNSUPPORTED     # X of one sample over 64 KiB
    assert fused(L, dense=0) == INVALID
    assert fused(L, dense=FAKE + 4) == INVALID
    assert fused(L, out=0) == INVALID
    assert fused(L, flags=4) == INVALID
    assert fused(L, B=0, nnz=1) == INVALID
    assert fused(L, B=0, nnz=0) == OK


def test_interact_rejects(L):
    f = L.dlrm_interact_fwd
    assert f(FAKE, FAKE, 4, 0, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 4, 66, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 4, 5, 6, FAKE, None) == UNSUPPORTED
    assert f(FAKE, FAKE, 4, 5, 1024, FAKE, None) == UNSUPPORTED
    assert f(None, FAKE, 4, 5, 16, FAKE, None) == INVALID
    assert f(FAKE, None, 4, 5, 16, FAKE, None) == INVALID
    assert f(FAKE + 4, FAKE, 4, 5, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, -1, 5, 16, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 0, 5, 16, FAKE, None) == OK
    b = L.dlrm_interact_bwd
    assert b(None, FAKE, FAKE, 4, 5, 16, FAKE, FAKE, None) == INVALID
    assert b(FAKE, FAKE, FAKE, 4, 5, 16, FAKE, None, None) == INVALID
    assert b(FAKE, FAKE, FAKE, 4, 5, 16, FAKE + 8, FAKE, None) == INVALID
    assert b(FAKE, FAKE, FAKE, 4, 5, 6, FAKE, FAKE, None) == UNSUPPORTED


def test_sgd_dense_multi_rejects(L):
    f = L.dlrm_sgd_dense_multi
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    assert f(65, arr(FAKE), None, arr(FAKE), i64s(1), 0.1, None) == INVALID   # more than 64 parameters
    assert f(-1, None, None, None, None, 0.1, None) == INVALID
    assert f(0, None, None, None, None, 0.1, None) == OK                      # nothing to do
    assert f(1, None, None, arr(FAKE), i64s(1), 0.1, None) == INVALID
    assert f(1, arr(FAKE), None, arr(FAKE), i64s(-1), 0.1, None) == INVALID
    assert f(1, arr(0), None, arr(FAKE), i64s(4), 0.1, None) == INVALID       # null parameter


def test_workspace_size(L):
    ws = lambda rows, D, B, nnz: binding.emb_bag_bwd_workspace_size(rows, D, B, nnz)
    assert ws([100], 6, 4, 10) == 0          # D must be a multiple of 4
    assert ws([100], 260, 4, 10) == 0        # and of 8 above 256
    assert ws([100], 1024, 4, 10) == 0
    for D in (4, 12, 24, 48, 96, 136, 200, 264, 384, 504):
        assert ws([100], D, 4, 10) > 0, D    # any other row of 16-byte multiples
    a, b = ws([100, 200], 128, 64, 1000), ws([100, 200], 128, 64, 100000)
    assert 0 < a < b
    assert a % 256 == 0 and b % 256 == 0
    assert ws([100], 128, 4, 0) > 0           # valid for an empty batch too


def test_workspace_size_covers_smaller_batches(L):
    """A workspace sized for nnz lookups serves every smaller batch: sizes never decrease with nnz,
    also where batches below 2^18 lookups switch to shorter segment-reduce chunks (more partials)."""
    ws = lambda D, nnz: binding.emb_bag_bwd_workspace_size([1000, 5000], D, 64, nnz)
    for D in (4, 16, 128, 200, 512):
        sizes = [ws(D, n) for n in (1, 4096, (1 << 18) - 2, (1 << 18) - 1, 1 << 18, (1 << 18) + 1, 1 << 19)]
        assert all(a <= b for a, b in zip(sizes, sizes[1:])), (D, sizes)


def bwd(L, T=1, D=16, dtype=0, B=4, nnz=4, rows=None, ws=FAKE, wsz=None, grad=FAKE, state=None,
        tables=None, flags=0):
    rows = rows if rows is not None else [10] * T
    r = i64s(*rows)
    tables = tables if tables is not None else ptrs(*[FAKE] * T)
    state = state if state is not None else ptrs(*[FAKE] * T)
    if wsz is None:
        wsz = binding.emb_bag_bwd_workspace_size(rows, D, B, nnz)
    return L.emb_bag_bwd_adagrad(tables, state, r, T, D, dtype, FAKE, FAKE, None, B, nnz, grad,
                                 0.01, 1e-8, ws, wsz, None, None, None, None, flags, None)


def test_emb_bag_bwd_rejects(L):
    assert bwd(L, D=6) == UNSUPPORTED          # rows of 24 bytes: not a multiple of 16
    assert bwd(L, D=260) == UNSUPPORTED        # fp32 above 256 needs a multiple of 8
    assert bwd(L, D=4, dtype=1) == UNSUPPORTED  # bf16 rows below 16 bytes
    assert bwd(L, D=12, dtype=1) == UNSUPPORTED  # 24-byte bf16 rows
    assert bwd(L, rows=[1 << 31, 1 << 31, 5], T=3) == UNSUPPORTED  # keys beyond 32 bits
    assert bwd(L, state=ptrs(0)) == INVALID
    assert bwd(L, grad=0) == INVALID
    assert bwd(L, grad=FAKE + 4) == INVALID
    assert bwd(L, ws=0) == WORKSPACE
    assert bwd(L, ws=FAKE + 16) == WORKSPACE    # workspace must be 256-byte aligned
    need = binding.emb_bag_bwd_workspace_size([10], 16, 4, 4)
    assert bwd(L, wsz=need - 1) == WORKSPACE
    assert bwd(L, flags=2) == INVALID
    assert bwd(L, B=0, nnz=2) == INVALID


def test_trace_api_without_gpu(L):
    binding.dlrm_trace_enable(True)
    assert binding.dlrm_trace_read() == {}
    binding.dlrm_trace_enable(False)
    n = ctypes.c_int32(0)
    assert L.dlrm_trace_read(-1, None, None, None, ctypes.byref(n)) == INVALID


def test_synth_fill_rejects(L):
    f = L.dlrm_synth_fill_table
    assert f(None, 0, 10, 16, 0, 1, 1.0, None) == INVALID
    assert f(FAKE, 0, 0, 16, 0, 1, 1.0, None) == INVALID
    assert f(FAKE, 0, 10, 6, 0, 1, 1.0, None) == INVALID
    assert f(FAKE, 2, 10, 16, 0, 1, 1.0, None) == INVALID
    assert f(FAKE + 4, 0, 10, 16, 0, 1, 1.0, None) == INVALID


def test_dense_layer_calls_reject(L):
    ws = binding.dlrm_linear_workspace_size(64, 32, 16)
    assert ws > (32 << 20) and binding.dlrm_linear_workspace_size(0, 32, 16) == 0
    # the weight gradient of a 16384-row batch is split in 8 slices of 2048 rows
    assert binding.dlrm_linear_workspace_size(16384, 1024, 1024) >= 8 * 1024 * 1024 * 4
    f = lambda M=64, N=32, K=16, act=1, yt=1, y=FAKE, wsz=ws: L.dlrm_linear_fwd(FAKE, FAKE, FAKE, M, N, K, act, y, yt,
                                                                                FAKE, wsz, None)
    assert f(N=12) == UNSUPPORTED       # rows of 16 bytes: N, K multiples of 8
    assert f(K=20) == UNSUPPORTED
    assert f(M=0) == INVALID
    assert f(act=3) == INVALID
    assert f(yt=2) == INVALID
    assert f(y=0) == INVALID
    assert f(y=FAKE + 8) == INVALID
    assert f(wsz=ws - 1) == WORKSPACE
    bw = lambda dy=FAKE, y=FAKE, act=1, dz=FAKE, wsz=ws: L.dlrm_linear_bwd(dy, y, 1, act, FAKE, FAKE, 64, 32, 16, dz,
                                                                           None, FAKE, FAKE, FAKE, wsz, None)
    assert bw(dy=0) == INVALID
    assert bw(y=None, act=1) == INVALID   # ReLU needs the forward output
    assert bw(dz=0) == INVALID
    assert bw(wsz=100) == WORKSPACE
    hws = binding.dlrm_bce_head_workspace_size(64, 256)
    h = lambda K=256, wsz=hws, x=FAKE: L.dlrm_bce_head(x, FAKE, FAKE, FAKE, 64, K, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                       wsz, None)
    assert h(K=2048) == UNSUPPORTED
    assert h(K=12) == UNSUPPORTED
    assert h(x=0) == INVALID
    assert h(wsz=hws - 1) == WORKSPACE
    assert L.dlrm_sgd_dense(FAKE, None, FAKE, -1, 0.1, None) == INVALID
    assert L.dlrm_sgd_dense(None, None, None, 0, 0.1, None) == OK
    assert L.dlrm_cast_rows(FAKE, 0, 16, 4, 17, FAKE, 1, 16, None) == INVALID   # cols > dst_cols
    assert L.dlrm_cast_rows(FAKE, 0, 8, 4, 13, FAKE, 1, 16, None) == INVALID    # cols > src_ld
    assert L.dlrm_cast_rows(FAKE, 3, 16, 4, 13, FAKE, 1, 16, None) == INVALID


def test_size_limits_rejected(L):
    """Positions and bags are 32-bit on the device: nnz >= 2^31 or T*B >= 2^31 is refused on the
    host by every entry point that takes a batch, before any workspace or device access."""
    big = 1 << 31
    assert fwd(L, nnz=big) == UNSUPPORTED
    assert fwd(L, B=big // 2, T=2, tables=ptrs(FAKE, FAKE), rows=i64s(1, 1)) == UNSUPPORTED
    assert fused(L, nnz=big) == UNSUPPORTED
    rows = [10]
    for n, B in ((big, 4), (4, big)):
        assert L.emb_bag_bwd_update(ptrs(FAKE), ptrs(FAKE), i64s(*rows), 1, 16, 0, FAKE, FAKE, 0, None, B, n, FAKE,
                                    0, 0.01, 1e-8, FAKE, 1, None, None, None, None, 0, None) == UNSUPPORTED
        assert L.emb_bag_bwd_plan(i64s(*rows), 1, 16, FAKE, FAKE, 0, None, B, n, FAKE, 1, None, None, None, None,
                                  0, None) == UNSUPPORTED
        assert L.emb_bag_bwd_apply(ptrs(FAKE), ptrs(FAKE), i64s(*rows), 1, 16, 0, B, n, 0, FAKE, 0, 0.01, 1e-8,
                                   FAKE, 1, None, None) == UNSUPPORTED


def test_probes_reject(L):
    r = L.dlrm_probe_read
    assert r(None, 1024, FAKE, 8, None) == INVALID
    assert r(FAKE, 1000, FAKE, 8, None) == INVALID     # not a multiple of 16 bytes
    assert r(FAKE, 0, FAKE, 8, None) == INVALID
    assert r(FAKE + 8, 1024, FAKE, 8, None) == INVALID
    assert r(FAKE, 1024, FAKE, 0, None) == INVALID
    g = L.dlrm_probe_gather
    assert g(FAKE, 0, 256, FAKE, 4, FAKE, 8, None) == INVALID
    assert g(FAKE, 10, 24, FAKE, 4, FAKE, 8, None) == INVALID      # not a multiple of 16
    assert g(FAKE, 10, 2048, FAKE, 4, FAKE, 8, None) == INVALID    # above 1024 bytes
    assert g(FAKE, 10, 48, FAKE, 4, FAKE, 8, None) == INVALID      # 3 lanes per row
    assert g(FAKE, 10, 256, None, 4, FAKE, 8, None) == INVALID
    assert g(FAKE, 10, 256, FAKE, 1 << 31, FAKE, 8, None) == INVALID
    assert g(FAKE, 10, 256, FAKE, 0, FAKE, 8, None) == OK          # nothing to read


def test_noalloc_refuses_batches_beyond_its_scratch(L):
    """The allocation-free backward sizes the batch on the host: one whose workspace exceeds the
    fixed scratch is refused with DLRM_ERR_WORKSPACE before any device access."""
    cap = binding.emb_bag_bwd_noalloc_max_bytes()
    assert cap == 64 << 20
    big = 4 << 20
    assert binding.emb_bag_bwd_workspace_size([1000], 128, 1, big) > cap
    rc = L.emb_bag_bwd_update_noalloc(ptrs(FAKE), ptrs(FAKE), i64s(1000), 1, 128, 0, FAKE, FAKE, 0, None, 1, big,
                                      FAKE, 0, 0.01, 1e-8, None, None, None, None, 0, None)
    assert rc == WORKSPACE
    # the ordinary argument checks come first
    assert L.emb_bag_bwd_update_noalloc(ptrs(FAKE), ptrs(FAKE), i64s(1000), 1, 260, 0, FAKE, FAKE, 0, None, 1, 4,
                                        FAKE, 0, 0.01, 1e-8, None, None, None, None, 0, None) == UNSUPPORTED


def test_interact_fwd_ex_rejects(L):
    f = L.dlrm_interact_fwd_ex
    assert f(FAKE, FAKE, 4, 5, 16, FAKE, 3, None) == INVALID          # no such path
    assert f(FAKE, FAKE, 4, 5, 16, FAKE, -1, None) == INVALID
    assert f(FAKE, FAKE, 4, 200, 16, FAKE, 1, None) == INVALID        # N beyond 65
    assert f(FAKE, FAKE, 4, 27, 1024, FAKE, 2, None) == UNSUPPORTED   # D above 512
    assert f(FAKE, FAKE, 4, 27, 12, FAKE, 2, None) == UNSUPPORTED     # VALU: D not a multiple of 16
    assert f(FAKE, FAKE, 4, 65, 256, FAKE, 2, None) == UNSUPPORTED    # VALU: one sample's X over 64 KiB
    assert f(FAKE, FAKE, 0, 27, 128, FAKE, 2, None) == OK             # empty batch
