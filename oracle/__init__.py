"""CPU oracle for the DLRM sparse path (numpy front end of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg.  The GPU library and its Python binding never
import it.  It shares no code with the GPU path; both take their inputs from
the package's seeded generator module.

All results are fp64.  Each function also returns the sum of the absolute
values of the terms behind every output, the scale of the error measure
``|gpu - oracle| / scale``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1

_lib = None


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` with gcc (plain C99 + OpenMP) into ``liboracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.oracle_emb_bag_fwd.argtypes = [i32, i32, i32, p, p, p, p, p, i64, p, p, i32]
        L.oracle_interact_fwd.argtypes = [p, p, i64, i32, i32, p, p, i32]
        L.oracle_emb_interact_fwd.argtypes = [i32, i32, i32, p, p, p, p, p, i64, p, p, p, i32]
        L.oracle_interact_bwd.argtypes = [p, p, p, i64, i32, i32, p, p, p, p, i32]
        L.oracle_emb_bag_bwd_adagrad.argtypes = [i32, i32, i32, p, p, p, p, p, p, i64, i64, p,
                                                 f32, f32, p, p, p, p, p, p]
        L.oracle_emb_bag_bwd_sgd.argtypes = [i32, i32, i32, p, p, p, p, p, i64, i64, p, f32,
                                             p, p, p, p, p]
        for f in (L.oracle_emb_bag_bwd_sgd, L.oracle_emb_bag_fwd, L.oracle_interact_fwd, L.oracle_emb_interact_fwd, L.oracle_interact_bwd,
                  L.oracle_emb_bag_bwd_adagrad):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: oracle precondition failed (code {rc})")


def _tables(tables: Sequence[np.ndarray]):
    dtype = BF16 if tables[0].dtype == np.uint16 else F32
    arrs = [np.ascontiguousarray(t, dtype=np.uint16 if dtype == BF16 else np.float32) for t in tables]
    ptrs = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    rows = np.array([a.shape[0] for a in arrs], dtype=np.int64)
    return dtype, arrs, ptrs, rows


def emb_bag_fwd(tables: Sequence[np.ndarray], indices: np.ndarray, offsets: np.ndarray,
                weights: Optional[np.ndarray], B: int, threads: int = 0):
    """Pooled embeddings [B, T, D] (fp64) and their error scale."""
    dtype, arrs, ptrs, rows = _tables(tables)
    T, D = len(arrs), arrs[0].shape[1]
    indices = np.ascontiguousarray(indices, dtype=np.int64)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    out = np.zeros((B, T, D), dtype=np.float64)
    mag = np.zeros((B, T, D), dtype=np.float64)
    _check(lib().oracle_emb_bag_fwd(T, D, dtype, ptrs, _ptr(rows), _ptr(indices), _ptr(offsets),
                                    _ptr(w), B, _ptr(out), _ptr(mag), threads), "emb_bag_fwd")
    return out, mag


def interact_fwd(dense: np.ndarray, pooled: np.ndarray, threads: int = 0):
    """Interaction output [B, N(N-1)/2 + D] (fp64) and its error scale."""
    dense = np.ascontiguousarray(dense, dtype=np.float32)
    pooled = np.ascontiguousarray(pooled, dtype=np.float32)
    B, D = dense.shape
    N = pooled.shape[1] + 1
    P = N * (N - 1) // 2
    out = np.zeros((B, P + D), dtype=np.float64)
    mag = np.zeros((B, P + D), dtype=np.float64)
    _check(lib().oracle_interact_fwd(_ptr(dense), _ptr(pooled), B, N, D, _ptr(out), _ptr(mag),
                                     threads), "interact_fwd")
    return out, mag


def emb_interact_fwd(tables: Sequence[np.ndarray], indices: np.ndarray, offsets: np.ndarray,
                     weights: Optional[np.ndarray], B: int, dense: np.ndarray, threads: int = 0):
    """Lookup fused with the interaction: [B, N(N-1)/2 + D] (fp64, pooled rows unrounded) and
    its error scale.  N = T + 1."""
    dtype, arrs, ptrs, rows = _tables(tables)
    T, D = len(arrs), arrs[0].shape[1]
    indices = np.ascontiguousarray(indices, dtype=np.int64)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    dense = np.ascontiguousarray(dense, dtype=np.float32)
    if dense.shape != (B, D):
        raise ValueError("dense must be [B, D]")
    N = T + 1
    P = N * (N - 1) // 2
    out = np.zeros((B, P + D), dtype=np.float64)
    mag = np.zeros((B, P + D), dtype=np.float64)
    _check(lib().oracle_emb_interact_fwd(T, D, dtype, ptrs, _ptr(rows), _ptr(indices), _ptr(offsets),
                                         _ptr(w), B, _ptr(dense), _ptr(out), _ptr(mag), threads),
           "emb_interact_fwd")
    return out, mag


def interact_bwd(grad_out: np.ndarray, dense: np.ndarray, pooled: np.ndarray, threads: int = 0):
    """(grad_dense [B,D], grad_pooled [B,N-1,D], scale_dense, scale_pooled), all fp64."""
    grad_out = np.ascontiguousarray(grad_out, dtype=np.float32)
    dense = np.ascontiguousarray(dense, dtype=np.float32)
    pooled = np.ascontiguousarray(pooled, dtype=np.float32)
    B, D = dense.shape
    N = pooled.shape[1] + 1
    gd = np.zeros((B, D), dtype=np.float64)
    gp = np.zeros((B, N - 1, D), dtype=np.float64)
    md = np.zeros_like(gd)
    mp = np.zeros_like(gp)
    _check(lib().oracle_interact_bwd(_ptr(grad_out), _ptr(dense), _ptr(pooled), B, N, D,
                                     _ptr(gd), _ptr(gp), _ptr(md), _ptr(mp), threads),
           "interact_bwd")
    return gd, gp, md, mp


class AdagradResult:
    def __init__(self, unique_keys, seg_offsets, perm, new_rows, new_state, rowbase):
        self.unique_keys = unique_keys      # int64 [U]
        self.seg_offsets = seg_offsets      # int64 [U+1]
        self.perm = perm                    # int32 [nnz]
        self.new_rows = new_rows            # fp64 [U, D]
        self.new_state = new_state          # fp64 [U]
        self.rowbase = rowbase              # int64 [T+1]

    @property
    def U(self) -> int:
        return int(self.unique_keys.shape[0])

    def table_and_row(self):
        """(t, r) of every unique key."""
        t = np.searchsorted(self.rowbase, self.unique_keys, side="right") - 1
        return t, self.unique_keys - self.rowbase[t]


def emb_bag_bwd_adagrad(tables: Sequence[np.ndarray], states: Sequence[np.ndarray],
                        indices: np.ndarray, offsets: np.ndarray, weights: Optional[np.ndarray],
                        B: int, grad_pooled: np.ndarray, lr: float, eps: float) -> AdagradResult:
    dtype, arrs, ptrs, rows = _tables(tables)
    T, D = len(arrs), arrs[0].shape[1]
    st = [np.ascontiguousarray(s, dtype=np.float32) for s in states]
    sptrs = (ctypes.c_void_p * T)(*[s.ctypes.data for s in st])
    indices = np.ascontiguousarray(indices, dtype=np.int64)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    g = np.ascontiguousarray(grad_pooled, dtype=np.float32)
    nnz = int(indices.shape[0])
    n1 = max(nnz, 1)
    uk = np.zeros(n1, dtype=np.int64)
    so = np.zeros(n1 + 1, dtype=np.int64)
    pm = np.zeros(n1, dtype=np.int32)
    nu = np.zeros(1, dtype=np.int64)
    nr = np.zeros((n1, D), dtype=np.float64)
    ns = np.zeros(n1, dtype=np.float64)
    _check(lib().oracle_emb_bag_bwd_adagrad(
        T, D, dtype, ptrs, sptrs, _ptr(rows), _ptr(indices), _ptr(offsets), _ptr(w), B, nnz,
        _ptr(g), float(lr), float(eps), _ptr(uk), _ptr(so), _ptr(pm), _ptr(nu), _ptr(nr),
        _ptr(ns)), "emb_bag_bwd_adagrad")
    U = int(nu[0])
    rowbase = np.zeros(T + 1, dtype=np.int64)
    np.cumsum(rows, out=rowbase[1:])
    return AdagradResult(uk[:U].copy(), so[:U + 1].copy(), pm[:nnz].copy(), nr[:U].copy(),
                         ns[:U].copy(), rowbase)


def emb_bag_bwd_sgd(tables: Sequence[np.ndarray], indices: np.ndarray, offsets: np.ndarray,
                    weights: Optional[np.ndarray], B: int, grad_pooled: np.ndarray,
                    lr: float) -> AdagradResult:
    """Plain SGD on the looked-up rows: E[r] - lr * G_r for each unique row (new_state is empty)."""
    dtype, arrs, ptrs, rows = _tables(tables)
    T, D = len(arrs), arrs[0].shape[1]
    indices = np.ascontiguousarray(indices, dtype=np.int64)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    g = np.ascontiguousarray(grad_pooled, dtype=np.float32)
    nnz = int(indices.shape[0])
    n1 = max(nnz, 1)
    uk = np.zeros(n1, dtype=np.int64)
    so = np.zeros(n1 + 1, dtype=np.int64)
    pm = np.zeros(n1, dtype=np.int32)
    nu = np.zeros(1, dtype=np.int64)
    nr = np.zeros((n1, D), dtype=np.float64)
    _check(lib().oracle_emb_bag_bwd_sgd(
        T, D, dtype, ptrs, _ptr(rows), _ptr(indices), _ptr(offsets), _ptr(w), B, nnz, _ptr(g),
        float(lr), _ptr(uk), _ptr(so), _ptr(pm), _ptr(nu), _ptr(nr)), "emb_bag_bwd_sgd")
    U = int(nu[0])
    rowbase = np.zeros(T + 1, dtype=np.int64)
    np.cumsum(rows, out=rowbase[1:])
    return AdagradResult(uk[:U].copy(), so[:U + 1].copy(), pm[:nnz].copy(), nr[:U].copy(),
                         np.zeros(0), rowbase)


def rel_err(got: np.ndarray, ref: np.ndarray, scale: np.ndarray) -> float:
    """max_o |got - ref| / scale_o; where scale_o == 0 the two must be equal (else inf)."""
    got = np.asarray(got, dtype=np.float64)
    diff = np.abs(got - ref)
    zero = scale == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(diff[~zero] / scale[~zero]))
