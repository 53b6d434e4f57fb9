"""Python binding of ``libdlrm_sparse.so`` (ctypes; argument marshalling only).

Each function has the name of the C entry point it calls and passes device
pointers of torch tensors plus the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback: if the
library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdlrm_sparse.so")

DLRM_F32, DLRM_BF16 = 0, 1
DLRM_INDEX_I64, DLRM_INDEX_I32 = 0, 1
DLRM_OPT_ADAGRAD, DLRM_OPT_SGD = 0, 1
DLRM_ACT_NONE, DLRM_ACT_RELU = 0, 1
DLRM_FLAG_CHECK_INDICES = 1

_lib = None


class DlrmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m recommendation_model_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64, u32, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                          ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float,
                                          ctypes.c_size_t)
        L.emb_bag_fwd.argtypes = [p, p, i32, i32, i32, p, p, p, i64, i64, p, u32, p]
        L.emb_bag_fwd_ex.argtypes = [p, p, i32, i32, i32, p, p, i32, p, i64, i64, p, i32, u32, p]
        L.emb_bag_bwd_update.argtypes = [p, p, p, i32, i32, i32, p, p, i32, p, i64, i64, p, i32, f32, f32,
                                         p, sz, p, p, p, p, u32, p]
        L.emb_bag_bwd_plan.argtypes = [p, i32, i32, p, p, i32, p, i64, i64, p, sz, p, p, p, p, u32, p]
        L.emb_bag_bwd_apply.argtypes = [p, p, p, i32, i32, i32, i64, i64, i32, p, i32, f32, f32, p, sz, p, p]
        L.dlrm_interact_fwd.argtypes = [p, p, i64, i32, i32, p, p]
        L.emb_bag_interact_fwd.argtypes = [p, p, i32, i32, i32, p, p, p, i64, i64, p, p, u32, p]
        L.dlrm_interact_bwd.argtypes = [p, p, p, i64, i32, i32, p, p, p]
        L.emb_bag_bwd_workspace_size.argtypes = [i32, p, i32, i64, i64]
        L.emb_bag_bwd_workspace_size.restype = sz
        L.emb_bag_bwd_adagrad.argtypes = [p, p, p, i32, i32, i32, p, p, p, i64, i64, p, f32, f32,
                                          p, sz, p, p, p, p, u32, p]
        L.dlrm_linear_workspace_size.argtypes = [i64, i32, i32]
        L.dlrm_linear_workspace_size.restype = sz
        L.dlrm_bce_head_workspace_size.argtypes = [i64, i32]
        L.dlrm_bce_head_workspace_size.restype = sz
        L.dlrm_linear_fwd.argtypes = [p, p, p, i64, i32, i32, i32, p, i32, p, sz, p]
        L.dlrm_linear_bwd.argtypes = [p, p, i32, i32, p, p, i64, i32, i32, p, p, p, p, p, sz, p]
        L.dlrm_bce_head.argtypes = [p, p, p, p, i64, i32, p, p, p, p, p, p, sz, p]
        L.dlrm_sgd_dense.argtypes = [p, p, p, i64, f32, p]
        L.dlrm_sgd_dense_multi.argtypes = [i32, p, p, p, p, f32, p]
        L.dlrm_cast_rows.argtypes = [p, i32, i64, i64, i32, p, i32, i32, p]
        for f in (L.dlrm_linear_fwd, L.dlrm_linear_bwd, L.dlrm_bce_head, L.dlrm_sgd_dense, L.dlrm_cast_rows):
            f.restype = ctypes.c_int
        L.dlrm_status_string.argtypes = [ctypes.c_int]
        L.dlrm_status_string.restype = ctypes.c_char_p
        L.dlrm_synth_fill_table.argtypes = [p, i32, i64, i32, i32, u64, f32, p]
        L.dlrm_trace_enable.argtypes = [ctypes.c_int]
        L.dlrm_trace_read.argtypes = [i32, p, p, p, p]
        for f in (L.emb_bag_fwd, L.emb_bag_fwd_ex, L.emb_bag_bwd_update, L.dlrm_interact_fwd, L.emb_bag_interact_fwd, L.dlrm_interact_bwd, L.emb_bag_bwd_adagrad,
                  L.dlrm_synth_fill_table, L.dlrm_trace_enable, L.dlrm_trace_read):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().dlrm_status_string(int(status)).decode()


dlrm_status_string = status_string


def _check(rc: int, what: str):
    if rc != 0:
        raise DlrmError(rc, what)


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DLRM_F32
    if t.dtype == torch.bfloat16:
        return DLRM_BF16
    raise TypeError(f"table dtype {t.dtype} is not float32 or bfloat16")


def _tables(tables: Sequence[torch.Tensor]):
    T = len(tables)
    if T == 0:
        raise ValueError("no tables")
    D = tables[0].shape[1]
    code = _dtype_code(tables[0])
    for t in tables:
        if t.dim() != 2 or t.shape[1] != D or _dtype_code(t) != code or not t.is_contiguous():
            raise ValueError("tables must be contiguous [V_t, D] of one dtype")
    ptrs = (ctypes.c_void_p * T)(*[t.data_ptr() for t in tables])
    rows = (ctypes.c_int64 * T)(*[t.shape[0] for t in tables])
    return T, D, code, ptrs, rows


def _index_code(indices: torch.Tensor, offsets: torch.Tensor) -> int:
    if indices.dtype != offsets.dtype or indices.dtype not in (torch.int64, torch.int32):
        raise ValueError("indices and offsets must both be int64 or both int32")
    if not (indices.is_contiguous() and offsets.is_contiguous()):
        raise ValueError("indices and offsets must be contiguous")
    return DLRM_INDEX_I32 if indices.dtype == torch.int32 else DLRM_INDEX_I64


def _contig(t: Optional[torch.Tensor], dtype, name):
    if t is None:
        return None
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous {dtype}")
    return t


def emb_bag_fwd(tables: Sequence[torch.Tensor], indices: torch.Tensor, offsets: torch.Tensor,
                per_sample_weights: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """Pooled embeddings [B, T, D] fp32 (C: emb_bag_fwd)."""
    T, D, code, ptrs, rows = _tables(tables)
    indices = _contig(indices, torch.int64, "indices")
    offsets = _contig(offsets, torch.int64, "offsets")
    w = _contig(per_sample_weights, torch.float32, "per_sample_weights")
    B = (offsets.numel() - 1) // T
    if offsets.numel() != T * B + 1:
        raise ValueError("offsets must have T*B+1 entries")
    dev = tables[0].device
    if out is None:
        out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    _check(lib().emb_bag_fwd(ptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), _ptr(w), B,
                             indices.numel(), _ptr(out), flags, _stream(dev)), "emb_bag_fwd")
    return out


def emb_bag_fwd_ex(tables: Sequence[torch.Tensor], indices: torch.Tensor, offsets: torch.Tensor,
                   per_sample_weights: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.float32, flags: int = 0) -> torch.Tensor:
    """Pooled embeddings [B, T, D] in out_dtype (fp32 or bf16), int64 or int32 indices and
    offsets (C: emb_bag_fwd_ex)."""
    T, D, code, ptrs, rows = _tables(tables)
    icode = _index_code(indices, offsets)
    w = _contig(per_sample_weights, torch.float32, "per_sample_weights")
    ocode = {torch.float32: DLRM_F32, torch.bfloat16: DLRM_BF16}[out_dtype]
    B = (offsets.numel() - 1) // T
    if offsets.numel() != T * B + 1:
        raise ValueError("offsets must have T*B+1 entries")
    dev = tables[0].device
    if out is None:
        out = torch.empty((B, T, D), dtype=out_dtype, device=dev)
    if out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be contiguous of out_dtype")
    _check(lib().emb_bag_fwd_ex(ptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), icode, _ptr(w), B,
                                indices.numel(), _ptr(out), ocode, flags, _stream(dev)), "emb_bag_fwd_ex")
    return out


def dlrm_interact_fwd(dense: torch.Tensor, pooled: torch.Tensor,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[B, N(N-1)/2 + D] fp32 (C: dlrm_interact_fwd); pooled is [B, N-1, D]."""
    dense = _contig(dense, torch.float32, "dense")
    pooled = _contig(pooled, torch.float32, "pooled")
    B, D = dense.shape
    N = pooled.shape[1] + 1
    P = N * (N - 1) // 2
    if out is None:
        out = torch.empty((B, P + D), dtype=torch.float32, device=dense.device)
    _check(lib().dlrm_interact_fwd(_ptr(dense), _ptr(pooled), B, N, D, _ptr(out),
                                   _stream(dense.device)), "dlrm_interact_fwd")
    return out


def emb_bag_interact_fwd(tables: Sequence[torch.Tensor], indices: torch.Tensor, offsets: torch.Tensor,
                         per_sample_weights: Optional[torch.Tensor], dense: torch.Tensor,
                         out: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """[B, N(N-1)/2 + D] fp32, N = T + 1: lookup fused with the interaction (C: emb_bag_interact_fwd)."""
    T, D, code, ptrs, rows = _tables(tables)
    indices = _contig(indices, torch.int64, "indices")
    offsets = _contig(offsets, torch.int64, "offsets")
    w = _contig(per_sample_weights, torch.float32, "per_sample_weights")
    dense = _contig(dense, torch.float32, "dense")
    B = (offsets.numel() - 1) // T
    if offsets.numel() != T * B + 1 or tuple(dense.shape) != (B, D):
        raise ValueError("offsets must have T*B+1 entries and dense must be [B, D]")
    N = T + 1
    dev = tables[0].device
    if out is None:
        out = torch.empty((B, N * (N - 1) // 2 + D), dtype=torch.float32, device=dev)
    _check(lib().emb_bag_interact_fwd(ptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), _ptr(w), B,
                                      indices.numel(), _ptr(dense), _ptr(out), flags, _stream(dev)),
           "emb_bag_interact_fwd")
    return out


def dlrm_interact_bwd(grad_out: torch.Tensor, dense: torch.Tensor, pooled: torch.Tensor,
                      grad_dense: Optional[torch.Tensor] = None,
                      grad_pooled: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(grad_dense [B, D], grad_pooled [B, N-1, D]) (C: dlrm_interact_bwd)."""
    grad_out = _contig(grad_out, torch.float32, "grad_out")
    dense = _contig(dense, torch.float32, "dense")
    pooled = _contig(pooled, torch.float32, "pooled")
    B, D = dense.shape
    N = pooled.shape[1] + 1
    if grad_dense is None:
        grad_dense = torch.empty_like(dense)
    if grad_pooled is None:
        grad_pooled = torch.empty_like(pooled)
    _check(lib().dlrm_interact_bwd(_ptr(grad_out), _ptr(dense), _ptr(pooled), B, N, D,
                                   _ptr(grad_dense), _ptr(grad_pooled), _stream(dense.device)),
           "dlrm_interact_bwd")
    return grad_dense, grad_pooled


def emb_bag_bwd_workspace_size(rows: Sequence[int], D: int, B: int, nnz: int) -> int:
    T = len(rows)
    r = (ctypes.c_int64 * T)(*rows)
    return int(lib().emb_bag_bwd_workspace_size(T, r, D, B, nnz))


class AdagradOutputs:
    """Optional integer outputs of emb_bag_bwd_adagrad (device tensors)."""

    def __init__(self, nnz: int, device):
        n1 = max(nnz, 1)
        self.unique_keys = torch.empty(n1, dtype=torch.int64, device=device)
        self.segment_offsets = torch.empty(n1 + 1, dtype=torch.int64, device=device)
        self.sorted_pos = torch.empty(n1, dtype=torch.int32, device=device)
        self.num_unique = torch.empty(1, dtype=torch.int64, device=device)


def emb_bag_bwd_adagrad(tables: Sequence[torch.Tensor], state: Sequence[torch.Tensor],
                        indices: torch.Tensor, offsets: torch.Tensor,
                        per_sample_weights: Optional[torch.Tensor], grad_pooled: torch.Tensor,
                        lr: float, eps: float, workspace: Optional[torch.Tensor] = None,
                        outputs: Optional[AdagradOutputs] = None, flags: int = 0) -> Optional[AdagradOutputs]:
    """Row-wise Adagrad on the tables and states, in place (C: emb_bag_bwd_adagrad)."""
    T, D, code, ptrs, rows = _tables(tables)
    if len(state) != T:
        raise ValueError("one state vector per table")
    for s, t in zip(state, tables):
        if s.dtype != torch.float32 or s.numel() != t.shape[0] or not s.is_contiguous():
            raise ValueError("state[t] must be contiguous fp32 [V_t]")
    sptrs = (ctypes.c_void_p * T)(*[s.data_ptr() for s in state])
    indices = _contig(indices, torch.int64, "indices")
    offsets = _contig(offsets, torch.int64, "offsets")
    w = _contig(per_sample_weights, torch.float32, "per_sample_weights")
    grad_pooled = _contig(grad_pooled, torch.float32, "grad_pooled")
    B = (offsets.numel() - 1) // T
    nnz = indices.numel()
    dev = tables[0].device
    need = emb_bag_bwd_workspace_size([t.shape[0] for t in tables], D, B, nnz)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    o = outputs
    _check(lib().emb_bag_bwd_adagrad(
        ptrs, sptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), _ptr(w), B, nnz,
        _ptr(grad_pooled), float(lr), float(eps), _ptr(workspace), workspace.numel(),
        _ptr(o.unique_keys) if o else None, _ptr(o.segment_offsets) if o else None,
        _ptr(o.sorted_pos) if o else None, _ptr(o.num_unique) if o else None, flags,
        _stream(dev)), "emb_bag_bwd_adagrad")
    return o


def emb_bag_bwd_update(tables: Sequence[torch.Tensor], state: Optional[Sequence[torch.Tensor]],
                       indices: torch.Tensor, offsets: torch.Tensor,
                       per_sample_weights: Optional[torch.Tensor], grad_pooled: torch.Tensor,
                       optimizer: int, lr: float, eps: float = 0.0,
                       workspace: Optional[torch.Tensor] = None, outputs: Optional[AdagradOutputs] = None,
                       flags: int = 0) -> Optional[AdagradOutputs]:
    """Embedding backward with DLRM_OPT_ADAGRAD (state required) or DLRM_OPT_SGD (state may be
    None), int64 or int32 indices and offsets (C: emb_bag_bwd_update)."""
    T, D, code, ptrs, rows = _tables(tables)
    icode = _index_code(indices, offsets)
    sptrs = None
    if state is not None:
        if len(state) != T:
            raise ValueError("one state vector per table")
        for st, t in zip(state, tables):
            if st.dtype != torch.float32 or st.numel() != t.shape[0] or not st.is_contiguous():
                raise ValueError("state[t] must be contiguous fp32 [V_t]")
        sptrs = (ctypes.c_void_p * T)(*[st.data_ptr() for st in state])
    w = _contig(per_sample_weights, torch.float32, "per_sample_weights")
    grad_pooled = _contig(grad_pooled, torch.float32, "grad_pooled")
    B = (offsets.numel() - 1) // T
    nnz = indices.numel()
    dev = tables[0].device
    need = emb_bag_bwd_workspace_size([t.shape[0] for t in tables], D, B, nnz)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    o = outputs
    _check(lib().emb_bag_bwd_update(
        ptrs, sptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), icode, _ptr(w), B, nnz,
        _ptr(grad_pooled), int(optimizer), float(lr), float(eps), _ptr(workspace), workspace.numel(),
        _ptr(o.unique_keys) if o else None, _ptr(o.segment_offsets) if o else None,
        _ptr(o.sorted_pos) if o else None, _ptr(o.num_unique) if o else None, flags,
        _stream(dev)), "emb_bag_bwd_update")
    return o


def emb_bag_bwd_plan(rows: Sequence[int], D: int, indices: torch.Tensor, offsets: torch.Tensor,
                     per_sample_weights: Optional[torch.Tensor], workspace: torch.Tensor,
                     outputs: Optional[AdagradOutputs] = None, flags: int = 0) -> Optional[AdagradOutputs]:
    """The batch-only half of the embedding backward (C: emb_bag_bwd_plan), on the current stream
    of the indices' device; `rows` are the tables' row counts."""
    T = len(rows)
    r = (ctypes.c_int64 * T)(*rows)
    icode = _index_code(indices, offsets)
    w = _contig(per_sample_weights, torch.float32, "per_sample_weights")
    B = (offsets.numel() - 1) // T
    nnz = indices.numel()
    o = outputs
    _check(lib().emb_bag_bwd_plan(
        r, T, D, _ptr(indices), _ptr(offsets), icode, _ptr(w), B, nnz, _ptr(workspace), workspace.numel(),
        _ptr(o.unique_keys) if o else None, _ptr(o.segment_offsets) if o else None,
        _ptr(o.sorted_pos) if o else None, _ptr(o.num_unique) if o else None, flags,
        _stream(indices.device)), "emb_bag_bwd_plan")
    return o


def emb_bag_bwd_apply(tables: Sequence[torch.Tensor], state: Optional[Sequence[torch.Tensor]], B: int, nnz: int,
                      weighted: bool, grad_pooled: torch.Tensor, optimizer: int, lr: float, eps: float,
                      workspace: torch.Tensor, outputs: Optional[AdagradOutputs] = None) -> None:
    """The update half of the embedding backward from a planned workspace (C: emb_bag_bwd_apply);
    `outputs` is the plan's, when it was given one (its segment offsets are read)."""
    T, D, code, ptrs, rows = _tables(tables)
    sptrs = None
    if state is not None:
        if len(state) != T:
            raise ValueError("one state vector per table")
        for st, t in zip(state, tables):
            if st.dtype != torch.float32 or st.numel() != t.shape[0] or not st.is_contiguous():
                raise ValueError("state[t] must be contiguous fp32 [V_t]")
        sptrs = (ctypes.c_void_p * T)(*[st.data_ptr() for st in state])
    grad_pooled = _contig(grad_pooled, torch.float32, "grad_pooled")
    _check(lib().emb_bag_bwd_apply(
        ptrs, sptrs, rows, T, D, code, int(B), int(nnz), 1 if weighted else 0, _ptr(grad_pooled), int(optimizer),
        float(lr), float(eps), _ptr(workspace), workspace.numel(),
        _ptr(outputs.segment_offsets) if outputs is not None else None, _stream(tables[0].device)),
        "emb_bag_bwd_apply")


def dlrm_synth_fill_table(table: torch.Tensor, t: int, seed: int, scale: float) -> None:
    """Fill ``table`` with the counter-hash contents of table ``t`` (input generation)."""
    if not table.is_contiguous() or table.dim() != 2:
        raise ValueError("table must be contiguous [V, D]")
    _check(lib().dlrm_synth_fill_table(_ptr(table), _dtype_code(table), table.shape[0],
                                       table.shape[1], t, seed, float(scale),
                                       _stream(table.device)), "dlrm_synth_fill_table")


# ---------------------------------------------------------------- dense layers (dlrm_mlp.h)

_TORCH_CODE = {torch.float32: DLRM_F32, torch.bfloat16: DLRM_BF16}


def dlrm_linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().dlrm_linear_workspace_size(M, N, K))


def dlrm_bce_head_workspace_size(M: int, K: int) -> int:
    return int(lib().dlrm_bce_head_workspace_size(M, K))


def _ws(nbytes: int, dev, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return workspace


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.bfloat16 or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous bf16")
    return t


def dlrm_linear_fwd(x: torch.Tensor, W: torch.Tensor, b: torch.Tensor, act: int = DLRM_ACT_RELU,
                    y: Optional[torch.Tensor] = None, y_dtype: torch.dtype = torch.bfloat16,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = act(x W^T + b), x [M][K] bf16, W [N][K] bf16, b [N] fp32 (C: dlrm_linear_fwd)."""
    x, W = _bf16(x, "x"), _bf16(W, "W")
    b = _contig(b, torch.float32, "b")
    M, K = x.shape
    N = W.shape[0]
    if W.shape[1] != K or b.numel() != N:
        raise ValueError("shapes do not match")
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=x.device)
    ws = _ws(dlrm_linear_workspace_size(M, N, K), x.device, workspace)
    _check(lib().dlrm_linear_fwd(_ptr(x), _ptr(W), _ptr(b), M, N, K, act, _ptr(y), _TORCH_CODE[y.dtype], _ptr(ws),
                                 ws.numel(), _stream(x.device)), "dlrm_linear_fwd")
    return y


def dlrm_linear_bwd(dy: torch.Tensor, y: Optional[torch.Tensor], act: int, x: torch.Tensor, W: torch.Tensor,
                    want_dx: bool = True, dz_bf16: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None,
                    dW: Optional[torch.Tensor] = None, db: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """(dx or None, dW, db) of y = act(x W^T + b) given dy fp32 (C: dlrm_linear_bwd)."""
    dy = _contig(dy, torch.float32, "dy")
    x, W = _bf16(x, "x"), _bf16(W, "W")
    M, K = x.shape
    N = W.shape[0]
    dev = x.device
    if dz_bf16 is None:
        dz_bf16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if want_dx and dx is None:
        dx = torch.empty((M, K), dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.empty((N, K), dtype=torch.float32, device=dev)
    if db is None:
        db = torch.empty(N, dtype=torch.float32, device=dev)
    ycode = _TORCH_CODE[y.dtype] if y is not None else DLRM_F32
    ws = _ws(dlrm_linear_workspace_size(M, N, K), dev, workspace)
    _check(lib().dlrm_linear_bwd(_ptr(dy), _ptr(y), ycode, act, _ptr(x), _ptr(W), M, N, K, _ptr(dz_bf16),
                                 _ptr(dx) if want_dx else None, _ptr(dW), _ptr(db), _ptr(ws), ws.numel(),
                                 _stream(dev)), "dlrm_linear_bwd")
    return (dx if want_dx else None), dW, db


def dlrm_bce_head(x: torch.Tensor, w: torch.Tensor, b: torch.Tensor, t: torch.Tensor,
                  workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None) -> dict:
    """Sigmoid head + mean BCE, forward and backward: dict p, loss, dx, dw, db (C: dlrm_bce_head)."""
    x, w = _bf16(x, "x"), _bf16(w, "w")
    b = _contig(b, torch.float32, "b")
    t = _contig(t, torch.float32, "t")
    M, K = x.shape
    dev = x.device
    o = out if out is not None else {
        "p": torch.empty(M, dtype=torch.float32, device=dev), "loss": torch.empty(1, dtype=torch.float32, device=dev),
        "dx": torch.empty((M, K), dtype=torch.float32, device=dev), "dw": torch.empty(K, dtype=torch.float32, device=dev),
        "db": torch.empty(1, dtype=torch.float32, device=dev)}
    ws = _ws(dlrm_bce_head_workspace_size(M, K), dev, workspace)
    _check(lib().dlrm_bce_head(_ptr(x), _ptr(w), _ptr(b), _ptr(t), M, K, _ptr(o["p"]), _ptr(o["loss"]), _ptr(o["dx"]),
                               _ptr(o["dw"]), _ptr(o["db"]), _ptr(ws), ws.numel(), _stream(dev)), "dlrm_bce_head")
    return o


def dlrm_sgd_dense(w32: torch.Tensor, w16: Optional[torch.Tensor], g: torch.Tensor, lr: float) -> None:
    """w32 -= lr * g; w16 <- bf16(w32) when given (C: dlrm_sgd_dense)."""
    w32 = _contig(w32, torch.float32, "w32")
    g = _contig(g, torch.float32, "g")
    if w16 is not None and (w16.numel() != w32.numel()):
        raise ValueError("w16 must match w32")
    if g.numel() != w32.numel():
        raise ValueError("g must match w32")
    _check(lib().dlrm_sgd_dense(_ptr(w32), _ptr(w16) if w16 is not None else None, _ptr(g), w32.numel(), float(lr),
                                _stream(w32.device)), "dlrm_sgd_dense")


def dlrm_sgd_dense_multi(params: Sequence, lr: float) -> None:
    """For each (w32, w16 or None, g): w32 -= lr * g and w16 <- bf16(w32), in one launch
    (C: dlrm_sgd_dense_multi)."""
    count = len(params)
    w32s, w16s, gs, ns = [], [], [], []
    for w32, w16, g in params:
        if w32.dtype != torch.float32 or not w32.is_contiguous():
            raise ValueError("w32 must be contiguous fp32")
        if g.dtype != torch.float32 or not g.is_contiguous() or g.numel() != w32.numel():
            raise ValueError("g must be contiguous fp32 of w32's size")
        if w16 is not None and (w16.numel() != w32.numel() or not w16.is_contiguous()):
            raise ValueError("w16 must match w32")
        w32s.append(w32.data_ptr())
        w16s.append(w16.data_ptr() if w16 is not None else None)
        gs.append(g.data_ptr())
        ns.append(w32.numel())
    if count == 0:
        return
    vp = ctypes.c_void_p * count
    _check(lib().dlrm_sgd_dense_multi(count, vp(*w32s), vp(*w16s), vp(*gs), (ctypes.c_int64 * count)(*ns), float(lr),
                                      _stream(params[0][0].device)), "dlrm_sgd_dense_multi")


def dlrm_cast_rows(src: torch.Tensor, cols: int, dst_cols: int, dst_dtype: torch.dtype,
                   dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dst [M][dst_cols]: the first `cols` columns of src converted, the rest zero (C: dlrm_cast_rows)."""
    if src.dim() != 2 or src.stride(1) != 1:
        raise ValueError("src must be a 2-D matrix with packed rows")
    M = src.shape[0]
    if dst is None:
        dst = torch.empty((M, dst_cols), dtype=dst_dtype, device=src.device)
    _check(lib().dlrm_cast_rows(_ptr(src), _TORCH_CODE[src.dtype], src.stride(0), M, cols, _ptr(dst),
                                _TORCH_CODE[dst.dtype], dst_cols, _stream(src.device)), "dlrm_cast_rows")
    return dst


def dlrm_trace_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events (C: dlrm_trace_enable)."""
    _check(lib().dlrm_trace_enable(1 if on else 0), "dlrm_trace_enable")


def dlrm_trace_read(max_entries: int = 64) -> dict:
    """{kernel name: (launches, total ms)} since the last read (C: dlrm_trace_read)."""
    names = ctypes.create_string_buffer(64 * max_entries)
    launches = (ctypes.c_int64 * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    n = ctypes.c_int32(0)
    _check(lib().dlrm_trace_read(max_entries, names, launches, ms, ctypes.byref(n)), "dlrm_trace_read")
    out = {}
    for i in range(n.value):
        name = names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
        out[name] = (int(launches[i]), float(ms[i]))
    return out
