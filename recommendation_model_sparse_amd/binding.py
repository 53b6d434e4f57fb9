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
DLRM_GRAM_AUTO, DLRM_GRAM_MFMA, DLRM_GRAM_VALU = 0, 1, 2

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
        L.dlrm_interact_fwd_ex.argtypes = [p, p, i64, i32, i32, p, i32, p]
        L.dlrm_interact_fwd_ex.restype = ctypes.c_int
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
        L.emb_bag_bwd_update_noalloc.argtypes = [p, p, p, i32, i32, i32, p, p, i32, p, i64, i64, p, i32, f32,
                                                 f32, p, p, p, p, u32, p]
        L.emb_bag_bwd_update_noalloc.restype = ctypes.c_int
        L.emb_bag_bwd_noalloc_max_bytes.argtypes = []
        L.emb_bag_bwd_noalloc_max_bytes.restype = sz
        L.dlrm_probe_read.argtypes = [p, u64, p, u32, p]
        L.dlrm_probe_gather.argtypes = [p, i64, i32, p, i64, p, u32, p]
        L.dlrm_trace_enable.argtypes = [ctypes.c_int]
        L.dlrm_trace_read.argtypes = [i32, p, p, p, p]
        for f in (L.emb_bag_fwd, L.emb_bag_fwd_ex, L.emb_bag_bwd_update, L.dlrm_interact_fwd, L.emb_bag_interact_fwd, L.dlrm_interact_bwd, L.emb_bag_bwd_adagrad,
                  L.dlrm_synth_fill_table, L.dlrm_trace_enable, L.dlrm_trace_read, L.dlrm_probe_read,
                  L.dlrm_probe_gather):
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


# ---------------------------------------------------------------- argument checks
#
# The C entry points see plain pointers and sizes, so they cannot tell a CPU tensor, a wrong-sized
# output or a buffer of the wrong type from a good one; a kernel would read or write out of bounds.
# Every wrapper therefore checks each tensor (type, dtype, exact shape, contiguity, one CUDA device,
# workspace and output sizes) and raises ValueError before it calls the library.

def _need(t, name, dtype=None, shape=None, min_numel: Optional[int] = None) -> torch.Tensor:
    """`name` is a string, or a callable giving it (only called to word an error)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{_name(name)} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None:
        ok = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in ok:
            raise ValueError(f"{_name(name)} must be {' or '.join(str(d) for d in ok)}, got {t.dtype}")
    if shape is not None and t.shape != shape:  # torch.Size compares with a tuple of ints
        raise ValueError(f"{_name(name)} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{_name(name)} must hold at least {min_numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{_name(name)} must be contiguous")
    return t


def _name(name) -> str:
    return name() if callable(name) else name


def _opt(t, name: str, dtype=None, shape=None, min_numel: Optional[int] = None):
    return None if t is None else _need(t, name, dtype, shape, min_numel)


def _device(*tensors) -> torch.device:
    """The one CUDA device every given tensor (None entries skipped) lives on."""
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a CUDA (HIP) device, got {dev}")
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"all tensors must be on {dev}, found one on {t.device}")
    return dev


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DLRM_F32
    if t.dtype == torch.bfloat16:
        return DLRM_BF16
    raise ValueError(f"table dtype {t.dtype} is not float32 or bfloat16")


def _tables(tables: Sequence[torch.Tensor]):
    T = len(tables)
    if T == 0:
        raise ValueError("no tables")
    for t in tables:
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError("tables must be 2-D tensors [V_t, D]")
    D = tables[0].shape[1]
    code = _dtype_code(tables[0])
    for t in tables:
        if t.shape[1] != D or _dtype_code(t) != code or not t.is_contiguous():
            raise ValueError("tables must be contiguous [V_t, D] of one dtype")
    ptrs = (ctypes.c_void_p * T)(*[t.data_ptr() for t in tables])
    rows = (ctypes.c_int64 * T)(*[t.shape[0] for t in tables])
    return T, D, code, ptrs, rows


def _states(state, tables, required: bool):
    if state is None:
        if required:
            raise ValueError("row-wise Adagrad needs one state vector per table")
        return None
    if len(state) != len(tables):
        raise ValueError("one state vector per table")
    for i, (st, t) in enumerate(zip(state, tables)):
        _need(st, lambda: f"state[{i}]", torch.float32, (t.shape[0],))
    return (ctypes.c_void_p * len(state))(*[st.data_ptr() for st in state])


class TableSet:
    """Tables, and optionally their row-wise Adagrad states, checked once for repeated calls.

    Every wrapper that takes a list of tables also takes a TableSet, and then takes its states
    when its `state` argument is None or the set's own list.  The per-call checks then reduce to
    re-reading the tensors' data pointers and row counts; if one changed (a tensor replaced in the
    set's lists, re-allocated or resized), the set is checked again in full before the call.  It
    behaves as the sequence of its tables."""

    def __init__(self, tables: Sequence[torch.Tensor], states: Optional[Sequence[torch.Tensor]] = None):
        # the caller's own lists are kept (not copies), so passing that state list to a call is
        # recognized as the set's, and a tensor swapped into either list is seen by the next call
        self.tables = tables if isinstance(tables, list) else list(tables)
        self.states = None if states is None else (states if isinstance(states, list) else list(states))
        self._build()

    def _pointers(self):
        return ([t.data_ptr() for t in self.tables] + [t.shape[0] for t in self.tables] +
                [s.data_ptr() for s in (self.states or ())] + [s.shape[0] for s in (self.states or ())])

    def _build(self):
        self.T, self.D, self.code, self.ptrs, self.rows = _tables(self.tables)
        self.row_counts = [int(t.shape[0]) for t in self.tables]
        self.sptrs = None if self.states is None else _states(self.states, self.tables, True)
        self.device = _device(*self.tables, *(self.states or ()))
        self._key = self._pointers()

    def refresh(self) -> "TableSet":
        if self._pointers() != self._key:
            self._build()
        return self

    def __len__(self):
        return len(self.tables)

    def __iter__(self):
        return iter(self.tables)

    def __getitem__(self, i):
        return self.tables[i]


def _prepared(tables, state=None, need_state=False, with_state=False):
    """(T, D, dtype code, table pointers, row counts as C array and as list, state pointers, the
    tensors whose device the call must check) of a table list or a TableSet."""
    if isinstance(tables, TableSet):
        tables.refresh()
        sptrs, extra = None, ()
        if with_state:
            if state is None or state is tables.states:
                if tables.sptrs is None and need_state:
                    raise ValueError("row-wise Adagrad needs one state vector per table")
                sptrs = tables.sptrs
            else:
                sptrs, extra = _states(state, tables.tables, need_state), tuple(state)
        return (tables.T, tables.D, tables.code, tables.ptrs, tables.rows, tables.row_counts, sptrs,
                (tables.tables[0],) + extra)
    T, D, code, ptrs, rows = _tables(tables)
    sptrs = _states(state, tables, need_state) if with_state else None
    dev_tensors = tuple(tables) + (tuple(state) if with_state and state is not None else ())
    return T, D, code, ptrs, rows, [int(t.shape[0]) for t in tables], sptrs, dev_tensors


def _batch(T: int, indices, offsets, per_sample_weights, index_dtypes=(torch.int64,)):
    """Checks the CSR batch; returns (indices, offsets, weights, index code, B, nnz)."""
    _need(indices, "indices", index_dtypes)
    _need(offsets, "offsets", indices.dtype)
    if indices.dim() != 1 or offsets.dim() != 1:
        raise ValueError("indices and offsets must be 1-D")
    B = (offsets.numel() - 1) // T
    if offsets.numel() < 1 or offsets.numel() != T * B + 1:
        raise ValueError(f"offsets must have T*B+1 entries (T={T}), got {offsets.numel()}")
    nnz = indices.numel()
    w = _opt(per_sample_weights, "per_sample_weights", torch.float32, (nnz,))
    code = DLRM_INDEX_I32 if indices.dtype == torch.int32 else DLRM_INDEX_I64
    return indices, offsets, w, code, B, nnz


def _outputs(o, nnz: int):
    """The optional integer outputs of the embedding backward, each sized for nnz lookups."""
    if o is None:
        return None
    _need(o.unique_keys, "outputs.unique_keys", torch.int64, min_numel=nnz)
    _need(o.segment_offsets, "outputs.segment_offsets", torch.int64, min_numel=nnz + 1)
    _need(o.sorted_pos, "outputs.sorted_pos", torch.int32, min_numel=nnz)
    _need(o.num_unique, "outputs.num_unique", torch.int64, min_numel=1)
    return o


def _workspace(workspace, need: int, dev):
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    return workspace


def emb_bag_fwd(tables: Sequence[torch.Tensor], indices: torch.Tensor, offsets: torch.Tensor,
                per_sample_weights: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """Pooled embeddings [B, T, D] fp32 (C: emb_bag_fwd)."""
    T, D, code, ptrs, rows, _, _, dt = _prepared(tables)
    indices, offsets, w, _, B, nnz = _batch(T, indices, offsets, per_sample_weights)
    out = _opt(out, "out", torch.float32, (B, T, D))
    dev = _device(*dt, indices, offsets, w, out)
    if out is None:
        out = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    _check(lib().emb_bag_fwd(ptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), _ptr(w), B,
                             nnz, _ptr(out), flags, _stream(dev)), "emb_bag_fwd")
    return out


def emb_bag_fwd_ex(tables: Sequence[torch.Tensor], indices: torch.Tensor, offsets: torch.Tensor,
                   per_sample_weights: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.float32, flags: int = 0) -> torch.Tensor:
    """Pooled embeddings [B, T, D] in out_dtype (fp32 or bf16), int64 or int32 indices and
    offsets (C: emb_bag_fwd_ex)."""
    T, D, code, ptrs, rows, _, _, dt = _prepared(tables)
    indices, offsets, w, icode, B, nnz = _batch(T, indices, offsets, per_sample_weights,
                                                (torch.int64, torch.int32))
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    ocode = DLRM_F32 if out_dtype == torch.float32 else DLRM_BF16
    out = _opt(out, "out", out_dtype, (B, T, D))
    dev = _device(*dt, indices, offsets, w, out)
    if out is None:
        out = torch.empty((B, T, D), dtype=out_dtype, device=dev)
    _check(lib().emb_bag_fwd_ex(ptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), icode, _ptr(w), B,
                                nnz, _ptr(out), ocode, flags, _stream(dev)), "emb_bag_fwd_ex")
    return out


def _interaction_shapes(dense: torch.Tensor, pooled: torch.Tensor):
    _need(dense, "dense", torch.float32)
    _need(pooled, "pooled", torch.float32)
    if dense.dim() != 2 or pooled.dim() != 3:
        raise ValueError("dense must be [B, D] and pooled [B, N-1, D]")
    B, D = dense.shape
    if pooled.shape[0] != B or pooled.shape[2] != D:
        raise ValueError(f"pooled must be [B={B}, N-1, D={D}], got {tuple(pooled.shape)}")
    N = pooled.shape[1] + 1
    return B, N, D, N * (N - 1) // 2


def dlrm_interact_fwd(dense: torch.Tensor, pooled: torch.Tensor,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[B, N(N-1)/2 + D] fp32 (C: dlrm_interact_fwd); pooled is [B, N-1, D]."""
    B, N, D, P = _interaction_shapes(dense, pooled)
    out = _opt(out, "out", torch.float32, (B, P + D))
    dev = _device(dense, pooled, out)
    if out is None:
        out = torch.empty((B, P + D), dtype=torch.float32, device=dev)
    _check(lib().dlrm_interact_fwd(_ptr(dense), _ptr(pooled), B, N, D, _ptr(out),
                                   _stream(dev)), "dlrm_interact_fwd")
    return out


def dlrm_interact_fwd_ex(dense: torch.Tensor, pooled: torch.Tensor, path: int = DLRM_GRAM_AUTO,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dlrm_interact_fwd with the Gram path chosen: DLRM_GRAM_AUTO, _MFMA or _VALU (C: dlrm_interact_fwd_ex)."""
    B, N, D, P = _interaction_shapes(dense, pooled)
    out = _opt(out, "out", torch.float32, (B, P + D))
    dev = _device(dense, pooled, out)
    if out is None:
        out = torch.empty((B, P + D), dtype=torch.float32, device=dev)
    _check(lib().dlrm_interact_fwd_ex(_ptr(dense), _ptr(pooled), B, N, D, _ptr(out), int(path), _stream(dev)),
           "dlrm_interact_fwd_ex")
    return out


def emb_bag_interact_fwd(tables: Sequence[torch.Tensor], indices: torch.Tensor, offsets: torch.Tensor,
                         per_sample_weights: Optional[torch.Tensor], dense: torch.Tensor,
                         out: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """[B, N(N-1)/2 + D] fp32, N = T + 1: lookup fused with the interaction (C: emb_bag_interact_fwd)."""
    T, D, code, ptrs, rows, _, _, dt = _prepared(tables)
    indices, offsets, w, _, B, nnz = _batch(T, indices, offsets, per_sample_weights)
    _need(dense, "dense", torch.float32, (B, D))
    N = T + 1
    out = _opt(out, "out", torch.float32, (B, N * (N - 1) // 2 + D))
    dev = _device(*dt, indices, offsets, w, dense, out)
    if out is None:
        out = torch.empty((B, N * (N - 1) // 2 + D), dtype=torch.float32, device=dev)
    _check(lib().emb_bag_interact_fwd(ptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), _ptr(w), B,
                                      nnz, _ptr(dense), _ptr(out), flags, _stream(dev)),
           "emb_bag_interact_fwd")
    return out


def dlrm_interact_bwd(grad_out: torch.Tensor, dense: torch.Tensor, pooled: torch.Tensor,
                      grad_dense: Optional[torch.Tensor] = None,
                      grad_pooled: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(grad_dense [B, D], grad_pooled [B, N-1, D]) (C: dlrm_interact_bwd)."""
    B, N, D, P = _interaction_shapes(dense, pooled)
    _need(grad_out, "grad_out", torch.float32, (B, P + D))
    grad_dense = _opt(grad_dense, "grad_dense", torch.float32, (B, D))
    grad_pooled = _opt(grad_pooled, "grad_pooled", torch.float32, (B, N - 1, D))
    dev = _device(grad_out, dense, pooled, grad_dense, grad_pooled)
    if grad_dense is None:
        grad_dense = torch.empty_like(dense)
    if grad_pooled is None:
        grad_pooled = torch.empty_like(pooled)
    _check(lib().dlrm_interact_bwd(_ptr(grad_out), _ptr(dense), _ptr(pooled), B, N, D,
                                   _ptr(grad_dense), _ptr(grad_pooled), _stream(dev)),
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


def _out_ptrs(o):
    if o is None:
        return None, None, None, None
    return _ptr(o.unique_keys), _ptr(o.segment_offsets), _ptr(o.sorted_pos), _ptr(o.num_unique)


def _out_tensors(o):
    return () if o is None else (o.unique_keys, o.segment_offsets, o.sorted_pos, o.num_unique)


def emb_bag_bwd_adagrad(tables: Sequence[torch.Tensor], state: Sequence[torch.Tensor],
                        indices: torch.Tensor, offsets: torch.Tensor,
                        per_sample_weights: Optional[torch.Tensor], grad_pooled: torch.Tensor,
                        lr: float, eps: float, workspace: Optional[torch.Tensor] = None,
                        outputs: Optional[AdagradOutputs] = None, flags: int = 0) -> Optional[AdagradOutputs]:
    """Row-wise Adagrad on the tables and states, in place (C: emb_bag_bwd_adagrad); `state` may
    be None when `tables` is a TableSet with states."""
    T, D, code, ptrs, rows, counts, sptrs, dt = _prepared(tables, state, True, True)
    indices, offsets, w, _, B, nnz = _batch(T, indices, offsets, per_sample_weights)
    _need(grad_pooled, "grad_pooled", torch.float32, (B, T, D))
    o = _outputs(outputs, nnz)
    need = emb_bag_bwd_workspace_size(counts, D, B, nnz)
    workspace = _opt(workspace, "workspace", torch.uint8, min_numel=need)
    dev = _device(*dt, indices, offsets, w, grad_pooled, workspace, *_out_tensors(o))
    workspace = _workspace(workspace, need, dev)
    _check(lib().emb_bag_bwd_adagrad(
        ptrs, sptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), _ptr(w), B, nnz,
        _ptr(grad_pooled), float(lr), float(eps), _ptr(workspace), workspace.numel(), *_out_ptrs(o), flags,
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
    T, D, code, ptrs, rows, counts, sptrs, dt = _prepared(tables, state, optimizer == DLRM_OPT_ADAGRAD, True)
    indices, offsets, w, icode, B, nnz = _batch(T, indices, offsets, per_sample_weights,
                                                (torch.int64, torch.int32))
    _need(grad_pooled, "grad_pooled", torch.float32, (B, T, D))
    o = _outputs(outputs, nnz)
    need = emb_bag_bwd_workspace_size(counts, D, B, nnz)
    workspace = _opt(workspace, "workspace", torch.uint8, min_numel=need)
    dev = _device(*dt, indices, offsets, w, grad_pooled, workspace, *_out_tensors(o))
    workspace = _workspace(workspace, need, dev)
    _check(lib().emb_bag_bwd_update(
        ptrs, sptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), icode, _ptr(w), B, nnz,
        _ptr(grad_pooled), int(optimizer), float(lr), float(eps), _ptr(workspace), workspace.numel(),
        *_out_ptrs(o), flags, _stream(dev)), "emb_bag_bwd_update")
    return o


def emb_bag_bwd_noalloc_max_bytes() -> int:
    return int(lib().emb_bag_bwd_noalloc_max_bytes())


def emb_bag_bwd_update_noalloc(tables: Sequence[torch.Tensor], state: Optional[Sequence[torch.Tensor]],
                               indices: torch.Tensor, offsets: torch.Tensor,
                               per_sample_weights: Optional[torch.Tensor], grad_pooled: torch.Tensor,
                               optimizer: int, lr: float, eps: float = 0.0,
                               outputs: Optional[AdagradOutputs] = None, flags: int = 0) -> Optional[AdagradOutputs]:
    """emb_bag_bwd_update with the library's fixed per-GPU scratch as the workspace: allocates
    nothing (C: emb_bag_bwd_update_noalloc).  Calls that overlap on one GPU race."""
    T, D, code, ptrs, rows, _, sptrs, dt = _prepared(tables, state, optimizer == DLRM_OPT_ADAGRAD, True)
    indices, offsets, w, icode, B, nnz = _batch(T, indices, offsets, per_sample_weights,
                                                (torch.int64, torch.int32))
    _need(grad_pooled, "grad_pooled", torch.float32, (B, T, D))
    o = _outputs(outputs, nnz)
    dev = _device(*dt, indices, offsets, w, grad_pooled, *_out_tensors(o))
    _check(lib().emb_bag_bwd_update_noalloc(
        ptrs, sptrs, rows, T, D, code, _ptr(indices), _ptr(offsets), icode, _ptr(w), B, nnz,
        _ptr(grad_pooled), int(optimizer), float(lr), float(eps), *_out_ptrs(o), flags, _stream(dev)),
        "emb_bag_bwd_update_noalloc")
    return o


def emb_bag_bwd_plan(rows: Sequence[int], D: int, indices: torch.Tensor, offsets: torch.Tensor,
                     per_sample_weights: Optional[torch.Tensor], workspace: torch.Tensor,
                     outputs: Optional[AdagradOutputs] = None, flags: int = 0) -> Optional[AdagradOutputs]:
    """The batch-only half of the embedding backward (C: emb_bag_bwd_plan), on the current stream
    of the indices' device; `rows` are the tables' row counts."""
    T = len(rows)
    r = (ctypes.c_int64 * T)(*rows)
    indices, offsets, w, icode, B, nnz = _batch(T, indices, offsets, per_sample_weights,
                                                (torch.int64, torch.int32))
    o = _outputs(outputs, nnz)
    _need(workspace, "workspace", torch.uint8, min_numel=emb_bag_bwd_workspace_size(rows, D, B, nnz))
    dev = _device(indices, offsets, w, workspace, *_out_tensors(o))
    _check(lib().emb_bag_bwd_plan(
        r, T, D, _ptr(indices), _ptr(offsets), icode, _ptr(w), B, nnz, _ptr(workspace), workspace.numel(),
        *_out_ptrs(o), flags, _stream(dev)), "emb_bag_bwd_plan")
    return o


def emb_bag_bwd_apply(tables: Sequence[torch.Tensor], state: Optional[Sequence[torch.Tensor]], B: int, nnz: int,
                      weighted: bool, grad_pooled: torch.Tensor, optimizer: int, lr: float, eps: float,
                      workspace: torch.Tensor, outputs: Optional[AdagradOutputs] = None) -> None:
    """The update half of the embedding backward from a planned workspace (C: emb_bag_bwd_apply);
    `outputs` is the plan's, when it was given one (its segment offsets are read)."""
    T, D, code, ptrs, rows, counts, sptrs, dt = _prepared(tables, state, optimizer == DLRM_OPT_ADAGRAD, True)
    B, nnz = int(B), int(nnz)
    _need(grad_pooled, "grad_pooled", torch.float32, (B, T, D))
    seg = None
    if outputs is not None:
        seg = _need(outputs.segment_offsets, "outputs.segment_offsets", torch.int64, min_numel=nnz + 1)
    _need(workspace, "workspace", torch.uint8, min_numel=emb_bag_bwd_workspace_size(counts, D, B, nnz))
    dev = _device(*dt, grad_pooled, workspace, seg)
    _check(lib().emb_bag_bwd_apply(
        ptrs, sptrs, rows, T, D, code, B, nnz, 1 if weighted else 0, _ptr(grad_pooled), int(optimizer),
        float(lr), float(eps), _ptr(workspace), workspace.numel(), _ptr(seg), _stream(dev)),
        "emb_bag_bwd_apply")


def dlrm_synth_fill_table(table: torch.Tensor, t: int, seed: int, scale: float) -> None:
    """Fill ``table`` with the counter-hash contents of table ``t`` (input generation)."""
    _need(table, "table", (torch.float32, torch.bfloat16))
    if table.dim() != 2:
        raise ValueError("table must be [V, D]")
    dev = _device(table)
    _check(lib().dlrm_synth_fill_table(_ptr(table), _dtype_code(table), table.shape[0],
                                       table.shape[1], t, seed, float(scale),
                                       _stream(dev)), "dlrm_synth_fill_table")


# ---------------------------------------------------------------- HBM read probes (dlrm_probe.h)

def dlrm_probe_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Stream-read every byte of ``buf`` once (C: dlrm_probe_read); ``sink`` is uint32/int32 scratch."""
    _need(buf, "buf")
    _need(sink, "sink", (torch.int32,))
    nbytes = buf.numel() * buf.element_size()
    if nbytes == 0 or nbytes % 16:
        raise ValueError("buf must hold a positive multiple of 16 bytes")
    dev = _device(buf, sink)
    _check(lib().dlrm_probe_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(dev)), "dlrm_probe_read")


def dlrm_probe_gather(table: torch.Tensor, idx: torch.Tensor, sink: torch.Tensor) -> None:
    """Read rows ``idx`` of the 2-D ``table`` with no output (C: dlrm_probe_gather)."""
    _need(table, "table")
    if table.dim() != 2:
        raise ValueError("table must be [rows, cols]")
    _need(idx, "idx", torch.int64)
    _need(sink, "sink", (torch.int32,))
    dev = _device(table, idx, sink)
    _check(lib().dlrm_probe_gather(_ptr(table), table.shape[0], table.shape[1] * table.element_size(), _ptr(idx),
                                   idx.numel(), _ptr(sink), sink.numel(), _stream(dev)), "dlrm_probe_gather")


# ---------------------------------------------------------------- dense layers (dlrm_mlp.h)

_TORCH_CODE = {torch.float32: DLRM_F32, torch.bfloat16: DLRM_BF16}


def dlrm_linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().dlrm_linear_workspace_size(M, N, K))


def dlrm_bce_head_workspace_size(M: int, K: int) -> int:
    return int(lib().dlrm_bce_head_workspace_size(M, K))


def _ws(nbytes: int, dev, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    """The caller's workspace when it is large enough, else a new one."""
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
        if workspace.device != dev:
            raise ValueError(f"workspace must be on {dev}, found it on {workspace.device}")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return workspace


def _mat(t, name: str, dtype) -> torch.Tensor:
    _need(t, name, dtype)
    if t.dim() != 2:
        raise ValueError(f"{name} must be a matrix, got shape {tuple(t.shape)}")
    return t


def dlrm_linear_fwd(x: torch.Tensor, W: torch.Tensor, b: torch.Tensor, act: int = DLRM_ACT_RELU,
                    y: Optional[torch.Tensor] = None, y_dtype: torch.dtype = torch.bfloat16,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = act(x W^T + b), x [M][K] bf16, W [N][K] bf16, b [N] fp32 (C: dlrm_linear_fwd)."""
    M, K = _mat(x, "x", torch.bfloat16).shape
    N = _mat(W, "W", torch.bfloat16).shape[0]
    if W.shape[1] != K:
        raise ValueError(f"W must be [N, K={K}], got {tuple(W.shape)}")
    _need(b, "b", torch.float32, (N,))
    y = _opt(y, "y", (torch.float32, torch.bfloat16) if y is not None else None, (M, N))
    dev = _device(x, W, b, y)
    if y is None:
        if y_dtype not in _TORCH_CODE:
            raise ValueError(f"y_dtype must be float32 or bfloat16, got {y_dtype}")
        y = torch.empty((M, N), dtype=y_dtype, device=dev)
    ws = _ws(dlrm_linear_workspace_size(M, N, K), dev, workspace)
    _check(lib().dlrm_linear_fwd(_ptr(x), _ptr(W), _ptr(b), M, N, K, act, _ptr(y), _TORCH_CODE[y.dtype], _ptr(ws),
                                 ws.numel(), _stream(dev)), "dlrm_linear_fwd")
    return y


def dlrm_linear_bwd(dy: torch.Tensor, y: Optional[torch.Tensor], act: int, x: torch.Tensor, W: torch.Tensor,
                    want_dx: bool = True, dz_bf16: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None,
                    dW: Optional[torch.Tensor] = None, db: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """(dx or None, dW, db) of y = act(x W^T + b) given dy fp32 (C: dlrm_linear_bwd)."""
    M, K = _mat(x, "x", torch.bfloat16).shape
    N = _mat(W, "W", torch.bfloat16).shape[0]
    if W.shape[1] != K:
        raise ValueError(f"W must be [N, K={K}], got {tuple(W.shape)}")
    _need(dy, "dy", torch.float32, (M, N))
    if act == DLRM_ACT_RELU and y is None:
        raise ValueError("the ReLU backward needs the forward output y")
    y = _opt(y, "y", (torch.float32, torch.bfloat16), (M, N))
    dz_bf16 = _opt(dz_bf16, "dz_bf16", torch.bfloat16, (M, N))
    dx = _opt(dx, "dx", torch.float32, (M, K)) if want_dx else None
    dW = _opt(dW, "dW", torch.float32, (N, K))
    db = _opt(db, "db", torch.float32, (N,))
    dev = _device(dy, y, x, W, dz_bf16, dx, dW, db)
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
    M, K = _mat(x, "x", torch.bfloat16).shape
    _need(w, "w", torch.bfloat16, (K,))
    _need(b, "b", torch.float32, (1,))
    _need(t, "t", torch.float32, (M,))
    if out is not None:
        for k, shp in (("p", (M,)), ("loss", (1,)), ("dx", (M, K)), ("dw", (K,)), ("db", (1,))):
            _need(out[k], f"out[{k!r}]", torch.float32, shp)
    dev = _device(x, w, b, t, *(out.values() if out is not None else ()))
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
    _need(w32, "w32", torch.float32)
    _need(g, "g", torch.float32, tuple(w32.shape))
    w16 = _opt(w16, "w16", torch.bfloat16, tuple(w32.shape))
    dev = _device(w32, w16, g)
    _check(lib().dlrm_sgd_dense(_ptr(w32), _ptr(w16), _ptr(g), w32.numel(), float(lr),
                                _stream(dev)), "dlrm_sgd_dense")


def dlrm_sgd_dense_multi(params: Sequence, lr: float) -> None:
    """For each (w32, w16 or None, g): w32 -= lr * g and w16 <- bf16(w32), in one launch
    (C: dlrm_sgd_dense_multi)."""
    count = len(params)
    if count == 0:
        return
    w32s, w16s, gs, ns, every = [], [], [], [], []
    for i, (w32, w16, g) in enumerate(params):
        _need(w32, f"params[{i}].w32", torch.float32)
        _need(g, f"params[{i}].g", torch.float32, tuple(w32.shape))
        _opt(w16, f"params[{i}].w16", torch.bfloat16, tuple(w32.shape))
        every += [w32, w16, g]
        w32s.append(w32.data_ptr())
        w16s.append(w16.data_ptr() if w16 is not None else None)
        gs.append(g.data_ptr())
        ns.append(w32.numel())
    dev = _device(*every)
    vp = ctypes.c_void_p * count
    _check(lib().dlrm_sgd_dense_multi(count, vp(*w32s), vp(*w16s), vp(*gs), (ctypes.c_int64 * count)(*ns), float(lr),
                                      _stream(dev)), "dlrm_sgd_dense_multi")


def dlrm_cast_rows(src: torch.Tensor, cols: int, dst_cols: int, dst_dtype: torch.dtype,
                   dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dst [M][dst_cols]: the first `cols` columns of src converted, the rest zero (C: dlrm_cast_rows)."""
    if not isinstance(src, torch.Tensor) or src.dim() != 2 or src.stride(1) != 1:
        raise ValueError("src must be a 2-D matrix with packed rows")
    if src.dtype not in _TORCH_CODE:
        raise ValueError(f"src must be float32 or bfloat16, got {src.dtype}")
    if not (0 <= cols <= src.shape[1] and cols <= dst_cols):
        raise ValueError(f"need cols <= src columns ({src.shape[1]}) and cols <= dst_cols ({dst_cols})")
    M = src.shape[0]
    if dst_dtype not in _TORCH_CODE:
        raise ValueError(f"dst_dtype must be float32 or bfloat16, got {dst_dtype}")
    dst = _opt(dst, "dst", dst_dtype, (M, dst_cols))
    dev = _device(src, dst)
    if dst is None:
        dst = torch.empty((M, dst_cols), dtype=dst_dtype, device=dev)
    _check(lib().dlrm_cast_rows(_ptr(src), _TORCH_CODE[src.dtype], src.stride(0), M, cols, _ptr(dst),
                                _TORCH_CODE[dst.dtype], dst_cols, _stream(dev)), "dlrm_cast_rows")
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
