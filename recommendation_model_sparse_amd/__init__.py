"""MI355X-native DLRM sparse hot path: embedding-bag lookup, dot-product
interaction (forward/backward) and the sparse row-wise Adagrad step, as HIP
kernels for gfx950 behind a C ABI (``include/dlrm_sparse.h``).

The functions below are thin ctypes wrappers of that ABI; see ``binding``.
"""
from .binding import (  # noqa: F401
    DLRM_ACT_NONE,
    DLRM_ACT_RELU,
    dlrm_bce_head,
    dlrm_bce_head_workspace_size,
    dlrm_cast_rows,
    dlrm_linear_bwd,
    dlrm_linear_fwd,
    dlrm_linear_workspace_size,
    dlrm_sgd_dense,
    dlrm_sgd_dense_multi,
    DLRM_BF16,
    DLRM_F32,
    DLRM_FLAG_CHECK_INDICES,
    DLRM_INDEX_I32,
    DLRM_INDEX_I64,
    DLRM_OPT_ADAGRAD,
    DLRM_OPT_SGD,
    AdagradOutputs,
    DlrmError,
    dlrm_interact_bwd,
    dlrm_interact_fwd,
    dlrm_probe_gather,
    dlrm_probe_read,
    dlrm_status_string,
    dlrm_synth_fill_table,
    dlrm_trace_enable,
    dlrm_trace_read,
    emb_bag_bwd_adagrad,
    emb_bag_bwd_update,
    emb_bag_bwd_plan,
    emb_bag_bwd_apply,
    emb_bag_bwd_workspace_size,
    emb_bag_fwd,
    emb_bag_fwd_ex,
    emb_bag_interact_fwd,
)
