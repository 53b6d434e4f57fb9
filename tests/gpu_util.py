"""Helpers shared by the GPU parity tests (host-side marshalling and error measures)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from recommendation_model_sparse_amd import synth

DEV = torch.device("cuda:0")


def say(*a):
    """Print and flush before a GPU step, so a failing run names its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def rel_err(got, ref, scale) -> float:
    got = np.asarray(got, dtype=np.float64)
    diff = np.abs(got - ref)
    zero = scale == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    return float(np.max(diff[~zero] / scale[~zero])) if np.any(~zero) else 0.0


def row_inf_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / ||ref||_inf."""
    num = np.max(np.abs(got.astype(np.float64) - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if len(num) else 0.0


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 2.0 ** -133)


def random_csr(rng, T, B, rows, lengths="multi", max_len=40, weighted=False, hot=None):
    """Table-major CSR batch with the given length mode; ``hot`` forces one row per table."""
    if lengths == "onehot":
        L = np.ones(T * B, dtype=np.int64)
    elif lengths == "empty":
        L = np.zeros(T * B, dtype=np.int64)
    else:
        L = rng.integers(0, max_len + 1, T * B)
    off = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(L, out=off[1:])
    idx = np.empty(int(off[-1]), dtype=np.int64)
    for t in range(T):
        a, b = off[t * B], off[(t + 1) * B]
        if hot is not None:
            idx[a:b] = min(hot, rows[t] - 1)
        else:
            idx[a:b] = rng.integers(0, rows[t], b - a)
    w = rng.standard_normal(len(idx)).astype(np.float32) if weighted else None
    return idx, off, w


def random_tables(rng, rows, D, dtype):
    out = []
    for v in rows:
        x = rng.standard_normal((v, D)).astype(np.float32)
        out.append(synth.f32_to_bf16_bits(x) if dtype == "bf16" else x)
    return out


def device_tables(wl) -> list:
    """Tables of a workload built on the device (hashed) or copied (small normal-init ones)."""
    if wl.init == "normal":
        return [to_dev(t) for t in wl.host_tables()]
    from recommendation_model_sparse_amd import dlrm_synth_fill_table
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    st = wl.seed_tab()
    tabs = []
    for t, v in enumerate(wl.rows):
        x = torch.empty((v, wl.D), dtype=dt, device=DEV)
        dlrm_synth_fill_table(x, t, st, float(synth.table_scale(v)))
        tabs.append(x)
    return tabs
