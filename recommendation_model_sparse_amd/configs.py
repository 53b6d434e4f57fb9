"""The five synthetic workloads of the DLRM sparse path.

Sizes follow the workloads the embedding-bag/interaction path is measured on:
a tiny correctness case, a one-hot fp32 case, a multi-hot bf16 case, one GPU's
share of very large bf16 tables, and a training step on the one-hot shapes.
Seeds are ``20261200 + k``.  Table row counts that are drawn (log-uniform) come
from the workload's own table stream, so they are fixed by the seed.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .synth import Workload, rng_for, S_TABLES

SEED_BASE = 20261200


def log_uniform_rows(seed: int, T: int, lo: float, hi: float) -> list:
    rng = rng_for(seed, S_TABLES, 1)
    v = np.exp(rng.uniform(math.log(lo), math.log(hi), T))
    return [int(min(max(round(x), lo), hi)) for x in v]


def make_config(k: int, **overrides) -> Workload:
    seed = SEED_BASE + k
    if k == 1:
        wl = Workload(name="tiny", seed=seed, T=3, D=16, dtype="f32", B=64, rows=[1000] * 3,
                      init="normal", init_std=0.01, bags="onehot", dist="uniform",
                      note="3 fp32 tables 1000x16 N(0,0.01); B=64; one-hot uniform; N=4")
    elif k == 2:
        wl = Workload(name="onehot-f32", seed=seed, T=26, D=128, dtype="f32", B=2048,
                      rows=log_uniform_rows(seed, 26, 1e3, 4e6), init="hash", bags="onehot",
                      dist="zipf", alpha=1.05,
                      note="26 fp32 tables D=128, V log-uniform [1e3,4e6]; B=2048; one-hot Zipf(1.05); N=27")
    elif k == 3:
        wl = Workload(name="multihot-bf16", seed=seed, T=26, D=128, dtype="bf16", B=16384,
                      rows=log_uniform_rows(seed, 26, 1e3, 1e7), init="hash", bags="geom",
                      bag_lo=1, bag_hi=100, bag_mean=20.0, dist="zipf", alpha=1.05,
                      note="26 bf16 tables D=128, V log-uniform [1e3,1e7]; B=16384; bag length "
                           "truncated geometric [1,100] mean 20; Zipf(1.05); N=27")
    elif k == 4:
        wl = Workload(name="bigtables-bf16", seed=seed, T=8, D=128, dtype="bf16", B=65536,
                      rows=[50_000_000] * 8, init="hash", bags="onehot", dist="uniform",
                      alpha=1.2,
                      note="8 bf16 tables of 50M rows, D=128 (102.4 GB); B=65536; one-hot, "
                           "uniform or Zipf(1.2); N=9")
    elif k == 5:
        base = make_config(2)
        wl = base.with_(name="train-onehot-f32", seed=seed, rows=list(base.rows),
                        note="training step on the one-hot fp32 shapes: interaction backward, "
                             "sort/unique/segment-reduce, row-wise Adagrad lr=0.01 eps=1e-8")
    else:
        raise ValueError(f"no workload {k}")
    return wl.with_(**overrides) if overrides else wl
