"""Seeded synthetic inputs for the DLRM sparse path.

This module only draws inputs: table sizes, table contents, CSR bags, per-lookup
weights, dense vectors and upstream gradients.  It holds none of the method's
arithmetic (no pooling, no dot products, no optimiser), so both the GPU path and
the CPU oracle may take their inputs from it.

Every stream is a numpy ``SeedSequence([seed, stream, batch])``, so any batch can
be regenerated on its own.  Table contents for the large workloads come from a
counter hash (SplitMix64, Steele, Lea & Flood, OOPSLA 2014) so that any element
can be regenerated anywhere: here in numpy, or on the device by the library's
fill kernel (``dlrm_synth_fill_table``), which implements the same definition.

The hash value of element (t, r, d) of a table with V_t rows:

    c  = (t << 50) | (r << 12) | d
    h  = splitmix64(seed_tab ^ splitmix64(c))
    m  = h >> 40                                   (24 uniform bits)
    x  = fp32( fp32(2*m - 2**24) * 2**-24 ) * a_t  (one fp32 multiply, RN)
    a_t = fp32(1 / sqrt(V_t))                      (computed in fp64, rounded once)

so x is uniform on [-a_t, a_t).  bf16 tables store RNE(x).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

# stream ids inside one workload seed
S_INDICES, S_LENGTHS, S_WEIGHTS, S_DENSE, S_GRADS, S_TABLES = 0, 1, 2, 3, 4, 5
S_FEATURES, S_LABELS = 6, 7  # raw dense features and 0/1 clicks of the full training step

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function applied to counter ``x`` (uint64, wrapping)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x + _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def rng_for(seed: int, stream: int, batch: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, batch])))


def table_seed(seed: int) -> int:
    """64-bit key of the table hash for one workload seed."""
    return int(np.random.SeedSequence([seed, S_TABLES, 0xFEED]).generate_state(1, np.uint64)[0])


def table_scale(V: int) -> np.float32:
    return np.float32(1.0 / math.sqrt(float(V)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, as uint16 bit patterns (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def hash_rows_f32(t: int, rows: np.ndarray, D: int, seed_tab: int, a_t: np.float32) -> np.ndarray:
    """fp32 values of rows ``rows`` of hashed table ``t``: array [len(rows), D]."""
    r = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    d = np.arange(D, dtype=np.uint64).reshape(1, -1)
    c = (np.uint64(t) << np.uint64(50)) | (r << np.uint64(12)) | d
    h = splitmix64(np.uint64(seed_tab) ^ splitmix64(c))
    m = (h >> np.uint64(40)).astype(np.int64)
    unit = ((2 * m - (1 << 24)).astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)
    return (unit * np.float32(a_t)).astype(np.float32)


def hash_rows(t: int, rows: np.ndarray, D: int, seed_tab: int, a_t: np.float32, dtype: str) -> np.ndarray:
    """Rows of hashed table ``t`` in storage form: float32, or uint16 bf16 bits."""
    x = hash_rows_f32(t, rows, D, seed_tab, a_t)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


# ---------------------------------------------------------------------------
# distributions
# ---------------------------------------------------------------------------

def truncated_geometric_p(lo: int, hi: int, mean: float) -> float:
    """p such that P(L=k) ∝ (1-p)^(k-lo) on [lo, hi] has exactly the given mean (bisection, fp64)."""
    k = np.arange(lo, hi + 1, dtype=np.float64)

    def m(p):
        w = (1.0 - p) ** (k - lo)
        return float((k * w).sum() / w.sum())

    a, b = 1e-12, 1.0 - 1e-12  # m(a) ~ (lo+hi)/2, m(b) ~ lo; m decreasing in p
    for _ in range(200):
        c = 0.5 * (a + b)
        if m(c) > mean:
            a = c
        else:
            b = c
    return 0.5 * (a + b)


def truncated_geometric(rng: np.random.Generator, n: int, lo: int, hi: int, mean: float) -> np.ndarray:
    p = truncated_geometric_p(lo, hi, mean)
    k = np.arange(lo, hi + 1, dtype=np.float64)
    w = (1.0 - p) ** (k - lo)
    cdf = np.cumsum(w / w.sum())
    cdf[-1] = 1.0
    u = rng.random(n)
    return (np.searchsorted(cdf, u, side="right") + lo).astype(np.int64)


_ZIPF_CDF: Dict[Tuple[int, float], np.ndarray] = {}


def _zipf_cdf(V: int, alpha: float) -> np.ndarray:
    key = (V, alpha)
    c = _ZIPF_CDF.get(key)
    if c is None:
        c = np.arange(1, V + 1, dtype=np.float64)
        np.power(c, -alpha, out=c)
        np.cumsum(c, out=c)
        c /= c[-1]
        if len(_ZIPF_CDF) > 4:
            _ZIPF_CDF.clear()
        _ZIPF_CDF[key] = c
    return c


def zipf_scatter(V: int, t: int) -> Tuple[int, int]:
    """(A, C): rank k (0-based) maps to row (A*k + C) mod V, A coprime to V, so hot rows are spread."""
    A = 2654435761 % V if V > 1 else 0  # 2654435761 is prime and > any V used here
    C = (t * 0x9E3779B1 + 12345) % V if V > 1 else 0
    return A, C


def zipf_rows(rng: np.random.Generator, V: int, alpha: float, n: int, t: int) -> np.ndarray:
    """n draws from the finite-support Zipf(alpha) over ranks 1..V (inverse CDF), scattered to rows."""
    if V == 1:
        return np.zeros(n, dtype=np.int64)
    cdf = _zipf_cdf(V, alpha)
    k = np.searchsorted(cdf, rng.random(n), side="right")
    np.minimum(k, V - 1, out=k)
    A, C = zipf_scatter(V, t)
    return ((A * k.astype(np.int64) + C) % V).astype(np.int64)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    """Shapes and distributions of one synthetic workload."""

    name: str
    seed: int
    T: int
    D: int
    dtype: str                 # "f32" | "bf16" (table storage)
    B: int
    rows: List[int]            # V_t
    init: str                  # "normal" (N(0, init_std)) | "hash" (U(±1/sqrt(V_t)) by hash)
    init_std: float = 0.01
    bags: str = "onehot"       # "onehot" | "geom"
    bag_lo: int = 1
    bag_hi: int = 100
    bag_mean: float = 20.0
    dist: str = "uniform"      # "uniform" | "zipf"
    alpha: float = 1.05
    weighted: bool = False
    grad_std: float = 1e-3
    lr: float = 0.01
    eps: float = 1e-8
    note: str = ""

    @property
    def N(self) -> int:
        return self.T + 1

    @property
    def P(self) -> int:
        return self.N * (self.N - 1) // 2

    @property
    def elem_size(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def table_bytes(self) -> int:
        return int(sum(self.rows)) * self.D * self.elem_size

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    # -- tables ------------------------------------------------------------
    def seed_tab(self) -> int:
        return table_seed(self.seed)

    def scales(self) -> List[np.float32]:
        return [table_scale(v) for v in self.rows]

    def host_tables(self) -> List[np.ndarray]:
        """Whole tables on the host (small workloads only): float32 [V,D] or uint16 bf16 bits."""
        if self.init == "normal":
            rng = rng_for(self.seed, S_TABLES, 0)
            out = []
            for v in self.rows:
                x = (rng.standard_normal((v, self.D)) * self.init_std).astype(np.float32)
                out.append(f32_to_bf16_bits(x) if self.dtype == "bf16" else x)
            return out
        st = self.seed_tab()
        return [hash_rows(t, np.arange(v), self.D, st, table_scale(v), self.dtype)
                for t, v in enumerate(self.rows)]

    def table_rows(self, t: int, rows: np.ndarray) -> np.ndarray:
        """Selected rows of table t in storage form, without building the whole table."""
        rows = np.asarray(rows, dtype=np.int64)
        if self.init == "normal":
            return self.host_tables()[t][rows]
        return hash_rows(t, rows, self.D, self.seed_tab(), table_scale(self.rows[t]), self.dtype)

    # -- one batch -----------------------------------------------------------
    def batch(self, i: int = 0, weighted: Optional[bool] = None) -> "Batch":
        weighted = self.weighted if weighted is None else weighted
        T, B = self.T, self.B
        if self.bags == "onehot":
            lengths = np.ones(T * B, dtype=np.int64)
        else:
            lengths = truncated_geometric(rng_for(self.seed, S_LENGTHS, i), T * B,
                                          self.bag_lo, self.bag_hi, self.bag_mean)
        offsets = np.zeros(T * B + 1, dtype=np.int64)
        np.cumsum(lengths, out=offsets[1:])
        nnz = int(offsets[-1])
        indices = np.empty(nnz, dtype=np.int64)
        rng = rng_for(self.seed, S_INDICES, i)
        for t in range(T):
            a, b = int(offsets[t * B]), int(offsets[(t + 1) * B])
            if self.dist == "zipf":
                indices[a:b] = zipf_rows(rng, self.rows[t], self.alpha, b - a, t)
            else:
                indices[a:b] = rng.integers(0, self.rows[t], b - a)
        weights = (rng_for(self.seed, S_WEIGHTS, i).random(nnz).astype(np.float32)
                   if weighted else None)
        dense = rng_for(self.seed, S_DENSE, i).standard_normal((B, self.D)).astype(np.float32)
        return Batch(self, i, offsets, indices, weights, dense)


@dataclass
class Batch:
    wl: Workload
    i: int
    offsets: np.ndarray        # int64 [T*B+1], bag (t, b) has id t*B + b
    indices: np.ndarray        # int64 [nnz]
    weights: Optional[np.ndarray]  # float32 [nnz] or None
    dense: np.ndarray          # float32 [B, D]
    _grad: Optional[np.ndarray] = field(default=None, repr=False)

    @property
    def nnz(self) -> int:
        return int(self.indices.shape[0])

    def grad_out(self) -> np.ndarray:
        """Upstream gradient of the interaction output, N(0, grad_std), float32 [B, P+D]."""
        if self._grad is None:
            wl = self.wl
            g = rng_for(wl.seed, S_GRADS, self.i).standard_normal((wl.B, wl.P + wl.D))
            self._grad = (g * wl.grad_std).astype(np.float32)
        return self._grad

    def grad_pooled(self) -> np.ndarray:
        """A stand-alone pooled gradient N(0, grad_std), float32 [B, T, D] (for isolated backward tests)."""
        wl = self.wl
        g = rng_for(wl.seed, S_GRADS, 1000 + self.i).standard_normal((wl.B, wl.T, wl.D))
        return (g * wl.grad_std).astype(np.float32)

    def features(self, n: int = 13) -> np.ndarray:
        """Raw dense features of the full training step, N(0, 1), float32 [B, n]."""
        return rng_for(self.wl.seed, S_FEATURES, self.i).standard_normal((self.wl.B, n)).astype(np.float32)

    def labels(self, rate: float = 0.25) -> np.ndarray:
        """0/1 clicks of the full training step, Bernoulli(rate), float32 [B]."""
        return (rng_for(self.wl.seed, S_LABELS, self.i).random(self.wl.B) < rate).astype(np.float32)

    def bag_lengths(self) -> np.ndarray:
        return np.diff(self.offsets)

    def sample_subset(self, samples: np.ndarray) -> Tuple["Workload", "Batch", List[np.ndarray]]:
        """Restrict to the batch rows ``samples`` and to the table rows they touch.

        Returns a small workload whose table t holds exactly the distinct rows of table t
        that the selected bags reference, in ascending row order, a batch with indices
        remapped into those small tables, and for each table the original row ids.  The
        remap is monotone, so sort order, segments and every per-bag result are unchanged.
        """
        wl = self.wl
        samples = np.asarray(samples, dtype=np.int64)
        S = len(samples)
        T, B = wl.T, wl.B
        lens = self.bag_lengths()
        new_len = np.empty(T * S, dtype=np.int64)
        pieces, wpieces, row_ids, new_rows = [], [], [], []
        for t in range(T):
            bags = t * B + samples
            L = lens[bags]
            new_len[t * S:(t + 1) * S] = L
            starts = self.offsets[bags]
            # positions of the selected bags, in order: start of each bag + rank inside it
            excl = np.cumsum(L) - L
            pos = np.repeat(starts - excl, L) + np.arange(int(L.sum()), dtype=np.int64)
            idx = self.indices[pos]
            uniq, inv = np.unique(idx, return_inverse=True)
            if len(uniq) == 0:
                uniq = np.zeros(1, dtype=np.int64)
            row_ids.append(uniq)
            new_rows.append(int(len(uniq)))
            pieces.append(inv.astype(np.int64).reshape(-1))
            if self.weights is not None:
                wpieces.append(self.weights[pos])
        offsets = np.zeros(T * S + 1, dtype=np.int64)
        np.cumsum(new_len, out=offsets[1:])
        indices = np.concatenate(pieces) if pieces else np.zeros(0, dtype=np.int64)
        weights = np.concatenate(wpieces) if self.weights is not None else None
        sub_wl = wl.with_(B=S, rows=new_rows, name=wl.name + "/subset")
        sub = Batch(sub_wl, self.i, offsets, indices, weights, self.dense[samples].copy())
        return sub_wl, sub, row_ids


def subset_tables(wl: Workload, row_ids: List[np.ndarray]) -> List[np.ndarray]:
    """Host copies of just the rows ``row_ids[t]`` of each table of ``wl``."""
    return [wl.table_rows(t, r) for t, r in enumerate(row_ids)]
