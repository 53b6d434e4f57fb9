"""Pins of the oracle's error scales (CPU only).

Every floating-point parity gate divides |gpu - oracle| by the scale S the oracle
returns beside each value: the sum of the absolute values of the terms that the
output adds (the forward-error scale of recursive summation).  A scale that came
out too large would loosen every gate without failing anything else, so each one
is pinned here to something other than the oracle itself:

  * hand-worked signed examples (tests/golden, "scales"), where S != |value|;
  * the same sums of absolute terms built from library routines in fp64 on the
    absolute inputs: torch.nn.functional.embedding_bag on |E| with |w| (pooling),
    torch.bmm on |X| (the dots), |G| times |X| by torch.bmm plus |g_dense|
    (the interaction backward);
  * inputs with no cancellation (all terms of one sign), where S equals |value|;
  * and a check that an inflated or deflated scale fails these pins.

The definitions: robocikowo.com "DLRM", paragraph "Forward pass", stages 2-4
(the lookup of one row per feature, its pooling, the pairwise dots of the N
vectors, the strict upper triangle followed by the dense vector); the backward
is the derivative of that map.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from recommendation_model_sparse_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))["scales"]


def as_f64(table):
    if table.dtype == np.uint16:
        return synth.bf16_bits_to_f32(table).astype(np.float64)
    return table.astype(np.float64)


def problem(seed, T, V, D, B, max_len, weighted, dtype="f32", positive=False):
    rng = np.random.default_rng(seed)
    mk = (lambda s: np.abs(rng.standard_normal(s))) if positive else rng.standard_normal
    tables = []
    for _ in range(T):
        x = mk((V, D)).astype(np.float32)
        tables.append(synth.f32_to_bf16_bits(x) if dtype == "bf16" else x)
    lengths = rng.integers(0, max_len + 1, T * B)
    off = np.zeros(T * B + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    idx = rng.integers(0, V, int(off[-1])).astype(np.int64)
    w = mk(int(off[-1])).astype(np.float32) if weighted else None
    return tables, idx, off, w


# ---------------------------------------------------------------- independent scale builders

def pool_scale_ref(tables, idx, off, w, B):
    """sum_j |w_j| |E_t[idx_j]| per bag: embedding_bag in fp64 on the absolute table and weights."""
    T = len(tables)
    out = []
    for t in range(T):
        lo, hi = off[t * B], off[(t + 1) * B]
        ti = torch.from_numpy(idx[lo:hi])
        to = torch.from_numpy(off[t * B:(t + 1) * B] - lo)
        aw = None if w is None else torch.from_numpy(np.abs(w[lo:hi].astype(np.float64)))
        out.append(torch.nn.functional.embedding_bag(ti, torch.from_numpy(np.abs(as_f64(tables[t]))), to,
                                                     mode="sum", per_sample_weights=aw).numpy())
    return np.stack(out, 1)


def interact_scale_ref(dense, pooled):
    """sum_d |x_i[d]| |x_j[d]| at the strict upper triangle (torch.bmm on |X|), then |dense|."""
    N = pooled.shape[1] + 1
    A = torch.from_numpy(np.abs(np.concatenate([dense[:, None, :], pooled], 1).astype(np.float64)))
    iu = torch.triu_indices(N, N, 1)
    S = torch.bmm(A, A.transpose(1, 2).contiguous())[:, iu[0], iu[1]]
    return torch.cat([S, A[:, 0]], 1).numpy()


def interact_bwd_scale_ref(g, dense, pooled):
    """sum_{j != i} |G_ij| |x_j[d]| (|G| times |X| by torch.bmm; the zero diagonal of G drops
    j = i), plus |g_dense| on row 0."""
    B, N, D = pooled.shape[0], pooled.shape[1] + 1, dense.shape[1]
    P = N * (N - 1) // 2
    A = torch.from_numpy(np.abs(np.concatenate([dense[:, None, :], pooled], 1).astype(np.float64)))
    G = torch.zeros(B, N, N, dtype=torch.float64)
    iu = torch.triu_indices(N, N, 1)
    ag = torch.from_numpy(np.abs(g[:, :P].astype(np.float64)))
    G[:, iu[0], iu[1]] = ag
    G[:, iu[1], iu[0]] = ag
    M = torch.bmm(G, A).numpy()
    return M[:, 0] + np.abs(g[:, P:].astype(np.float64)), M[:, 1:]


def close(a, b, rtol=1e-13):
    return a.shape == b.shape and bool(np.all(np.abs(a - b) <= rtol * np.abs(b)))


# ---------------------------------------------------------------- hand examples

def test_pool_scale_hand_example():
    tab = np.array(GOLD["pool_table"], dtype=np.float32)
    idx = np.array(GOLD["pool_indices"], dtype=np.int64)
    off = np.array(GOLD["pool_offsets"], dtype=np.int64)
    w = np.array(GOLD["pool_weights"], dtype=np.float32)
    out, s = oracle.emb_bag_fwd([tab], idx, off, None, 3)
    assert np.array_equal(out[:, 0], np.array(GOLD["pool_sum"], np.float64))
    assert np.array_equal(s[:, 0], np.array(GOLD["pool_sum_scale"], np.float64))
    out, s = oracle.emb_bag_fwd([tab], idx, off, w, 3)
    assert np.array_equal(out[:, 0], np.array(GOLD["pool_weighted"], np.float64))
    assert np.array_equal(s[:, 0], np.array(GOLD["pool_weighted_scale"], np.float64))


def test_interact_scale_hand_example():
    out, s = oracle.interact_fwd(np.array(GOLD["dense"], np.float32), np.array(GOLD["pooled"], np.float32))
    assert np.array_equal(out, np.array(GOLD["interact_out"], np.float64))
    assert np.array_equal(s, np.array(GOLD["interact_scale"], np.float64))


def test_interact_bwd_scale_hand_example():
    gd, gp, sd, sp = oracle.interact_bwd(np.array(GOLD["grad_out"], np.float32), np.array(GOLD["dense"], np.float32),
                                         np.array(GOLD["pooled"], np.float32))
    assert np.array_equal(gd, np.array(GOLD["grad_dense"], np.float64))
    assert np.array_equal(gp, np.array(GOLD["grad_pooled"], np.float64))
    assert np.array_equal(sd, np.array(GOLD["grad_dense_scale"], np.float64))
    assert np.array_equal(sp, np.array(GOLD["grad_pooled_scale"], np.float64))


# ---------------------------------------------------------------- library routines on |inputs|

@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_scale_vs_embedding_bag_of_abs(weighted, dtype):
    T, V, D, B = 4, 29, 12, 21
    tables, idx, off, w = problem(31, T, V, D, B, 9, weighted, dtype)
    _, s = oracle.emb_bag_fwd(tables, idx, off, w, B)
    assert close(s, pool_scale_ref(tables, idx, off, w, B))


@pytest.mark.parametrize("N,D,B", [(2, 5, 3), (4, 16, 7), (27, 16, 3), (9, 33, 4)])
def test_interact_scale_vs_bmm_of_abs(N, D, B):
    rng = np.random.default_rng(N * 7 + D)
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    _, s = oracle.interact_fwd(dense, pooled)
    assert close(s, interact_scale_ref(dense, pooled))


@pytest.mark.parametrize("N,D,B", [(2, 3, 2), (5, 7, 3), (27, 16, 2)])
def test_interact_bwd_scale_vs_bmm_of_abs(N, D, B):
    rng = np.random.default_rng(N * 11 + D)
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    g = rng.standard_normal((B, N * (N - 1) // 2 + D)).astype(np.float32)
    _, _, sd, sp = oracle.interact_bwd(g, dense, pooled)
    rd, rp = interact_bwd_scale_ref(g, dense, pooled)
    assert close(sd, rd) and close(sp, rp)


# ---------------------------------------------------------------- no cancellation: S = |value|

def test_scales_equal_abs_value_without_cancellation():
    """With every term of one sign there is nothing to cancel, so each scale is |value| up to
    fp64 rounding of the two sums."""
    T, V, D, B = 3, 17, 8, 9
    tables, idx, off, w = problem(41, T, V, D, B, 6, True, positive=True)
    out, s = oracle.emb_bag_fwd(tables, idx, off, w, B)
    assert close(s, np.abs(out), 1e-14)
    rng = np.random.default_rng(42)
    N = 6
    dense = np.abs(rng.standard_normal((B, D))).astype(np.float32)
    pooled = np.abs(rng.standard_normal((B, N - 1, D))).astype(np.float32)
    out, s = oracle.interact_fwd(dense, pooled)
    assert close(s, np.abs(out), 1e-14)
    g = np.abs(rng.standard_normal((B, N * (N - 1) // 2 + D))).astype(np.float32)
    gd, gp, sd, sp = oracle.interact_bwd(g, dense, pooled)
    assert close(sd, np.abs(gd), 1e-14) and close(sp, np.abs(gp), 1e-14)
    # and with signs flipped throughout, the values flip while the scales stay
    out2, s2 = oracle.interact_fwd(-dense, pooled)
    assert np.array_equal(s2, s) and close(np.abs(out2[:, :N * (N - 1) // 2]), s[:, :N * (N - 1) // 2], 1e-14)


# ---------------------------------------------------------------- the pins reject a wrong scale

@pytest.mark.parametrize("factor", [2.0, 0.5, 1.0 + 1e-9])
def test_a_wrong_scale_fails_the_pins(factor):
    """A scale off by any factor (twice, half, or a part in 1e9) is rejected by each pin above."""
    T, V, D, B = 3, 23, 8, 11
    tables, idx, off, w = problem(51, T, V, D, B, 7, True)
    _, s = oracle.emb_bag_fwd(tables, idx, off, w, B)
    ref = pool_scale_ref(tables, idx, off, w, B)
    assert close(s, ref) and not close(s * factor, ref)
    rng = np.random.default_rng(52)
    N = 5
    dense = rng.standard_normal((B, D)).astype(np.float32)
    pooled = rng.standard_normal((B, N - 1, D)).astype(np.float32)
    _, s = oracle.interact_fwd(dense, pooled)
    ref = interact_scale_ref(dense, pooled)
    assert close(s, ref) and not close(s * factor, ref)
    g = rng.standard_normal((B, N * (N - 1) // 2 + D)).astype(np.float32)
    _, _, sd, sp = oracle.interact_bwd(g, dense, pooled)
    rd, rp = interact_bwd_scale_ref(g, dense, pooled)
    assert close(sd, rd) and not close(sd * factor, rd)
    assert close(sp, rp) and not close(sp * factor, rp)


# ---------------------------------------------------------------- dense layers (oracle/mlp.py)

def test_mlp_backward_scales_hand_example():
    """The hand-worked ReLU layer (tests/golden "mlp"): dz = [[0,0],[1,0]], so the scales are
    |dz||W| = [[0,0],[1,1]], |dz|^T|x| = [[3,1],[0,0]] and sum|dz| = [1,0]; the head at z = 0
    with x = 0 has z scale |b| = 0, dw scale 0 and db scale sum|dz| = 0.5."""
    from oracle import mlp
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))["mlp"]
    _, _, z = mlp.linear_fwd(g["x"], g["W"], g["b"], relu=True)
    _, _, _, sdx, sdw, sdb = mlp.linear_bwd(g["dy"], z, g["x"], g["W"], relu=True)
    assert np.array_equal(sdx, [[0, 0], [1, 1]])
    assert np.array_equal(sdw, [[3, 1], [0, 0]])
    assert np.array_equal(sdb, [1, 0])
    h = mlp.bce_head(g["head_x"], g["head_w"], g["head_b"], g["head_t"])
    assert np.array_equal(h["z_scale"], [0, 0]) and np.array_equal(h["dw_scale"], [0]) and h["db_scale"] == 0.5


def test_mlp_scales_vs_torch_on_abs():
    """Each dense-layer scale equals the same product taken by torch in fp64 on absolute values."""
    from oracle import mlp
    rng = np.random.default_rng(61)
    M, K, N = 7, 12, 5
    x = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K))
    b = rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    T = lambda a: torch.from_numpy(np.abs(np.asarray(a, np.float64)))
    _, s, z = mlp.linear_fwd(x, W, b, relu=True)
    assert close(s, (T(x) @ T(W).T + T(b)).numpy())
    dz = dy * (z > 0)
    _, _, _, sdx, sdw, sdb = mlp.linear_bwd(dy, z, x, W, relu=True)
    assert close(sdx, (T(dz) @ T(W)).numpy()) and close(sdw, (T(dz).T @ T(x)).numpy())
    assert close(sdb, T(dz).sum(0).numpy())
    w1, t = rng.standard_normal(K), (rng.random(M) < 0.3).astype(np.float64)
    h = mlp.bce_head(x, w1, -0.7, t)
    assert close(h["z_scale"], (T(x) @ T(w1) + 0.7).numpy())
    assert close(h["dw_scale"], (T(x).T @ T(h["dz"])).numpy())
    assert abs(h["db_scale"] - float(T(h["dz"]).sum())) <= 1e-15
    # an inflated scale is rejected by the same comparison
    assert not close(2 * s, (T(x) @ T(W).T + T(b)).numpy())
