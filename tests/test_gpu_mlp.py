"""GPU parity of the dense layers (dlrm_mlp.h; needs an MI355X) against oracle/mlp.py.

Error measure: |gpu - oracle| / scale with scale the sum of the absolute values of the terms
(R19).  Gates, derived from the arithmetic:
  - fp32 GEMM outputs: gamma_K = K * 2^-24 (recursive summation bound; K <= 1024 -> 6.1e-5);
  - bf16 outputs and the GEMMs that take the bf16-rounded dz: 2^-9 (one rounding) + gamma_K,
    held to 2^-8;
  - fixed-order fp32 column sums over M rows in blocks of 32: (32 + M/32) * 2^-24 -> 1e-4.
The ReLU mask is a decision taken in floating point, so both sides take it from one forward output
(y > 0) that the backward receives as an input: the oracle's own forward, rounded to the layer's
output type.  Every oracle input is generated on the host.
"""
import zlib

import numpy as np
import pytest
import torch

from oracle import mlp
from recommendation_model_sparse_amd import (
    DLRM_ACT_NONE,
    DLRM_ACT_RELU,
    dlrm_bce_head,
    dlrm_cast_rows,
    dlrm_linear_bwd,
    dlrm_linear_fwd,
    dlrm_sgd_dense,
    dlrm_sgd_dense_multi,
    synth,
)

from gpu_util import DEV, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def bf16_pair(a: np.ndarray):
    """(device bf16 tensor, host fp64 values) of the bf16 rounding of a."""
    bits = synth.f32_to_bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
    return to_dev(bits), synth.bf16_bits_to_f32(bits).astype(np.float64)


def host_f64(t: torch.Tensor) -> np.ndarray:
    h = to_host(t)
    return synth.bf16_bits_to_f32(h).astype(np.float64) if t.dtype == torch.bfloat16 else h.astype(np.float64)


def gamma(K):
    return K * 2.0 ** -24


@pytest.mark.parametrize("M,K,N", [(1, 16, 8), (300, 16, 512), (300, 480, 1024), (4099, 1024, 128),
                                   (16384, 256, 512), (8192, 512, 64), (257, 256, 1024), (64, 64, 64)])
@pytest.mark.parametrize("act", [DLRM_ACT_RELU, DLRM_ACT_NONE])
@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_linear_fwd_bwd(M, K, N, act, ydt):
    rng = np.random.default_rng(zlib.crc32(f"lin-{M}-{K}-{N}-{act}-{ydt}".encode()))
    x_d, x = bf16_pair(rng.standard_normal((M, K)))
    W_d, W = bf16_pair(rng.standard_normal((N, K)) / np.sqrt(K))
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    say(f"[mlp] linear M={M} K={K} N={N} act={act} y={ydt}")
    y_d = dlrm_linear_fwd(x_d, W_d, to_dev(b), act, y_dtype=ydt)
    y_d2 = dlrm_linear_fwd(x_d, W_d, to_dev(b), act, y_dtype=ydt)
    torch.cuda.synchronize()
    assert torch.equal(y_d.view(torch.int16) if ydt == torch.bfloat16 else y_d.view(torch.int32),
                       y_d2.view(torch.int16) if ydt == torch.bfloat16 else y_d2.view(torch.int32))
    y = host_f64(y_d)
    ref, scale, _ = mlp.linear_fwd(x, W, b, act == DLRM_ACT_RELU)
    gate = gamma(K) if ydt == torch.float32 else 2.0 ** -8
    err = rel_err(y, ref, scale)
    say(f"   fwd max rel err {err:.3e} (gate {gate:.2e})")
    assert err <= gate

    # backward: the forward output it takes (the ReLU mask) is the oracle's, rounded as the layer
    # stores it, on both sides
    if ydt == torch.bfloat16:
        y_in_d, y_in = bf16_pair(ref)
    else:
        y_in = ref.astype(np.float32)
        y_in_d, y_in = to_dev(y_in), y_in.astype(np.float64)
    dy = rng.standard_normal((M, N)).astype(np.float32)
    for want_dx in (True, False):
        dx_d, dW_d, db_d = dlrm_linear_bwd(to_dev(dy), y_in_d, act, x_d, W_d, want_dx=want_dx)
        torch.cuda.synchronize()
        mask_src = y_in if act == DLRM_ACT_RELU else np.ones_like(y_in)
        rdx, rdW, rdb, sdx, sdW, sdb = mlp.linear_bwd(dy, mask_src, x, W, act == DLRM_ACT_RELU)
        e_dW = rel_err(dW_d.cpu().numpy(), rdW, sdW)
        e_db = rel_err(db_d.cpu().numpy(), rdb, sdb)
        say(f"   bwd dW {e_dW:.3e} db {e_db:.3e}")
        assert e_dW <= 2.0 ** -8
        assert e_db <= 1e-4
        if want_dx:
            e_dx = rel_err(dx_d.cpu().numpy(), rdx, sdx)
            say(f"   bwd dx {e_dx:.3e}")
            assert e_dx <= 2.0 ** -8
        else:
            assert dx_d is None


@pytest.mark.parametrize("M,K", [(1, 8), (300, 256), (16384, 256), (1000, 1024), (2051, 64), (257, 120),
                                 (777, 200), (4099, 512), (130, 520), (5, 1016)])
def test_bce_head(M, K):
    rng = np.random.default_rng(M * 7 + K)
    x_d, x = bf16_pair(np.maximum(rng.standard_normal((M, K)), 0))
    w_d, w = bf16_pair(rng.standard_normal(K) / np.sqrt(K))
    b = np.array([0.3], np.float32)
    t = (rng.random(M) < 0.25).astype(np.float32)
    say(f"[mlp] bce head M={M} K={K}")
    o = dlrm_bce_head(x_d, w_d, to_dev(b), to_dev(t))
    o2 = dlrm_bce_head(x_d, w_d, to_dev(b), to_dev(t))
    torch.cuda.synchronize()
    for k in o:
        assert torch.equal(o[k].view(torch.int32), o2[k].view(torch.int32)), k
    r = mlp.bce_head(x, w, float(b[0]), t)
    # p: error of z (gamma_K of its scale) times |dp/dz| <= 1/4, plus the fp32 sigmoid's own rounding
    dp = np.abs(o["p"].cpu().numpy() - r["p"])
    assert np.all(dp <= 0.25 * gamma(K) * r["z_scale"] + 4e-7)
    loss = float(o["loss"].item())
    assert abs(loss - r["loss"]) <= 1e-5 * max(1.0, abs(r["loss"]))
    # dz = (p - t)/M carries the error of p; dx = dz w, dw = x^T dz, db = sum dz
    dz_err = (0.25 * gamma(K) * r["z_scale"] + 4e-7) / M
    assert np.all(np.abs(o["dx"].cpu().numpy() - r["dx"]) <= np.outer(dz_err, np.abs(w)) + 1e-6 * np.abs(r["dx"]) + 1e-30)
    assert np.all(np.abs(o["dw"].cpu().numpy() - r["dw"]) <= np.abs(x).T @ dz_err + 1e-4 * r["dw_scale"] + 1e-30)
    assert abs(float(o["db"].item()) - r["db"]) <= dz_err.sum() + 1e-4 * r["db_scale"]


def test_sgd_dense_and_cast_rows():
    rng = np.random.default_rng(11)
    n = 100003
    w = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    w32 = to_dev(w)
    w16 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    say("[mlp] sgd dense")
    dlrm_sgd_dense(w32, w16, to_dev(g), 0.05)
    torch.cuda.synchronize()
    got = w32.cpu().numpy()
    ref = mlp.sgd(w, g, float(np.float32(0.05)))
    assert np.all(np.abs(got - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-30)
    assert np.array_equal(to_host(w16), synth.f32_to_bf16_bits(got))
    # cast with padding and back
    M = 777
    a = rng.standard_normal((M, 479)).astype(np.float32)
    say("[mlp] cast rows")
    p16 = dlrm_cast_rows(to_dev(a), 479, 480, torch.bfloat16)
    torch.cuda.synchronize()
    h = to_host(p16)
    assert np.array_equal(h[:, :479], synth.f32_to_bf16_bits(a)) and np.all(h[:, 479] == 0)
    big = to_dev(np.pad(a, ((0, 0), (0, 1))))
    crop = dlrm_cast_rows(big, 479, 479, torch.float32)
    assert np.array_equal(crop.cpu().numpy(), a)


@pytest.mark.parametrize("M,src_ld,cols,dst_cols,sdt,ddt", [
    (70000, 13, 13, 16, "f32", "bf16"),   # more rows than the grid's 65535: each block takes several
    (5, 7, 3, 5, "bf16", "f32"),          # odd destination width: element stores
    (300, 104, 100, 100, "bf16", "bf16"),
    (1, 1, 1, 1, "f32", "f32"),
    (33, 480, 479, 480, "f32", "f32")])
def test_cast_rows_shapes(M, src_ld, cols, dst_cols, sdt, ddt):
    rng = np.random.default_rng(M + cols)
    a = rng.standard_normal((M, src_ld)).astype(np.float32)
    if sdt == "bf16":
        src, a64 = bf16_pair(a)
        a = a64.astype(np.float32)
    else:
        src = to_dev(a)
    say(f"[mlp] cast rows M={M} {sdt}[{src_ld}] -> {ddt}[{dst_cols}] ({cols} columns)")
    out = dlrm_cast_rows(src, cols, dst_cols, torch.bfloat16 if ddt == "bf16" else torch.float32)
    torch.cuda.synchronize()
    want = np.zeros((M, dst_cols), np.float32)
    want[:, :cols] = a[:, :cols]
    if ddt == "bf16":
        assert np.array_equal(to_host(out), synth.f32_to_bf16_bits(want))
    else:
        assert np.array_equal(out.cpu().numpy(), want)


def test_sgd_dense_multi_equals_single():
    """One launch over many parameters (sizes 0, 1, ragged, several blocks) gives the bits of the
    per-parameter call."""
    rng = np.random.default_rng(5)
    sizes = [1, 0, 1023, 1024, 1025, 70000, 13, 4096 * 3 + 7]
    single, multi = [], []
    for k, n in enumerate(sizes):
        w = rng.standard_normal(n).astype(np.float32)
        g = rng.standard_normal(n).astype(np.float32)
        with16 = k % 2 == 0
        for lst in (single, multi):
            w32 = to_dev(w)
            w16 = torch.empty(n, dtype=torch.bfloat16, device=DEV) if with16 else None
            lst.append((w32, w16, to_dev(g)))
    say("[mlp] sgd dense multi")
    for w32, w16, g in single:
        dlrm_sgd_dense(w32, w16, g, 0.03)
    dlrm_sgd_dense_multi(multi, 0.03)
    torch.cuda.synchronize()
    for (a32, a16, _), (b32, b16, _) in zip(single, multi):
        assert torch.equal(a32.view(torch.int32), b32.view(torch.int32))
        if a16 is not None:
            assert torch.equal(a16.view(torch.int16), b16.view(torch.int16))
