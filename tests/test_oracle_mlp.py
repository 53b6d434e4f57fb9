"""Pins of the dense-layer oracle (oracle/mlp.py) to things other than itself (CPU only):
a hand-worked example, torch autograd and torch.nn.functional in fp64, torch.optim.SGD, and
closed forms of the sigmoid / cross-entropy."""
import json
import os

import numpy as np
import torch

from oracle import mlp

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def test_linear_and_head_hand_example():
    g = GOLD["mlp"]
    y, scale, z = mlp.linear_fwd(g["x"], g["W"], g["b"], relu=True)
    assert np.array_equal(z, np.array(g["z"]))
    assert np.array_equal(y, np.array(g["y"]))
    assert np.array_equal(scale, np.array(g["scale"]))
    dx, dW, db, *_ = mlp.linear_bwd(g["dy"], z, g["x"], g["W"], relu=True)
    assert np.array_equal(dx, np.array(g["dx"]))
    assert np.array_equal(dW, np.array(g["dW"]))
    assert np.array_equal(db, np.array(g["db"]))
    h = mlp.bce_head(g["head_x"], g["head_w"], g["head_b"], g["head_t"])
    assert np.array_equal(h["p"], np.array(g["head_p"]))
    assert abs(h["loss"] - np.log(2.0)) < 1e-15
    assert np.array_equal(h["dz"], np.array(g["head_dz"]))


def test_stack_vs_torch_autograd():
    """Two ReLU layers and the head, forward and backward, against torch autograd in fp64."""
    rng = np.random.default_rng(5)
    M, K0, K1, K2 = 37, 13, 24, 16
    x = rng.standard_normal((M, K0))
    W1, b1 = rng.standard_normal((K1, K0)) * 0.3, rng.standard_normal(K1) * 0.1
    W2, b2 = rng.standard_normal((K2, K1)) * 0.3, rng.standard_normal(K2) * 0.1
    w3, b3 = rng.standard_normal(K2) * 0.3, 0.2
    t = (rng.random(M) < 0.3).astype(np.float64)

    y1, _, z1 = mlp.linear_fwd(x, W1, b1, relu=True)
    y2, _, z2 = mlp.linear_fwd(y1, W2, b2, relu=True)
    h = mlp.bce_head(y2, w3, b3, t)
    dy1, dW2, db2, *_ = mlp.linear_bwd(h["dx"], z2, y1, W2, relu=True)
    dx, dW1, db1, *_ = mlp.linear_bwd(dy1, z1, x, W1, relu=True)

    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tx, tW1, tb1, tW2, tb2, tw3 = T(x), T(W1), T(b1), T(W2), T(b2), T(w3)
    tb3 = T(np.array(b3))
    a1 = torch.relu(torch.nn.functional.linear(tx, tW1, tb1))
    a2 = torch.relu(torch.nn.functional.linear(a1, tW2, tb2))
    logit = a2 @ tw3 + tb3
    loss = torch.nn.functional.binary_cross_entropy_with_logits(logit, torch.tensor(t))
    loss.backward()
    assert abs(h["loss"] - loss.item()) <= 1e-14
    assert np.allclose(h["p"], torch.sigmoid(logit).detach().numpy(), rtol=1e-14, atol=1e-16)
    for ours, ref in ((dx, tx), (dW1, tW1), (db1, tb1), (dW2, tW2), (db2, tb2), (h["dw"], tw3)):
        assert np.allclose(ours, ref.grad.numpy(), rtol=1e-12, atol=1e-15)
    assert abs(h["db"] - tb3.grad.item()) <= 1e-14


def test_sigmoid_and_loss_closed_forms():
    z = np.array([-60.0, -3.0, 0.0, 3.0, 60.0])
    p = mlp.sigmoid(z)
    assert p[2] == 0.5 and np.allclose(p + mlp.sigmoid(-z), 1.0, rtol=0, atol=4e-16)
    x = z[:, None]
    for t in (0.0, 1.0):
        h = mlp.bce_head(x, np.array([1.0]), 0.0, np.full(5, t))
        ref = torch.nn.functional.binary_cross_entropy_with_logits(
            torch.tensor(z), torch.full((5,), t, dtype=torch.float64), reduction="none").numpy()
        # torch forms log(1 + e^-|z|) without log1p, so it loses values below ~1e-16 (it gives 0 at
        # z = -60, t = 0): compare to the rounding of O(1) losses; the tiny loss is pinned below
        assert np.allclose(h["loss_i"], ref, rtol=1e-14, atol=1e-15)
    # the loss of the right answer at |z| = 60 is e^-60, not 0 and not a log of 0
    h = mlp.bce_head(np.array([[60.0]]), np.array([1.0]), 0.0, np.array([1.0]))
    assert abs(h["loss"] - np.exp(-60.0)) <= 1e-30


def test_sgd_vs_torch_optim():
    rng = np.random.default_rng(6)
    w, g = rng.standard_normal(50), rng.standard_normal(50)
    p = torch.nn.Parameter(torch.tensor(w))
    opt = torch.optim.SGD([p], lr=0.03)
    p.grad = torch.tensor(g)
    opt.step()
    assert np.allclose(mlp.sgd(w, g, 0.03), p.detach().numpy(), rtol=1e-15, atol=0)
