"""CPU oracle of the dense layers either side of the sparse path (fp64 numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU
baseline leg; the GPU library never imports it and shares no code with it.

What it computes (robocikowo.com "DLRM", paragraph "Forward pass": stage (1) the bottom MLP of
fully connected layers with ReLU, stage (4) the top MLP of fully connected layers with a sigmoid
at the end, trained on cross-entropy against the clicks; its paragraph on the top MLP):

  linear layer      y = act(x W^T + b),  W [N][K], b [N], act = ReLU or identity
  head              z = x w + b (one unit), p = sigmoid(z)
  loss              mean over the batch of -(t log p + (1 - t) log(1 - p)), t the 0/1 click
  backward          the derivative of the above (dz = (p - t) / M for the mean loss)
  SGD               w <- w - lr * dw

Every function works in fp64 on the values it is given (the GPU's bf16 weights and activations
widen exactly) and also returns the error scale of each output: the sum of the absolute values
of the terms it adds.
"""
from __future__ import annotations

import numpy as np


def linear_fwd(x, W, b, relu: bool):
    """(y, scale): y = act(x W^T + b); scale = |x| |W|^T + |b| (before the activation)."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    b = np.asarray(b, np.float64)
    z = x @ W.T + b
    scale = np.abs(x) @ np.abs(W).T + np.abs(b)
    y = np.maximum(z, 0.0) if relu else z
    return y, scale, z


def linear_bwd(dy, z, x, W, relu: bool):
    """Gradients of y = act(x W^T + b) given dy: (dx, dW, db, scales of each).

    z is the pre-activation; ReLU passes the gradient where z > 0."""
    dy = np.asarray(dy, np.float64)
    dz = dy * (np.asarray(z) > 0) if relu else dy
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    dx = dz @ W
    dW = dz.T @ x
    db = dz.sum(axis=0)
    return dx, dW, db, np.abs(dz) @ np.abs(W), np.abs(dz).T @ np.abs(x), np.abs(dz).sum(axis=0)


def sigmoid(z):
    z = np.asarray(z, np.float64)
    return np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.abs(z))), np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))


def bce_head(x, w, b, t):
    """One-unit head with a sigmoid and the mean binary cross-entropy.

    Returns dict with p [M], loss, and the gradients dx [M][K], dw [K], db of the mean loss."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    t = np.asarray(t, np.float64)
    M = x.shape[0]
    z = x @ w + float(b)
    p = sigmoid(z)
    # -(t log p + (1-t) log(1-p)) written with log(1 + e^-|z|) so that it is exact for large |z|
    loss_i = np.maximum(z, 0.0) - z * t + np.log1p(np.exp(-np.abs(z)))
    dz = (p - t) / M
    return {"z": z, "p": p, "loss": float(loss_i.mean()), "loss_i": loss_i, "dz": dz,
            "dx": np.outer(dz, w), "dw": x.T @ dz, "db": float(dz.sum()),
            "z_scale": np.abs(x) @ np.abs(w) + abs(float(b)),
            "dw_scale": np.abs(x).T @ np.abs(dz), "db_scale": float(np.abs(dz).sum())}


def sgd(w, g, lr):
    return np.asarray(w, np.float64) - float(lr) * np.asarray(g, np.float64)
