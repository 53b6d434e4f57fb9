"""One full DLRM training step on one GPU, as a sequence of the library's C-ABI calls.

robocikowo.com "DLRM", paragraph "Forward pass", stages (1)-(4) and the training sentence:
dense features -> bottom MLP (FC + ReLU) -> the D-wide dense vector; sparse features -> bag
lookups; pairwise dots of the N = T + 1 vectors (strict upper triangle) concatenated with the
dense vector -> top MLP (FC + ReLU) -> one unit with a sigmoid -> binary cross-entropy against
the clicks; then the backward pass, SGD on the dense layers and row-wise Adagrad on the tables.

This module only orders the calls and owns the buffers (argument marshalling); every step runs in
the library's kernels (hipBLASLt for the plain GEMMs).  Dense weights are kept as fp32 masters
with bf16 copies for the GEMMs; activations are bf16 between layers, the dense vector and the
interaction are fp32.  Widths are padded to multiples of 8 (16-byte bf16 rows): the dense input
features with zero columns, the interaction output 479 -> 480 with a zero column whose weights
stay zero (their gradient is zero).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np
import torch

from . import binding as L
from .synth import f32_to_bf16_bits


def _pad8(n: int) -> int:
    return (n + 7) // 8 * 8


@dataclass
class DenseLayer:
    W32: torch.Tensor   # [N][K] fp32 master
    W16: torch.Tensor   # [N][K] bf16 copy
    b: torch.Tensor     # [N] fp32
    dW: torch.Tensor
    db: torch.Tensor


def _init_layer(rng: np.random.Generator, N: int, K: int, K_used: int, dev) -> DenseLayer:
    """Uniform(+-1/sqrt(fan_in)) weights over the first K_used input columns, zero padding."""
    a = 1.0 / np.sqrt(K_used)
    W = np.zeros((N, K), np.float32)
    W[:, :K_used] = rng.uniform(-a, a, (N, K_used)).astype(np.float32)
    b = rng.uniform(-a, a, N).astype(np.float32)
    W32 = torch.from_numpy(W).to(dev)
    W16 = torch.from_numpy(f32_to_bf16_bits(W).view(np.int16)).view(torch.bfloat16).to(dev)
    return DenseLayer(W32, W16, torch.from_numpy(b).to(dev), torch.empty_like(W32), torch.empty(N, device=dev))


class DlrmStep:
    """Buffers and weights of one DLRM on one GPU; `step` runs a full training step."""

    def __init__(self, tables: Sequence[torch.Tensor], states: Sequence[torch.Tensor], B: int, n_dense: int,
                 bottom: Sequence[int], top: Sequence[int], lr_dense: float, lr_emb: float, eps: float,
                 seed: int, max_nnz: int, overlap: bool = True):
        self.tables, self.states = list(tables), list(states)
        # the tables and states checked once for the step's calls (each call re-reads only their
        # pointers and row counts)
        self.tabset = L.TableSet(self.tables, self.states)
        # overlap: a second stream takes the bottom MLP's forward (beside the lookup), the
        # batch-only half of the embedding backward (key sort and segments, beside the top MLP's
        # and the interaction's backward) and the bottom MLP's backward (beside the embedding
        # update); events order each against the caller's stream
        self.overlap = overlap
        dev = self.tables[0].device
        self.dev = dev
        self.B, self.T, self.D = B, len(tables), tables[0].shape[1]
        self.N = self.T + 1
        self.P = self.N * (self.N - 1) // 2
        self.lr_dense, self.lr_emb, self.eps = lr_dense, lr_emb, eps
        if bottom[-1] != self.D:
            raise ValueError("the bottom MLP must end at the embedding width D")
        rng = np.random.default_rng(seed)
        self.F, self.Fp = n_dense, _pad8(n_dense)
        self.I, self.Ip = self.P + self.D, _pad8(self.P + self.D)
        widths_b = [self.Fp] + list(bottom)
        used_b = [self.F] + list(bottom)
        self.bottom: List[DenseLayer] = [_init_layer(rng, widths_b[i + 1], widths_b[i], used_b[i], dev)
                                         for i in range(len(bottom))]
        widths_t = [self.Ip] + list(top)
        used_t = [self.I] + list(top)
        self.top: List[DenseLayer] = [_init_layer(rng, widths_t[i + 1], widths_t[i], used_t[i], dev)
                                      for i in range(len(top))]
        if top[-1] % 8:
            raise ValueError("the last top width must be a multiple of 8")
        self.head = _init_layer(rng, 1, top[-1], top[-1], dev)
        bf = dict(dtype=torch.bfloat16, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        # activations (bottom outputs bf16 except the last, the fp32 dense vector)
        self.x0 = torch.empty((B, self.Fp), **bf)
        self.hb = [torch.empty((B, n), **bf) for n in bottom[:-1]] + [torch.empty((B, self.D), **f32)]
        self.pooled = torch.empty((B, self.T, self.D), **f32)
        self.inter = torch.empty((B, self.I), **f32)
        self.t0 = torch.empty((B, self.Ip), **bf)
        self.ht = [torch.empty((B, n), **bf) for n in top]
        self.labels = torch.empty(B, **f32)
        # gradients and scratch
        widest = max(max(bottom), max(top), self.Ip, self.Fp)
        self.ws = torch.empty(L.dlrm_linear_workspace_size(B, widest, widest), dtype=torch.uint8, device=dev)
        self.hws = torch.empty(L.dlrm_bce_head_workspace_size(B, top[-1]), dtype=torch.uint8, device=dev)
        self.dz = torch.empty(B * widest, **bf)
        self.grad_a = torch.empty(B * widest, **f32)
        self.grad_b = torch.empty(B * widest, **f32)
        self.dinter = torch.empty((B, self.I), **f32)
        self.gdense = torch.empty((B, self.D), **f32)
        self.gpooled = torch.empty_like(self.pooled)
        self.head_out = {"p": torch.empty(B, **f32), "loss": torch.empty(1, **f32),
                         "dx": torch.empty((B, top[-1]), **f32), "dw": torch.empty(top[-1], **f32),
                         "db": torch.empty(1, **f32)}
        rows = [t.shape[0] for t in self.tables]
        self.rows = rows
        self.emb_ws = torch.empty(L.emb_bag_bwd_workspace_size(rows, self.D, B, max_nnz), dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev)  # default priority
        self.plan_done = torch.cuda.Event()
        self.dense_ready = torch.cuda.Event()
        self.bottom_fwd_done = torch.cuda.Event()
        self.bottom_done = torch.cuda.Event()

    def _mat(self, flat: torch.Tensor, rows: int, cols: int) -> torch.Tensor:
        return flat[:rows * cols].view(rows, cols)

    def forward(self, idx: torch.Tensor, off: torch.Tensor, dense_x: torch.Tensor, labels: torch.Tensor):
        if self.overlap:
            # the bottom MLP runs on the second stream while the lookup runs here
            main = torch.cuda.current_stream(self.dev)
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                self._bottom_forward(dense_x)
                self.bottom_fwd_done.record(self.side)
            L.emb_bag_fwd(self.tabset, idx, off, None, out=self.pooled)
            main.wait_event(self.bottom_fwd_done)
        else:
            self._bottom_forward(dense_x)
            L.emb_bag_fwd(self.tabset, idx, off, None, out=self.pooled)
        L.dlrm_interact_fwd(self.hb[-1], self.pooled, out=self.inter)
        L.dlrm_cast_rows(self.inter, self.I, self.Ip, torch.bfloat16, dst=self.t0)
        x = self.t0
        for i, layer in enumerate(self.top):
            L.dlrm_linear_fwd(x, layer.W16, layer.b, L.DLRM_ACT_RELU, y=self.ht[i], workspace=self.ws)
            x = self.ht[i]
        self.labels.copy_(labels)
        # the head needs a 16-byte-row input: the last top width is a multiple of 8
        L.dlrm_bce_head(x, self.head.W16.view(-1), self.head.b, self.labels, workspace=self.hws, out=self.head_out)
        return self.head_out

    def backward_and_update(self, idx: torch.Tensor, off: torch.Tensor, outputs=None):
        B = self.B
        if self.overlap:
            main = torch.cuda.current_stream(self.dev)
            # after everything already on the caller's stream (the previous update read the workspace)
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                L.emb_bag_bwd_plan(self.rows, self.D, idx, off, None, self.emb_ws, outputs=outputs)
                self.plan_done.record(self.side)
        # head: its own gradients came with the forward
        dy = self.head_out["dx"]
        ins = [self.t0] + self.ht[:-1]
        bufs = [self.grad_a, self.grad_b]
        for i in range(len(self.top) - 1, -1, -1):
            layer = self.top[i]
            K = ins[i].shape[1]
            dx = self._mat(bufs[i % 2], B, K)
            L.dlrm_linear_bwd(dy, self.ht[i], L.DLRM_ACT_RELU, ins[i], layer.W16, want_dx=True,
                              dz_bf16=self._mat(self.dz, B, layer.W16.shape[0]), dx=dx, dW=layer.dW, db=layer.db,
                              workspace=self.ws)
            dy = dx
        L.dlrm_cast_rows(dy, self.I, self.I, torch.float32, dst=self.dinter)  # drop the pad column
        L.dlrm_interact_bwd(self.dinter, self.hb[-1], self.pooled, grad_dense=self.gdense, grad_pooled=self.gpooled)
        if self.overlap:
            # the bottom MLP's backward needs only the dense gradient: it runs on the second stream
            # (after the sort) while the embedding update runs here; the two share no buffer
            self.dense_ready.record(main)
            main.wait_event(self.plan_done)
            L.emb_bag_bwd_apply(self.tabset, self.states, B, idx.numel(), False, self.gpooled, L.DLRM_OPT_ADAGRAD,
                                self.lr_emb, self.eps, self.emb_ws, outputs=outputs)
            with torch.cuda.stream(self.side):
                self.side.wait_event(self.dense_ready)
                self._bottom_backward(bufs)
                self.bottom_done.record(self.side)
            main.wait_event(self.bottom_done)
        else:
            L.emb_bag_bwd_adagrad(self.tabset, self.states, idx, off, None, self.gpooled, self.lr_emb, self.eps,
                                  workspace=self.emb_ws, outputs=outputs)
            self._bottom_backward(bufs)
        # SGD on every dense parameter, in one launch
        params = []
        for layer in self.bottom + self.top:
            params += [(layer.W32, layer.W16, layer.dW), (layer.b, None, layer.db)]
        h = self.head
        params += [(h.W32.view(-1), h.W16.view(-1), self.head_out["dw"]), (h.b, None, self.head_out["db"])]
        L.dlrm_sgd_dense_multi(params, self.lr_dense)

    def _bottom_forward(self, dense_x):
        L.dlrm_cast_rows(dense_x, self.F, self.Fp, torch.bfloat16, dst=self.x0)
        x = self.x0
        for i, layer in enumerate(self.bottom):
            L.dlrm_linear_fwd(x, layer.W16, layer.b, L.DLRM_ACT_RELU, y=self.hb[i], workspace=self.ws)
            x = self.hb[i]

    def _bottom_backward(self, bufs):
        B = self.B
        dy = self.gdense
        ins = [self.x0] + self.hb[:-1]
        for i in range(len(self.bottom) - 1, -1, -1):
            layer = self.bottom[i]
            K = ins[i].shape[1]
            dx = self._mat(bufs[i % 2], B, K) if i > 0 else None
            L.dlrm_linear_bwd(dy, self.hb[i], L.DLRM_ACT_RELU, ins[i], layer.W16, want_dx=i > 0,
                              dz_bf16=self._mat(self.dz, B, layer.W16.shape[0]), dx=dx, dW=layer.dW, db=layer.db,
                              workspace=self.ws)
            dy = dx

    def step(self, idx, off, dense_x, labels, outputs=None):
        out = self.forward(idx, off, dense_x, labels)
        self.backward_and_update(idx, off, outputs)
        return out
