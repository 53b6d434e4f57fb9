"""A full DLRM training step on the GPU (bottom MLP, lookup, interaction, top MLP, sigmoid + BCE,
backward, SGD on the dense layers, row-wise Adagrad on the tables), checked against the oracle's
own step (needs an MI355X).

The oracle runs the whole step on the host from the same initial parameters, features, labels,
tables and lookups, in fp64, applying the step's storage roundings to its own values (bf16
activations between layers, the fp32 dense vector, pooled rows and interaction).  No GPU value
enters it.  Each link of the chain, forward or backward, rounds one operand to bf16 (2^-9) on each
side, so a result k links from the exact inputs is compared norm-wise, ||gpu - oracle|| <= k * 2^-8
||oracle|| (the gradients of a link are bilinear in two operands that each carry their own depth;
the larger is used).  Element-wise gates hold where the inputs are exact: the bf16 input rows bit
for bit, the first bottom layer's output (one GEMM and one bf16 rounding from exact inputs) within
its fp32 accumulation bound plus the roundings, the pooled rows within 1e-5 of their error scale,
untouched table rows bit for bit.  The
isolated kernels are checked element-wise against the oracle on host inputs in test_gpu_mlp.py and
test_gpu_parity.py; this test checks that the step wires them together.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mlp
from recommendation_model_sparse_amd import AdagradOutputs, synth
from recommendation_model_sparse_amd.dlrm_step import DlrmStep
from recommendation_model_sparse_amd.synth import Workload, subset_tables

from gpu_util import DEV, bf16_half_ulp, device_tables, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu
E = 2.0 ** -8  # one bf16 rounding on each side


def f64(t: torch.Tensor) -> np.ndarray:
    h = to_host(t)
    return synth.bf16_bits_to_f32(h).astype(np.float64) if t.dtype == torch.bfloat16 else h.astype(np.float64)


def bf16r(x: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def f32r(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float32).astype(np.float64)


def nrel(got, ref) -> float:
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref) / (den if den > 0 else 1.0))


REPORT = []


def close(got, ref, k, what):
    e = nrel(got, ref)
    REPORT.append((what, e, k))
    assert e <= k * E, f"{what}: {e:.3e} > {k} * 2^-8"


class OracleStep:
    """The oracle's forward, backward and updates of one step, with the link depth of each result."""

    def __init__(self, wl, b, feats, labels, m, params):
        B = wl.B
        self.params = params
        x = np.zeros((B, m.Fp))
        x[:, :m.F] = bf16r(feats)
        self.x0 = x
        self.hb = []
        for i, layer in enumerate(m.bottom):
            W, bb, _, _ = params[id(layer)]
            y, _, _ = mlp.linear_fwd(x, W, bb, relu=True)
            x = f32r(y) if i == len(m.bottom) - 1 else bf16r(y)
            self.hb.append(x)
        self.kb = len(m.bottom)
        tables = subset_tables(wl, [np.arange(v) for v in wl.rows])
        self.pooled, self.pooled_scale = oracle.emb_bag_fwd(tables, b.indices, b.offsets, None, B)
        self.dense32, self.pooled32 = self.hb[-1].astype(np.float32), self.pooled.astype(np.float32)
        self.inter, _ = oracle.interact_fwd(self.dense32, self.pooled32)
        x = np.zeros((B, m.Ip))
        x[:, :m.I] = bf16r(f32r(self.inter))
        self.t0 = x
        self.ht = []
        for layer in m.top:
            W, bb, _, _ = params[id(layer)]
            y, _, _ = mlp.linear_fwd(x, W, bb, relu=True)
            x = bf16r(y)
            self.ht.append(x)
        self.kt = self.kb + 2 + len(m.top)  # depth of the last top activation (kb + 3 + i for layer i)
        hw, hbias, _, _ = params[id(m.head)]
        self.head = h = mlp.bce_head(x, hw.reshape(-1), float(hbias[0]), labels)
        # backward
        dy, self.top_grads, k = self.chain(h["dx"], self.ht, [self.t0] + self.ht[:-1], m.top, self.kt + 1)
        self.dinter, self.kdi = dy[:, :m.I], k
        self.gdense, self.gpooled, _, _ = oracle.interact_bwd(self.dinter.astype(np.float32), self.dense32,
                                                               self.pooled32)
        self.kdx = k + 1
        _, self.bottom_grads, _ = self.chain(self.gdense, self.hb, [self.x0] + self.hb[:-1], m.bottom, self.kdx)

    def chain(self, dy, acts, ins, layers, k):
        """Backward through `layers` from dy (depth k): dx, [(layer index, dW, db, depth)], depth."""
        grads = []
        for i in range(len(layers) - 1, -1, -1):
            W = self.params[id(layers[i])][0]
            dx, dW, db, *_ = mlp.linear_bwd(dy, acts[i], ins[i], W, relu=True)
            k += 1  # the bf16 rounding of dz
            grads.append((i, dW, db, k))
            dy = dx
        return dy, grads, k


@pytest.mark.parametrize("overlap", [True, False])
def test_full_training_step(overlap):
    wl = Workload(name="step", seed=4242, T=8, D=64, dtype="bf16", B=512,
                  rows=[1000, 50000, 3000, 7, 20000, 900, 12345, 64], init="hash", bags="geom",
                  bag_lo=1, bag_hi=20, bag_mean=5.0, dist="zipf", alpha=1.05)
    b = wl.batch(0)
    feats, labels = b.features(13), b.labels()
    tabs = device_tables(wl)
    states = [torch.zeros(v, dtype=torch.float32, device=DEV) for v in wl.rows]
    say(f"[step] T={wl.T} D={wl.D} B={wl.B} nnz={b.nnz} overlap={overlap}")
    lr_dense, lr_emb = 0.05, 0.01
    m = DlrmStep(tabs, states, wl.B, 13, bottom=[64, 64], top=[128, 64], lr_dense=lr_dense, lr_emb=lr_emb,
                 eps=1e-8, seed=7, max_nnz=b.nnz, overlap=overlap)
    # the initial parameters (the oracle's inputs): bf16 copies, the GEMM operands, and fp32 masters
    params = {id(l): (f64(l.W16), l.b.cpu().numpy().astype(np.float64), l.W32.cpu().numpy().astype(np.float64),
                      l.b.cpu().numpy().astype(np.float64)) for l in m.bottom + m.top + [m.head]}
    idx, off = to_dev(b.indices), to_dev(b.offsets)
    outs = AdagradOutputs(b.nnz, DEV)
    m.forward(idx, off, to_dev(feats), to_dev(labels))
    torch.cuda.synchronize()
    gpu = {"x0": f64(m.x0), "hb": [f64(h) for h in m.hb], "pooled": f64(m.pooled), "inter": f64(m.inter),
           "t0": f64(m.t0), "ht": [f64(h) for h in m.ht], "p": m.head_out["p"].cpu().numpy().astype(np.float64),
           "loss": float(m.head_out["loss"].item()), "dw": m.head_out["dw"].cpu().numpy().astype(np.float64)}
    m.backward_and_update(idx, off, outputs=outs)
    torch.cuda.synchronize()
    o = OracleStep(wl, b, feats, labels, m, params)
    REPORT.clear()

    # ---- forward
    assert np.array_equal(gpu["x0"], o.x0)
    # the first layer is one GEMM and one bf16 rounding from exact inputs (x0 and W bit-equal on both
    # sides): element-wise, the fp32 accumulation error gamma_K * scale plus the two roundings (half
    # a bf16 ulp of each side's value)
    W0, b0, _, _ = params[id(m.bottom[0])]
    _, s0, _ = mlp.linear_fwd(o.x0, W0, b0, relu=True)
    K0 = o.x0.shape[1]
    gate0 = bf16_half_ulp(o.hb[0]) + bf16_half_ulp(gpu["hb"][0]) + (K0 + 2) * 2.0 ** -24 * s0  # K products and the bias
    assert np.all(np.abs(gpu["hb"][0] - o.hb[0]) <= gate0)
    for i in range(len(m.bottom)):
        close(gpu["hb"][i], o.hb[i], i + 1, f"bottom layer {i}")
    assert rel_err(gpu["pooled"], o.pooled, o.pooled_scale) <= 1e-5
    close(gpu["inter"], o.inter, o.kb + 1, "interaction")
    close(gpu["t0"], o.t0, o.kb + 2, "top input")
    for i in range(len(m.top)):
        close(gpu["ht"][i], o.ht[i], o.kb + 3 + i, f"top layer {i}")
    h = o.head
    close(gpu["p"], h["p"], o.kt, "click probability")
    assert abs(gpu["loss"] - h["loss"]) <= o.kt * E * h["loss"]
    close(gpu["dw"], h["dw"], o.kt + 1, "head dw")

    # ---- backward
    for layers, grads, tag in ((m.top, o.top_grads, "top"), (m.bottom, o.bottom_grads, "bottom")):
        for (i, dW, db, k) in grads:
            close(layers[i].dW.cpu().numpy(), dW, k, f"{tag} dW {i}")
            close(layers[i].db.cpu().numpy(), db, k, f"{tag} db {i}")
    close(m.dinter.cpu().numpy(), o.dinter, o.kdi, "interaction input gradient")
    close(m.gdense.cpu().numpy(), o.gdense, o.kdx, "dense-vector gradient")
    close(m.gpooled.cpu().numpy(), o.gpooled, o.kdx, "pooled gradient")
    # padded input columns keep zero weights
    assert np.all(m.bottom[0].W32.cpu().numpy()[:, 13:] == 0) and np.all(m.top[0].W32.cpu().numpy()[:, m.I:] == 0)

    # ---- SGD: the oracle's step from the same fp32 masters; the update lr * dW is within the
    # gradient's gate and the new master within one fp32 rounding more; the bf16 copy is the new
    # master rounded
    for layers, grads in ((m.top, o.top_grads), (m.bottom, o.bottom_grads)):
        for (i, dW, db, k) in grads:
            layer = layers[i]
            _, _, W32, b32 = params[id(layer)]
            got = layer.W32.cpu().numpy().astype(np.float64)
            want = mlp.sgd(W32, dW, lr_dense)
            assert np.linalg.norm(got - want) <= lr_dense * k * E * np.linalg.norm(dW) + 2.0 ** -23 * np.linalg.norm(want)
            assert np.array_equal(to_host(layer.W16), synth.f32_to_bf16_bits(layer.W32.cpu().numpy()))
            gotb = layer.b.cpu().numpy().astype(np.float64)
            wantb = mlp.sgd(b32, db, lr_dense)
            assert np.linalg.norm(gotb - wantb) <= lr_dense * k * E * np.linalg.norm(db) + 2.0 ** -23 * np.linalg.norm(wantb)

    # ---- row-wise Adagrad with the oracle's pooled gradient: each touched row's update w' - w is
    # within the pooled gradient's gate (twice: the step divides by the gradient's own RMS) plus
    # the bf16 rounding of the stored row; untouched rows and states are unchanged
    sub_wl, sub, row_ids = b.sample_subset(np.arange(wl.B))
    host_tabs = subset_tables(wl, row_ids)
    r = oracle.emb_bag_bwd_adagrad(host_tabs, [np.zeros(len(x), np.float32) for x in row_ids], sub.indices,
                                   sub.offsets, None, wl.B, o.gpooled.astype(np.float32), lr_emb, 1e-8)
    assert int(outs.num_unique.item()) == r.U
    tt, rr = r.table_and_row()
    rng = np.random.default_rng(5)
    for t in range(wl.T):
        sel = tt == t
        rows_t = row_ids[t][rr[sel]]
        w0 = synth.bf16_bits_to_f32(host_tabs[t][rr[sel]]).astype(np.float64)
        got = synth.bf16_bits_to_f32(to_host(tabs[t])[rows_t]).astype(np.float64)
        ref = r.new_rows[sel]
        gate = 2 * o.kdx * E * np.linalg.norm(ref - w0) + 2.0 ** -9 * np.linalg.norm(ref)
        assert np.linalg.norm(got - ref) <= gate, f"table {t}"
        gs = states[t][torch.from_numpy(rows_t).to(DEV)].cpu().numpy().astype(np.float64)
        assert nrel(gs, r.new_state[sel]) <= 2 * o.kdx * E, f"table {t} state"
        cand = np.setdiff1d(rng.integers(0, wl.rows[t], 256), row_ids[t])
        if len(cand):
            dc = torch.from_numpy(cand).to(DEV)
            assert np.array_equal(to_host(tabs[t][dc]), wl.table_rows(t, cand))
            assert torch.all(states[t][dc] == 0)
    worst = max(REPORT, key=lambda x: x[1] / x[2])
    say(f"   step checked against the oracle's step: U={r.U}; largest error {worst[1]:.2e} ({worst[0]}, "
        f"gate {worst[2]} * 2^-8)")
    del tabs, states
    torch.cuda.empty_cache()


def test_overlapped_step_matches_one_stream():
    """The step with the sort and the bottom MLP's backward on a second stream, against the same
    model stepped on one stream: every kernel and its order within each stream are the same, so
    two steps leave every dense parameter, table row and state bit for bit equal (a missing wait
    between the streams would let a kernel read a buffer before it is written, or after it is
    reused)."""
    wl = Workload(name="ovl", seed=99, T=6, D=64, dtype="bf16", B=2048,
                  rows=[5000, 300, 80000, 17, 4096, 1200], init="hash", bags="geom",
                  bag_lo=1, bag_hi=24, bag_mean=6.0, dist="zipf", alpha=1.05)
    batches = [wl.batch(i) for i in range(2)]
    models = []
    for overlap in (True, False):
        tabs = device_tables(wl)
        states = [torch.zeros(v, dtype=torch.float32, device=DEV) for v in wl.rows]
        m = DlrmStep(tabs, states, wl.B, 13, bottom=[128, 64], top=[256, 128, 64], lr_dense=0.05, lr_emb=0.01,
                     eps=1e-8, seed=11, max_nnz=max(b.nnz for b in batches), overlap=overlap)
        say(f"[step] overlap={overlap} B={wl.B} nnz={[b.nnz for b in batches]}")
        for b in batches:
            m.step(to_dev(b.indices), to_dev(b.offsets), to_dev(b.features(13)), to_dev(b.labels()))
        torch.cuda.synchronize()
        models.append((m, tabs, states))
    (a, ta, sa), (c, tc, sc) = models
    for la, lc in zip(a.bottom + a.top + [a.head], c.bottom + c.top + [c.head]):
        assert torch.equal(la.W32, lc.W32) and torch.equal(la.b, lc.b) and torch.equal(la.W16, lc.W16)
    for t in range(wl.T):
        assert torch.equal(ta[t], tc[t]), f"table {t}"
        assert torch.equal(sa[t], sc[t]), f"state {t}"
    del models, a, c, ta, tc, sa, sc
    torch.cuda.empty_cache()
