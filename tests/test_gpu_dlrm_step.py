"""A full DLRM training step on the GPU (bottom MLP, lookup, interaction, top MLP, sigmoid + BCE,
backward, SGD on the dense layers, row-wise Adagrad on the tables), checked link by link against
the oracle on the GPU's own inputs to each link (needs an MI355X).

Gates: the per-layer gates of test_gpu_mlp.py and the sparse-path gates of test_gpu_parity.py.
The dense-layer gradients are checked through an fp64 oracle backward chain started from the
head's input gradient: each GPU layer rounds dz to bf16 once (2^-9), so after the L layers of a
chain the gate is L * 2^-9 plus the fp32 bounds, held to 2^-7 for the at most 3 layers here.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mlp
from recommendation_model_sparse_amd import AdagradOutputs, synth
from recommendation_model_sparse_amd.dlrm_step import DlrmStep
from recommendation_model_sparse_amd.synth import Workload, subset_tables

from gpu_util import DEV, device_tables, rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def f64(t: torch.Tensor) -> np.ndarray:
    h = to_host(t)
    return synth.bf16_bits_to_f32(h).astype(np.float64) if t.dtype == torch.bfloat16 else h.astype(np.float64)


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
    m = DlrmStep(tabs, states, wl.B, 13, bottom=[64, 64], top=[128, 64], lr_dense=0.05, lr_emb=0.01,
                 eps=1e-8, seed=7, max_nnz=b.nnz, overlap=overlap)
    before = {id(l): (f64(l.W16), l.b.cpu().numpy().astype(np.float64), l.W32.cpu().numpy().copy(),
                      l.b.cpu().numpy().copy()) for l in m.bottom + m.top + [m.head]}
    idx, off = to_dev(b.indices), to_dev(b.offsets)
    outs = AdagradOutputs(b.nnz, DEV)
    m.forward(idx, off, to_dev(feats), to_dev(labels))
    torch.cuda.synchronize()
    # keep what the backward overwrites or what we check the backward against
    fwd = {"x0": f64(m.x0), "hb": [f64(h) for h in m.hb], "pooled": f64(m.pooled), "inter": f64(m.inter),
           "t0": f64(m.t0), "ht": [f64(h) for h in m.ht], "p": m.head_out["p"].cpu().numpy().astype(np.float64),
           "loss": float(m.head_out["loss"].item()), "hdx": m.head_out["dx"].cpu().numpy().astype(np.float64)}
    m.backward_and_update(idx, off, outputs=outs)
    torch.cuda.synchronize()

    # ---- forward, link by link
    assert np.array_equal(to_host(m.x0)[:, :13], synth.f32_to_bf16_bits(feats)) and np.all(fwd["x0"][:, 13:] == 0)
    x = fwd["x0"]
    for i, layer in enumerate(m.bottom):
        W, bb, _, _ = before[id(layer)]
        ref, scale, _ = mlp.linear_fwd(x, W, bb, relu=True)
        gate = 2.0 ** -8 if i < len(m.bottom) - 1 else W.shape[1] * 2.0 ** -24  # bf16 / fp32 output
        assert rel_err(fwd["hb"][i], ref, scale) <= gate, f"bottom layer {i}"
        x = fwd["hb"][i]
    ref, scale = oracle.emb_bag_fwd(subset_tables(wl, [np.arange(v) for v in wl.rows]), b.indices, b.offsets,
                                    None, wl.B)
    assert rel_err(fwd["pooled"], ref, scale) <= 1e-5
    ref, scale = oracle.interact_fwd(fwd["hb"][-1].astype(np.float32), fwd["pooled"].astype(np.float32))
    assert rel_err(fwd["inter"], ref, scale) <= 1e-5
    assert np.array_equal(to_host(m.t0)[:, :m.I], synth.f32_to_bf16_bits(fwd["inter"].astype(np.float32)))
    x = fwd["t0"]
    for i, layer in enumerate(m.top):
        W, bb, _, _ = before[id(layer)]
        ref, scale, _ = mlp.linear_fwd(x, W, bb, relu=True)
        assert rel_err(fwd["ht"][i], ref, scale) <= 2.0 ** -8, f"top layer {i}"
        x = fwd["ht"][i]
    hw, hb, _, _ = before[id(m.head)]
    h = mlp.bce_head(fwd["ht"][-1], hw.reshape(-1), float(hb[0]), labels)
    K = fwd["ht"][-1].shape[1]
    assert np.all(np.abs(fwd["p"] - h["p"]) <= 0.25 * K * 2.0 ** -24 * h["z_scale"] + 4e-7)
    assert abs(fwd["loss"] - h["loss"]) <= 1e-5 * max(1.0, h["loss"])
    say(f"   loss {fwd['loss']:.6f} (oracle on the GPU's head input {h['loss']:.6f})")

    # ---- backward: the top chain from the head's input gradient, in fp64 on the GPU activations.
    # The error scale of a chain is the absolute values carried through it, S <- (S * mask) |W|,
    # started from |the chain's GPU input|: every link adds at most one bf16 rounding of dz.
    def chain(dy, outs, ins, layers, tag):
        S = np.abs(dy)
        for i in range(len(layers) - 1, -1, -1):
            layer = layers[i]
            W = before[id(layer)][0]
            mask = outs[i] > 0
            dx, dW, db, *_ = mlp.linear_bwd(dy, outs[i], ins[i], W, relu=True)
            Sdz = S * mask
            assert rel_err(layer.dW.cpu().numpy(), dW, Sdz.T @ np.abs(ins[i])) <= 2.0 ** -7, f"{tag} dW {i}"
            assert rel_err(layer.db.cpu().numpy(), db, Sdz.sum(axis=0)) <= 2.0 ** -7, f"{tag} db {i}"
            dy, S = dx, Sdz @ np.abs(W)
        return dy, S

    dtop, Stop = chain(fwd["hdx"], fwd["ht"], [fwd["t0"]] + fwd["ht"][:-1], m.top, "top")
    dinter = m.dinter.cpu().numpy()
    assert rel_err(dinter, dtop[:, :m.I], Stop[:, :m.I]) <= 2.0 ** -7
    # the interaction backward on the GPU's own upstream gradient
    rd, rp, md, mp = oracle.interact_bwd(dinter, fwd["hb"][-1].astype(np.float32), fwd["pooled"].astype(np.float32))
    assert rel_err(m.gdense.cpu().numpy(), rd, md) <= 1e-5
    assert rel_err(m.gpooled.cpu().numpy(), rp, mp) <= 1e-5
    # the bottom chain from the GPU's dense-vector gradient
    chain(m.gdense.cpu().numpy().astype(np.float64), fwd["hb"], [fwd["x0"]] + fwd["hb"][:-1], m.bottom, "bottom")
    # padded input columns keep zero weights
    assert np.all(m.bottom[0].W32.cpu().numpy()[:, 13:] == 0) and np.all(m.top[0].W32.cpu().numpy()[:, m.I:] == 0)

    # ---- SGD on every dense parameter: fp32 master minus lr * gradient, bf16 copy refreshed
    lr = np.float32(0.05)
    for layer, g, gb in [(l, l.dW, l.db) for l in m.bottom + m.top] + [(m.head, m.head_out["dw"], m.head_out["db"])]:
        _, _, W32, b32 = before[id(layer)]
        want = (W32.reshape(-1).astype(np.float64) - float(lr) * g.cpu().numpy().reshape(-1).astype(np.float64))
        got = layer.W32.cpu().numpy().reshape(-1)
        assert np.all(np.abs(got - want) <= 2.0 ** -24 * np.abs(want) + 1e-30)
        assert np.array_equal(to_host(layer.W16).reshape(-1), synth.f32_to_bf16_bits(got))
        wantb = b32.astype(np.float64) - float(lr) * gb.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(layer.b.cpu().numpy() - wantb) <= 2.0 ** -24 * np.abs(wantb) + 1e-30)

    # ---- row-wise Adagrad on the tables with the GPU's pooled gradient
    gp = m.gpooled.cpu().numpy()
    sub_wl, sub, row_ids = b.sample_subset(np.arange(wl.B))
    r = oracle.emb_bag_bwd_adagrad(subset_tables(wl, row_ids), [np.zeros(len(x), np.float32) for x in row_ids],
                                   sub.indices, sub.offsets, None, wl.B, gp, 0.01, 1e-8)
    assert int(outs.num_unique.item()) == r.U
    tt, rr = r.table_and_row()
    for t in range(wl.T):
        sel = tt == t
        rows_t = row_ids[t][rr[sel]]
        got = synth.bf16_bits_to_f32(to_host(tabs[t])[rows_t]).astype(np.float64)
        ref = r.new_rows[sel]
        tol = np.abs(ref) * 2.0 ** -8 + 1e-4 * np.max(np.abs(ref), axis=1, keepdims=True)
        assert np.all(np.abs(got - ref) <= tol), f"table {t}"
    say(f"   step checked: U={r.U}")
    del tabs, states
    torch.cuda.empty_cache()
