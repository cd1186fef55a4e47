"""GPU parity of the _ex options against the oracle: logit_scale, the z-loss term
alone, and accumulation into existing gradients."""

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import functional as F
from lm_head_cross_flce_amd import synth
from oracle import flce_oracle as O

from flce_gpu_util import GRAD_RTOL, LOSS_RTOL, LSE_RTOL, device_inputs, rel, to_f64

pytestmark = pytest.mark.gpu

W_ = synth.WORKLOADS
CASES = {
    "c3_small": synth.scaled(W_["n8192_h4096_v128256"], "c3_small", N=600, H=328, V=2083, n_ignored=30),
    "f32_none": synth.scaled(W_["tiny_f32"], "f32_none", N=300, H=136, V=1100, n_ignored=11, label_smoothing=0.1,
                             z_loss_scale=1e-3, reduction="none", grad="vector_normal", seed=8),
}
_inp = {}


def inputs(name):
    if name not in _inp:
        _inp[name] = synth.make_inputs(CASES[name])
    return _inp[name]


def oracle(inp, alpha=1.0, reduction=None):
    w = inp.w
    red = reduction or w.reduction
    g = inp.grad
    if red != w.reduction:
        g = np.full(w.N, g[0], dtype=np.float32) if red == "none" else g[:1]
    x, W, b = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    f = O.forward(x, W, b, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, red, logit_scale=alpha)
    bw = O.backward(x, W, b, inp.targets, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, red,
                    logit_scale=alpha)
    return f, bw, g


@pytest.mark.parametrize("name,alpha", [("c3_small", 0.5), ("c3_small", -1.3), ("f32_none", 2.0)])
def test_logit_scale(name, alpha):
    inp = inputs(name)
    w = inp.w
    print(f"[gpu] logit_scale {alpha} {name}", flush=True)
    x, W, b, t, g = device_inputs(inp)
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                                   logit_scale=alpha)
    dx, dW, db = F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                 w.reduction, logit_scale=alpha)
    torch.cuda.synchronize()
    f, bw, _ = oracle(inp, alpha)
    tol = GRAD_RTOL[w.dtype]
    assert int(nv.item()) == f.n_valid
    assert rel(loss.cpu().numpy().astype(np.float64), f.loss) <= LOSS_RTOL
    assert rel(lse.cpu().numpy().astype(np.float64), f.lse) <= LSE_RTOL
    assert rel(to_f64(dx), bw.dx) <= tol and rel(to_f64(dW), bw.dW) <= tol
    if bw.db is not None:
        assert rel(to_f64(db), bw.db) <= tol


@pytest.mark.parametrize("red", ["none", "sum", "mean"])
def test_z_loss_term_alone(red):
    inp = inputs("c3_small")
    w = inp.w
    print(f"[gpu] z-loss term {red}", flush=True)
    x, W, b, t, g = device_inputs(inp)
    loss, lse, nv, zl = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, red,
                                       return_z_loss=True)
    torch.cuda.synchronize()
    f, _, _ = oracle(inp, reduction=red)
    assert zl.shape == loss.shape
    assert rel(zl.cpu().numpy().astype(np.float64), f.z_loss) <= LOSS_RTOL
    assert rel(loss.cpu().numpy().astype(np.float64), f.loss) <= LOSS_RTOL


@pytest.mark.parametrize("name,slab", [("c3_small", None), ("c3_small", "512"), ("c3_small", "1024"),
                                       ("f32_none", None), ("f32_none", "256")])
def test_accumulate_into_existing_gradients(monkeypatch, name, slab):
    # one slab and several (with no override and with 1024 columns these
    # shapes split each slab's columns in K parts, each with an fp32
    # accumulator; with 512 or 256 columns dx is its own accumulator: bf16
    # holds the fp32 values' high halves, fp32 the values themselves)
    if slab:
        monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", slab)
    inp = inputs(name)
    w = inp.w
    print(f"[gpu] accumulate {name} slab={slab}", flush=True)
    f, bw, _ = oracle(inp)
    x, W, b, t, g = device_inputs(inp)
    gen = torch.Generator(device="cpu").manual_seed(5)

    def prefill(ref, like):
        v = torch.randn(like.shape, generator=gen, dtype=torch.float64) * float(np.std(ref))
        return v.to(like.dtype).to(like.device)

    dx0, dW0 = prefill(bw.dx, x), prefill(bw.dW, W)
    db0 = prefill(bw.db, b) if b is not None else None
    out = (dx0.clone(), dW0.clone(), db0.clone() if db0 is not None else None)
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                    out=out, accumulate=True)
    torch.cuda.synchronize()
    tol = GRAD_RTOL[w.dtype]
    assert rel(to_f64(out[0]), to_f64(dx0) + bw.dx) <= tol
    assert rel(to_f64(out[1]), to_f64(dW0) + bw.dW) <= tol
    if db0 is not None:
        assert rel(to_f64(out[2]), to_f64(db0) + bw.db) <= tol


def test_module_with_logit_scale():
    inp = inputs("c3_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    x.requires_grad_(True)
    W.requires_grad_(True)
    print("[gpu] module with logit_scale", flush=True)
    mod = F.FusedLinearCrossEntropyLoss(w.ignore_index, w.label_smoothing, w.z_loss_scale, "mean", logit_scale=0.8)
    loss = mod(x, t, W, b)
    loss.backward(g.reshape(()))
    torch.cuda.synchronize()
    f, bw, _ = oracle(inp, 0.8)
    assert rel(np.array([loss.item()]), f.loss) <= LOSS_RTOL
    assert rel(to_f64(x.grad), bw.dx) <= GRAD_RTOL["bf16"] and rel(to_f64(W.grad), bw.dW) <= GRAD_RTOL["bf16"]
