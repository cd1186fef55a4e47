"""GPU parity with fp16 inputs: the HIP library against the fp64 CPU oracle.

fp16 x, W and b run the same kernels as bf16 with the fp16 MFMA and conversions;
the backward's dlogits slab holds dz times a power-of-two scale so that
values near c_n / V stay in half's normal range.  The oracle takes the fp16
values exactly (fp16 -> fp64 is exact).  Bar: loss relative error <= 1e-3,
dx/dW/db relative Frobenius error <= 1e-2 (the bf16 bar; fp16 carries three
more mantissa bits), exact zeros where the oracle's result is zero.

The reduced cases keep the workloads' distributions.  They check that the
slab scale (2^22 at c3_f16) is applied and cancelled exactly in every
product: a missing factor would be off by orders of magnitude.  How much the
scale matters for accuracy grows with the mean's count and the vocabulary: at
c3_f16 an unscaled dz of c_n p ~ 1e-6 sits among fp16's subnormals (spacing
6e-8), which doubles the dx error (3e-4 -> 6e-4, both inside the bar); at the
full-size Llama-3-sized head (c_n p ~ 1e-9) every softmax term would flush to
zero, which the full-size fp16 test covers.
"""

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import functional as F
from lm_head_cross_flce_amd import synth
from oracle import flce_oracle as O

from flce_gpu_util import GRAD_RTOL, LOSS_RTOL, LSE_RTOL, device_inputs, rel, run, to_f64

pytestmark = pytest.mark.gpu

W_ = synth.WORKLOADS


def _case(base, name, **kw):
    return synth.scaled(W_[base], name, dtype="f16", **kw)


CASES = {
    "c3_f16": _case("n8192_h4096_v128256", "c3_f16", N=600, H=328, V=2083, n_ignored=30),
    "c2_f16": _case("n4096_h2048_v32000", "c2_f16", N=520, H=256, V=3001),
    "c4_f16": _case("n32768_h2048_v128000", "c4_f16", N=1024, H=264, V=4000),
    "c5_f16": _case("n16384_h1024_v256000", "c5_f16", N=777, H=128, V=5003),
    "sum_f16": _case("n8192_h4096_v128256", "sum_f16", N=300, H=200, V=1500, n_ignored=7,
                     reduction="sum", grad="scalar_normal", seed=7),
}

_inp = {}
_ref = {}


def inputs(name):
    if name not in _inp:
        _inp[name] = synth.make_inputs(CASES[name])
    return _inp[name]


def oracle(name):
    if name not in _ref:
        inp = inputs(name)
        w = inp.w
        x, W, b = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
        f = O.forward(x, W, b, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
        bw = O.backward(x, W, b, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                        w.reduction)
        _ref[name] = (f, bw)
    return _ref[name]


def check(name, got):
    f, bw = oracle(name)
    tol = GRAD_RTOL["f16"]
    assert got["n_valid"] == f.n_valid
    assert rel(got["loss"], f.loss) <= LOSS_RTOL, (rel(got["loss"], f.loss), got["loss"][:4], f.loss[:4])
    assert rel(got["lse"], f.lse) <= LSE_RTOL, rel(got["lse"], f.lse)
    assert rel(got["dx"], bw.dx) <= tol, ("dx", rel(got["dx"], bw.dx))
    assert rel(got["dW"], bw.dW) <= tol, ("dW", rel(got["dW"], bw.dW))
    if bw.db is not None:
        assert rel(got["db"], bw.db) <= tol, ("db", rel(got["db"], bw.db))
    ignored = inputs(name).targets == CASES[name].ignore_index
    assert np.all(got["dx"][ignored] == 0.0)


@pytest.mark.parametrize("name", list(CASES))
def test_f16_parity(name):
    print(f"[gpu] f16 parity {name}", flush=True)
    got = run(inputs(name))
    check(name, got)


def test_f16_forced_slabs_and_k_split(monkeypatch):
    # 1024-column slabs: three slabs at V = 2083, and these token counts split
    # the input-gradient product in two K parts (the last slab's second part
    # is empty); the scale must cancel in every accumulator.
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "1024")
    for name in ("c3_f16", "c5_f16"):
        print(f"[gpu] f16 forced slabs {name}", flush=True)
        check(name, run(inputs(name)))


@pytest.mark.parametrize("accumulate", [False, True])
def test_f16_split_dx_accumulator(monkeypatch, accumulate):
    # 256-column slabs give one K part, so dx accumulates over nine slabs as
    # fp32 values split in two: the high halves in dx itself, the low halves in
    # the workspace.  With accumulate, dx's old values are added on the first
    # slab, before its high halves replace them.
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "256")
    name = "c3_f16"
    inp = inputs(name)
    w = inp.w
    print(f"[gpu] f16 split dx accumulator, accumulate={accumulate}", flush=True)
    if not accumulate:
        check(name, run(inp))
        return
    f, bw = oracle(name)
    x, W, b, t, g = device_inputs(inp)
    gen = torch.Generator(device="cpu").manual_seed(8)
    dx0 = (torch.randn(x.shape, generator=gen, dtype=torch.float64) * float(np.std(bw.dx))).to(x.dtype).to(x.device)
    out = (dx0.clone(), None, None)
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                    need_dW=False, need_db=False, out=out, accumulate=True)
    torch.cuda.synchronize()
    assert rel(to_f64(out[0]), to_f64(dx0) + bw.dx) <= GRAD_RTOL["f16"]


def test_f16_all_ignored_gives_exact_zeros():
    w = _case("n8192_h4096_v128256", "f16_all_ignored", N=300, H=64, V=700, n_ignored=300)
    print("[gpu] f16 all ignored", flush=True)
    got = run(synth.make_inputs(w))
    assert got["n_valid"] == 0
    assert np.all(got["loss"] == 0.0)
    assert np.all(got["dx"] == 0.0) and np.all(got["dW"] == 0.0) and np.all(got["db"] == 0.0)


def test_f16_accumulate_and_logit_scale():
    name = "c3_f16"
    inp = inputs(name)
    w = inp.w
    print("[gpu] f16 accumulate", flush=True)
    f, bw = oracle(name)
    x, W, b, t, g = device_inputs(inp)
    gen = torch.Generator(device="cpu").manual_seed(6)

    def prefill(ref, like):
        v = torch.randn(like.shape, generator=gen, dtype=torch.float64) * float(np.std(ref))
        return v.to(like.dtype).to(like.device)

    dx0, dW0, db0 = prefill(bw.dx, x), prefill(bw.dW, W), prefill(bw.db, b)
    out = (dx0.clone(), dW0.clone(), db0.clone())
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                    out=out, accumulate=True)
    torch.cuda.synchronize()
    tol = GRAD_RTOL["f16"]
    assert rel(to_f64(out[0]), to_f64(dx0) + bw.dx) <= tol
    assert rel(to_f64(out[1]), to_f64(dW0) + bw.dW) <= tol
    assert rel(to_f64(out[2]), to_f64(db0) + bw.db) <= tol
    # a logit scale multiplies the coefficients the slab scale is chosen from
    print("[gpu] f16 logit scale", flush=True)
    alpha = -1.3
    xs, Ws, bs = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    fr = O.forward(xs, Ws, bs, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                   logit_scale=alpha)
    br = O.backward(xs, Ws, bs, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                    w.reduction, logit_scale=alpha)
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                                   logit_scale=alpha)
    dx, dW, db = F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                 w.reduction, logit_scale=alpha)
    torch.cuda.synchronize()
    assert rel(loss.cpu().numpy().astype(np.float64), fr.loss) <= LOSS_RTOL
    assert rel(to_f64(dx), br.dx) <= tol and rel(to_f64(dW), br.dW) <= tol and rel(to_f64(db), br.db) <= tol


def test_f16_deterministic():
    inp = inputs("c3_f16")
    print("[gpu] f16 determinism", flush=True)
    a = run(inp, raw=True)
    b = run(inp, raw=True)
    for k in ("dx", "dW", "db"):
        assert torch.equal(a[k], b[k])
    assert np.array_equal(a["loss"], b["loss"]) and np.array_equal(a["lse"], b["lse"])
