"""GPU parity sweep: seeded random small problems against the fp64 CPU oracle.

Each case draws its shape and options from a fixed seed: N in [1, 700], H a
multiple of 8 in [8, 400], V in [1, 3000], bf16 / fp16 / fp32 inputs, bias on
or off, label smoothing, z-loss, any reduction, a random share of ignored
rows (all of them sometimes), a logit scale, and uniform or Zipf targets.
The shapes are ragged in every dimension, and most of them split the
input-gradient product along K (few output tiles) or run several vocabulary
slabs.  Every case runs through all three schedules: flce_forward +
flce_backward, the kept-slab pair (half of those cases with 512-column
slabs, so the kept slab is one of several), and the fused schedule in
256-token chunks.  Bar: loss relative error <= 1e-3 (relative 2-norm for reduction
none), lse <= 1e-5, gradients <= 1e-2 (bf16, fp16) or 1e-5 (fp32) relative
Frobenius error; exact zeros where the oracle's result is zero.  fp16
gradients are compared with the exact result rounded to fp16: with means over
hundreds of rows and logit scales below 1, some gradients here approach
half's subnormal range, where the output format alone costs up to about 1%.
"""

import math

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import functional as F
from lm_head_cross_flce_amd import synth
from oracle import flce_oracle as O

from flce_gpu_util import GRAD_RTOL, LOSS_RTOL, LSE_RTOL, device_inputs, rel, to_f64

pytestmark = pytest.mark.gpu

N_CASES = 120


def draw_case(k):
    rng = np.random.default_rng(1000 + k)
    N = int(rng.integers(1, 701))
    H = 8 * int(rng.integers(1, 51))
    V = int(rng.integers(1, 3001))
    dtype = ["bf16", "f16", "f32"][k % 3]
    red = ["mean", "sum", "none"][int(rng.integers(0, 3))]
    grad = {"mean": "scalar_normal", "sum": "scalar_normal", "none": "vector_normal"}[red]
    frac = [0.0, 0.05, 0.5, 1.0][int(rng.integers(0, 4))]
    w = synth.Workload(
        f"sweep{k}", N=N, H=H, V=V, dtype=dtype,
        b_std=math.sqrt(0.02) if rng.random() < 0.5 else None,
        targets="zipf" if rng.random() < 0.3 else "uniform",
        n_ignored=int(round(frac * N)),
        label_smoothing=[0.0, 0.1, 0.5][int(rng.integers(0, 3))],
        z_loss_scale=[0.0, 1e-4, 1e-2][int(rng.integers(0, 3))],
        reduction=red, grad=grad, seed=2000 + k)
    scale = [1.0, 1.0, 0.5, -1.3, 2.0][int(rng.integers(0, 5))]
    return w, scale


_oracle_cache = {}


def _oracle(k, inp, w, scale):
    if k not in _oracle_cache:
        _oracle_cache.clear()   # the schedules of one case run back to back
        x64, W64, b64 = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
        f = O.forward(x64, W64, b64, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                      logit_scale=scale)
        bw = O.backward(x64, W64, b64, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                        w.reduction, logit_scale=scale)
        _oracle_cache[k] = (f, bw)
    return _oracle_cache[k]


@pytest.mark.parametrize("schedule", ["recompute", "keep", "fused"])
@pytest.mark.parametrize("k", range(N_CASES))
def test_sweep(k, schedule, monkeypatch):
    # keep: the kept-slab pair (flce_forward_keep + flce_backward_kept); on
    # even cases with 512-column slabs, so the kept slab is one of several.
    # fused: flce_fused_forward_backward in chunks of 256 tokens.
    w, scale = draw_case(k)
    if schedule == "keep" and k % 2 == 0:
        monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")
    print(f"[gpu] sweep {k} {schedule}: N={w.N} H={w.H} V={w.V} {w.dtype} bias={w.b_std is not None} "
          f"eps={w.label_smoothing} s={w.z_loss_scale} {w.reduction} ignored={w.n_ignored} scale={scale}",
          flush=True)
    inp = synth.make_inputs(w)
    x, W, b, t, g = device_inputs(inp)
    if schedule == "fused":
        loss, lse, nv, dx, dW, db = F.flce_fused_forward_backward(x, W, b, t, g, w.label_smoothing, w.z_loss_scale,
                                                                  w.ignore_index, w.reduction, chunk_tokens=256,
                                                                  logit_scale=scale)
    elif schedule == "keep":
        loss, lse, nv, keep = F.flce_forward_keep(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                                  w.reduction, logit_scale=scale)
        dx, dW, db = F.flce_backward_kept(x, W, b, t, lse, nv, g, keep, w.label_smoothing, w.z_loss_scale,
                                          w.ignore_index, w.reduction, logit_scale=scale)
    else:
        loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                                       logit_scale=scale)
        dx, dW, db = F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                     w.reduction, logit_scale=scale)
    torch.cuda.synchronize()
    f, bw = _oracle(k, inp, w, scale)
    tol = GRAD_RTOL[w.dtype]
    assert int(nv.item()) == f.n_valid
    got_loss = loss.cpu().numpy().astype(np.float64)
    if np.all(f.loss == 0):
        assert np.all(got_loss == 0)
    else:
        assert rel(got_loss, f.loss) <= LOSS_RTOL, (rel(got_loss, f.loss), got_loss[:4], f.loss[:4])
    valid = inp.targets != w.ignore_index
    if valid.any():
        got_lse = lse.cpu().numpy().astype(np.float64)
        assert rel(got_lse[valid], f.lse[valid]) <= LSE_RTOL
    for name, got, ref in (("dx", dx, bw.dx), ("dW", dW, bw.dW), ("db", db, bw.db)):
        if ref is None:
            assert got is None
            continue
        g64 = to_f64(got)
        if w.dtype == "f16":
            ref = ref.astype(np.float16).astype(np.float64)
        if np.all(ref == 0):
            assert np.all(g64 == 0), name
        else:
            assert rel(g64, ref) <= tol, (name, rel(g64, ref))
    # ignored rows: exactly zero input gradient
    assert np.all(to_f64(dx)[~valid] == 0)
