"""GPU parity: the HIP library against the fp64 CPU oracle, element by element.

Sizes here let the oracle finish in seconds while spanning several 256-wide
tiles in every dimension plus ragged tails (N, V not multiples of 256; H not a
multiple of the 64-wide K stage).  The bar: loss relative error <= 1e-3 (for
reduction "none" the relative 2-norm over rows), dx/dW/db relative Frobenius
error <= 1e-2 for bf16 inputs and <= 1e-5 for fp32 inputs; exact zeros where
the oracle's result is zero.
"""

import os

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
    return synth.scaled(W_[base], name, **kw)


# Reduced-size versions of the five workloads (same distributions and options).
CASES = {
    "tiny_f32": W_["tiny_f32"],
    "c2_small": _case("n4096_h2048_v32000", "c2_small", N=520, H=256, V=3001),
    "c3_small": _case("n8192_h4096_v128256", "c3_small", N=600, H=328, V=2083, n_ignored=30),
    "c4_small": _case("n32768_h2048_v128000", "c4_small", N=1024, H=264, V=4000),
    "c5_small": _case("n16384_h1024_v256000", "c5_small", N=777, H=128, V=5003),
    "c5_whole": _case("n16384_h1024_v256000", "c5_whole", N=512, H=128, V=5003),
    # whole tiles in every dimension (N and V multiples of 256): the forward's, the kept-value forward's and the
    # recompute's instances without partial-tile code; with a bias (c3), and without one at a logit scale of 1
    # (c5, c2: the kept-value forward reads the logits straight from its accumulators)
    "c3_whole": _case("n8192_h4096_v128256", "c3_whole", N=512, H=256, V=2048, n_ignored=20),
    "c5_whole_unit": _case("n16384_h1024_v256000", "c5_whole_unit", N=512, H=128, V=2048),
    "c2_whole": _case("n4096_h2048_v32000", "c2_whole", N=256, H=256, V=1024),
    "sum_bias": _case("n8192_h4096_v128256", "sum_bias", N=300, H=200, V=1500, n_ignored=7,
                      reduction="sum", grad="scalar_normal", seed=7),
    "f32_none": _case("tiny_f32", "f32_none", N=300, H=136, V=1100, n_ignored=11, label_smoothing=0.1,
                      z_loss_scale=1e-3, reduction="none", grad="vector_normal", seed=8),
    "f32_sum_nobias": _case("tiny_f32", "f32_sum_nobias", N=129, H=64, V=777, b_std=None, n_ignored=0,
                            reduction="sum", grad="scalar_normal", seed=9),
    "n1_v1": _case("tiny_f32", "n1_v1", N=1, H=8, V=1, n_ignored=0, z_loss_scale=0.01, seed=10),
    "bf16_v_lt_tile": _case("n8192_h4096_v128256", "bf16_v_lt_tile", N=33, H=72, V=100, n_ignored=3, seed=11),
    # with 1024-column slabs the last slab has 6 columns: the second input-gradient K part is empty
    "f32_v1030": _case("tiny_f32", "f32_v1030", N=64, H=128, V=1030, seed=12),
    # H not a multiple of 8: the binding pads x and W with zero columns
    "bf16_h100": _case("n8192_h4096_v128256", "bf16_h100", N=130, H=100, V=700, n_ignored=5, seed=14),
    "f32_h13": _case("tiny_f32", "f32_h13", N=40, H=13, V=300, seed=15),
    # extreme aspect ratios: a million-row vocabulary (3907 vocabulary tiles over 256 phases of one token tile),
    # a hidden size past 8192 that is no multiple of the 64-deep K block or the 256-wide output tile, and
    # 20000 tokens (79 token tiles, the last 32 rows) against a tiny head
    "bf16_v1m": _case("n8192_h4096_v128256", "bf16_v1m", N=64, H=64, V=1_000_003, n_ignored=2, seed=16),
    "bf16_h8200": _case("n8192_h4096_v128256", "bf16_h8200", N=300, H=8200, V=1500, n_ignored=4, seed=17),
    "bf16_n20000": _case("n8192_h4096_v128256", "bf16_n20000", N=20000, H=64, V=700, n_ignored=100, seed=18),
    # fp32 inputs over several ragged tiles in every dimension (6 x 3 x 20), with bias, smoothing and z-loss
    "f32_mid": _case("tiny_f32", "f32_mid", N=1300, H=520, V=5003, n_ignored=40, label_smoothing=0.1,
                     z_loss_scale=1e-4, seed=19),
}

_oracle_cache = {}
_input_cache = {}


def inputs(name):
    if name not in _input_cache:
        _input_cache[name] = synth.make_inputs(CASES[name])
    return _input_cache[name]


def oracle(name, reduction=None):
    key = (name, reduction)
    if key not in _oracle_cache:
        inp = inputs(name)
        w = inp.w
        red = reduction or w.reduction
        g = inp.grad
        if red != w.reduction:
            g = np.full(w.N, g[0], dtype=np.float32) if red == "none" else g[:1]
        x, W, b = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
        f = O.forward(x, W, b, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, red)
        bw = O.backward(x, W, b, inp.targets, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, red)
        _oracle_cache[key] = (f, bw)
    return _oracle_cache[key]


def check(name, got, f, bw, need=(True, True, True)):
    w = CASES[name]
    tol = GRAD_RTOL[w.dtype]
    assert got["n_valid"] == f.n_valid
    assert rel(got["loss"], f.loss) <= LOSS_RTOL, (rel(got["loss"], f.loss), got["loss"][:4], f.loss[:4])
    assert rel(got["lse"], f.lse) <= LSE_RTOL, rel(got["lse"], f.lse)
    if need[0]:
        assert rel(got["dx"], bw.dx) <= tol, ("dx", rel(got["dx"], bw.dx))
    if need[1]:
        assert rel(got["dW"], bw.dW) <= tol, ("dW", rel(got["dW"], bw.dW))
    if need[2] and bw.db is not None:
        assert rel(got["db"], bw.db) <= tol, ("db", rel(got["db"], bw.db))


@pytest.mark.parametrize("name", list(CASES))
def test_parity(name):
    print(f"[gpu] parity case {name}", flush=True)
    got = run(inputs(name))
    f, bw = oracle(name)
    check(name, got, f, bw)


@pytest.mark.parametrize("red", ["none", "sum", "mean"])
def test_parity_all_reductions(red):
    print(f"[gpu] reductions c3_small {red}", flush=True)
    got = run(inputs("c3_small"), reduction=red)
    f, bw = oracle("c3_small", red)
    check("c3_small", got, f, bw)


@pytest.mark.parametrize("cols", ["256", "512", "1024"])
def test_forced_small_slabs(monkeypatch, cols):
    # Many vocabulary slabs: the fp32 dx accumulator carries across launches.
    # 1024 columns: these token counts give the input-gradient product too few
    # tiles for the GPU, so each slab's columns are split in two K parts (each
    # with its own accumulator, summed at the end); the last slabs of c3_small
    # and f32_v1030 leave the second part without columns.
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", cols)
    for name in ("c3_small", "c5_small", "f32_none") + (("f32_v1030",) if cols == "1024" else ()):
        print(f"[gpu] forced slabs {cols} {name}", flush=True)
        got = run(inputs(name))
        f, bw = oracle(name)
        check(name, got, f, bw)


@pytest.mark.parametrize("cols", ["512", "1024"])
@pytest.mark.parametrize("name", ["c4_small", "c5_whole"])
def test_whole_tile_slabs_then_a_ragged_one(monkeypatch, cols, name):
    # N a multiple of 256 and slabs of whole tiles: every slab but the last
    # (4000 or 5003 columns) runs the recompute instance without the
    # partial-tile masks and token checks, the last one the instance with them.
    # c4_small has a bias (db partials), c5_whole none.
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", cols)
    print(f"[gpu] whole-tile slabs {cols} {name}", flush=True)
    got = run(inputs(name))
    f, bw = oracle(name)
    check(name, got, f, bw)


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (True, True, False)])
def test_partial_gradients(need):
    print(f"[gpu] partial gradients {need}", flush=True)
    got = run(inputs("c3_small"), need=need)
    f, bw = oracle("c3_small")
    for k, flag in zip(("dx", "dW", "db"), need):
        assert (got[k] is None) == (not flag)
    check("c3_small", got, f, bw, need)


def test_all_ignored_gives_exact_zeros():
    w = _case("n8192_h4096_v128256", "all_ignored", N=300, H=64, V=700, n_ignored=300)
    inp = synth.make_inputs(w)
    print("[gpu] all ignored", flush=True)
    got = run(inp)
    assert got["n_valid"] == 0
    assert np.all(got["loss"] == 0.0)
    assert np.all(got["dx"] == 0.0) and np.all(got["dW"] == 0.0) and np.all(got["db"] == 0.0)
    got = run(inp, reduction="none")
    assert np.all(got["loss"] == 0.0)


def test_ignore_index_inside_vocabulary():
    w = _case("n8192_h4096_v128256", "ign5", N=260, H=64, V=300, n_ignored=0,
              ignore_index=5, seed=12)
    inp = synth.make_inputs(w)
    inp.targets[::7] = 5
    _input_cache["ign5"], CASES["ign5"] = inp, w
    print("[gpu] ignore_index 5", flush=True)
    got = run(inp)
    f, bw = oracle("ign5")
    assert f.n_valid == int(np.sum(inp.targets != 5))
    check("ign5", got, f, bw)


@pytest.mark.parametrize("dtype,b_mean", [("bf16", -120.0), ("f16", -20.0), ("f32", -105.0)])
def test_ragged_vocabulary_with_very_negative_lse(dtype, b_mean):
    # V = 1001 leaves a ragged last vocabulary tile, and a bias far below zero
    # puts lse near b_mean (softmax is shift-invariant, so the exact gradients
    # are ordinary).  The dlogits slab's padded vocabulary rows must hold
    # zeros: the input-gradient product reads the slab up to the next multiple
    # of 8 columns, where an unmasked c e^(-lse) overflows to inf and times
    # W's zero rows gives NaN (fp16's slab is scaled to ~2^13 per unit of c, so
    # lse ~ -13 suffices; fp32 arithmetic overflows past lse ~ -94 here).
    name = f"ragged_neg_lse_{dtype}"
    w = _case("n8192_h4096_v128256", name, dtype=dtype, N=300, H=136, V=1001, n_ignored=9,
              label_smoothing=0.0, z_loss_scale=0.0, b_std=0.1, b_mean=b_mean, seed=13)
    inp = synth.make_inputs(w)
    _input_cache[name], CASES[name] = inp, w
    print(f"[gpu] ragged vocabulary, lse ~ {b_mean}, {dtype}", flush=True)
    got = run(inp)
    f, bw = oracle(name)
    assert f.lse.max() < b_mean + 10.0
    for k in ("dx", "dW", "db"):
        assert np.all(np.isfinite(got[k])), k
    check(name, got, f, bw)


def test_deterministic():
    inp = inputs("c3_small")
    dev = device_inputs(inp)
    print("[gpu] determinism", flush=True)
    a = run(inp, dev_inputs=dev)
    b = run(inp, dev_inputs=dev)
    for k in ("loss", "lse", "dx", "dW", "db"):
        assert np.array_equal(a[k], b[k]), k


def test_autograd_module():
    inp = inputs("c3_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    x.requires_grad_(True)
    W.requires_grad_(True)
    b.requires_grad_(True)
    mod = F.FusedLinearCrossEntropyLoss(w.ignore_index, w.label_smoothing, w.z_loss_scale, "mean")
    print("[gpu] autograd module", flush=True)
    loss = mod(x.view(2, w.N // 2, w.H), t.view(2, -1), W, b)
    assert loss.shape == ()
    loss.backward(g.reshape(()))
    torch.cuda.synchronize()
    f, bw = oracle("c3_small")
    assert rel(np.array([loss.item()]), f.loss) <= LOSS_RTOL
    assert rel(to_f64(x.grad), bw.dx) <= GRAD_RTOL["bf16"]
    assert rel(to_f64(W.grad), bw.dW) <= GRAD_RTOL["bf16"]
    assert rel(to_f64(b.grad), bw.db) <= GRAD_RTOL["bf16"]


def test_module_frozen_weight_and_none_reduction():
    inp = inputs("c5_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    x.requires_grad_(True)
    print("[gpu] frozen weight, none", flush=True)
    loss = F.fused_linear_cross_entropy_loss(x, t, W, None, w.ignore_index, w.label_smoothing,
                                             w.z_loss_scale, "none")
    assert loss.shape == (w.N,)
    loss.backward(g)
    torch.cuda.synchronize()
    f, bw = oracle("c5_small")
    assert rel(loss.detach().cpu().numpy().astype(np.float64), f.loss) <= LOSS_RTOL
    assert rel(to_f64(x.grad), bw.dx) <= GRAD_RTOL["bf16"]
    assert W.grad is None


def _nan_guarded(a, extra_rows):
    """``a`` copied to the front of a buffer whose remaining ``extra_rows`` rows are NaN."""
    flat = a.reshape(-1)
    row = a.shape[1] if a.dim() == 2 else 1
    buf = torch.full((flat.numel() + extra_rows * row,), float("nan"), dtype=a.dtype, device=a.device)
    buf[: flat.numel()] = flat
    return buf[: flat.numel()].view(a.shape)


@pytest.mark.parametrize("name", ["sum_bias", "c3_small", "f32_none", "bf16_v_lt_tile"])
def test_no_reads_past_operands_or_of_unwritten_memory(name):
    # x, W and b end where NaN rows begin; the workspaces and the gradient
    # outputs start as NaN bytes.  A read past an operand's last row, or of
    # workspace or output memory that the library did not write first, would
    # carry NaN into the results.
    inp = inputs(name)
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    x, W = _nan_guarded(x, 300), _nan_guarded(W, 300)
    b = _nan_guarded(b, 300) if b is not None else None
    fb, bb = F.flce_workspace_size(w.N, w.H, w.V, x.dtype, b is not None, w.reduction)
    wsf = torch.full((max(fb, 1),), 0xFF, dtype=torch.uint8, device=x.device)
    wsb = torch.full((max(bb, 1),), 0xFF, dtype=torch.uint8, device=x.device)
    out = (torch.full_like(x, float("nan")), torch.full_like(W, float("nan")),
           torch.full_like(b, float("nan")) if b is not None else None)
    print(f"[gpu] NaN-guarded operands {name}", flush=True)
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                                   workspace=wsf)
    dx, dW, db = F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                 w.reduction, workspace=wsb, out=out)
    torch.cuda.synchronize()
    got = {"loss": loss.cpu().numpy().astype(np.float64), "lse": lse.cpu().numpy().astype(np.float64),
           "n_valid": int(nv.cpu().item()), "dx": to_f64(dx), "dW": to_f64(dW),
           "db": None if db is None else to_f64(db)}
    f, bw = oracle(name)
    check(name, got, f, bw)


def test_padded_hidden_size_with_accumulation():
    # H = 100: the padded gradients are sliced back, and accumulation adds to
    # the caller's unpadded buffers.
    inp = inputs("bf16_h100")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    print("[gpu] padded H with accumulation", flush=True)
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    f, bw = oracle("bf16_h100")
    # start from values of the gradients' own size (the exact ones, times -0.5, in bf16)
    base = tuple(torch.from_numpy(-0.5 * r).to(x.device).to(torch.bfloat16) for r in (bw.dx, bw.dW, bw.db))
    out = tuple(o.clone() for o in base)
    F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                    out=out, accumulate=True)
    torch.cuda.synchronize()
    for got, b0, ref, name in zip(out, base, (bw.dx, bw.dW, bw.db), ("dx", "dW", "db")):
        assert rel(to_f64(got), to_f64(b0) + ref) <= GRAD_RTOL["bf16"], name


def test_binding_rejects_bad_out_and_ctx_tensors():
    inp = inputs("c3_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    args = (x, W, b, t)
    opts = (w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    bad_outs = [
        (torch.empty(w.N - 1, w.H, dtype=x.dtype, device=x.device), None, None),          # too small
        (torch.empty(w.N, w.H, dtype=torch.float32, device=x.device), None, None),        # wrong dtype
        (None, torch.empty(w.H, w.V, dtype=x.dtype, device=x.device).t(), None),          # not contiguous
        (None, None, torch.empty(w.V + 1, dtype=x.dtype, device=x.device)),               # wrong length
    ]
    print("[gpu] binding argument checks", flush=True)
    for out in bad_outs:
        with pytest.raises(ValueError):
            F.flce_backward(*args, lse, nv, g, *opts, out=out)
    with pytest.raises(ValueError):
        F.flce_backward(*args, lse[:-1], nv, g, *opts)
    with pytest.raises(ValueError):
        F.flce_backward(*args, lse.double(), nv, g, *opts)
    with pytest.raises(ValueError):
        F.flce_backward(*args, lse, nv.int(), g, *opts)
    with pytest.raises(ValueError):
        F.flce_backward(*args, lse, nv, g, *opts, accumulate=True)
