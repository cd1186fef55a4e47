"""GPU parity of the recompute schedule with the first vocabulary slab kept
(flce_forward_keep + flce_backward_kept) against the fp64 CPU oracle.

The forward keeps the first slab's logits as e = exp(z - m_h) in the input
dtype (the fused schedule's form); the backward turns them into that slab's
dlogits in place and recomputes only the other slabs.  At the reduced sizes
here the whole vocabulary fits in one slab unless FLCE_DEBUG_SLAB_COLS forces
narrower slabs (then the forward runs both of its launches and the backward
both kinds of slab).  The bar is the recompute schedule's: loss relative
error <= 1e-3, gradients' relative Frobenius error <= 1e-2 for bf16/fp16 and
<= 1e-5 for fp32, each row within 4x the bar, exact zeros where the oracle's
result is zero.
"""

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import functional as F
from lm_head_cross_flce_amd import synth
from oracle import flce_oracle as O

from flce_gpu_util import (GRAD_RTOL, LOSS_RTOL, LSE_RTOL, check_close, device_inputs, rel, row_rel_max,
                           ROW_FACTOR, to_f64)
from test_gpu_parity import CASES, _nan_guarded, inputs, oracle

pytestmark = pytest.mark.gpu


def run_keep(inp, reduction=None, need=(True, True, True), dev_inputs=None, keep=None, fwd_ws=None, bwd_ws=None,
             out=None, logit_scale=1.0, accumulate=False, return_z_loss=False):
    w = inp.w
    red = reduction or w.reduction
    x, W, b, t, g = dev_inputs or device_inputs(inp)
    if red != w.reduction:
        g = (g.expand(w.N) if red == "none" else g[:1]).contiguous()
    res = F.flce_forward_keep(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, red, workspace=fwd_ws,
                              logit_scale=logit_scale, return_z_loss=return_z_loss, keep=keep)
    loss, lse, nv, kb = res[:4]
    dx, dW, db = F.flce_backward_kept(x, W, b, t, lse, nv, g, kb, w.label_smoothing, w.z_loss_scale,
                                      w.ignore_index, red, need_dx=need[0], need_dW=need[1], need_db=need[2],
                                      workspace=bwd_ws, out=out, logit_scale=logit_scale, accumulate=accumulate)
    torch.cuda.synchronize()
    got = {"loss": loss.cpu().numpy().astype(np.float64), "lse": lse.cpu().numpy().astype(np.float64),
           "n_valid": int(nv.cpu().item()), "dx": None if dx is None else to_f64(dx),
           "dW": None if dW is None else to_f64(dW), "db": None if db is None else to_f64(db)}
    if return_z_loss:
        got["z_loss"] = res[4].cpu().numpy().astype(np.float64)
    return got


def check_keep(w, got, f, bw, need=(True, True, True)):
    tol = GRAD_RTOL[w.dtype]
    assert got["n_valid"] == f.n_valid
    assert rel(got["loss"], f.loss) <= LOSS_RTOL, (rel(got["loss"], f.loss), got["loss"][:4], f.loss[:4])
    assert rel(got["lse"], f.lse) <= LSE_RTOL, rel(got["lse"], f.lse)
    for k, ref, flag in (("dx", bw.dx, need[0]), ("dW", bw.dW, need[1]), ("db", bw.db, need[2])):
        if not flag or ref is None:
            continue
        assert rel(got[k], ref) <= tol, (k, rel(got[k], ref))
        assert row_rel_max(got[k], ref) <= ROW_FACTOR * tol, (k, row_rel_max(got[k], ref))


@pytest.mark.parametrize("name", list(CASES))
def test_keep_parity(name):
    print(f"[gpu] keep {name}", flush=True)
    got = run_keep(inputs(name))
    f, bw = oracle(name)
    check_keep(CASES[name], got, f, bw)


@pytest.mark.parametrize("cols", ["256", "512", "1024"])
def test_keep_forced_small_slabs(monkeypatch, cols):
    # The kept slab is one of several: the forward's plain launch covers the
    # rest of the vocabulary and the backward recomputes the other slabs into
    # the kept slab's buffer.  1024 columns split the dx product's K in two.
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", cols)
    for name in ("c3_small", "c5_small", "f32_none", "sum_bias") + (("f32_v1030",) if cols == "1024" else ()):
        print(f"[gpu] keep, slabs of {cols}: {name}", flush=True)
        got = run_keep(inputs(name))
        f, bw = oracle(name)
        check_keep(CASES[name], got, f, bw)


@pytest.mark.parametrize("name", ["c3_whole", "c5_whole_unit", "c2_whole"])
def test_keep_whole_tiles_several_slabs(monkeypatch, name):
    # N and V multiples of 256 with 512-column slabs: the kept-value forward on
    # the first 512 rows, the forward on the rest and the recompute all run
    # their whole-tile instances.
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")
    print(f"[gpu] keep, whole tiles, slabs of 512: {name}", flush=True)
    got = run_keep(inputs(name))
    f, bw = oracle(name)
    check_keep(CASES[name], got, f, bw)


def test_slab_cols_knob(monkeypatch):
    # The documented FLCE_SLAB_COLS narrows the slabs for both calls and the
    # workspace queries the binding makes: 256 columns give c3_small nine slabs,
    # the kept slab and dx accumulated in place over the other eight.
    monkeypatch.setenv("FLCE_SLAB_COLS", "256")
    print("[gpu] FLCE_SLAB_COLS=256 keep", flush=True)
    got = run_keep(inputs("c3_small"))
    f, bw = oracle("c3_small")
    check_keep(CASES["c3_small"], got, f, bw)


@pytest.mark.parametrize("red", ["none", "sum", "mean"])
def test_keep_all_reductions(red, monkeypatch):
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")
    print(f"[gpu] keep reductions {red}", flush=True)
    got = run_keep(inputs("c3_small"), reduction=red)
    f, bw = oracle("c3_small", red)
    check_keep(CASES["c3_small"], got, f, bw)


@pytest.mark.parametrize("cols", [None, "512"])
def test_keep_f16(cols, monkeypatch):
    if cols:
        monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", cols)
    w = synth.scaled(synth.WORKLOADS["n8192_h4096_v128256"], "c3_keep_f16", dtype="f16", N=600, H=328, V=2083,
                     n_ignored=30)
    inp = synth.make_inputs(w)
    print(f"[gpu] keep f16, slabs {cols}", flush=True)
    got = run_keep(inp)
    x, W, b = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    f = O.forward(x, W, b, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    bw = O.backward(x, W, b, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    check_keep(w, got, f, bw)


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True)])
def test_keep_partial_gradients(need, monkeypatch):
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")
    print(f"[gpu] keep partial gradients {need}", flush=True)
    got = run_keep(inputs("c3_small"), need=need)
    f, bw = oracle("c3_small")
    for k, flag in zip(("dx", "dW", "db"), need):
        assert (got[k] is None) == (not flag)
    check_keep(CASES["c3_small"], got, f, bw, need)


@pytest.mark.parametrize("dtype,b_mean", [("bf16", -120.0), ("f16", -20.0), ("f32", -105.0)])
def test_keep_ragged_vocabulary_with_very_negative_lse(dtype, b_mean):
    # As for the recompute: the kept slab's padded rows must hold zeros for the
    # dx product, which reads up to the next multiple of 8 columns.
    w = synth.scaled(synth.WORKLOADS["n8192_h4096_v128256"], f"keep_neg_lse_{dtype}", dtype=dtype, N=300, H=136,
                     V=1001, n_ignored=9, label_smoothing=0.0, z_loss_scale=0.0, b_std=0.1, b_mean=b_mean, seed=13)
    inp = synth.make_inputs(w)
    print(f"[gpu] keep ragged vocabulary, lse ~ {b_mean}, {dtype}", flush=True)
    got = run_keep(inp)
    x, W, b = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    f = O.forward(x, W, b, inp.targets, 0.0, 0.0, w.ignore_index, w.reduction)
    bw = O.backward(x, W, b, inp.targets, inp.grad, 0.0, 0.0, w.ignore_index, w.reduction)
    for k in ("dx", "dW", "db"):
        assert np.all(np.isfinite(got[k])), k
    check_keep(w, got, f, bw)


def test_keep_options_scale_zloss_accumulate(monkeypatch):
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")
    inp = inputs("c3_small")
    w = inp.w
    alpha = 0.5
    x64, W64, b64 = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    f = O.forward(x64, W64, b64, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                  logit_scale=alpha)
    bw = O.backward(x64, W64, b64, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                    w.reduction, logit_scale=alpha)
    dev = device_inputs(inp)
    print("[gpu] keep options", flush=True)
    got = run_keep(inp, dev_inputs=dev, logit_scale=alpha, return_z_loss=True)
    check_keep(w, got, f, bw)
    assert rel(got["z_loss"], f.z_loss) <= LOSS_RTOL
    base = tuple(torch.from_numpy(-0.5 * r).to(dev[0].device).to(torch.bfloat16) for r in (bw.dx, bw.dW, bw.db))
    out = tuple(o.clone() for o in base)
    run_keep(inp, dev_inputs=dev, out=out, logit_scale=alpha, accumulate=True)
    for got_t, b0, ref, name in zip(out, base, (bw.dx, bw.dW, bw.db), ("dx", "dW", "db")):
        assert rel(to_f64(got_t), to_f64(b0) + ref) <= GRAD_RTOL["bf16"], name


def test_keep_all_ignored_gives_exact_zeros():
    w = synth.scaled(synth.WORKLOADS["n8192_h4096_v128256"], "keep_all_ignored", N=300, H=64, V=700,
                     n_ignored=300)
    print("[gpu] keep all ignored", flush=True)
    got = run_keep(synth.make_inputs(w))
    assert got["n_valid"] == 0 and np.all(got["loss"] == 0.0)
    assert np.all(got["dx"] == 0.0) and np.all(got["dW"] == 0.0) and np.all(got["db"] == 0.0)


@pytest.mark.parametrize("cols", [None, "512"])
@pytest.mark.parametrize("name", ["c3_small", "f32_none", "bf16_v_lt_tile"])
def test_keep_no_reads_past_operands_or_of_unwritten_memory(name, cols, monkeypatch):
    # Operands end where NaN rows begin; the keep buffer, both workspaces and
    # the outputs start as NaN bytes.
    if cols:
        monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", cols)
    inp = inputs(name)
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    x, W = _nan_guarded(x, 300), _nan_guarded(W, 300)
    b = _nan_guarded(b, 300) if b is not None else None
    fb, kb, bb = F.flce_keep_workspace_size(w.N, w.H, w.V, x.dtype, b is not None, w.reduction)
    nan_bytes = lambda n: torch.full((max(n, 1),), 0xFF, dtype=torch.uint8, device=x.device)
    out = (torch.full_like(x, float("nan")), torch.full_like(W, float("nan")),
           torch.full_like(b, float("nan")) if b is not None else None)
    print(f"[gpu] keep NaN-guarded operands {name}, slabs {cols}", flush=True)
    got = run_keep(inp, dev_inputs=(x, W, b, t, g), keep=nan_bytes(kb), fwd_ws=nan_bytes(fb), bwd_ws=nan_bytes(bb),
                   out=out)
    f, bw = oracle(name)
    check_keep(w, got, f, bw)


def test_keep_deterministic():
    inp = inputs("c3_small")
    dev = device_inputs(inp)
    print("[gpu] keep determinism", flush=True)
    a = run_keep(inp, dev_inputs=dev)
    b = run_keep(inp, dev_inputs=dev)
    for k in ("loss", "lse", "dx", "dW", "db"):
        assert np.array_equal(a[k], b[k]), k


def test_keep_autograd_and_second_backward():
    # keep_first_slab: the first backward consumes the kept logits; a second
    # backward through the same graph recomputes every slab.
    inp = inputs("c3_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    for p in (x, W, b):
        p.requires_grad_(True)
    mod = F.FusedLinearCrossEntropyLoss(w.ignore_index, w.label_smoothing, w.z_loss_scale, "mean",
                                        keep_first_slab=True)
    print("[gpu] keep autograd", flush=True)
    loss = mod(x, t, W, b)
    loss.backward(g.reshape(()), retain_graph=True)
    torch.cuda.synchronize()
    f, bw = oracle("c3_small")
    assert rel(np.array([loss.item()]), f.loss) <= LOSS_RTOL
    grads = [to_f64(p.grad) for p in (x, W, b)]
    for gr, ref in zip(grads, (bw.dx, bw.dW, bw.db)):
        assert rel(gr, ref) <= GRAD_RTOL["bf16"]
    for p in (x, W, b):
        p.grad = None
    loss.backward(g.reshape(()))
    torch.cuda.synchronize()
    for p, ref in zip((x, W, b), (bw.dx, bw.dW, bw.db)):
        assert rel(to_f64(p.grad), ref) <= GRAD_RTOL["bf16"]


FULL = ["n4096_h2048_v32000", "n8192_h4096_v128256", "n32768_h2048_v128000", "n16384_h1024_v256000",
        "n8192_h4096_v128256_f16"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_keep_full_size_dense(name):
    # Full size with every row live, in the launch configuration the benchmark
    # times: all of lse, the loss, dx and db and ~50 dW rows against the
    # oracle's dense pass (rows 0 and 255 lie in the kept slab; the sampled
    # rows mostly in recomputed ones).  fp16 outputs are compared with the
    # exact result rounded to fp16, and held to twice the bar against the
    # exact result, as the recompute schedule's full-size check does.
    from test_gpu_fullsize import _out
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    tol = GRAD_RTOL[w.dtype]
    print(f"[gpu] keep full size {name}: GPU run", flush=True)
    x, W, b, t, g = device_inputs(inp)
    loss, lse, nv, keep = F.flce_forward_keep(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                              w.reduction)
    dx, dW, db = F.flce_backward_kept(x, W, b, t, lse, nv, g, keep, w.label_smoothing, w.z_loss_scale,
                                      w.ignore_index, w.reduction)
    torch.cuda.synchronize()
    T = O.count_valid(inp.targets, w.ignore_index)
    assert int(nv.item()) == T
    slab = F._lib.flce_backward_slab_cols(w.N, w.H, w.V, F._dtype_code(x))
    cols = np.unique(np.concatenate([[0, 1, 255, 256, min(slab, w.V) - 1, min(slab, w.V - 1), w.V - 1],
                                     O.sample_rows(w.V, 40, seed=w.seed + 5),
                                     inp.targets[inp.targets != w.ignore_index][:8]]))
    got_dx = to_f64(dx)
    got_dW = to_f64(dW[torch.from_numpy(cols).to(dW.device)])
    got_db = None if db is None else to_f64(db)
    got_loss, got_lse = loss.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    del x, W, b, t, g, dx, dW, db, keep
    torch.cuda.empty_cache()
    print(f"[gpu] keep full size {name}: oracle", flush=True)
    d = O.dense_columns(inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b"), inp.targets, inp.grad, cols,
                        w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    assert rel(got_loss, d.loss) <= LOSS_RTOL
    check_close(got_lse, d.lse, LSE_RTOL, "lse")
    check_close(got_dx, _out(d.dx, w.dtype), tol, "dx")
    check_close(got_dW, _out(d.dW_cols, w.dtype), tol, "dW rows")
    if got_db is not None:
        check_close(got_db, _out(d.db, w.dtype), tol, "db")
    if w.dtype == "f16":
        assert rel(got_dx, d.dx) <= 2 * tol and rel(got_dW, d.dW_cols) <= 2 * tol


@pytest.mark.timeout(600)
def test_keep_more_token_tiles_than_one_grid_dimension_holds():
    # 65537 token tiles of 256 (N = 16,777,472) with H = 8 and V = 300: the
    # in-place dlogits pass and every token-tiled launch take more blocks than
    # a second grid dimension allows (65535).  Reduction none makes each row's
    # loss, lse and dx a function of that row alone, so the oracle checks
    # sampled rows: the first and last tokens, both sides of tile boundaries
    # near the start, the middle and the 65535th/65536th tiles, and random rows.
    N = 65537 * 256
    w = synth.scaled(synth.WORKLOADS["n16384_h1024_v256000"], "keep_many_tiles", N=N, H=8, V=300)
    inp = synth.make_inputs(w)
    print(f"[gpu] keep with {N} tokens (65537 token tiles)", flush=True)
    x, W, b, t, g = device_inputs(inp)
    loss, lse, nv, keep = F.flce_forward_keep(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                              w.reduction)
    dx, dW, db = F.flce_backward_kept(x, W, b, t, lse, nv, g, keep, w.label_smoothing, w.z_loss_scale,
                                      w.ignore_index, w.reduction)
    torch.cuda.synchronize()
    assert int(nv.item()) == O.count_valid(inp.targets, w.ignore_index)
    assert bool(torch.isfinite(dW.float()).all())
    rows = np.unique(np.concatenate([
        [0, 1, 255, 256, 257, N // 2 - 1, N // 2, 65535 * 256 - 1, 65535 * 256, 65536 * 256 - 1, 65536 * 256,
         N - 2, N - 1], O.sample_rows(N, 40, seed=77)]))
    idx = torch.from_numpy(rows).to(x.device)
    got_loss = loss[idx].cpu().numpy().astype(np.float64)
    got_lse = lse[idx].cpu().numpy().astype(np.float64)
    got_dx = to_f64(dx[idx])
    del x, W, b, t, g, keep, dx, dW, db, loss, lse, nv
    torch.cuda.empty_cache()
    x64 = synth.bf16_bits_to_f64(inp.x[rows])
    W64 = inp.as_f64("W")
    f = O.forward(x64, W64, None, inp.targets[rows], w.label_smoothing, w.z_loss_scale, w.ignore_index, "none")
    bw = O.backward(x64, W64, None, inp.targets[rows], inp.grad[rows], w.label_smoothing, w.z_loss_scale,
                    w.ignore_index, "none")
    assert rel(got_loss, f.loss) <= LOSS_RTOL
    check_close(got_lse, f.lse, LSE_RTOL, "lse")
    check_close(got_dx, bw.dx, GRAD_RTOL["bf16"], "dx rows")
