"""GPU parity of the fused schedule (gradients formed while the forward runs,
one token chunk at a time) against the fp64 CPU oracle.

The schedule keeps each chunk's logits as e = exp(z - m_h) in the input dtype
between its logits product and its dlogits, and accumulates dW over the chunks
in dW's own dtype, so its rounding differs from the recompute schedule's; the
bar is the same: loss relative error <= 1e-3, gradients' relative Frobenius
error <= 1e-2 for bf16/fp16 and <= 1e-5 for fp32, each row within 4x the bar,
exact zeros where the oracle's result is zero.  Chunks of 256 tokens make
several chunks with a ragged last one at these sizes; chunk 0 is the default
(equal extra memory to the recompute schedule).
"""

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import functional as F
from lm_head_cross_flce_amd import synth
from oracle import flce_oracle as O

from flce_gpu_util import (GRAD_RTOL, LOSS_RTOL, LSE_RTOL, check_close, device_inputs, rel, row_rel_max,
                           ROW_FACTOR, to_f64)
from test_gpu_parity import CASES, inputs, oracle

pytestmark = pytest.mark.gpu

F16_CASE = synth.scaled(synth.WORKLOADS["n8192_h4096_v128256"], "c3_fused_f16", dtype="f16", N=600, H=328,
                        V=2083, n_ignored=30)


def run_fused(inp, chunk=0, reduction=None, need=(True, True, True), dev_inputs=None, **kw):
    w = inp.w
    red = reduction or w.reduction
    x, W, b, t, g = dev_inputs or device_inputs(inp)
    if red != w.reduction:
        g = (g.expand(w.N) if red == "none" else g[:1]).contiguous()
    res = F.flce_fused_forward_backward(x, W, b, t, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, red,
                                        need_dx=need[0], need_dW=need[1], need_db=need[2], chunk_tokens=chunk,
                                        **kw)
    torch.cuda.synchronize()
    loss, lse, nv, dx, dW, db = res[:6]
    out = {"loss": loss.cpu().numpy().astype(np.float64), "lse": lse.cpu().numpy().astype(np.float64),
           "n_valid": int(nv.cpu().item()), "dx": None if dx is None else to_f64(dx),
           "dW": None if dW is None else to_f64(dW), "db": None if db is None else to_f64(db)}
    if len(res) > 6:
        out["z_loss"] = res[6].cpu().numpy().astype(np.float64)
    return out


def check_fused(w, got, f, bw, need=(True, True, True)):
    tol = GRAD_RTOL[w.dtype]
    assert got["n_valid"] == f.n_valid
    assert rel(got["loss"], f.loss) <= LOSS_RTOL, (rel(got["loss"], f.loss), got["loss"][:4], f.loss[:4])
    assert rel(got["lse"], f.lse) <= LSE_RTOL, rel(got["lse"], f.lse)
    for k, ref, flag in (("dx", bw.dx, need[0]), ("dW", bw.dW, need[1]), ("db", bw.db, need[2])):
        if not flag or ref is None:
            continue
        assert rel(got[k], ref) <= tol, (k, rel(got[k], ref))
        assert row_rel_max(got[k], ref) <= ROW_FACTOR * tol, (k, row_rel_max(got[k], ref))


NAMES = ["tiny_f32", "c2_small", "c3_small", "c4_small", "c5_small", "sum_bias", "f32_none", "bf16_v_lt_tile",
         "f32_v1030", "c3_whole", "c5_whole_unit", "c2_whole"]


@pytest.mark.parametrize("chunk", [0, 256])
@pytest.mark.parametrize("name", NAMES)
def test_fused_parity(name, chunk):
    print(f"[gpu] fused {name} chunk {chunk}", flush=True)
    got = run_fused(inputs(name), chunk)
    f, bw = oracle(name)
    check_fused(CASES[name], got, f, bw)


@pytest.mark.parametrize("red", ["none", "sum", "mean"])
def test_fused_all_reductions(red):
    print(f"[gpu] fused reductions {red}", flush=True)
    got = run_fused(inputs("c3_small"), 256, reduction=red)
    f, bw = oracle("c3_small", red)
    check_fused(CASES["c3_small"], got, f, bw)


@pytest.mark.parametrize("chunk", [0, 256])
def test_fused_f16(chunk):
    inp = synth.make_inputs(F16_CASE)
    w = inp.w
    print(f"[gpu] fused f16 chunk {chunk}", flush=True)
    got = run_fused(inp, chunk)
    x, W, b = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    f = O.forward(x, W, b, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    bw = O.backward(x, W, b, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    check_fused(w, got, f, bw)


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True)])
def test_fused_partial_gradients(need):
    print(f"[gpu] fused partial gradients {need}", flush=True)
    got = run_fused(inputs("c3_small"), 256, need=need)
    f, bw = oracle("c3_small")
    for k, flag in zip(("dx", "dW", "db"), need):
        assert (got[k] is None) == (not flag)
    check_fused(CASES["c3_small"], got, f, bw, need)


def test_fused_options_scale_zloss_accumulate():
    # logit scale and the z-loss output against the oracle; accumulation into
    # buffers that hold gradient-sized values adds to them.
    inp = inputs("c3_small")
    w = inp.w
    alpha = 0.5
    x64, W64, b64 = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    f = O.forward(x64, W64, b64, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                  logit_scale=alpha)
    bw = O.backward(x64, W64, b64, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                    w.reduction, logit_scale=alpha)
    dev = device_inputs(inp)
    print("[gpu] fused options", flush=True)
    got = run_fused(inp, 256, dev_inputs=dev, logit_scale=alpha, return_z_loss=True)
    check_fused(w, got, f, bw)
    assert rel(got["z_loss"], f.z_loss) <= LOSS_RTOL
    base = tuple(torch.from_numpy(-0.5 * r).to(dev[0].device).to(torch.bfloat16) for r in (bw.dx, bw.dW, bw.db))
    out = tuple(o.clone() for o in base)
    x, W, b, t, g = dev
    F.flce_fused_forward_backward(x, W, b, t, g, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                                  chunk_tokens=256, out=out, accumulate=True, logit_scale=alpha)
    torch.cuda.synchronize()
    for got_t, b0, ref, name in zip(out, base, (bw.dx, bw.dW, bw.db), ("dx", "dW", "db")):
        assert rel(to_f64(got_t), to_f64(b0) + ref) <= GRAD_RTOL["bf16"], name


def test_fused_all_ignored_gives_exact_zeros():
    w = synth.scaled(synth.WORKLOADS["n8192_h4096_v128256"], "fused_all_ignored", N=300, H=64, V=700,
                     n_ignored=300)
    print("[gpu] fused all ignored", flush=True)
    got = run_fused(synth.make_inputs(w), 256)
    assert got["n_valid"] == 0 and np.all(got["loss"] == 0.0)
    assert np.all(got["dx"] == 0.0) and np.all(got["dW"] == 0.0) and np.all(got["db"] == 0.0)


def test_fused_deterministic():
    inp = inputs("c3_small")
    dev = device_inputs(inp)
    print("[gpu] fused determinism", flush=True)
    a = run_fused(inp, 256, dev_inputs=dev)
    b = run_fused(inp, 256, dev_inputs=dev)
    for k in ("loss", "lse", "dx", "dW", "db"):
        assert np.array_equal(a[k], b[k]), k


def test_fused_no_reads_past_operands_or_of_unwritten_memory():
    # As for the recompute schedule: operands end where NaN rows begin, the
    # workspace and the outputs start as NaN bytes.
    name = "c3_small"
    inp = inputs(name)
    w = inp.w
    x, W, b, t, g = device_inputs(inp)

    def guarded(a, extra):
        flat = a.reshape(-1)
        row = a.shape[1] if a.dim() == 2 else 1
        buf = torch.full((flat.numel() + extra * row,), float("nan"), dtype=a.dtype, device=a.device)
        buf[: flat.numel()] = flat
        return buf[: flat.numel()].view(a.shape)

    x, W, b = guarded(x, 300), guarded(W, 300), guarded(b, 300)
    nbytes, _ = F.flce_fused_workspace_size(w.N, w.H, w.V, x.dtype, True, 256)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=x.device)
    out = (torch.full_like(x, float("nan")), torch.full_like(W, float("nan")), torch.full_like(b, float("nan")))
    print("[gpu] fused NaN-guarded operands", flush=True)
    loss, lse, nv, dx, dW, db = F.flce_fused_forward_backward(x, W, b, t, g, w.label_smoothing, w.z_loss_scale,
                                                              w.ignore_index, w.reduction, chunk_tokens=256,
                                                              workspace=ws, out=out)
    torch.cuda.synchronize()
    got = {"loss": loss.cpu().numpy().astype(np.float64), "lse": lse.cpu().numpy().astype(np.float64),
           "n_valid": int(nv.cpu().item()), "dx": to_f64(dx), "dW": to_f64(dW), "db": to_f64(db)}
    f, bw = oracle(name)
    check_fused(w, got, f, bw)


FULL = ["n4096_h2048_v32000", "n8192_h4096_v128256", "n16384_h1024_v256000"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_fused_full_size_dense(name):
    # The default (equal-memory) chunking at full size: all of lse, the loss,
    # dx and db and ~50 dW rows against the oracle's dense pass.
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    tol = GRAD_RTOL[w.dtype]
    print(f"[gpu] fused full size {name}: GPU run", flush=True)
    dev = device_inputs(inp)
    x, W, b, t, g = dev
    loss, lse, nv, dx, dW, db = F.flce_fused_forward_backward(x, W, b, t, g, w.label_smoothing, w.z_loss_scale,
                                                              w.ignore_index, w.reduction)
    torch.cuda.synchronize()
    T = O.count_valid(inp.targets, w.ignore_index)
    assert int(nv.item()) == T
    cols = np.unique(np.concatenate([[0, 1, 255, 256, w.V - 1], O.sample_rows(w.V, 40, seed=w.seed + 5),
                                     inp.targets[inp.targets != w.ignore_index][:8]]))
    got_dx = to_f64(dx)
    got_dW = to_f64(dW[torch.from_numpy(cols).to(dW.device)])
    got_db = None if db is None else to_f64(db)
    got_loss, got_lse = loss.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    del dev, x, W, b, t, g, dx, dW, db
    torch.cuda.empty_cache()
    print(f"[gpu] fused full size {name}: oracle", flush=True)
    d = O.dense_columns(inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b"), inp.targets, inp.grad, cols,
                        w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    assert rel(got_loss, d.loss) <= LOSS_RTOL
    check_close(got_lse, d.lse, LSE_RTOL, "lse")
    check_close(got_dx, d.dx, tol, "dx")
    check_close(got_dW, d.dW_cols, tol, "dW rows")
    if got_db is not None:
        check_close(got_db, d.db, tol, "db")
