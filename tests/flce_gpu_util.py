"""Helpers shared by the GPU parity tests: device transfer, runs, error norms."""

from __future__ import annotations

import numpy as np
import torch

from lm_head_cross_flce_amd import functional as F
from lm_head_cross_flce_amd import synth

# Tolerances of the parity bar: loss relative error, gradient relative
# Frobenius error by input dtype.
LOSS_RTOL = 1e-3
GRAD_RTOL = {"bf16": 1e-2, "f16": 1e-2, "f32": 1e-5}
LSE_RTOL = 1e-5
# Per-row (2-D outputs) and per-element (1-D outputs) bound, beside the
# Frobenius bar: each row's relative error may be at most ROW_FACTOR times
# the tensor's bar.  A row's error is a sum of the same independent rounding
# terms as the whole tensor's, so typical rows sit near the Frobenius figure;
# a wrong row (a wrong index, a missing or doubled term) errs by O(1).  Rows
# far smaller than the tensor's typical row are measured against
# ROW_FLOOR x the typical row norm instead, since their relative error is
# dominated by the rounding of their larger neighbours' shared terms.
ROW_FACTOR = 4.0
ROW_FLOOR = 0.1


def to_torch(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def device_inputs(inp: synth.Inputs, dev="cuda"):
    w = inp.w
    x = to_torch(inp.x, w.dtype, dev)
    W = to_torch(inp.W, w.dtype, dev)
    b = to_torch(inp.b, w.dtype, dev) if inp.b is not None else None
    t = torch.from_numpy(inp.targets).to(dev)
    g = torch.from_numpy(inp.grad).to(dev)
    return x, W, b, t, g


def run(inp: synth.Inputs, reduction=None, need=(True, True, True), dev_inputs=None, raw=False):
    """Forward + backward on the GPU; returns fp64 numpy results (device tensors for
    the gradients when ``raw``)."""
    w = inp.w
    red = reduction or w.reduction
    x, W, b, t, g = dev_inputs or device_inputs(inp)
    if red != w.reduction:
        g = (g.expand(w.N) if red == "none" else g[:1]).contiguous()
    loss, lse, nv = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, red)
    dx, dW, db = F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                 red, need_dx=need[0], need_dW=need[1], need_db=need[2])
    torch.cuda.synchronize()
    if raw:
        return {"loss": loss.cpu().numpy().astype(np.float64), "lse": lse.cpu().numpy().astype(np.float64),
                "n_valid": int(nv.cpu().item()), "dx": dx, "dW": dW, "db": db}
    return {
        "loss": loss.cpu().numpy().astype(np.float64),
        "lse": lse.cpu().numpy().astype(np.float64),
        "n_valid": int(nv.cpu().item()),
        "dx": None if dx is None else to_f64(dx),
        "dW": None if dW is None else to_f64(dW),
        "db": None if db is None else to_f64(db),
    }


def rel(a: np.ndarray, ref: np.ndarray) -> float:
    """Relative Frobenius error; exact zeros are required where ref is zero."""
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.all(np.asarray(a) == 0.0) else float("inf")
    return float(np.linalg.norm(np.asarray(a) - ref) / nr)


def row_rel_max(a: np.ndarray, ref: np.ndarray, floor: float = ROW_FLOOR) -> float:
    """Largest per-row relative error (per element for 1-D arrays), each row's
    reference norm floored at ``floor`` times the root-mean-square row norm.
    Where the whole reference is zero, exact zeros are required."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if a.shape != ref.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {ref.shape}")
    if ref.ndim == 1:
        a, ref = a[:, None], ref[:, None]
    err = np.linalg.norm(a - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    typical = float(np.sqrt(np.mean(nrm * nrm)))
    if typical == 0.0:
        return 0.0 if np.all(a == 0.0) else float("inf")
    return float(np.max(err / np.maximum(nrm, floor * typical)))


def check_close(a, ref, tol: float, what: str = "") -> None:
    """The parity bar: relative Frobenius error <= tol and every row within
    ROW_FACTOR * tol (see row_rel_max)."""
    e = rel(a, ref)
    r = row_rel_max(a, ref)
    print(f"  {what}: frobenius {e:.3e}, worst row {r:.3e}", flush=True)
    assert e <= tol, (what, "frobenius", e, tol)
    assert r <= ROW_FACTOR * tol, (what, "row", r, ROW_FACTOR * tol)
