"""flce_forward_noalloc, through the C ABI, against flce_forward_ex.

The entry point runs the forward's kernels with their partials in the
library's static per-GPU scratch instead of a caller's workspace.  Two calls in
a row, the second with a smaller problem (and other options), must each give
exactly what flce_forward_ex gives for the same arguments (the same kernels
and the same fixed-order reductions, so bit-identical), and the first must
also meet the oracle bar.  Then the first problem again: the array holds the
second call's contents, which the forward overwrites before it reads them.
"""

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import _lib, synth
from oracle import flce_oracle as O

from flce_gpu_util import LOSS_RTOL, LSE_RTOL, device_inputs, rel

pytestmark = pytest.mark.gpu

_DT = {"bf16": _lib.FLCE_BF16, "f16": _lib.FLCE_F16, "f32": _lib.FLCE_F32}

BIG = synth.scaled(synth.WORKLOADS["n8192_h4096_v128256"], "noalloc_big", N=600, H=328, V=2083, n_ignored=30)
SMALL = synth.scaled(synth.WORKLOADS["n16384_h1024_v256000"], "noalloc_small", N=70, H=64, V=300, seed=21)


def _outputs(w, dev, want_zl):
    n = w.N if w.reduction == "none" else 1
    loss = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((w.N,), float("nan"), dtype=torch.float32, device=dev)
    nv = torch.full((1,), -1, dtype=torch.int64, device=dev)
    zl = torch.full((n,), float("nan"), dtype=torch.float32, device=dev) if want_zl else None
    return loss, lse, nv, zl


def _both(inp, logit_scale, want_zl, stream):
    """(noalloc outputs, workspace outputs) for the same arguments."""
    w = inp.w
    x, W, b, t, _ = device_inputs(inp)
    dev = x.device
    red = _lib.REDUCTIONS[w.reduction]
    args = (x.data_ptr(), W.data_ptr(), b.data_ptr() if b is not None else None, t.data_ptr(), w.N, w.H, w.V,
            _DT[w.dtype], w.label_smoothing, w.z_loss_scale, w.ignore_index, red)
    fwd_bytes, _ = _lib.flce_workspace_size(w.N, w.H, w.V, _DT[w.dtype], b is not None, red)
    assert fwd_bytes <= _lib.FORWARD_SCRATCH_BYTES
    ws = torch.empty(fwd_bytes, dtype=torch.uint8, device=dev)
    a = _outputs(w, dev, want_zl)
    r = _outputs(w, dev, want_zl)
    oa = _lib.options(logit_scale, False, a[3].data_ptr() if want_zl else None)
    orf = _lib.options(logit_scale, False, r[3].data_ptr() if want_zl else None)
    stream.wait_stream(torch.cuda.current_stream())   # inputs and outputs were written on the current stream
    with torch.cuda.stream(stream):
        print(f"[gpu] no-alloc forward {w.name}: N={w.N} H={w.H} V={w.V}", flush=True)
        _lib.flce_forward_noalloc(*args, oa, a[0].data_ptr(), a[1].data_ptr(), a[2].data_ptr(),
                                  stream.cuda_stream)
        _lib.flce_forward_ex(*args, orf, r[0].data_ptr(), r[1].data_ptr(), r[2].data_ptr(), ws.data_ptr(),
                             fwd_bytes, stream.cuda_stream)
    torch.cuda.synchronize()
    return a, r


def _same(a, r):
    for k, (u, v) in enumerate(zip(a, r)):
        if u is None:
            assert v is None
            continue
        assert torch.equal(u, v), (k, u[:4], v[:4])


def test_noalloc_forward_matches_the_workspace_entry_point():
    big, small = synth.make_inputs(BIG), synth.make_inputs(SMALL)
    stream = torch.cuda.Stream()
    a1, r1 = _both(big, 1.0, True, stream)
    _same(a1, r1)
    a2, r2 = _both(small, 0.75, False, torch.cuda.current_stream())
    _same(a2, r2)
    a3, _ = _both(big, 1.0, True, stream)
    _same(a3, r1)
    # the first problem also meets the oracle bar
    w = big.w
    f = O.forward(big.as_f64("x"), big.as_f64("W"), big.as_f64("b"), big.targets, w.label_smoothing,
                  w.z_loss_scale, w.ignore_index, w.reduction)
    assert int(a1[2].item()) == f.n_valid
    assert rel(a1[0].cpu().numpy().astype(np.float64), f.loss) <= LOSS_RTOL
    assert rel(a1[1].cpu().numpy().astype(np.float64), f.lse) <= LSE_RTOL
    assert rel(a1[3].cpu().numpy().astype(np.float64), f.z_loss) <= LOSS_RTOL

