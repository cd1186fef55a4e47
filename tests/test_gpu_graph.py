"""HIP graph capture of the entry points that take caller-owned buffers.

The library allocates nothing and never synchronises the host, so a caller
may capture its launches into a graph: here the benchmark's step (the
kept-slab forward and backward, with caller-owned workspaces and keep
buffer) and the no-allocation forward.  Each graph is replayed three times,
with eager work between the replays (the outputs are refilled with NaN), and
every replay must equal the eager result bit for bit.
"""

import pytest
import torch

from lm_head_cross_flce_amd import _lib
from lm_head_cross_flce_amd import functional as F

from flce_gpu_util import device_inputs
from test_gpu_parity import inputs

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up launch outside the capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def _replay_and_compare(graph, outs, ref):
    for i in range(3):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), (i, k)


def test_graph_of_the_kept_slab_step(monkeypatch):
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")   # several slabs, the first kept
    inp = inputs("c3_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    N, H, V = w.N, w.H, w.V
    dev = x.device
    red = _lib.REDUCTIONS[w.reduction]
    fb, kb, bb = F.flce_keep_workspace_size(N, H, V, x.dtype, True, w.reduction)
    ws_f = torch.empty(fb, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bb, dtype=torch.uint8, device=dev)
    keep = torch.empty(kb, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int64, device=dev)
    dx, dW, db = torch.empty_like(x), torch.empty_like(W), torch.empty_like(b)

    def step():
        s = torch.cuda.current_stream().cuda_stream
        _lib.flce_forward_keep(x.data_ptr(), W.data_ptr(), b.data_ptr(), t.data_ptr(), N, H, V, _lib.FLCE_BF16,
                               w.label_smoothing, w.z_loss_scale, w.ignore_index, red, None, loss.data_ptr(),
                               lse.data_ptr(), nv.data_ptr(), keep.data_ptr(), kb, ws_f.data_ptr(), fb, s)
        _lib.flce_backward_kept(x.data_ptr(), W.data_ptr(), b.data_ptr(), t.data_ptr(), N, H, V, _lib.FLCE_BF16,
                                w.label_smoothing, w.z_loss_scale, w.ignore_index, red, None, lse.data_ptr(),
                                nv.data_ptr(), g.data_ptr(), keep.data_ptr(), kb, dx.data_ptr(), dW.data_ptr(),
                                db.data_ptr(), ws_b.data_ptr(), bb, s)

    print("[gpu] graph: kept-slab step, eager", flush=True)
    step()
    torch.cuda.synchronize()
    outs = (loss, lse, nv, dx, dW, db)
    ref = tuple(o.clone() for o in outs)
    print("[gpu] graph: kept-slab step, capture and replays", flush=True)
    graph = _capture(step)
    _replay_and_compare(graph, outs, ref)


def test_graph_of_the_no_allocation_forward():
    inp = inputs("c3_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    N, H, V = w.N, w.H, w.V
    dev = x.device
    red = _lib.REDUCTIONS[w.reduction]
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int64, device=dev)

    def fwd():
        _lib.flce_forward_noalloc(x.data_ptr(), W.data_ptr(), b.data_ptr(), t.data_ptr(), N, H, V,
                                  _lib.FLCE_BF16, w.label_smoothing, w.z_loss_scale, w.ignore_index, red, None,
                                  loss.data_ptr(), lse.data_ptr(), nv.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)

    print("[gpu] graph: no-allocation forward, eager", flush=True)
    fwd()
    torch.cuda.synchronize()
    outs = (loss, lse, nv)
    ref = tuple(o.clone() for o in outs)
    print("[gpu] graph: no-allocation forward, capture and replays", flush=True)
    graph = _capture(fwd)
    _replay_and_compare(graph, outs, ref)
