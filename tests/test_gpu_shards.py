"""GPU parity of the vocabulary-shard entry points against the full-vocabulary oracle.

W's rows are split into uneven shards (one of a few rows, one not aligned to a
256-row tile, one holding no target) that run one after another on one GPU:
flce_shard_forward per shard, flce_shard_merge of the stacked statistics, then
flce_shard_backward per shard with the fp32 dx partials summed into one buffer.
The merged loss, lse and count, the summed dx, and the concatenated dW and db
must meet the same bar as the unsharded path (the oracle is the plain
definition over all V rows).
"""

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
    "c5_small": synth.scaled(W_["n16384_h1024_v256000"], "c5_small", N=777, H=128, V=5003),
    "f32_none": synth.scaled(W_["tiny_f32"], "f32_none", N=300, H=136, V=1100, n_ignored=11, label_smoothing=0.1,
                             z_loss_scale=1e-3, reduction="none", grad="vector_normal", seed=8),
}


def splits(V, targets):
    """Uneven shard boundaries: a 7-row shard, tile-unaligned cuts, and one shard
    (found by search) that holds no target."""
    cuts = {0, V, 7, (3 * V) // 10, (3 * V) // 10 + 300, (3 * V) // 4}
    tset = set(int(t) for t in targets if 0 <= t < V)
    for a in range(V // 2, V - 3):
        if not any(a <= t < a + 3 for t in tset):
            cuts |= {a, a + 3}      # a 3-row shard without targets
            break
    c = sorted(x for x in cuts if 0 <= x <= V)
    return [(a, b) for a, b in zip(c[:-1], c[1:]) if b > a]


def run_shards(inp, order=None):
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    sh = splits(w.V, inp.targets)
    stats = [F.flce_shard_forward(x, W[a:e], None if b is None else b[a:e], t, a, w.V, w.label_smoothing,
                                  w.ignore_index) for a, e in sh]
    stack = torch.stack(stats if order is None else [stats[i] for i in order])
    loss, lse, nv = F.flce_shard_merge(stack, t, w.V, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                       w.reduction)
    dx = torch.empty(w.N, w.H, dtype=torch.float32, device=x.device)
    dWs, dbs = [], []
    for k, (a, e) in enumerate(sh):
        _, dW, db = F.flce_shard_backward(x, W[a:e], None if b is None else b[a:e], t, a, w.V, lse, nv, g,
                                          w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction,
                                          dx_partial=dx, accumulate_dx=k > 0)
        dWs.append(dW)
        dbs.append(db)
    torch.cuda.synchronize()
    return sh, {
        "loss": loss.cpu().numpy().astype(np.float64), "lse": lse.cpu().numpy().astype(np.float64),
        "n_valid": int(nv.cpu().item()), "dx": dx.cpu().numpy().astype(np.float64),
        "dW": to_f64(torch.cat(dWs)), "db": None if b is None else to_f64(torch.cat(dbs)),
    }


@pytest.mark.parametrize("name", list(CASES))
def test_shards_match_full_vocabulary_oracle(name):
    inp = synth.make_inputs(CASES[name])
    w = inp.w
    print(f"[gpu] vocabulary shards {name}", flush=True)
    sh, got = run_shards(inp)
    assert len(sh) >= 5 and min(e - a for a, e in sh) <= 7
    x, W, b = inp.as_f64("x"), inp.as_f64("W"), inp.as_f64("b")
    f = O.forward(x, W, b, inp.targets, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    bw = O.backward(x, W, b, inp.targets, inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    tol = GRAD_RTOL[w.dtype]
    assert got["n_valid"] == f.n_valid
    assert rel(got["loss"], f.loss) <= LOSS_RTOL
    assert rel(got["lse"], f.lse) <= LSE_RTOL
    assert rel(got["dx"], bw.dx) <= tol, ("dx", rel(got["dx"], bw.dx))
    assert rel(got["dW"], bw.dW) <= tol, ("dW", rel(got["dW"], bw.dW))
    if bw.db is not None:
        assert rel(got["db"], bw.db) <= tol, ("db", rel(got["db"], bw.db))


def test_merge_is_independent_of_shard_order():
    inp = synth.make_inputs(CASES["c3_small"])
    print("[gpu] shard order", flush=True)
    sh, a = run_shards(inp)
    _, b = run_shards(inp, order=list(reversed(range(len(sh)))))
    assert a["n_valid"] == b["n_valid"]
    assert rel(b["lse"], a["lse"]) <= 1e-6 and rel(b["loss"], a["loss"]) <= 1e-6
