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
    "c3_f16": synth.scaled(W_["n8192_h4096_v128256"], "c3_f16", N=600, H=328, V=2083, n_ignored=30, dtype="f16"),
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


@pytest.mark.timeout(900)
def test_full_size_eight_shards():
    # The benchmarked Llama-3-sized head in 8 shards of 16032 rows (not tile
    # aligned): lse, per-row losses and dx rows against the oracle on sampled
    # rows; lse against the unsharded forward; dW and db bit-identical to the
    # unsharded backward given the same lse (every dlogit is computed the same
    # way and db's partials are summed in the same order).
    name = "n8192_h4096_v128256"
    inp = synth.make_inputs(synth.WORKLOADS[name])
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    P = 8
    cuts = [k * w.V // P for k in range(P + 1)]
    print(f"[gpu] full size {name}: {P} shards", flush=True)
    stats = torch.stack([F.flce_shard_forward(x, W[a:e], b[a:e], t, a, w.V, w.label_smoothing, w.ignore_index)
                         for a, e in zip(cuts[:-1], cuts[1:])])
    loss, lse, nv = F.flce_shard_merge(stats, t, w.V, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                       w.reduction)
    loss_none, _, _ = F.flce_shard_merge(stats, t, w.V, w.label_smoothing, w.z_loss_scale, w.ignore_index, "none")
    dx = torch.empty(w.N, w.H, dtype=torch.float32, device=x.device)
    dWs, dbs = [], []
    for k, (a, e) in enumerate(zip(cuts[:-1], cuts[1:])):
        _, dW, db = F.flce_shard_backward(x, W[a:e], b[a:e], t, a, w.V, lse, nv, g, w.label_smoothing,
                                          w.z_loss_scale, w.ignore_index, w.reduction, dx_partial=dx,
                                          accumulate_dx=k > 0)
        dWs.append(dW)
        dbs.append(db)
    dW = torch.cat(dWs)
    db = torch.cat(dbs)
    del dWs, dbs, stats
    torch.cuda.synchronize()
    T = O.count_valid(inp.targets, w.ignore_index)
    assert int(nv.item()) == T
    np.testing.assert_allclose(loss.item(), loss_none.double().sum().item() / T, rtol=1e-5)
    print(f"[gpu] full size {name}: unsharded run", flush=True)
    _, ref_lse, _ = F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    assert rel(lse.double().cpu().numpy(), ref_lse.double().cpu().numpy()) <= 1e-6
    # the unsharded backward given the shards' merged lse: identical dlogits
    ref_dx, ref_dW, ref_db = F.flce_backward(x, W, b, t, lse, nv, g, w.label_smoothing, w.z_loss_scale,
                                             w.ignore_index, w.reduction)
    assert torch.equal(dW, ref_dW) and torch.equal(db, ref_db)
    assert rel(to_f64(dx.to(torch.bfloat16)), to_f64(ref_dx)) <= 1e-2
    del ref_dx, ref_dW, ref_db
    torch.cuda.empty_cache()
    rows = O.sample_rows(w.N, 12, seed=w.seed)
    print(f"[gpu] full size {name}: oracle on {rows.size} rows", flush=True)
    r = O.rows(synth.bf16_bits_to_f64(inp.x[rows]), inp.as_f64("W"), inp.as_f64("b"), inp.targets[rows], T,
               inp.grad, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    assert rel(lse.cpu().numpy().astype(np.float64)[rows], r["lse"]) <= LSE_RTOL
    assert rel(loss_none.cpu().numpy().astype(np.float64)[rows], r["row_loss"]) <= LOSS_RTOL
    assert rel(dx[torch.from_numpy(rows).to(dx.device)].cpu().numpy().astype(np.float64), r["dx"]) <= GRAD_RTOL["bf16"]
