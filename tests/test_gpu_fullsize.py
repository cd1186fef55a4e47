"""GPU parity at the full workload sizes, in the benchmarked launch configuration.

Two checks for each workload:

(a) the workload's own inputs, every token live as drawn: the GPU runs the
    full problem; the oracle makes one pass over row chunks that hold the
    logits over the whole vocabulary (one logits product and one dx product
    in fp64) and gives every token's lse, per-row loss and dx row, all of db,
    and ~60 chosen dW rows, each summed over all N tokens (the first rows,
    the ragged last tile, both sides of every backward slab boundary,
    frequent target rows, random rows).  Each is held to the Frobenius bar
    and to a per-row bound (ROW_FACTOR times the bar); the reduced loss must
    also equal the per-row losses summed (divided by the count for mean);
(b) the same shapes with all but 16 rows ignored: every output is then a
    function of 16 rows, so the oracle checks loss, all of dx, all of db and
    sampled dW rows exactly (the launch grid and slab sequence are unchanged:
    ignored rows only get a zero coefficient).
"""

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import _lib, synth
from oracle import flce_oracle as O

from flce_gpu_util import GRAD_RTOL, LOSS_RTOL, LSE_RTOL, check_close, device_inputs, rel, run, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

FULL = ["n4096_h2048_v32000", "n8192_h4096_v128256", "n32768_h2048_v128000", "n16384_h1024_v256000",
        "n8192_h4096_v128256_f16"]


def _out(ref, dtype):
    """The reference as the output dtype can hold it, for fp16.  With a mean
    over ~7800 rows and W ~ N(0, 1/H), |dx| is about 2e-6 at the Llama-3-sized
    head: subnormal in fp16 (spacing 6e-8), so rounding the exact result to
    fp16 alone costs about 1% (the reason fp16 training scales its loss).
    Compared with the rounded reference, the tolerance measures the kernels'
    own error.  bf16 and fp32 outputs have fp32's exponent range and are
    compared with the exact result."""
    return ref.astype(np.float16).astype(np.float64) if dtype == "f16" else ref


def _x_rows(inp, rows):
    """Exact fp64 copy of the chosen rows of x."""
    if inp.w.dtype == "bf16":
        return synth.bf16_bits_to_f64(inp.x[rows])
    return inp.x[rows].astype(np.float64)


@pytest.fixture(scope="module")
def cache():
    return {}


def _inputs(cache, name):
    if name not in cache:
        inp = synth.make_inputs(synth.WORKLOADS[name])
        cache.clear()  # keep one workload resident at a time
        cache[name] = (inp, inp.as_f64("W"), inp.as_f64("b"))
    return cache[name]


def _dense_cols(w, targets):
    """dW rows the dense check compares: the first rows and a tile boundary,
    the ragged last tile, both sides of every backward slab boundary, the
    most frequent and some other target rows, and random rows."""
    V = w.V
    code = {"bf16": _lib.FLCE_BF16, "f16": _lib.FLCE_F16, "f32": _lib.FLCE_F32}[w.dtype]
    slab = _lib.flce_backward_slab_cols(w.N, w.H, V, code)
    picks = [0, 1, 7, 8, 255, 256, V - 9, V - 8, V - 2, V - 1]
    for k in range(1, -(-V // slab)):
        picks += [k * slab - 1, k * slab]
    live = targets[targets != w.ignore_index]
    ids, counts = np.unique(live, return_counts=True)
    picks += list(ids[np.argsort(-counts, kind="stable")[:8]])
    picks += list(ids[O.sample_rows(ids.size, 8, seed=w.seed + 4)])
    picks += list(O.sample_rows(V, 32, seed=w.seed + 3))
    return np.unique(np.clip(np.array(picks, dtype=np.int64), 0, V - 1))


@pytest.mark.parametrize("name", FULL)
def test_full_size_dense(cache, name):
    # Every token live as drawn: all of lse, the per-row losses, all of dx and
    # db, and ~60 dW rows (each a sum over all N tokens) against the oracle.
    inp, W64, b64 = _inputs(cache, name)
    w = inp.w
    tol = GRAD_RTOL[w.dtype]
    print(f"[gpu] full size dense {name}: GPU run", flush=True)
    dev = device_inputs(inp)
    got = run(inp, dev_inputs=dev, raw=True)
    got_none = got if w.reduction == "none" else run(inp, reduction="none", need=(False, False, False),
                                                     dev_inputs=dev)
    T = O.count_valid(inp.targets, w.ignore_index)
    assert got["n_valid"] == T
    # the reduced loss equals the per-row losses of the same launch configuration
    if w.reduction == "mean":
        np.testing.assert_allclose(got["loss"][0], got_none["loss"].sum() / T, rtol=1e-5)
    cols = _dense_cols(w, inp.targets)
    dx = to_f64(got["dx"])
    dW = to_f64(got["dW"][torch.from_numpy(cols).to(got["dW"].device)])
    db = None if got["db"] is None else to_f64(got["db"])
    assert bool(torch.isfinite(got["dW"]).all())
    lse, row_loss, loss = got["lse"], got_none["loss"], got["loss"]
    del got, got_none, dev
    torch.cuda.empty_cache()
    print(f"[gpu] full size dense {name}: oracle, {cols.size} dW rows", flush=True)
    d = O.dense_columns(inp.as_f64("x"), W64, b64, inp.targets, inp.grad, cols, w.label_smoothing,
                        w.z_loss_scale, w.ignore_index, w.reduction)
    assert d.n_valid == T
    assert rel(loss, d.loss) <= LOSS_RTOL, (rel(loss, d.loss), loss[:4], d.loss[:4])
    check_close(lse, d.lse, LSE_RTOL, "lse")
    check_close(row_loss, d.row_loss, LOSS_RTOL, "per-row loss")
    check_close(dx, _out(d.dx, w.dtype), tol, "dx")
    check_close(dW, _out(d.dW_cols, w.dtype), tol, "dW rows")
    if db is not None:
        check_close(db, _out(d.db, w.dtype), tol, "db")
    if w.dtype == "f16":
        # Against the exact (unrounded) result: rounding to fp16 alone costs
        # ~9.5e-3 of dx at this shape, so the kernels' error adds little.
        print(f"  f16 against the exact result: dx {rel(dx, d.dx):.3e}, dW rows {rel(dW, d.dW_cols):.3e}",
              flush=True)
        assert rel(dx, d.dx) <= 2 * tol and rel(dW, d.dW_cols) <= 2 * tol


@pytest.mark.parametrize("name", FULL)
def test_full_size_sixteen_live_rows(cache, name):
    inp, W64, b64 = _inputs(cache, name)
    w = inp.w
    live = O.sample_rows(w.N, 16, seed=w.seed + 1)
    targets = np.full(w.N, w.ignore_index, dtype=np.int64)
    targets[live] = inp.targets[live]
    targets[live[targets[live] == w.ignore_index]] = 3   # every chosen row is live
    sparse = synth.Inputs(w, inp.x, inp.W, inp.b, targets, inp.grad)
    print(f"[gpu] full size {name}: 16 live rows, GPU run", flush=True)
    got = run(sparse, raw=True)
    print(f"[gpu] full size {name}: oracle", flush=True)
    x_live = _x_rows(inp, live)
    g = inp.grad[live] if w.reduction == "none" else inp.grad
    r = O.rows(x_live, W64, b64, targets[live], 16, g, w.label_smoothing, w.z_loss_scale, w.ignore_index,
               w.reduction)
    assert got["n_valid"] == 16
    if w.reduction == "none":
        ref_loss = np.zeros(w.N)
        ref_loss[live] = r["row_loss"]
    elif w.reduction == "sum":
        ref_loss = np.array([r["row_loss"].sum()])
    else:
        ref_loss = np.array([r["row_loss"].sum() / 16])
    assert rel(got["loss"], ref_loss) <= LOSS_RTOL
    dev = got["dx"].device
    live_t = torch.from_numpy(live).to(dev)
    assert rel(to_f64(got["dx"][live_t]), _out(r["dx"], w.dtype)) <= GRAD_RTOL[w.dtype]
    dead = torch.ones(w.N, dtype=torch.bool, device=dev)
    dead[live_t] = False
    assert bool((got["dx"][dead] == 0).all())
    if got["db"] is not None:
        assert rel(to_f64(got["db"]), _out(r["dz"].sum(axis=0), w.dtype)) <= GRAD_RTOL[w.dtype]
    vs = np.unique(np.concatenate([targets[live], O.sample_rows(w.V, 48, seed=w.seed + 2)]))
    dW_ref = r["dz"][:, vs].T @ x_live
    assert rel(to_f64(got["dW"][torch.from_numpy(vs).to(dev)]), _out(dW_ref, w.dtype)) <= GRAD_RTOL[w.dtype]
    del got
    torch.cuda.empty_cache()
