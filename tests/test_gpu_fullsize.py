"""GPU parity at the full workload sizes, in the benchmarked launch configuration.

The oracle cannot afford the whole [N, V] problem here, so two checks are used
for each workload:

(a) the workload's own inputs: the GPU runs the full problem; the oracle
    recomputes sampled rows one by one (lse, the per-row loss of a
    reduction="none" run, the dx rows) and the reduced loss must equal the
    per-row losses summed (divided by the non-ignored count for mean);
(b) the same shapes with all but 16 rows ignored: every output is then a
    function of 16 rows, so the oracle checks loss, all of dx, all of db and
    sampled dW rows exactly (the launch grid and slab sequence are unchanged:
    ignored rows only get a zero coefficient).
"""

import numpy as np
import pytest
import torch

from lm_head_cross_flce_amd import synth
from oracle import flce_oracle as O

from flce_gpu_util import GRAD_RTOL, LOSS_RTOL, LSE_RTOL, device_inputs, rel, run, to_f64

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
N_SAMPLE = 12


@pytest.fixture(scope="module")
def cache():
    return {}


def _inputs(cache, name):
    if name not in cache:
        inp = synth.make_inputs(synth.WORKLOADS[name])
        cache.clear()  # keep one workload resident at a time
        cache[name] = (inp, inp.as_f64("W"), inp.as_f64("b"))
    return cache[name]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(cache, name):
    inp, W64, b64 = _inputs(cache, name)
    w = inp.w
    print(f"[gpu] full size {name}: GPU run", flush=True)
    dev = device_inputs(inp)
    got = run(inp, dev_inputs=dev, raw=True)
    got_none = got if w.reduction == "none" else run(inp, reduction="none", need=(False, False, False),
                                                     dev_inputs=dev)
    del dev
    torch.cuda.empty_cache()
    T = O.count_valid(inp.targets, w.ignore_index)
    assert got["n_valid"] == T
    # reduced loss equals the per-row losses of the same launch configuration
    if w.reduction == "mean":
        np.testing.assert_allclose(got["loss"][0], got_none["loss"].sum() / T, rtol=1e-5)
    rows = O.sample_rows(w.N, N_SAMPLE, seed=w.seed)
    print(f"[gpu] full size {name}: oracle on {rows.size} rows", flush=True)
    x_rows = _x_rows(inp, rows)
    g_rows = inp.grad[rows] if w.reduction == "none" else inp.grad
    r = O.rows(x_rows, W64, b64, inp.targets[rows], T, g_rows, w.label_smoothing, w.z_loss_scale,
               w.ignore_index, w.reduction)
    assert rel(got["lse"][rows], r["lse"]) <= LSE_RTOL
    assert rel(got_none["loss"][rows], r["row_loss"]) <= LOSS_RTOL
    rows_t = torch.from_numpy(rows).to(got["dx"].device)
    assert rel(to_f64(got["dx"][rows_t]), _out(r["dx"], w.dtype)) <= GRAD_RTOL[w.dtype]
    assert bool(torch.isfinite(got["dW"]).all()) and bool(torch.isfinite(got["dx"]).all())
    if got["db"] is not None:
        assert bool(torch.isfinite(got["db"]).all())


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
