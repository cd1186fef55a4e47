"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

The oracle is trusted for GPU parity only because these checks hold.  Each one
is independent of the oracle's own code: closed forms, invariants, central
finite differences, PyTorch's fp64 CPU cross entropy (used as a check only, for
the case it covers) and a separately written pure-Python brute force.  The last
section plants mistakes in a copy of the oracle and shows a pin catches each.
"""

import math

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import flce_oracle as O

RED = ("none", "sum", "mean")


def _rand_problem(rng, N, H, V, bias=True, n_ign=0, scale=1.0):
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * scale / math.sqrt(H)
    b = rng.standard_normal(V) * 0.3 if bias else None
    t = rng.integers(0, V, N)
    if n_ign:
        t[rng.choice(N, n_ign, replace=False)] = -100
    return x, W, b, t


def _grad(rng, red, N):
    return rng.standard_normal(N) if red == "none" else np.array([rng.standard_normal()])


def _scalar_objective(fwd, red, g):
    """sum_n g_n l_n for none, g * loss otherwise (its gradient is the backward's)."""
    if red == "none":
        return float(np.dot(g, fwd.loss))
    return float(g[0] * fwd.loss[0])


# --- P1: lse identity and shift invariance (PR 239 lse derivation) -----------

def test_p1_lse_equals_direct_logsumexp():
    rng = np.random.default_rng(1)
    x, W, b, t = _rand_problem(rng, 16, 12, 37)
    f = O.forward(x, W, b, t, reduction="none")
    z = x @ W.T + b
    direct = np.log(np.sum(np.exp(z), axis=1))
    np.testing.assert_allclose(f.lse, direct, rtol=1e-13, atol=1e-13)


def test_p1_lse_large_magnitude_stays_finite():
    # logits ~ +-1000: the direct formula overflows, m + log d does not.
    rng = np.random.default_rng(2)
    x, W, b, t = _rand_problem(rng, 4, 8, 9)
    f = O.forward(x * 1000.0, W, b, t, reduction="none")
    z = (x * 1000.0) @ W.T + b
    m = z.max(axis=1)
    np.testing.assert_allclose(f.lse, m + np.log(np.sum(np.exp(z - m[:, None]), axis=1)), rtol=1e-14)
    assert np.all(np.isfinite(f.lse))


@pytest.mark.parametrize("eps", [0.0, 0.2])
def test_p1_shift_invariance(eps):
    rng = np.random.default_rng(3)
    x, W, b, t = _rand_problem(rng, 10, 6, 15, n_ign=2)
    g = np.array([0.7])
    f0 = O.forward(x, W, b, t, eps=eps, reduction="sum")
    f1 = O.forward(x, W, b + 5.0, t, eps=eps, reduction="sum")
    np.testing.assert_allclose(f1.lse, f0.lse + 5.0, rtol=1e-13)
    np.testing.assert_allclose(f1.loss, f0.loss, rtol=1e-12)
    g0 = O.backward(x, W, b, t, g, eps=eps, reduction="sum")
    g1 = O.backward(x, W, b + 5.0, t, g, eps=eps, reduction="sum")
    np.testing.assert_allclose(g1.dx, g0.dx, atol=1e-12)
    np.testing.assert_allclose(g1.dW, g0.dW, atol=1e-12)
    np.testing.assert_allclose(g1.db, g0.db, atol=1e-12)


# --- P2: uniform logits give loss = log V (closed form, all terms) ------------

@pytest.mark.parametrize("eps,s,red", [(0.0, 0.0, "mean"), (0.1, 1e-2, "sum"),
                                       (0.05, 1e-4, "none"), (1.0, 0.5, "mean")])
def test_p2_uniform_logits_closed_form(eps, s, red):
    rng = np.random.default_rng(4)
    N, H, V, c = 7, 5, 13, 0.75
    x = rng.standard_normal((N, H))
    W = np.zeros((V, H))
    b = np.full(V, c)
    t = rng.integers(0, V, N)
    t[2] = -100
    g = _grad(rng, red, N)
    f = O.forward(x, W, b, t, eps=eps, s=s, reduction=red)
    lse = c + math.log(V)
    np.testing.assert_allclose(f.lse, lse, rtol=1e-14)
    valid = t != -100
    T = int(valid.sum())
    row = np.where(valid, math.log(V) + s * lse * lse, 0.0)
    expect = {"none": row, "sum": [row.sum()], "mean": [row.sum() / T]}[red]
    np.testing.assert_allclose(f.loss, expect, rtol=1e-13)
    bw = O.backward(x, W, b, t, g, eps=eps, s=s, reduction=red)
    cn = {"none": g, "sum": np.full(N, g[0]), "mean": np.full(N, g[0] / T)}[red] * valid
    dz = np.tile(((1 + 2 * s * lse) - eps) / V, (N, V))
    dz[np.arange(N)[valid], t[valid]] -= 1 - eps
    dz *= cn[:, None]
    np.testing.assert_allclose(bw.dx, 0.0, atol=1e-15)
    np.testing.assert_allclose(bw.dW, dz.T @ x, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(bw.db, dz.sum(0), rtol=1e-12, atol=1e-15)


# --- P3: softmax rows sum to one (PR 239, d lse / dz = softmax) ---------------

@pytest.mark.parametrize("s", [0.0, 1e-2])
def test_p3_dlogit_rows_sum(s):
    rng = np.random.default_rng(5)
    x, W, b, t = _rand_problem(rng, 9, 7, 21, n_ign=2)
    g = rng.standard_normal(9)
    r = O.rows(x, W, b, t, int((t != -100).sum()), g, eps=0.1, s=s, reduction="none")
    valid = t != -100
    cn = np.where(valid, g, 0.0)
    np.testing.assert_allclose(r["dz"].sum(axis=1), cn * 2 * s * r["lse"], atol=1e-14)
    bw = O.backward(x, W, b, t, g, eps=0.1, s=s, reduction="none")
    np.testing.assert_allclose(bw.db.sum(), np.sum(cn * 2 * s * r["lse"]), atol=1e-13)


# --- P4: ignored rows (fla kernel early exit; total counts non-ignored) -------

@pytest.mark.parametrize("red", RED)
def test_p4_ignored_rows_equal_deleted_rows(red):
    rng = np.random.default_rng(6)
    x, W, b, t = _rand_problem(rng, 12, 6, 17, n_ign=4)
    g = _grad(rng, red, 12)
    keep = t != -100
    f = O.forward(x, W, b, t, eps=0.1, s=1e-2, reduction=red)
    bw = O.backward(x, W, b, t, g, eps=0.1, s=1e-2, reduction=red)
    assert np.all(f.row_loss[~keep] == 0.0)
    assert np.all(bw.dx[~keep] == 0.0)
    gk = g[keep] if red == "none" else g
    fk = O.forward(x[keep], W, b, t[keep], eps=0.1, s=1e-2, reduction=red)
    bk = O.backward(x[keep], W, b, t[keep], gk, eps=0.1, s=1e-2, reduction=red)
    if red == "none":
        np.testing.assert_allclose(f.loss[keep], fk.loss, rtol=1e-13)
    else:
        np.testing.assert_allclose(f.loss, fk.loss, rtol=1e-13)
    np.testing.assert_allclose(bw.dW, bk.dW, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(bw.db, bk.db, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(bw.dx[keep], bk.dx, rtol=1e-12, atol=1e-15)


def test_p4_all_ignored_gives_zero():
    rng = np.random.default_rng(7)
    x, W, b, _ = _rand_problem(rng, 5, 4, 9)
    t = np.full(5, -100)
    for red in RED:
        f = O.forward(x, W, b, t, eps=0.1, s=1e-2, reduction=red)
        assert f.n_valid == 0 and np.all(f.loss == 0.0)
        bw = O.backward(x, W, b, t, _grad(rng, red, 5), eps=0.1, s=1e-2, reduction=red)
        assert np.all(bw.dx == 0) and np.all(bw.dW == 0) and np.all(bw.db == 0)


def test_p4_ignore_index_inside_vocab_wins():
    rng = np.random.default_rng(8)
    x, W, b, t = _rand_problem(rng, 6, 4, 9)
    t[1] = 3
    f = O.forward(x, W, b, t, ignore_index=3, reduction="none")
    assert f.row_loss[1] == 0.0 and f.n_valid == int(np.sum(t != 3))


def test_p4_out_of_range_target_raises():
    rng = np.random.default_rng(9)
    x, W, b, t = _rand_problem(rng, 4, 4, 9)
    t[0] = 9
    with pytest.raises(ValueError):
        O.forward(x, W, b, t)


# --- P5: reductions (fla kernel: mean divides loss and grads by total) --------

def test_p5_reduction_relations():
    rng = np.random.default_rng(10)
    x, W, b, t = _rand_problem(rng, 11, 5, 13, n_ign=3)
    T = int((t != -100).sum())
    fn = O.forward(x, W, b, t, eps=0.1, s=1e-2, reduction="none")
    fs = O.forward(x, W, b, t, eps=0.1, s=1e-2, reduction="sum")
    fm = O.forward(x, W, b, t, eps=0.1, s=1e-2, reduction="mean")
    np.testing.assert_allclose(fs.loss[0], fn.loss.sum(), rtol=1e-14)
    np.testing.assert_allclose(fm.loss[0], fs.loss[0] / T, rtol=1e-14)
    g = 1.7
    bm = O.backward(x, W, b, t, [g], eps=0.1, s=1e-2, reduction="mean")
    bs = O.backward(x, W, b, t, [g / T], eps=0.1, s=1e-2, reduction="sum")
    bn = O.backward(x, W, b, t, np.full(11, g / T), eps=0.1, s=1e-2, reduction="none")
    for a, c in ((bm, bs), (bs, bn)):
        np.testing.assert_allclose(a.dx, c.dx, rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(a.dW, c.dW, rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(a.db, c.db, rtol=1e-12, atol=1e-16)


# --- P6: textbook special case (PyTorch fp64 CPU cross entropy, s = 0) --------

@pytest.mark.parametrize("red", RED)
@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("bias", [True, False])
def test_p6_matches_torch_cross_entropy(red, eps, bias):
    rng = np.random.default_rng(11)
    N, H, V = 24, 16, 50
    x, W, b, t = _rand_problem(rng, N, H, V, bias=bias, n_ign=5, scale=3.0)
    g = _grad(rng, red, N)
    xt = torch.tensor(x, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True) if bias else None
    z = torch.nn.functional.linear(xt, Wt, bt)
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(t), ignore_index=-100,
                                             label_smoothing=eps, reduction=red)
    loss.backward(torch.tensor(g if red == "none" else g[0]))
    f = O.forward(x, W, b, t, eps=eps, reduction=red)
    bw = O.backward(x, W, b, t, g, eps=eps, reduction=red)
    np.testing.assert_allclose(f.loss.reshape(-1), loss.detach().numpy().reshape(-1), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bw.dx, xt.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(bw.dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-14)
    if bias:
        np.testing.assert_allclose(bw.db, bt.grad.numpy(), rtol=1e-10, atol=1e-14)


# --- P7: central finite differences (pins PR 239's z-loss and smoothing grads) -

@pytest.mark.parametrize("eps", [0.0, 0.1])
@pytest.mark.parametrize("s", [0.0, 1e-2])
@pytest.mark.parametrize("red", RED)
@pytest.mark.parametrize("bias", [True, False])
def test_p7_finite_differences(eps, s, red, bias):
    rng = np.random.default_rng(12)
    N, H, V = 5, 4, 7
    x, W, b, t = _rand_problem(rng, N, H, V, bias=bias, n_ign=1, scale=2.0)
    g = _grad(rng, red, N)
    bw = O.backward(x, W, b, t, g, eps=eps, s=s, reduction=red)

    def obj(xx, WW, bb):
        return _scalar_objective(O.forward(xx, WW, bb, t, eps=eps, s=s, reduction=red), red, g)

    h = 1e-5
    targets = [("x", x, bw.dx), ("W", W, bw.dW)] + ([("b", b, bw.db)] if bias else [])
    for name, arr, analytic in targets:
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            fp = obj(x, W, b)
            arr[idx] = old - h
            fm = obj(x, W, b)
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        err = np.linalg.norm(num - analytic) / max(np.linalg.norm(analytic), 1e-300)
        assert err < 1e-6, (name, err)


# --- P8: brute force agrees with the numpy oracle ----------------------------

@pytest.mark.parametrize("red", RED)
@pytest.mark.parametrize("bias", [True, False])
def test_p8_brute_force(red, bias):
    rng = np.random.default_rng(13)
    N, H, V = 6, 5, 11
    x, W, b, t = _rand_problem(rng, N, H, V, bias=bias, n_ign=2, scale=2.0)
    g = _grad(rng, red, N)
    eps, s = 0.1, 1e-2
    loss, lse, rl, dx, dW, db = brute.run(x.tolist(), W.tolist(), None if b is None else b.tolist(),
                                          t.tolist(), g.tolist(), eps, s, -100, red)
    f = O.forward(x, W, b, t, eps=eps, s=s, reduction=red)
    bw = O.backward(x, W, b, t, g, eps=eps, s=s, reduction=red)
    np.testing.assert_allclose(f.loss, loss, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f.lse, lse, rtol=1e-12)
    np.testing.assert_allclose(bw.dx, dx, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(bw.dW, dW, rtol=1e-12, atol=1e-13)
    if bias:
        np.testing.assert_allclose(bw.db, db, rtol=1e-12, atol=1e-13)


def test_rows_matches_full_oracle():
    rng = np.random.default_rng(14)
    x, W, b, t = _rand_problem(rng, 20, 8, 31, n_ign=3)
    g = rng.standard_normal(20)
    T = int((t != -100).sum())
    for red in RED:
        gg = g if red == "none" else g[:1]
        f = O.forward(x, W, b, t, eps=0.1, s=1e-2, reduction=red)
        bw = O.backward(x, W, b, t, gg, eps=0.1, s=1e-2, reduction=red)
        sel = np.array([0, 3, 19])
        r = O.rows(x[sel], W, b, t[sel], T, gg[sel] if red == "none" else gg, eps=0.1, s=1e-2, reduction=red)
        np.testing.assert_allclose(r["lse"], f.lse[sel], rtol=1e-14)
        np.testing.assert_allclose(r["row_loss"], f.row_loss[sel], rtol=1e-14)
        np.testing.assert_allclose(r["dx"], bw.dx[sel], rtol=1e-12, atol=1e-16)


@pytest.mark.parametrize("red", RED)
@pytest.mark.parametrize("bias", [True, False])
def test_dense_columns_matches_full_oracle_and_brute_force(red, bias):
    # The all-token check of large problems: lse, per-row loss, dx, all of db
    # and chosen dW rows, against the full oracle (rows per chunk smaller than
    # N, so several chunks are summed) and against the pure-loop brute force.
    rng = np.random.default_rng(16)
    N, H, V = 9, 6, 13
    x, W, b, t = _rand_problem(rng, N, H, V, bias=bias, n_ign=2, scale=2.0)
    g = _grad(rng, red, N)
    eps, s, alpha = 0.1, 1e-2, 1.3
    cols = np.array([0, 4, 12, int(t[t >= 0][0])])
    d = O.dense_columns(x, W, b, t, g, cols, eps=eps, s=s, reduction=red, rows_per_chunk=4, logit_scale=alpha)
    f = O.forward(x, W, b, t, eps=eps, s=s, reduction=red, logit_scale=alpha)
    bw = O.backward(x, W, b, t, g, eps=eps, s=s, reduction=red, logit_scale=alpha)
    assert d.n_valid == f.n_valid
    np.testing.assert_allclose(d.loss, f.loss, rtol=1e-13)
    np.testing.assert_allclose(d.lse, f.lse, rtol=1e-14)
    np.testing.assert_allclose(d.row_loss, f.row_loss, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(d.dx, bw.dx, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(d.dW_cols, bw.dW[cols], rtol=1e-12, atol=1e-16)
    loss, lse, rl, dx, dW, db = brute.run(x.tolist(), W.tolist(), None if b is None else b.tolist(), t.tolist(),
                                          g.tolist(), eps, s, -100, red, logit_scale=alpha)
    np.testing.assert_allclose(d.dW_cols, np.array(dW)[cols], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(d.dx, np.array(dx), rtol=1e-12, atol=1e-13)
    if bias:
        np.testing.assert_allclose(d.db, bw.db, rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(d.db, np.array(db), rtol=1e-12, atol=1e-13)
    # Without a bias db is still the dlogits' column sums: dW's rows against
    # a bias-free problem agree with the same sums formed by the brute force.
    else:
        _, _, _, _, _, db_b = brute.run(x.tolist(), W.tolist(), [0.0] * V, t.tolist(), g.tolist(), eps, s,
                                        -100, red, logit_scale=alpha)
        np.testing.assert_allclose(d.db, np.array(db_b), rtol=1e-12, atol=1e-13)
    d2 = O.dense_columns(x, W, b, t, g, cols, eps=eps, s=s, reduction=red, logit_scale=alpha, want_dx=False)
    assert d2.dx is None
    np.testing.assert_array_equal(d2.dW_cols, O.dense_columns(x, W, b, t, g, cols, eps=eps, s=s, reduction=red,
                                                              logit_scale=alpha).dW_cols)


def test_dense_columns_rejects_columns_outside_the_vocabulary():
    rng = np.random.default_rng(17)
    x, W, b, t = _rand_problem(rng, 4, 3, 5)
    with pytest.raises(ValueError):
        O.dense_columns(x, W, b, t, np.ones(1), [5])


# --- P9: scale sanity (not a pin): unit-variance logits give ~ log V + 1/2 ----

def test_p9_scale_sanity():
    rng = np.random.default_rng(15)
    N, H, V = 64, 256, 4000
    x = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) / math.sqrt(H)
    t = rng.integers(0, V, N)
    f = O.forward(x, W, None, t)
    assert abs(f.loss[0] - (math.log(V) + 0.5)) < 0.3


# --- Planted mistakes: each must be caught by a pin above ---------------------

def _fd_error(monkeypatch_target=None):
    rng = np.random.default_rng(16)
    N, H, V = 4, 3, 6
    x, W, b, t = _rand_problem(rng, N, H, V, n_ign=1, scale=2.0)
    g = np.array([0.9])
    eps, s = 0.1, 1e-2
    bw = O.backward(x, W, b, t, g, eps=eps, s=s, reduction="mean")
    h = 1e-5
    num = np.zeros_like(W)
    for idx in np.ndindex(W.shape):
        old = W[idx]
        W[idx] = old + h
        fp = O.forward(x, W, b, t, eps=eps, s=s).loss[0] * g[0]
        W[idx] = old - h
        fm = O.forward(x, W, b, t, eps=eps, s=s).loss[0] * g[0]
        W[idx] = old
        num[idx] = (fp - fm) / (2 * h)
    return np.linalg.norm(num - bw.dW) / np.linalg.norm(bw.dW)


def test_planted_mistakes_are_caught(monkeypatch):
    assert _fd_error() < 1e-6
    good_dlogits, good_row_loss, good_lse = O._dlogits, O._row_loss, O._lse

    # 1. sign of the eps/V term flipped (the garbled inline form on the PR page)
    def bad_sign(z, lse, t, valid, c, eps, s, V, scale=1.0):
        return good_dlogits(z, lse, t, valid, c, eps, s, V, scale) + 2 * scale * c[:, None] * eps / V
    monkeypatch.setattr(O, "_dlogits", bad_sign)
    assert _fd_error() > 1e-3
    monkeypatch.setattr(O, "_dlogits", good_dlogits)

    # 2. z-loss term dropped from the gradient
    def no_zloss_grad(z, lse, t, valid, c, eps, s, V, scale=1.0):
        return good_dlogits(z, lse, t, valid, c, eps, 0.0, V, scale)
    monkeypatch.setattr(O, "_dlogits", no_zloss_grad)
    assert _fd_error() > 1e-3
    monkeypatch.setattr(O, "_dlogits", good_dlogits)

    # 3. lse read literally as "m + d"
    def garbled_lse(z):
        m = np.max(z, axis=1)
        return m + np.sum(np.exp(z - m[:, None]), axis=1)
    monkeypatch.setattr(O, "_lse", garbled_lse)
    rng = np.random.default_rng(17)
    x, W, b, t = _rand_problem(rng, 6, 4, 9)
    z = x @ W.T + b
    assert not np.allclose(O.forward(x, W, b, t).lse, np.log(np.exp(z).sum(1)), rtol=1e-6)
    monkeypatch.setattr(O, "_lse", good_lse)

    # 4. smoothing weight on the wrong term of the loss
    def bad_loss(z, lse, t, valid, eps, s, V):
        return good_row_loss(z, lse, t, valid, 0.0, s, V)
    monkeypatch.setattr(O, "_row_loss", bad_loss)
    assert _fd_error() > 1e-3
    monkeypatch.setattr(O, "_row_loss", good_row_loss)


# --- logit_scale (fla cross_entropy_kernel; forward driver's scaled lse) -------

@pytest.mark.parametrize("alpha", [0.5, 2.5, -1.3])
@pytest.mark.parametrize("red", RED)
def test_logit_scale_equals_scaled_weights_chain_rule(alpha, red):
    # a (x W^T + b) = x (a W)^T + a b: the same loss; by the chain rule dx is
    # the same and the weight and bias gradients are a times those of (aW, ab).
    rng = np.random.default_rng(31)
    x, W, b, t = _rand_problem(rng, 9, 6, 14, n_ign=2)
    g = _grad(rng, red, 9)
    kw = dict(eps=0.1, s=1e-2, reduction=red)
    f1 = O.forward(x, W, b, t, logit_scale=alpha, **kw)
    f2 = O.forward(x, alpha * W, alpha * b, t, **kw)
    np.testing.assert_allclose(f1.loss, f2.loss, rtol=1e-12)
    np.testing.assert_allclose(f1.lse, f2.lse, rtol=1e-12)
    np.testing.assert_allclose(f1.z_loss, f2.z_loss, rtol=1e-12)
    b1 = O.backward(x, W, b, t, g, logit_scale=alpha, **kw)
    b2 = O.backward(x, alpha * W, alpha * b, t, g, **kw)
    np.testing.assert_allclose(b1.dx, b2.dx, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(b1.dW, alpha * b2.dW, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(b1.db, alpha * b2.db, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("alpha,eps,red", [(0.7, 0.0, "mean"), (3.0, 0.2, "sum"), (-0.4, 0.05, "none")])
def test_logit_scale_matches_torch_cross_entropy(alpha, eps, red):
    # PyTorch fp64 cross entropy of the scaled logits, with autograd gradients
    # (s = 0: torch has no z-loss).
    rng = np.random.default_rng(32)
    x, W, b, t = _rand_problem(rng, 8, 5, 11, n_ign=1)
    g = _grad(rng, red, 8)
    xt = torch.tensor(x, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    z = alpha * (xt @ Wt.T + bt)
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(t), ignore_index=-100, label_smoothing=eps,
                                             reduction=red)
    (loss * torch.tensor(g if red == "none" else g[0])).sum().backward()
    f = O.forward(x, W, b, t, eps=eps, reduction=red, logit_scale=alpha)
    bw = O.backward(x, W, b, t, g, eps=eps, reduction=red, logit_scale=alpha)
    np.testing.assert_allclose(f.loss, np.atleast_1d(loss.detach().numpy()), rtol=1e-12)
    np.testing.assert_allclose(bw.dx, xt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(bw.dW, Wt.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(bw.db, bt.grad.numpy(), rtol=1e-10, atol=1e-13)


def _fd_error_scaled(alpha=1.7):
    rng = np.random.default_rng(33)
    N, H, V = 4, 3, 6
    x, W, b, t = _rand_problem(rng, N, H, V, n_ign=1, scale=2.0)
    g = np.array([0.9])
    kw = dict(eps=0.1, s=1e-2, reduction="mean", logit_scale=alpha)
    bw = O.backward(x, W, b, t, g, **kw)
    h = 1e-5
    num_W = np.zeros_like(W)
    for idx in np.ndindex(W.shape):
        old = W[idx]
        W[idx] = old + h
        fp = O.forward(x, W, b, t, **kw).loss[0] * g[0]
        W[idx] = old - h
        fm = O.forward(x, W, b, t, **kw).loss[0] * g[0]
        W[idx] = old
        num_W[idx] = (fp - fm) / (2 * h)
    num_b = np.zeros_like(b)
    for j in range(V):
        old = b[j]
        b[j] = old + h
        fp = O.forward(x, W, b, t, **kw).loss[0] * g[0]
        b[j] = old - h
        fm = O.forward(x, W, b, t, **kw).loss[0] * g[0]
        b[j] = old
        num_b[j] = (fp - fm) / (2 * h)
    return max(np.max(np.abs(num_W - bw.dW)) / np.max(np.abs(num_W)),
               np.max(np.abs(num_b - bw.db)) / np.max(np.abs(num_b)))


def test_logit_scale_finite_differences():
    assert _fd_error_scaled() < 1e-6


def test_logit_scale_planted_mistake_is_caught(monkeypatch):
    good = O._dlogits

    def unscaled(z, lse, t, valid, c, eps, s, V, scale=1.0):   # forgets the scale on the gradient
        return good(z, lse, t, valid, c, eps, s, V, 1.0)
    monkeypatch.setattr(O, "_dlogits", unscaled)
    assert _fd_error_scaled() > 1e-3


def test_logit_scale_brute_force_agrees():
    rng = np.random.default_rng(34)
    x, W, b, t = _rand_problem(rng, 5, 4, 7, n_ign=1)
    g = np.array([1.3])
    loss, lse, rl, dx, dW, db = brute.run(x.tolist(), W.tolist(), b.tolist(), t.tolist(), g.tolist(), eps=0.1,
                                          s=1e-2, reduction="mean", logit_scale=-2.2)
    f = O.forward(x, W, b, t, eps=0.1, s=1e-2, reduction="mean", logit_scale=-2.2)
    bw = O.backward(x, W, b, t, g, eps=0.1, s=1e-2, reduction="mean", logit_scale=-2.2)
    np.testing.assert_allclose(f.loss, loss, rtol=1e-12)
    np.testing.assert_allclose(bw.dx, dx, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(bw.dW, dW, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(bw.db, db, rtol=1e-11, atol=1e-14)


# --- z-loss term reported alone (PR 239: L_total = L_ce + s lse^2) -------------

@pytest.mark.parametrize("red", RED)
def test_z_loss_term_alone(red):
    rng = np.random.default_rng(35)
    x, W, b, t = _rand_problem(rng, 10, 6, 13, n_ign=3)
    s = 3e-2
    f = O.forward(x, W, b, t, eps=0.1, s=s, reduction=red)
    f0 = O.forward(x, W, b, t, eps=0.1, s=0.0, reduction=red)
    # the CE part is unchanged: loss(s) - z_loss(s) = loss(s = 0)
    np.testing.assert_allclose(f.loss - f.z_loss, f0.loss, rtol=1e-12, atol=1e-14)
    lse = torch.logsumexp(torch.tensor(x @ W.T + b), dim=1).numpy()
    valid = t != -100
    rows = np.where(valid, s * lse * lse, 0.0)
    expect = {"none": rows, "sum": [rows.sum()], "mean": [rows.sum() / valid.sum()]}[red]
    np.testing.assert_allclose(f.z_loss, expect, rtol=1e-12)
