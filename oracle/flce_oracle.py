"""Fused linear cross entropy (FLCE): plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU path
and imports nothing from it.

It computes, slowly and obviously, what the fused GPU kernels compute quickly.
FLCE reaches exactly (up to rounding order) the result of the unfused
definition, so this oracle is that definition written out in fp64:

  logits          z[n, j] = sum_h x[n, h] W[j, h] + b[j]
                  (linear layer in nn.Linear layout: fla
                  fused_linear_cross_entropy.py, forward driver, the F.linear
                  call; weight is [vocab, hidden])
  log-sum-exp     m = max_j z, d = sum_j exp(z - m), lse = m + log d
                  (Liger-Kernel PR 239 "Support Z Loss in CE", the lse
                  derivation; the page prints "m + d", read as m + log d since
                  d is defined as the sum of exponentials)
  per-row loss    l = lse - (1 - eps) z_y - (eps / V) sum_j z_j + s lse^2
                  (fla cross_entropy_kernel: loss = lse - z_y, then the label
                  smoothing blend (1 - eps) H(q, p) + eps H(u, p); PR 239: total
                  loss = CE + lse_square_scale * lse^2)
  ignored rows    target == ignore_index gives l = 0 and zero gradient rows
                  (fla cross_entropy_kernel, the early exit on ignore_index)
  reduction       mean = sum l / T with T = number of non-ignored rows,
                  sum = sum l, none = the vector l
                  (fla forward driver: total = target.ne(ignore_index).sum();
                  DeepSpeed PR 8792 adds reduction "none")
  dlogits         dz[n, j] = c_n [ (1 + 2 s lse_n) p[n, j] - eps / V
                                   - (1 - eps) [j == y_n] ],  p = exp(z - lse)
                  c_n = g / T (mean), g (sum), g_n (none), 0 for ignored rows
                  (PR 239, the total derivative of CE plus z-loss; fla kernel
                  comments for the per-class form and the 1/total scaling)
  gradients       dx = dz W,  dW = dz^T x,  db_j = sum_n dz[n, j]
                  (fla forward driver: torch.mm(c_logits, weight),
                  c_logits.t() @ c_x, c_logits.sum(0))
  logit scale     with logit_scale a, every formula above applies to the
                  scaled logits a z (bias included), and the gradient of the
                  raw logits is a times the dlogits of the scaled ones
                  (fla forward driver: logsumexp_fwd(c_logits,
                  scale=logit_scale); cross_entropy_kernel: the loaded logits
                  and the target logit multiplied by logit_scale, and the
                  gradient (exp(z - lse) - eps) * logit_scale with the target
                  term (label_smoothing - 1) * logit_scale)
  z-loss term     s lse^2 of a row, reported alone as well (0 for ignored
                  rows), reduced like the loss

Readings where the pages are silent or garbled (each is also listed in the
design notes): all rows ignored gives loss 0 and zero gradients (the fla kernel
leaves every row at its zero init); an ignore_index inside [0, V) is treated as
ignored (the ignore test comes first); a non-ignored target outside [0, V) is
an error here; K in eps/K is V; the z-loss term is added per row and shares the
mean's 1/T; logits are never rounded (kept in fp64 here).

Inputs are arrays of any real dtype; everything is upcast to fp64 first (bf16
and fp32 widen exactly).  Memory is bounded by processing rows in chunks, so no
[N, V] array is ever held.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from contextlib import contextmanager
from dataclasses import dataclass
import os
from typing import Optional, Sequence

import numpy as np

try:
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover - optional: only affects speed
    threadpool_limits = None

REDUCTIONS = ("none", "sum", "mean")


@dataclass
class ForwardResult:
    loss: np.ndarray        # [N] for none, [1] otherwise
    lse: np.ndarray         # [N]
    row_loss: np.ndarray    # [N], zero for ignored rows
    n_valid: int
    z_loss: np.ndarray = None      # the z-loss term alone, reduced like loss
    row_z_loss: np.ndarray = None  # [N]


@dataclass
class BackwardResult:
    dx: np.ndarray          # [N, H]
    dW: np.ndarray          # [V, H]
    db: Optional[np.ndarray]  # [V] or None without bias


def _check(x, W, b, targets, eps, s, ignore_index, reduction):
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {REDUCTIONS}")
    if not (0.0 <= eps <= 1.0):
        raise ValueError("label smoothing must lie in [0, 1]")
    if s < 0.0:
        raise ValueError("z-loss scale must be >= 0")
    N, H = x.shape
    V, H2 = W.shape
    if H2 != H:
        raise ValueError("x and W disagree on the hidden size")
    if b is not None and b.shape != (V,):
        raise ValueError("bias must have shape [V]")
    t = np.asarray(targets).reshape(-1)
    if t.shape[0] != N:
        raise ValueError("targets must have one entry per row")
    valid = t != ignore_index
    bad = valid & ((t < 0) | (t >= V))
    if np.any(bad):
        raise ValueError("a non-ignored target lies outside [0, V)")
    return N, H, V, t.astype(np.int64), valid


def _logits(x64, W64, b64, scale=1.0):
    z = x64 @ W64.T
    if b64 is not None:
        z += b64[None, :]
    if scale != 1.0:
        z *= scale
    return z


def _lse(z):
    m = np.max(z, axis=1)
    d = np.sum(np.exp(z - m[:, None]), axis=1)
    return m + np.log(d)


def _row_loss(z, lse, t, valid, eps, s, V):
    rows = np.arange(z.shape[0])
    zy = np.where(valid, z[rows, np.where(valid, t, 0)], 0.0)
    l = lse - (1.0 - eps) * zy - (eps / V) * np.sum(z, axis=1) + s * lse * lse
    return np.where(valid, l, 0.0)


def _coeff(t_valid, grad, reduction, T, rows):
    """Upstream scale c_n for the given rows (0 for ignored rows)."""
    g = np.asarray(grad, dtype=np.float64).reshape(-1)
    if reduction == "none":
        c = g[rows]
    elif reduction == "sum":
        c = np.full(rows.shape[0], g[0])
    else:
        c = np.full(rows.shape[0], g[0] / T if T > 0 else 0.0)
    return np.where(t_valid, c, 0.0)


def _dlogits(z, lse, t, valid, c, eps, s, V, scale=1.0):
    """Gradient of the raw logits (before the logit scale), from the scaled z."""
    p = np.exp(z - lse[:, None])
    dz = (1.0 + 2.0 * s * lse)[:, None] * p - eps / V
    rows = np.arange(z.shape[0])
    tv = np.where(valid, t, 0)
    dz[rows, tv] -= np.where(valid, 1.0 - eps, 0.0)
    dz *= (c * scale)[:, None]
    return dz


def _reduce(rows_v, reduction, T):
    if reduction == "none":
        return rows_v.copy()
    if reduction == "sum":
        return np.array([np.sum(rows_v)])
    return np.array([np.sum(rows_v) / T if T > 0 else 0.0])


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _chunks(N, rows_per_chunk):
    return [(i, min(N, i + rows_per_chunk)) for i in range(0, N, rows_per_chunk)]


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


def _pool():
    return ThreadPoolExecutor(_workers())


@contextmanager
def _blas_per_chunk(nchunks):
    """While several row chunks run on the thread pool, each chunk's matrix
    products use one BLAS thread (the pool is the parallelism; BLAS pools
    inside every worker would oversubscribe the cores).  Execution only: the
    arithmetic is unchanged."""
    if nchunks > 1 and threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            yield
    else:
        yield


def forward(x, W, b, targets, eps=0.0, s=0.0, ignore_index=-100, reduction="mean",
            rows_per_chunk=256, logit_scale=1.0) -> ForwardResult:
    """Loss, per-row lse and the non-ignored count (and the z-loss term alone)."""
    N, H, V, t, valid = _check(x, W, b, targets, eps, s, ignore_index, reduction)
    W64, b64 = _f64(W), _f64(b)
    lse = np.empty(N)
    rl = np.empty(N)

    def work(c):
        lo, hi = c
        z = _logits(_f64(x[lo:hi]), W64, b64, logit_scale)
        lse[lo:hi] = _lse(z)
        rl[lo:hi] = _row_loss(z, lse[lo:hi], t[lo:hi], valid[lo:hi], eps, s, V)

    chunks = _chunks(N, rows_per_chunk)
    with _blas_per_chunk(len(chunks)), _pool() as ex:
        list(ex.map(work, chunks))
    T = int(np.sum(valid))
    rzl = np.where(valid, s * lse * lse, 0.0)
    return ForwardResult(_reduce(rl, reduction, T), lse, rl, T, _reduce(rzl, reduction, T), rzl)


def backward(x, W, b, targets, grad, eps=0.0, s=0.0, ignore_index=-100,
             reduction="mean", rows_per_chunk=256, logit_scale=1.0) -> BackwardResult:
    """dx, dW and db of the reduced loss, scaled by the upstream gradient."""
    N, H, V, t, valid = _check(x, W, b, targets, eps, s, ignore_index, reduction)
    W64, b64 = _f64(W), _f64(b)
    T = int(np.sum(valid))
    dx = np.empty((N, H))
    chunks = _chunks(N, rows_per_chunk)
    parts = [None] * len(chunks)

    def work(k):
        lo, hi = chunks[k]
        x64 = _f64(x[lo:hi])
        z = _logits(x64, W64, b64, logit_scale)
        lse = _lse(z)
        c = _coeff(valid[lo:hi], grad, reduction, T, np.arange(lo, hi))
        dz = _dlogits(z, lse, t[lo:hi], valid[lo:hi], c, eps, s, V, logit_scale)
        dx[lo:hi] = dz @ W64
        parts[k] = (dz.T @ x64, dz.sum(axis=0))

    dW = np.zeros((V, H))
    db = np.zeros(V)
    # Chunks run in parallel batches sized so their [V, H] partials stay under
    # ~2 GB; partials are added in chunk order.
    batch = max(1, min(_workers(), int(2e9 // (8 * V * H + 1))))
    with _blas_per_chunk(min(batch, len(chunks))), _pool() as ex:
        for k0 in range(0, len(chunks), batch):
            ks = range(k0, min(len(chunks), k0 + batch))
            list(ex.map(work, ks))
            for k in ks:
                pw, pb = parts[k]
                dW += pw
                db += pb
                parts[k] = None
    return BackwardResult(dx, dW, db if b is not None else None)


def rows(x_rows, W, b, targets_rows, T, grad_rows, eps=0.0, s=0.0, ignore_index=-100,
         reduction="mean", logit_scale=1.0):
    """Per-row outputs for a subset of rows, computed one row block at a time.

    ``T`` is the non-ignored count of the whole batch (it fixes the mean's
    scale); ``grad_rows`` holds the upstream gradient of these rows (none) or
    the scalar (sum/mean).  Returns lse, the per-row loss, the dlogits rows and
    the dx rows.  Used to check large problems on sampled rows.
    """
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {REDUCTIONS}")
    x64, W64, b64 = _f64(x_rows), _f64(W), _f64(b)
    V = W64.shape[0]
    t = np.asarray(targets_rows, dtype=np.int64).reshape(-1)
    valid = t != ignore_index
    if np.any(valid & ((t < 0) | (t >= V))):
        raise ValueError("a non-ignored target lies outside [0, V)")
    z = _logits(x64, W64, b64, logit_scale)
    lse = _lse(z)
    rl = _row_loss(z, lse, t, valid, eps, s, V)
    g = np.asarray(grad_rows, dtype=np.float64).reshape(-1)
    if reduction == "none":
        c = np.where(valid, g, 0.0)
    elif reduction == "sum":
        c = np.where(valid, g[0], 0.0)
    else:
        c = np.where(valid, g[0] / T if T > 0 else 0.0, 0.0)
    dz = _dlogits(z, lse, t, valid, c, eps, s, V, logit_scale)
    return {"lse": lse, "row_loss": rl, "dz": dz, "dx": dz @ W64}


@dataclass
class DenseColumnsResult:
    loss: np.ndarray        # reduced like the forward's loss
    lse: np.ndarray         # [N]
    row_loss: np.ndarray    # [N]
    n_valid: int
    db: np.ndarray          # [V]: sum over all rows of dz (formed with or without a bias)
    dW_cols: np.ndarray     # [len(cols), H]: rows ``cols`` of dW, summed over all N rows
    dx: Optional[np.ndarray]  # [N, H] if asked for


def dense_columns(x, W, b, targets, grad, cols, eps=0.0, s=0.0, ignore_index=-100, reduction="mean",
                  rows_per_chunk=256, logit_scale=1.0, want_dx=True) -> DenseColumnsResult:
    """Every token's lse, loss and dx row, all of db, and the dW rows ``cols``.

    The same definition as ``forward`` and ``backward`` (each row chunk holds
    its logits over the whole vocabulary, so its lse and its dlogits rows are
    complete), restricted to the outputs that a check of a large problem can
    afford: dW[j] = sum_n dz[n, j] x[n] only for j in ``cols``, so the cost
    is one logits product plus one dx product.  db_j = sum_n dz[n, j] and the
    dW rows sum the chunks' contributions in chunk order.
    """
    N, H, V, t, valid = _check(x, W, b, targets, eps, s, ignore_index, reduction)
    W64, b64 = _f64(W), _f64(b)
    cols = np.asarray(cols, dtype=np.int64).reshape(-1)
    if cols.size and (cols.min() < 0 or cols.max() >= V):
        raise ValueError("cols must lie in [0, V)")
    T = int(np.sum(valid))
    lse = np.empty(N)
    rl = np.empty(N)
    dx = np.empty((N, H)) if want_dx else None
    chunks = _chunks(N, rows_per_chunk)
    parts = [None] * len(chunks)

    def work(k):
        lo, hi = chunks[k]
        x64 = _f64(x[lo:hi])
        z = _logits(x64, W64, b64, logit_scale)
        lse[lo:hi] = _lse(z)
        rl[lo:hi] = _row_loss(z, lse[lo:hi], t[lo:hi], valid[lo:hi], eps, s, V)
        c = _coeff(valid[lo:hi], grad, reduction, T, np.arange(lo, hi))
        dz = _dlogits(z, lse[lo:hi], t[lo:hi], valid[lo:hi], c, eps, s, V, logit_scale)
        if want_dx:
            dx[lo:hi] = dz @ W64
        parts[k] = (dz.sum(axis=0), dz[:, cols].T @ x64)

    db = np.zeros(V)
    dWc = np.zeros((cols.size, H))
    with _blas_per_chunk(len(chunks)), _pool() as ex:
        list(ex.map(work, range(len(chunks))))
    for pb, pw in parts:
        db += pb
        dWc += pw
    return DenseColumnsResult(_reduce(rl, reduction, T), lse, rl, T, db, dWc, dx)


def count_valid(targets, ignore_index=-100) -> int:
    return int(np.sum(np.asarray(targets).reshape(-1) != ignore_index))


def loss_and_grads(x, W, b, targets, grad, eps=0.0, s=0.0, ignore_index=-100,
                   reduction="mean", rows_per_chunk=256, logit_scale=1.0):
    """Forward and backward in one pass over row chunks (the oracle timing leg)."""
    f = forward(x, W, b, targets, eps, s, ignore_index, reduction, rows_per_chunk, logit_scale)
    g = backward(x, W, b, targets, grad, eps, s, ignore_index, reduction, rows_per_chunk, logit_scale)
    return f, g


def sample_rows(N: int, k: int, seed: int = 0) -> np.ndarray:
    """k distinct row indices, always including the first and last row."""
    rng = np.random.default_rng(seed)
    k = min(k, N)
    picks = set([0, N - 1])
    while len(picks) < k:
        picks.add(int(rng.integers(0, N)))
    return np.array(sorted(picks), dtype=np.int64)


__all__: Sequence[str] = ("forward", "backward", "rows", "dense_columns", "count_valid", "loss_and_grads",
                          "sample_rows", "ForwardResult", "BackwardResult", "DenseColumnsResult", "REDUCTIONS")
