"""Pure-Python brute force of fused linear cross entropy, for tiny shapes.

TEST INFRASTRUCTURE ONLY (used to cross-check the numpy oracle; nothing on the
GPU path may import it).

Plain loops over Python floats, following the same definitions as the numpy
oracle but written separately: the logits of the linear layer (fla
fused_linear_cross_entropy.py, F.linear in the forward driver), log-sum-exp
through the running max m and d = sum exp(z - m) (Liger-Kernel PR 239, lse
derivation, read as m + log d), the label-smoothed loss plus the z-loss term
(fla cross_entropy_kernel loss blend; PR 239 L_total = L_ce + s lse^2) and the
dlogits of PR 239's total derivative, contracted into dx, dW and db as in the
fla forward driver.  math.fsum keeps every sum correctly rounded.
"""

from __future__ import annotations

import math


def run(x, W, b, targets, grad, eps=0.0, s=0.0, ignore_index=-100, reduction="mean", logit_scale=1.0):
    """Returns (loss, lse, row_loss, dx, dW, db) as nested Python lists.  logit_scale
    multiplies every logit (bias included) and the gradient of the raw logits (fla
    cross_entropy_kernel)."""
    N = len(x)
    H = len(x[0])
    V = len(W)
    T = sum(1 for t in targets if t != ignore_index)
    lse_all, row_loss, dz_all = [], [], []
    for n in range(N):
        z = []
        for j in range(V):
            acc = math.fsum(float(x[n][h]) * float(W[j][h]) for h in range(H))
            if b is not None:
                acc += float(b[j])
            z.append(logit_scale * acc)
        m = max(z)
        d = math.fsum(math.exp(zj - m) for zj in z)
        lse = m + math.log(d)
        lse_all.append(lse)
        y = targets[n]
        if y == ignore_index:
            row_loss.append(0.0)
            dz_all.append([0.0] * V)
            continue
        ce = lse - z[y]
        smooth = lse - math.fsum(z) / V          # cross entropy against uniform
        loss_n = (1.0 - eps) * ce + eps * smooth + s * lse * lse
        row_loss.append(loss_n)
        if reduction == "none":
            c = float(grad[n])
        elif reduction == "sum":
            c = float(grad[0])
        else:
            c = float(grad[0]) / T
        row = []
        for j in range(V):
            p = math.exp(z[j] - lse)
            g = (1.0 + 2.0 * s * lse) * p - eps / V
            if j == y:
                g -= 1.0 - eps
            row.append(c * logit_scale * g)
        dz_all.append(row)
    if reduction == "none":
        loss = list(row_loss)
    elif reduction == "sum":
        loss = [math.fsum(row_loss)]
    else:
        loss = [math.fsum(row_loss) / T if T else 0.0]
    dx = [[math.fsum(dz_all[n][j] * float(W[j][h]) for j in range(V)) for h in range(H)]
          for n in range(N)]
    dW = [[math.fsum(dz_all[n][j] * float(x[n][h]) for n in range(N)) for h in range(H)]
          for j in range(V)]
    db = [math.fsum(dz_all[n][j] for n in range(N)) for j in range(V)] if b is not None else None
    return loss, lse_all, row_loss, dx, dW, db
