"""PyTorch-facing binding of the FLCE library.

PyTorch supplies device memory and the current stream; every step of the
computation runs in libflce.so.  ``flce_forward`` / ``flce_backward`` take
tensors and mirror the C entry points of the same names; the autograd function
and module wrap them the way fla's FusedLinearCrossEntropyLoss wraps its
kernels (fla/modules/fused_linear_cross_entropy.py: the module flattens
[batch, seq, hidden] to [tokens, hidden]), with reduction "none" added and the
gradients produced in backward rather than in forward (DeepSpeed PR 8792).
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.FLCE_BF16, torch.float16: _lib.FLCE_F16, torch.float32: _lib.FLCE_F32}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16, float16 or float32")
    return _DTYPES[t.dtype]


def _reduction_code(reduction: str) -> int:
    if reduction not in _lib.REDUCTIONS:
        raise ValueError(f"reduction must be one of {tuple(_lib.REDUCTIONS)}")
    return _lib.REDUCTIONS[reduction]


def _prep(x, W, b, targets):
    if x.dim() != 2 or W.dim() != 2:
        raise ValueError("x must be [N, H] and W must be [V, H]")
    if not x.is_cuda:
        raise ValueError("tensors must live on a GPU")
    if W.shape[1] != x.shape[1]:
        raise ValueError("x and W disagree on the hidden size")
    if W.dtype != x.dtype or (b is not None and b.dtype != x.dtype):
        raise TypeError("x, W and b must share one dtype")
    if W.device != x.device or targets.device != x.device or (b is not None and b.device != x.device):
        raise ValueError("x, W, b and targets must be on one device")
    if b is not None and b.shape != (W.shape[0],):
        raise ValueError("b must be [V]")
    x = _pad_hidden(x.contiguous())
    W = _pad_hidden(W.contiguous())
    b = b.contiguous() if b is not None else None
    targets = targets.reshape(-1).to(torch.int64).contiguous()
    if targets.numel() != x.shape[0]:
        raise ValueError("targets must have one entry per row of x")
    return x, W, b, targets


def _pad_hidden(t: torch.Tensor) -> torch.Tensor:
    """The library moves rows in 16-byte pieces and needs H % 8 == 0: other H
    get zero columns up to the next multiple of 8 (a copy), which changes no
    logit, loss or gradient entry of the original columns."""
    H = t.shape[1]
    if H % 8 == 0:
        return t
    out = torch.zeros(t.shape[0], H + (-H) % 8, dtype=t.dtype, device=t.device)
    out[:, :H] = t
    return out


def _check_out(t: Optional[torch.Tensor], shape, like: torch.Tensor, what: str) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != like.dtype or t.device != like.device or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {like.dtype} tensor of shape {tuple(shape)} on {like.device}")


def _check_ctx(lse: torch.Tensor, n_valid: torch.Tensor, N: int, dev) -> None:
    if lse.dtype != torch.float32 or tuple(lse.shape) != (N,) or not lse.is_contiguous() or lse.device != dev:
        raise ValueError(f"lse must be a contiguous float32 [{N}] tensor on {dev} (as flce_forward returns it)")
    if n_valid.dtype != torch.int64 or n_valid.numel() != 1 or n_valid.device != dev:
        raise ValueError(f"n_valid must be an int64 [1] tensor on {dev} (as flce_forward returns it)")


def flce_workspace_size(N: int, H: int, V: int, dtype: torch.dtype, has_bias: bool,
                        reduction: str = "mean") -> Tuple[int, int]:
    return _lib.flce_workspace_size(N, H, V, _DTYPES[dtype], has_bias, _reduction_code(reduction))


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def flce_keep_workspace_size(N: int, H: int, V: int, dtype: torch.dtype, has_bias: bool,
                             reduction: str = "mean") -> Tuple[int, int, int]:
    """(forward bytes, keep bytes, backward bytes) of flce_forward_keep + flce_backward_kept."""
    return _lib.flce_keep_workspace_size(N, H, V, _DTYPES[dtype], has_bias, _reduction_code(reduction))


def flce_forward(x: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor], targets: torch.Tensor,
                 label_smoothing: float = 0.0, z_loss_scale: float = 0.0, ignore_index: int = -100,
                 reduction: str = "mean", workspace: Optional[torch.Tensor] = None, logit_scale: float = 1.0,
                 return_z_loss: bool = False):
    """Returns (loss, lse, n_valid): loss float32 [1] (sum/mean) or [N] (none); with
    return_z_loss, (loss, lse, n_valid, z_loss), z_loss the s * lse^2 term alone,
    shaped like loss.  The logits are logit_scale * (x W^T + b)."""
    return _forward(x, W, b, targets, label_smoothing, z_loss_scale, ignore_index, reduction, workspace,
                    logit_scale, return_z_loss, None)


def flce_forward_keep(x: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor], targets: torch.Tensor,
                      label_smoothing: float = 0.0, z_loss_scale: float = 0.0, ignore_index: int = -100,
                      reduction: str = "mean", workspace: Optional[torch.Tensor] = None, logit_scale: float = 1.0,
                      return_z_loss: bool = False, keep: Optional[torch.Tensor] = None):
    """flce_forward that also keeps the first vocabulary slab's logits for
    flce_backward_kept: returns (loss, lse, n_valid, keep) (with return_z_loss,
    z_loss last).  keep: a uint8 device buffer of at least the keep bytes of
    flce_keep_workspace_size to fill (allocated when None)."""
    return _forward(x, W, b, targets, label_smoothing, z_loss_scale, ignore_index, reduction, workspace,
                    logit_scale, return_z_loss, keep if keep is not None else True)


def _forward(x, W, b, targets, label_smoothing, z_loss_scale, ignore_index, reduction, workspace, logit_scale,
             return_z_loss, keep):
    x, W, b, targets = _prep(x, W, b, targets)
    N, H = x.shape
    V = W.shape[0]
    dt, red = _dtype_code(x), _reduction_code(reduction)
    dev = x.device
    if keep is None:
        fwd_bytes, _ = _lib.flce_workspace_size(N, H, V, dt, b is not None, red)
    else:
        fwd_bytes, keep_bytes, _ = _lib.flce_keep_workspace_size(N, H, V, dt, b is not None, red)
        if keep is True:
            keep = torch.empty(keep_bytes, dtype=torch.uint8, device=dev)
        elif keep.dtype != torch.uint8 or keep.device != dev or not keep.is_contiguous() or keep.numel() < keep_bytes:
            raise ValueError(f"keep must be a contiguous uint8 tensor of at least {keep_bytes} bytes on {dev}")
    if workspace is None or workspace.numel() < fwd_bytes:
        workspace = torch.empty(max(fwd_bytes, 1), dtype=torch.uint8, device=dev)
    loss = torch.empty(N if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int64, device=dev)
    z_loss = torch.empty_like(loss) if return_z_loss else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        if keep is not None:
            _lib.flce_forward_keep(x.data_ptr(), W.data_ptr(), _ptr(b), targets.data_ptr(), N, H, V, dt,
                                   float(label_smoothing), float(z_loss_scale), int(ignore_index), red,
                                   _lib.options(logit_scale, False, _ptr(z_loss)), loss.data_ptr(), lse.data_ptr(),
                                   n_valid.data_ptr(), keep.data_ptr(), keep.numel(), workspace.data_ptr(),
                                   workspace.numel(), stream)
        elif logit_scale == 1.0 and not return_z_loss:
            _lib.flce_forward(x.data_ptr(), W.data_ptr(), _ptr(b), targets.data_ptr(), N, H, V, dt,
                              float(label_smoothing), float(z_loss_scale), int(ignore_index), red,
                              loss.data_ptr(), lse.data_ptr(), n_valid.data_ptr(), workspace.data_ptr(),
                              workspace.numel(), stream)
        else:
            _lib.flce_forward_ex(x.data_ptr(), W.data_ptr(), _ptr(b), targets.data_ptr(), N, H, V, dt,
                                 float(label_smoothing), float(z_loss_scale), int(ignore_index), red,
                                 _lib.options(logit_scale, False, _ptr(z_loss)), loss.data_ptr(), lse.data_ptr(),
                                 n_valid.data_ptr(), workspace.data_ptr(), workspace.numel(), stream)
    out = (loss, lse, n_valid) if keep is None else (loss, lse, n_valid, keep)
    return out + (z_loss,) if return_z_loss else out


def flce_backward(x: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor], targets: torch.Tensor,
                  lse: torch.Tensor, n_valid: torch.Tensor, grad_loss: torch.Tensor,
                  label_smoothing: float = 0.0, z_loss_scale: float = 0.0, ignore_index: int = -100,
                  reduction: str = "mean", need_dx: bool = True, need_dW: bool = True,
                  need_db: bool = True, workspace: Optional[torch.Tensor] = None,
                  out: Optional[Tuple] = None, logit_scale: float = 1.0, accumulate: bool = False):
    """Returns (dx, dW, db) in the input dtype (None where not requested).  With
    accumulate, the gradients are added to the ``out`` tensors' contents."""
    return _backward(x, W, b, targets, lse, n_valid, grad_loss, label_smoothing, z_loss_scale, ignore_index,
                     reduction, need_dx, need_dW, need_db, workspace, out, logit_scale, accumulate, None)


def flce_backward_kept(x: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor], targets: torch.Tensor,
                       lse: torch.Tensor, n_valid: torch.Tensor, grad_loss: torch.Tensor, keep: torch.Tensor,
                       label_smoothing: float = 0.0, z_loss_scale: float = 0.0, ignore_index: int = -100,
                       reduction: str = "mean", need_dx: bool = True, need_dW: bool = True,
                       need_db: bool = True, workspace: Optional[torch.Tensor] = None,
                       out: Optional[Tuple] = None, logit_scale: float = 1.0, accumulate: bool = False):
    """flce_backward given the keep buffer that flce_forward_keep filled with
    the same arguments; consumes it (a second backward needs a new forward)."""
    if keep is None:
        raise ValueError("keep is the buffer flce_forward_keep returned")
    return _backward(x, W, b, targets, lse, n_valid, grad_loss, label_smoothing, z_loss_scale, ignore_index,
                     reduction, need_dx, need_dW, need_db, workspace, out, logit_scale, accumulate, keep)


def _backward(x, W, b, targets, lse, n_valid, grad_loss, label_smoothing, z_loss_scale, ignore_index, reduction,
              need_dx, need_dW, need_db, workspace, out, logit_scale, accumulate, keep):
    H0 = x.shape[1] if x.dim() == 2 else -1
    x, W, b, targets = _prep(x, W, b, targets)
    N, H = x.shape
    V = W.shape[0]
    dt, red = _dtype_code(x), _reduction_code(reduction)
    dev = x.device
    _check_ctx(lse, n_valid, N, dev)
    g = grad_loss.reshape(-1).to(device=dev, dtype=torch.float32).contiguous()
    if g.numel() != (N if reduction == "none" else 1):
        raise ValueError("grad_loss must have N entries for none and one otherwise")
    if keep is None:
        _, bwd_bytes = _lib.flce_workspace_size(N, H, V, dt, b is not None, red)
    else:
        _, keep_bytes, bwd_bytes = _lib.flce_keep_workspace_size(N, H, V, dt, b is not None, red)
        if keep.dtype != torch.uint8 or keep.device != dev or not keep.is_contiguous() or keep.numel() < keep_bytes:
            raise ValueError(f"keep must be the contiguous uint8 buffer flce_forward_keep filled ({keep_bytes} bytes)")
    if workspace is None or workspace.numel() < bwd_bytes:
        workspace = torch.empty(max(bwd_bytes, 1), dtype=torch.uint8, device=dev)
    if out is not None:
        dx, dW, db = out
        _check_out(dx, (N, H0), x, "out dx")
        _check_out(dW, (V, H0), x, "out dW")
        _check_out(db, (V,), x, "out db")
    else:
        if accumulate:
            raise ValueError("accumulate needs the out tensors to add to")
        dx = torch.empty(N, H0, dtype=x.dtype, device=dev) if need_dx else None
        dW = torch.empty(V, H0, dtype=x.dtype, device=dev) if need_dW else None
        db = torch.empty_like(b) if (need_db and b is not None) else None
    # H padded to a multiple of 8: the library writes padded gradients, whose
    # first H0 columns are the result (with accumulate, they start from out's).
    kx, kW = dx, dW
    if H != H0:
        kx = _pad_hidden(dx) if (dx is not None and accumulate) else (
            torch.empty(N, H, dtype=x.dtype, device=dev) if dx is not None else None)
        kW = _pad_hidden(dW) if (dW is not None and accumulate) else (
            torch.empty(V, H, dtype=x.dtype, device=dev) if dW is not None else None)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        if keep is not None:
            _lib.flce_backward_kept(x.data_ptr(), W.data_ptr(), _ptr(b), targets.data_ptr(), N, H, V, dt,
                                    float(label_smoothing), float(z_loss_scale), int(ignore_index), red,
                                    _lib.options(logit_scale, accumulate, None), lse.data_ptr(), n_valid.data_ptr(),
                                    g.data_ptr(), keep.data_ptr(), keep.numel(), _ptr(kx), _ptr(kW), _ptr(db),
                                    workspace.data_ptr(), workspace.numel(), stream)
        elif logit_scale == 1.0 and not accumulate:
            _lib.flce_backward(x.data_ptr(), W.data_ptr(), _ptr(b), targets.data_ptr(), N, H, V, dt,
                               float(label_smoothing), float(z_loss_scale), int(ignore_index), red,
                               lse.data_ptr(), n_valid.data_ptr(), g.data_ptr(), _ptr(kx), _ptr(kW), _ptr(db),
                               workspace.data_ptr(), workspace.numel(), stream)
        else:
            _lib.flce_backward_ex(x.data_ptr(), W.data_ptr(), _ptr(b), targets.data_ptr(), N, H, V, dt,
                                  float(label_smoothing), float(z_loss_scale), int(ignore_index), red,
                                  _lib.options(logit_scale, accumulate, None), lse.data_ptr(), n_valid.data_ptr(),
                                  g.data_ptr(), _ptr(kx), _ptr(kW), _ptr(db), workspace.data_ptr(),
                                  workspace.numel(), stream)
    if H != H0:
        if dx is not None:
            dx.copy_(kx[:, :H0])
        if dW is not None:
            dW.copy_(kW[:, :H0])
    return dx, dW, db


def flce_fused_workspace_size(N: int, H: int, V: int, dtype: torch.dtype, has_bias: bool,
                              chunk_tokens: int = 0) -> Tuple[int, int]:
    """(workspace bytes, tokens per chunk) of the fused schedule."""
    return _lib.flce_fused_workspace_size(N, H, V, _DTYPES[dtype], has_bias, chunk_tokens)


def flce_fused_forward_backward(x: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor], targets: torch.Tensor,
                                grad_loss: torch.Tensor, label_smoothing: float = 0.0, z_loss_scale: float = 0.0,
                                ignore_index: int = -100, reduction: str = "mean", need_dx: bool = True,
                                need_dW: bool = True, need_db: bool = True, chunk_tokens: int = 0,
                                workspace: Optional[torch.Tensor] = None, out: Optional[Tuple] = None,
                                logit_scale: float = 1.0, accumulate: bool = False,
                                return_z_loss: bool = False):
    """The fused schedule: loss and gradients in one pass, the gradients formed
    while the forward runs (grad_loss must be known up front: [1] for sum/mean,
    [N] for none).  Returns (loss, lse, n_valid, dx, dW, db) (and z_loss with
    return_z_loss); gradients are None where not requested."""
    if x.dim() == 2 and x.shape[1] % 8 != 0:
        raise ValueError("the fused schedule needs H % 8 == 0; pad x and W with zero columns")
    x, W, b, targets = _prep(x, W, b, targets)
    N, H = x.shape
    V = W.shape[0]
    dt, red = _dtype_code(x), _reduction_code(reduction)
    dev = x.device
    g = grad_loss.reshape(-1).to(device=dev, dtype=torch.float32).contiguous()
    if g.numel() != (N if reduction == "none" else 1):
        raise ValueError("grad_loss must have N entries for none and one otherwise")
    nbytes, _ = _lib.flce_fused_workspace_size(N, H, V, dt, b is not None, chunk_tokens)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if out is not None:
        dx, dW, db = out
        _check_out(dx, (N, H), x, "out dx")
        _check_out(dW, (V, H), x, "out dW")
        _check_out(db, (V,), x, "out db")
    else:
        if accumulate:
            raise ValueError("accumulate needs the out tensors to add to")
        dx = torch.empty_like(x) if need_dx else None
        dW = torch.empty_like(W) if need_dW else None
        db = torch.empty_like(b) if (need_db and b is not None) else None
    loss = torch.empty(N if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int64, device=dev)
    z_loss = torch.empty_like(loss) if return_z_loss else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.flce_fused_forward_backward(x.data_ptr(), W.data_ptr(), _ptr(b), targets.data_ptr(), N, H, V, dt,
                                         float(label_smoothing), float(z_loss_scale), int(ignore_index), red,
                                         _lib.options(logit_scale, accumulate, _ptr(z_loss)), g.data_ptr(),
                                         int(chunk_tokens), loss.data_ptr(), lse.data_ptr(), n_valid.data_ptr(),
                                         _ptr(dx), _ptr(dW), _ptr(db), workspace.data_ptr(), workspace.numel(),
                                         stream)
    res = (loss, lse, n_valid, dx, dW, db)
    return res + (z_loss,) if return_z_loss else res


def _shard_hidden(x: torch.Tensor) -> None:
    # The shard entry points hand the caller fp32 dx partials of x's width,
    # so they take H as the library does (a multiple of 8) rather than pad.
    if x.dim() == 2 and x.shape[1] % 8 != 0:
        raise ValueError("the vocabulary-shard entry points need H % 8 == 0; pad x and W with zero columns")


def flce_shard_workspace_size(N: int, H: int, V_shard: int, dtype: torch.dtype,
                              has_bias: bool) -> Tuple[int, int, int]:
    """(forward, merge, backward) workspace bytes of one vocabulary shard."""
    return _lib.flce_shard_workspace_size(N, H, V_shard, _DTYPES[dtype], has_bias)


def flce_shard_forward(x: torch.Tensor, W_shard: torch.Tensor, b_shard: Optional[torch.Tensor],
                       targets: torch.Tensor, vocab_start: int, V_total: int, label_smoothing: float = 0.0,
                       ignore_index: int = -100, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-token statistics float32 [N, 4] = (m, d, sum z, z_y) over the shard's rows
    W[vocab_start : vocab_start + V_shard] (W_shard); targets are global indices."""
    _shard_hidden(x)
    x, W_shard, b_shard, targets = _prep(x, W_shard, b_shard, targets)
    N, H = x.shape
    V_shard = W_shard.shape[0]
    dt, dev = _dtype_code(x), x.device
    fwd_bytes, _, _ = _lib.flce_shard_workspace_size(N, H, V_shard, dt, b_shard is not None)
    if workspace is None or workspace.numel() < fwd_bytes:
        workspace = torch.empty(max(fwd_bytes, 1), dtype=torch.uint8, device=dev)
    stats = torch.empty(N, 4, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.flce_shard_forward(x.data_ptr(), W_shard.data_ptr(), _ptr(b_shard), targets.data_ptr(), N, H, V_shard,
                                int(vocab_start), int(V_total), dt, float(label_smoothing), int(ignore_index),
                                stats.data_ptr(), workspace.data_ptr(), workspace.numel(), stream)
    return stats


def flce_shard_merge(stats: torch.Tensor, targets: torch.Tensor, V_total: int, label_smoothing: float = 0.0,
                     z_loss_scale: float = 0.0, ignore_index: int = -100, reduction: str = "mean",
                     workspace: Optional[torch.Tensor] = None):
    """Merge stacked shard statistics [num_shards, N, 4] into (loss, lse, n_valid), as
    flce_forward returns them for the whole head."""
    if stats.dim() != 3 or stats.shape[2] != 4 or stats.dtype != torch.float32:
        raise ValueError("stats must be float32 [num_shards, N, 4]")
    stats = stats.contiguous()
    num_shards, N = stats.shape[0], stats.shape[1]
    dev = stats.device
    targets = targets.reshape(-1).to(torch.int64).contiguous()
    _, merge_bytes, _ = _lib.flce_shard_workspace_size(N, 8, 1, _lib.FLCE_F32, False)
    if workspace is None or workspace.numel() < merge_bytes:
        workspace = torch.empty(max(merge_bytes, 1), dtype=torch.uint8, device=dev)
    loss = torch.empty(N if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    n_valid = torch.empty(1, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.flce_shard_merge(stats.data_ptr(), num_shards, targets.data_ptr(), N, int(V_total),
                              float(label_smoothing), float(z_loss_scale), int(ignore_index),
                              _reduction_code(reduction), loss.data_ptr(), lse.data_ptr(), n_valid.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), stream)
    return loss, lse, n_valid


def flce_shard_backward(x: torch.Tensor, W_shard: torch.Tensor, b_shard: Optional[torch.Tensor],
                        targets: torch.Tensor, vocab_start: int, V_total: int, lse: torch.Tensor,
                        n_valid: torch.Tensor, grad_loss: torch.Tensor, label_smoothing: float = 0.0,
                        z_loss_scale: float = 0.0, ignore_index: int = -100, reduction: str = "mean",
                        dx_partial: Optional[torch.Tensor] = None, accumulate_dx: bool = False,
                        need_dx: bool = True, need_dW: bool = True, need_db: bool = True,
                        workspace: Optional[torch.Tensor] = None):
    """Returns (dx_partial float32 [N, H], dW_shard, db_shard) (None where not requested).
    dx_partial: the buffer to write (or, with accumulate_dx, to add to); allocated if None."""
    _shard_hidden(x)
    x, W_shard, b_shard, targets = _prep(x, W_shard, b_shard, targets)
    N, H = x.shape
    V_shard = W_shard.shape[0]
    dt, red, dev = _dtype_code(x), _reduction_code(reduction), x.device
    _check_ctx(lse, n_valid, N, dev)
    g = grad_loss.reshape(-1).to(device=dev, dtype=torch.float32).contiguous()
    if g.numel() != (N if reduction == "none" else 1):
        raise ValueError("grad_loss must have N entries for none and one otherwise")
    if dx_partial is not None:
        if (dx_partial.shape != (N, H) or dx_partial.dtype != torch.float32 or not dx_partial.is_contiguous()
                or dx_partial.device != dev):
            raise ValueError(f"dx_partial must be a contiguous float32 [N, H] tensor on {dev}")
    elif need_dx:
        if accumulate_dx:
            raise ValueError("accumulate_dx needs dx_partial")
        dx_partial = torch.empty(N, H, dtype=torch.float32, device=dev)
    _, _, bwd_bytes = _lib.flce_shard_workspace_size(N, H, V_shard, dt, b_shard is not None)
    if workspace is None or workspace.numel() < bwd_bytes:
        workspace = torch.empty(max(bwd_bytes, 1), dtype=torch.uint8, device=dev)
    dW = torch.empty_like(W_shard) if need_dW else None
    db = torch.empty_like(b_shard) if (need_db and b_shard is not None) else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.flce_shard_backward(x.data_ptr(), W_shard.data_ptr(), _ptr(b_shard), targets.data_ptr(), N, H,
                                 V_shard, int(vocab_start), int(V_total), dt, float(label_smoothing),
                                 float(z_loss_scale), int(ignore_index), red, lse.data_ptr(), n_valid.data_ptr(),
                                 g.data_ptr(), _ptr(dx_partial), bool(accumulate_dx), _ptr(dW), _ptr(db),
                                 workspace.data_ptr(), workspace.numel(), stream)
    return dx_partial, dW, db


class FusedLinearCrossEntropyFunction(torch.autograd.Function):
    """loss = FLCE(x, target, weight, bias); saves only lse and the count."""

    @staticmethod
    def forward(ctx, x, target, weight, bias=None, ignore_index=-100, label_smoothing=0.0,
                z_loss_scale=0.0, reduction="mean", logit_scale=1.0, keep_first_slab=False):
        # keep_first_slab: the forward keeps the first vocabulary slab's logits
        # (flce_forward_keep) so the backward skips their recompute; the buffer
        # (about N x 16384 x 2 bytes) lives until the backward.
        if keep_first_slab:
            loss, lse, n_valid, keep = flce_forward_keep(x, weight, bias, target, label_smoothing, z_loss_scale,
                                                         ignore_index, reduction, logit_scale=logit_scale)
        else:
            (loss, lse, n_valid), keep = flce_forward(x, weight, bias, target, label_smoothing, z_loss_scale,
                                                      ignore_index, reduction, logit_scale=logit_scale), None
        ctx.save_for_backward(x, target, weight, bias, lse, n_valid)
        ctx.keep = keep
        ctx.opts = (ignore_index, label_smoothing, z_loss_scale, reduction, logit_scale)
        return loss if reduction == "none" else loss.reshape(())

    @staticmethod
    def backward(ctx, grad):
        x, target, weight, bias, lse, n_valid = ctx.saved_tensors
        ignore_index, eps, s, reduction, logit_scale = ctx.opts
        keep, ctx.keep = ctx.keep, None   # consumed: a second backward recomputes every slab
        args = (x, weight, bias, target, lse, n_valid, grad)
        kw = dict(label_smoothing=eps, z_loss_scale=s, ignore_index=ignore_index, reduction=reduction,
                  need_dx=ctx.needs_input_grad[0], need_dW=ctx.needs_input_grad[2],
                  need_db=bias is not None and ctx.needs_input_grad[3], logit_scale=logit_scale)
        if keep is not None:
            dx, dW, db = flce_backward_kept(*args, keep, **kw)
        else:
            dx, dW, db = flce_backward(*args, **kw)
        return dx, None, dW, db, None, None, None, None, None, None


def fused_linear_cross_entropy_loss(x, target, weight, bias=None, ignore_index=-100, label_smoothing=0.0,
                                    z_loss_scale=0.0, reduction="mean", logit_scale=1.0, keep_first_slab=False):
    """Functional form: x [N, H], target [N], weight [V, H], bias [V] or None."""
    return FusedLinearCrossEntropyFunction.apply(x, target, weight, bias, ignore_index, label_smoothing,
                                                 z_loss_scale, reduction, logit_scale, keep_first_slab)


class FusedLinearCrossEntropyLoss(torch.nn.Module):
    """Module form; x may be [..., H] and target [...]; they are flattened."""

    def __init__(self, ignore_index: int = -100, label_smoothing: float = 0.0, z_loss_scale: float = 0.0,
                 reduction: str = "mean", logit_scale: float = 1.0, keep_first_slab: bool = False):
        super().__init__()
        _reduction_code(reduction)
        self.logit_scale = logit_scale
        self.keep_first_slab = keep_first_slab
        self.ignore_index = ignore_index
        self.label_smoothing = label_smoothing
        self.z_loss_scale = z_loss_scale
        self.reduction = reduction

    def forward(self, x, target, weight, bias=None):
        return fused_linear_cross_entropy_loss(x.reshape(-1, x.shape[-1]), target.reshape(-1), weight, bias,
                                               self.ignore_index, self.label_smoothing, self.z_loss_scale,
                                               self.reduction, self.logit_scale, self.keep_first_slab)
