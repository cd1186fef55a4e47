"""ctypes binding of libflce.so: the C entry points under their own names.

Argument marshalling only.  Every step of the computation runs in the HIP
library; if the library is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce.so")

FLCE_OK = 0
FLCE_ERR_INVALID_ARGUMENT = 1
FLCE_ERR_UNSUPPORTED = 2
FLCE_ERR_WORKSPACE_TOO_SMALL = 3
FLCE_ERR_HIP = 4
FLCE_ERR_SCRATCH_TOO_SMALL = 5

# Bytes of the static device scratch of flce_forward_noalloc (FLCE_FORWARD_SCRATCH_BYTES).
FORWARD_SCRATCH_BYTES = 16 << 20

FLCE_F32 = 0
FLCE_BF16 = 1
FLCE_F16 = 2

REDUCTIONS = {"none": 0, "sum": 1, "mean": 2}

# Every symbol the public header declares.
EXPORTS = ("flce_workspace_size", "flce_forward", "flce_backward", "flce_forward_ex", "flce_backward_ex",
           "flce_forward_noalloc", "flce_fused_workspace_size", "flce_fused_forward_backward",
           "flce_keep_workspace_size", "flce_forward_keep", "flce_backward_kept",
           "flce_timing_start", "flce_timing_stop", "flce_timing_count", "flce_timing_read", "flce_timing_clear",
           "flce_status_string",
           "flce_backward_slab_cols", "flce_shard_workspace_size", "flce_shard_forward", "flce_shard_merge",
           "flce_shard_backward")

class FlceOptions(ctypes.Structure):
    """struct flce_options of flce.h."""
    _fields_ = [("logit_scale", ctypes.c_float), ("accumulate", ctypes.c_int), ("z_loss", ctypes.c_void_p)]


_lock = threading.Lock()
_lib = None


class FlceError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load libflce.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m lm_head_cross_flce_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        i64, sz, vp, f32, c_int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        lib.flce_workspace_size.argtypes = [i64, i64, i64, c_int, c_int, c_int,
                                            ctypes.POINTER(sz), ctypes.POINTER(sz)]
        lib.flce_workspace_size.restype = c_int
        lib.flce_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int,
                                     vp, vp, vp, vp, sz, vp]
        lib.flce_forward.restype = c_int
        lib.flce_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int,
                                      vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flce_backward.restype = c_int
        opt = ctypes.POINTER(FlceOptions)
        lib.flce_forward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int, opt,
                                        vp, vp, vp, vp, sz, vp]
        lib.flce_forward_ex.restype = c_int
        lib.flce_backward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int, opt,
                                         vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flce_backward_ex.restype = c_int
        lib.flce_forward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int, opt,
                                             vp, vp, vp, vp]
        lib.flce_forward_noalloc.restype = c_int
        lib.flce_fused_workspace_size.argtypes = [i64, i64, i64, c_int, c_int, i64, ctypes.POINTER(i64),
                                                  ctypes.POINTER(sz)]
        lib.flce_fused_workspace_size.restype = c_int
        lib.flce_fused_forward_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int, opt,
                                                    vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.flce_fused_forward_backward.restype = c_int
        lib.flce_keep_workspace_size.argtypes = [i64, i64, i64, c_int, c_int, c_int, ctypes.POINTER(sz),
                                                 ctypes.POINTER(sz), ctypes.POINTER(sz)]
        lib.flce_keep_workspace_size.restype = c_int
        lib.flce_forward_keep.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int, opt,
                                          vp, vp, vp, vp, sz, vp, sz, vp]
        lib.flce_forward_keep.restype = c_int
        lib.flce_backward_kept.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, f32, f32, i64, c_int, opt,
                                           vp, vp, vp, vp, sz, vp, vp, vp, vp, sz, vp]
        lib.flce_backward_kept.restype = c_int
        lib.flce_timing_start.argtypes = [c_int]
        lib.flce_timing_start.restype = c_int
        lib.flce_timing_stop.argtypes = []
        lib.flce_timing_stop.restype = c_int
        lib.flce_timing_count.argtypes = []
        lib.flce_timing_count.restype = i64
        lib.flce_timing_read.argtypes = [i64, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(f32)]
        lib.flce_timing_read.restype = c_int
        lib.flce_timing_clear.argtypes = []
        lib.flce_timing_clear.restype = c_int
        lib.flce_status_string.argtypes = [c_int]
        lib.flce_status_string.restype = ctypes.c_char_p
        lib.flce_backward_slab_cols.argtypes = [i64, i64, i64, c_int]
        lib.flce_backward_slab_cols.restype = i64
        lib.flce_shard_workspace_size.argtypes = [i64, i64, i64, c_int, c_int, ctypes.POINTER(sz),
                                                  ctypes.POINTER(sz), ctypes.POINTER(sz)]
        lib.flce_shard_workspace_size.restype = c_int
        lib.flce_shard_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, c_int, f32, i64, vp,
                                           vp, sz, vp]
        lib.flce_shard_forward.restype = c_int
        lib.flce_shard_merge.argtypes = [vp, i64, vp, i64, i64, f32, f32, i64, c_int, vp, vp, vp, vp, sz, vp]
        lib.flce_shard_merge.restype = c_int
        lib.flce_shard_backward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, c_int, f32, f32, i64,
                                            c_int, vp, vp, vp, vp, c_int, vp, vp, vp, sz, vp]
        lib.flce_shard_backward.restype = c_int
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().flce_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != FLCE_OK:
        raise FlceError(status, where)


def flce_workspace_size(N: int, H: int, V: int, dtype: int, has_bias: bool, reduction: int):
    """(forward_bytes, backward_bytes) for this problem."""
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load().flce_workspace_size(N, H, V, dtype, int(bool(has_bias)), reduction,
                                      ctypes.byref(f), ctypes.byref(b)), "flce_workspace_size")
    return f.value, b.value


def flce_backward_slab_cols(N: int, H: int, V: int, dtype: int) -> int:
    return int(load().flce_backward_slab_cols(N, H, V, dtype))


def flce_forward(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                 reduction, loss, lse, n_valid, workspace, workspace_bytes, stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_forward(x, W, b or None, targets, N, H, V, dtype, label_smoothing, z_loss_scale,
                               ignore_index, reduction, loss, lse, n_valid, workspace, workspace_bytes,
                               stream or None), "flce_forward")


def flce_backward(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                  reduction, lse, n_valid, grad_loss, dx, dW, db, workspace, workspace_bytes,
                  stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_backward(x, W, b or None, targets, N, H, V, dtype, label_smoothing, z_loss_scale,
                                ignore_index, reduction, lse, n_valid, grad_loss, dx or None, dW or None,
                                db or None, workspace, workspace_bytes, stream or None), "flce_backward")


def flce_shard_workspace_size(N: int, H: int, V_shard: int, dtype: int, has_bias: bool):
    """(forward_bytes, merge_bytes, backward_bytes) for one vocabulary shard."""
    f, m, b = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load().flce_shard_workspace_size(N, H, V_shard, dtype, int(bool(has_bias)), ctypes.byref(f),
                                            ctypes.byref(m), ctypes.byref(b)), "flce_shard_workspace_size")
    return f.value, m.value, b.value


def flce_shard_forward(x, W_shard, b_shard, targets, N, H, V_shard, vocab_start, V_total, dtype,
                       label_smoothing, ignore_index, stats, workspace, workspace_bytes, stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_shard_forward(x, W_shard, b_shard or None, targets, N, H, V_shard, vocab_start, V_total,
                                     dtype, label_smoothing, ignore_index, stats, workspace, workspace_bytes,
                                     stream or None), "flce_shard_forward")


def flce_shard_merge(stats, num_shards, targets, N, V_total, label_smoothing, z_loss_scale, ignore_index,
                     reduction, loss, lse, n_valid, workspace, workspace_bytes, stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_shard_merge(stats, num_shards, targets, N, V_total, label_smoothing, z_loss_scale,
                                   ignore_index, reduction, loss, lse, n_valid, workspace, workspace_bytes,
                                   stream or None), "flce_shard_merge")


def flce_shard_backward(x, W_shard, b_shard, targets, N, H, V_shard, vocab_start, V_total, dtype,
                        label_smoothing, z_loss_scale, ignore_index, reduction, lse, n_valid, grad_loss,
                        dx_partial, accumulate_dx, dW_shard, db_shard, workspace, workspace_bytes,
                        stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_shard_backward(x, W_shard, b_shard or None, targets, N, H, V_shard, vocab_start, V_total,
                                      dtype, label_smoothing, z_loss_scale, ignore_index, reduction, lse, n_valid,
                                      grad_loss, dx_partial or None, int(bool(accumulate_dx)), dW_shard or None,
                                      db_shard or None, workspace, workspace_bytes, stream or None),
           "flce_shard_backward")


def options(logit_scale: float = 1.0, accumulate: bool = False, z_loss=None) -> FlceOptions:
    """An flce_options value; z_loss is an integer device address or None."""
    return FlceOptions(float(logit_scale), int(bool(accumulate)), z_loss or None)


def flce_forward_ex(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                    reduction, opts, loss, lse, n_valid, workspace, workspace_bytes, stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_forward_ex(x, W, b or None, targets, N, H, V, dtype, label_smoothing, z_loss_scale,
                                  ignore_index, reduction, ctypes.byref(opts) if opts is not None else None,
                                  loss, lse, n_valid, workspace, workspace_bytes, stream or None),
           "flce_forward_ex")


def flce_backward_ex(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                     reduction, opts, lse, n_valid, grad_loss, dx, dW, db, workspace, workspace_bytes,
                     stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_backward_ex(x, W, b or None, targets, N, H, V, dtype, label_smoothing, z_loss_scale,
                                   ignore_index, reduction, ctypes.byref(opts) if opts is not None else None,
                                   lse, n_valid, grad_loss, dx or None, dW or None, db or None, workspace,
                                   workspace_bytes, stream or None), "flce_backward_ex")


def flce_forward_noalloc(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                         reduction, opts, loss, lse, n_valid, stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_forward_noalloc(x, W, b or None, targets, N, H, V, dtype, label_smoothing, z_loss_scale,
                                       ignore_index, reduction, ctypes.byref(opts) if opts is not None else None,
                                       loss, lse, n_valid, stream or None), "flce_forward_noalloc")


def flce_fused_workspace_size(N: int, H: int, V: int, dtype: int, has_bias: bool, chunk_tokens: int = 0):
    """(workspace bytes, chunk used) of the fused schedule."""
    c, b = ctypes.c_int64(0), ctypes.c_size_t(0)
    _check(load().flce_fused_workspace_size(N, H, V, dtype, int(bool(has_bias)), chunk_tokens, ctypes.byref(c),
                                            ctypes.byref(b)), "flce_fused_workspace_size")
    return b.value, c.value


def flce_fused_forward_backward(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                                reduction, opts, grad_loss, chunk_tokens, loss, lse, n_valid, dx, dW, db,
                                workspace, workspace_bytes, stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_fused_forward_backward(x, W, b or None, targets, N, H, V, dtype, label_smoothing,
                                              z_loss_scale, ignore_index, reduction,
                                              ctypes.byref(opts) if opts is not None else None, grad_loss,
                                              chunk_tokens, loss, lse, n_valid, dx or None, dW or None, db or None,
                                              workspace, workspace_bytes, stream or None),
           "flce_fused_forward_backward")


def flce_keep_workspace_size(N: int, H: int, V: int, dtype: int, has_bias: bool, reduction: int):
    """(forward_bytes, keep_bytes, backward_bytes) of the kept-first-slab pair."""
    f, k, b = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load().flce_keep_workspace_size(N, H, V, dtype, int(bool(has_bias)), reduction, ctypes.byref(f),
                                           ctypes.byref(k), ctypes.byref(b)), "flce_keep_workspace_size")
    return f.value, k.value, b.value


def flce_forward_keep(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                      reduction, opts, loss, lse, n_valid, keep, keep_bytes, workspace, workspace_bytes,
                      stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_forward_keep(x, W, b or None, targets, N, H, V, dtype, label_smoothing, z_loss_scale,
                                    ignore_index, reduction, ctypes.byref(opts) if opts is not None else None,
                                    loss, lse, n_valid, keep or None, keep_bytes, workspace, workspace_bytes,
                                    stream or None), "flce_forward_keep")


def flce_backward_kept(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                       reduction, opts, lse, n_valid, grad_loss, keep, keep_bytes, dx, dW, db, workspace,
                       workspace_bytes, stream) -> None:
    """Raw call: every tensor argument is an integer device address (or 0/None)."""
    _check(load().flce_backward_kept(x, W, b or None, targets, N, H, V, dtype, label_smoothing, z_loss_scale,
                                     ignore_index, reduction, ctypes.byref(opts) if opts is not None else None,
                                     lse, n_valid, grad_loss, keep or None, keep_bytes, dx or None, dW or None,
                                     db or None, workspace, workspace_bytes, stream or None),
           "flce_backward_kept")


def flce_timing_start(capacity: int) -> None:
    _check(load().flce_timing_start(int(capacity)), "flce_timing_start")


def flce_timing_stop() -> None:
    _check(load().flce_timing_stop(), "flce_timing_stop")


def flce_timing_clear() -> None:
    _check(load().flce_timing_clear(), "flce_timing_clear")


def flce_timing_log():
    """[(kernel, ms)] of the launches logged since flce_timing_start (waits for them)."""
    lib = load()
    out = []
    for i in range(int(lib.flce_timing_count())):
        name, ms = ctypes.c_char_p(), ctypes.c_float()
        _check(lib.flce_timing_read(i, ctypes.byref(name), ctypes.byref(ms)), "flce_timing_read")
        out.append((name.value.decode(), float(ms.value)))
    return out


def kernel_family(name: str) -> str:
    """"(bwd_dx_kernel<T, kDxFirst, false>)" -> "bwd_dx_kernel"."""
    return name.strip("() ").split("<")[0].strip()
