"""GPU check of the launch timing log (flce_timing_*): one entry per kernel
launch of the logged calls, in launch order, with positive durations."""

import pytest
import torch

from lm_head_cross_flce_amd import _lib
from lm_head_cross_flce_amd import functional as F

from flce_gpu_util import device_inputs
from test_gpu_parity import inputs

pytestmark = pytest.mark.gpu


def test_timing_log_names_every_launch(monkeypatch):
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")   # c3_small: 5 slabs, the first kept
    inp = inputs("c3_small")
    w = inp.w
    x, W, b, t, g = device_inputs(inp)
    print("[gpu] timing log", flush=True)
    _lib.flce_timing_start(256)
    try:
        loss, lse, nv, keep = F.flce_forward_keep(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                                                  w.reduction)
        F.flce_backward_kept(x, W, b, t, lse, nv, g, keep, w.label_smoothing, w.z_loss_scale, w.ignore_index,
                             w.reduction)
        _lib.flce_timing_stop()
        log = _lib.flce_timing_log()
    finally:
        _lib.flce_timing_clear()
    fams = [_lib.kernel_family(k) for k, _ in log]
    nslab = -(-w.V // 512)
    assert fams[:4] == ["fused_fwd_kernel", "fwd_lse_kernel", "fwd_combine_kernel", "fwd_finalize_kernel"], fams
    back = fams[4:]
    assert back[0] == "bwd_coef_kernel" and back[1] == "fused_dz_kernel", back
    assert back.count("bwd_dz_kernel") == nslab - 1
    assert back.count("bwd_dx_kernel") == nslab and back.count("bwd_dw_kernel") == nslab
    assert all(ms > 0.0 for _, ms in log)
    # logging off: later calls add nothing
    F.flce_forward(x, W, b, t, w.label_smoothing, w.z_loss_scale, w.ignore_index, w.reduction)
    torch.cuda.synchronize()
    assert _lib.load().flce_timing_count() == 0
