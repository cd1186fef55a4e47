"""Fused linear cross entropy for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libflce.so (C ABI in include/flce.h);
this package holds its ctypes binding, a thin PyTorch autograd/module shim and
the seeded synthetic-input generator used by the benchmark and the tests.
"""

from ._lib import FlceError, LIB_PATH, load  # noqa: F401

__all__ = ["FlceError", "LIB_PATH", "load", "functional", "synth"]


def __getattr__(name):
    # torch-dependent parts load on first use, so ``synth`` imports stay light.
    if name in ("functional", "synth", "build"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    if name in ("flce_forward", "flce_backward", "flce_workspace_size", "fused_linear_cross_entropy_loss",
                "FusedLinearCrossEntropyLoss", "FusedLinearCrossEntropyFunction"):
        from . import functional
        return getattr(functional, name)
    raise AttributeError(name)
