"""Builds the FLCE HIP library (libflce.so) in-tree for gfx950.

    python -m lm_head_cross_flce_amd.build [--verbose]

Each translation unit is compiled by hipcc in parallel, then linked into one
shared library next to this file.  Packed fp32 instructions are disabled for
all device code (-packed-fp32-ops).
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libflce.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["flce_kernels.hip", "flce_api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every source and link libflce.so; returns the library path."""
    with tempfile.TemporaryDirectory(prefix="flce_build_") as tmp:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
            if resource_usage:
                cmd.append("-Rpass-analysis=kernel-resource-usage")
            res = subprocess.run(cmd, capture_output=True, text=True)
            out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                            if "packed-fp32-ops" not in l)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{out}")
            if verbose and out.strip():
                print(out)
            return obj

        with ThreadPoolExecutor(len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = os.path.join(tmp, LIB_NAME)
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
        os.replace(tmp_lib, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv, resource_usage="--usage" in sys.argv)
    print(path)
