"""The host side of the C-ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

CPU only.  flce_api.hip (validation, workspace and chunk arithmetic, the
entry points) is compiled with host-side ASan and UBSan (device code is not
instrumented) and linked with launchers that only return an error, so no
kernel can run; the boundary tests then run against that library in a child
process with the sanitizer runtime preloaded.  Any sanitizer report ends the
child with a non-zero status.
"""

import glob
import os
import re
import shlex
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_head_cross_flce_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer"


def _runtime():
    libs = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return libs[-1] if libs else None


def _stub_launchers(path):
    """A translation unit defining every launcher of flce_launch.hpp as a
    function that returns hipErrorNotSupported."""
    decls = re.findall(r"^(hipError_t launch_\w+\([^;]*?\));", open(os.path.join(CSRC, "flce_launch.hpp")).read(),
                       re.M | re.S)
    body = "\n".join(d.replace("\n", " ") + " { return hipErrorNotSupported; }" for d in decls)
    with open(path, "w") as f:
        f.write('#include "flce_launch.hpp"\nnamespace flce {\n' + body + "\n}\n")
    return len(decls)


@pytest.mark.timeout(300)
def test_boundary_under_asan_and_ubsan():
    rt = _runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the ASan runtime is not available")
    with tempfile.TemporaryDirectory(prefix="flce_san_") as tmp:
        assert _stub_launchers(os.path.join(tmp, "stub.cpp")) >= 10
        inc = f"-I{os.path.join(ROOT, 'include')} -I{CSRC}"
        cmds = [
            f"{HIPCC} --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -Xclang -target-feature -Xclang "
            f"-packed-fp32-ops {inc} -c {os.path.join(CSRC, 'flce_api.hip')} -o {tmp}/api.o {SAN}",
            f"{HIPCC} -O1 -std=c++17 -fPIC {inc} -c {tmp}/stub.cpp -o {tmp}/stub.o",
            f"{HIPCC} -shared -fPIC -o {tmp}/libflce_san.so {tmp}/api.o {tmp}/stub.o {SAN} -shared-libsan",
        ]
        for c in cmds:
            r = subprocess.run(shlex.split(c), capture_output=True, text=True)
            assert r.returncode == 0, r.stdout + r.stderr
        child = (
            "import sys\n"
            f"sys.path.insert(0, {ROOT!r})\n"
            "import lm_head_cross_flce_amd._lib as L\n"
            f"L.LIB_PATH = {tmp + '/libflce_san.so'!r}\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_boundary.py')!r}]))\n"
        )
        env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env, cwd=ROOT)
        out = r.stdout + r.stderr
        assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
        assert re.search(r"\d+ passed", out), out[-2000:]
