"""CPU oracle for fused linear cross entropy.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its Python binding.

* ``flce_oracle`` - numpy fp64 definition, row-chunked (any size).
* ``brute`` - pure-Python loops for tiny shapes, to cross-check the former.

Every function is pinned by the CPU tests (closed forms, invariants, finite
differences, a textbook cross-entropy routine and the brute force).
"""
