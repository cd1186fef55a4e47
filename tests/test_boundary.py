"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/flce.h declares, and
reject bad arguments on the host before anything is enqueued.  Each call below
carries exactly one invalid argument, caught by validation, so no kernel is
ever launched with the placeholder addresses used here.
"""

import ctypes
import os
import re

import pytest

from lm_head_cross_flce_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")

# Placeholder addresses: 256-byte aligned, never dereferenced (validation fails first).
P = 0x100000
P2 = 0x200000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from lm_head_cross_flce_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*]+\s+)+\**(flce_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and they are real dynamic symbols of the shared object
    so = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert ctypes.cast(getattr(so, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert _lib.status_string(0) == "ok"
    for s in range(1, 6):
        assert _lib.status_string(s) not in ("ok", "unknown status")
    assert _lib.status_string(99) == "unknown status"


def test_workspace_size_arithmetic(lib):
    # forward: one fp32x4 partial per (phase, token) plus one fp32 per token
    f, b = _lib.flce_workspace_size(8192, 4096, 128256, _lib.FLCE_BF16, True, 2)
    NT, VT = 32, 501
    P = min(VT, 256 // NT)
    assert f >= P * 8192 * 16 + 8192 * 4
    slab = _lib.flce_backward_slab_cols(8192, 4096, 128256, _lib.FLCE_BF16)
    assert slab % 256 == 0 and slab >= 256
    # the dx accumulator keeps only its low 16-bit halves here (the high halves live in dx)
    need = 8192 * slab * 2 + 8192 * 4096 * 2 + NT * slab * 4 + 8192 * 20
    assert need <= b <= need + 8 * 256
    # extra memory at the Llama-3-sized head stays under 10% of the fp32 logits
    assert f + b < 0.1 * 8192 * 128256 * 4
    # no bias: no db partials
    _, b_nobias = _lib.flce_workspace_size(8192, 4096, 128256, _lib.FLCE_BF16, False, 2)
    assert b - b_nobias >= NT * slab * 4


def test_fp16_workspace_adds_the_slab_scale(lib):
    # fp16 inputs use the bf16 layout plus one 256-byte slot for the slab's scale {S, 1/S}
    for args in ((8192, 4096, 128256, True), (4096, 2048, 32000, False), (64, 128, 1000, True)):
        N, H, V, bias = args
        fh, bh = _lib.flce_workspace_size(N, H, V, _lib.FLCE_F16, bias, 2)
        fb, bb = _lib.flce_workspace_size(N, H, V, _lib.FLCE_BF16, bias, 2)
        assert fh == fb and bh == bb + 256
        assert _lib.flce_backward_slab_cols(N, H, V, _lib.FLCE_F16) == _lib.flce_backward_slab_cols(N, H, V, 1)
    fs, ms, bs = _lib.flce_shard_workspace_size(8192, 4096, 16032, _lib.FLCE_F16, True)
    _, _, bs16 = _lib.flce_shard_workspace_size(8192, 4096, 16032, _lib.FLCE_BF16, True)
    assert bs == bs16 + 256


def test_dx_accumulator_bytes_by_dtype_and_slab_count(lib):
    # one K part and several slabs: fp32 inputs accumulate in dx itself, 16-bit
    # inputs hold the fp32 low halves in the workspace; one slab: nothing
    N, H, V = 8192, 4096, 128256
    slab = _lib.flce_backward_slab_cols(N, H, V, _lib.FLCE_BF16)
    _, b16 = _lib.flce_workspace_size(N, H, V, _lib.FLCE_BF16, False, 2)
    _, b32 = _lib.flce_workspace_size(N, H, V, _lib.FLCE_F32, False, 2)
    slab32 = _lib.flce_backward_slab_cols(N, H, V, _lib.FLCE_F32)
    tail = N * 20
    assert N * slab * 2 + N * H * 2 + tail <= b16 <= N * slab * 2 + N * H * 2 + tail + 8 * 256
    assert N * slab32 * 4 + tail <= b32 <= N * slab32 * 4 + tail + 8 * 256
    # a vocabulary within one slab: no accumulator (N = 8192, H = 4096 never splits K)
    V1 = slab
    _, b1 = _lib.flce_workspace_size(N, H, V1, _lib.FLCE_BF16, False, 2)
    assert N * slab * 2 + tail <= b1 <= N * slab * 2 + tail + 8 * 256


def test_workspace_holds_one_dx_accumulator_per_k_part(lib):
    # N=4096, H=2048: the dx product has 16 x 8 = 128 output tiles, half the
    # 256 CUs, so each slab's columns are split in two parts with an fp32
    # [N, H] accumulator each; the Llama-3-sized head (512 tiles) keeps one.
    N, H, V = 4096, 2048, 32000
    slab = _lib.flce_backward_slab_cols(N, H, V, _lib.FLCE_BF16)
    _, b = _lib.flce_workspace_size(N, H, V, _lib.FLCE_BF16, False, 2)
    need = N * slab * 2 + 2 * N * H * 4 + N * 20
    assert need <= b <= need + 8 * 256
    # no split below 512 columns per part: a 1000-column vocabulary splits in two at most
    _, b1 = _lib.flce_workspace_size(64, 128, 1000, _lib.FLCE_F32, False, 2)
    slab1 = _lib.flce_backward_slab_cols(64, 128, 1000, _lib.FLCE_F32)
    need1 = 64 * slab1 * 4 + 2 * 64 * 128 * 4 + 64 * 20
    assert need1 <= b1 <= need1 + 8 * 256


def test_slab_width_heuristic(lib):
    # the wider of: one slab's dW tiles cover 256 CUs twice (once when the fp32 dx
    # accumulator is under 128 MiB), or the widest
    # slab within 256 MiB whose dW tiles fill whole rounds of 256 CUs; capped
    # at 1 GiB and at V rounded up to a tile
    assert _lib.flce_backward_slab_cols(8192, 4096, 128256, 1) == 16384
    assert _lib.flce_backward_slab_cols(4096, 2048, 32000, 1) == 32000
    assert _lib.flce_backward_slab_cols(32768, 2048, 128000, 1) == 16384
    assert _lib.flce_backward_slab_cols(16384, 1024, 256000, 1) == 16384   # small accumulator: one dW round
    assert _lib.flce_backward_slab_cols(64, 128, 1000, 0) == 1024     # capped at V rounded up
    assert _lib.flce_backward_slab_cols(64, 12, 1000, 0) == 0         # H % 8 != 0


def test_slab_cols_knob_trades_memory(lib, monkeypatch):
    # FLCE_SLAB_COLS narrows the slabs; 8192 columns keep the Llama-3-sized head's
    # extra memory (kept slab) under 10% of its bf16 logits
    monkeypatch.delenv("FLCE_DEBUG_SLAB_COLS", raising=False)
    base = sum(_lib.flce_keep_workspace_size(8192, 4096, 128256, _lib.FLCE_BF16, True, 2))
    monkeypatch.setenv("FLCE_SLAB_COLS", "8192")
    assert _lib.flce_backward_slab_cols(8192, 4096, 128256, 1) == 8192
    narrow = sum(_lib.flce_keep_workspace_size(8192, 4096, 128256, _lib.FLCE_BF16, True, 2))
    assert narrow < 0.1 * 8192 * 128256 * 2 < base
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")   # the documented knob wins
    assert _lib.flce_backward_slab_cols(8192, 4096, 128256, 1) == 8192
    monkeypatch.setenv("FLCE_SLAB_COLS", "1000")          # not a multiple of 256: ignored
    assert _lib.flce_backward_slab_cols(8192, 4096, 128256, 1) == 512


def test_slab_debug_override(lib, monkeypatch):
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "512")
    assert _lib.flce_backward_slab_cols(8192, 4096, 128256, 1) == 512
    monkeypatch.setenv("FLCE_DEBUG_SLAB_COLS", "100")   # not a multiple of 256: ignored
    assert _lib.flce_backward_slab_cols(8192, 4096, 128256, 1) == 16384


def _fwd(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, V=1000, dtype=0, eps=0.0, s=0.0, ign=-100,
                red=2, loss=P2, lse=P2, nv=P2, ws=P2, wsb=1 << 30, stream=None)
    args.update(over)
    return lib.flce_forward(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"], args["V"],
                            args["dtype"], args["eps"], args["s"], args["ign"], args["red"], args["loss"],
                            args["lse"], args["nv"], args["ws"], args["wsb"], args["stream"])


def _bwd(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, V=1000, dtype=0, eps=0.0, s=0.0, ign=-100,
                red=2, lse=P2, nv=P2, g=P2, dx=P2, dW=P2, db=None, ws=P2, wsb=1 << 30, stream=None)
    args.update(over)
    return lib.flce_backward(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"], args["V"],
                             args["dtype"], args["eps"], args["s"], args["ign"], args["red"], args["lse"],
                             args["nv"], args["g"], args["dx"], args["dW"], args["db"], args["ws"], args["wsb"],
                             args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(N=0), 1), (dict(H=0), 1), (dict(V=0), 1), (dict(N=-5), 1),
    (dict(H=12), 2), (dict(dtype=7), 2),
    (dict(eps=-0.1), 1), (dict(eps=1.5), 1), (dict(eps=float("nan")), 1),
    (dict(s=-1.0), 1), (dict(s=float("inf")), 1),
    (dict(red=3), 1), (dict(red=-1), 1),
    (dict(x=None), 1), (dict(W=None), 1), (dict(targets=None), 1),
    (dict(loss=None), 1), (dict(lse=None), 1), (dict(nv=None), 1),
    (dict(x=P + 8), 1), (dict(W=P + 2), 1), (dict(targets=P + 4), 1),
    (dict(wsb=16), 3), (dict(ws=None), 1), (dict(ws=P2 + 8), 1),
])
def test_forward_validation(lib, over, code):
    assert _fwd(lib, **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(N=0), 1), (dict(H=20), 2), (dict(eps=2.0), 1), (dict(s=-0.5), 1), (dict(red=9), 1),
    (dict(lse=None), 1), (dict(nv=None), 1), (dict(g=None), 1), (dict(x=None), 1),
    (dict(dx=P2 + 4), 1), (dict(dW=P2 + 8), 1),
    (dict(wsb=100), 3), (dict(ws=None), 1),
])
def test_backward_validation(lib, over, code):
    assert _bwd(lib, **over) == code


def test_backward_with_nothing_requested_is_a_no_op(lib):
    # dx, dW and db all NULL: returns OK without launching anything.
    assert _bwd(lib, dx=None, dW=None, db=None) == 0


def test_python_binding_raises_on_error(lib):
    with pytest.raises(_lib.FlceError) as e:
        _lib.flce_workspace_size(0, 128, 1000, 0, False, 2)
    assert e.value.status == _lib.FLCE_ERR_INVALID_ARGUMENT


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "lm_head_cross_flce_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def _sfwd(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, Vs=400, vs0=300, Vt=1000, dtype=0, eps=0.0, ign=-100,
                stats=P2, ws=P2, wsb=1 << 30, stream=None)
    args.update(over)
    return lib.flce_shard_forward(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"],
                                  args["Vs"], args["vs0"], args["Vt"], args["dtype"], args["eps"], args["ign"],
                                  args["stats"], args["ws"], args["wsb"], args["stream"])


def _smerge(lib, **over):
    args = dict(stats=P2, p=3, targets=P, N=64, Vt=1000, eps=0.0, s=0.0, ign=-100, red=2, loss=P2, lse=P2,
                nv=P2, ws=P2, wsb=1 << 30, stream=None)
    args.update(over)
    return lib.flce_shard_merge(args["stats"], args["p"], args["targets"], args["N"], args["Vt"], args["eps"],
                                args["s"], args["ign"], args["red"], args["loss"], args["lse"], args["nv"],
                                args["ws"], args["wsb"], args["stream"])


def _sbwd(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, Vs=400, vs0=300, Vt=1000, dtype=0, eps=0.0, s=0.0,
                ign=-100, red=2, lse=P2, nv=P2, g=P2, dx=P2, acc=0, dW=P2, db=None, ws=P2, wsb=1 << 30,
                stream=None)
    args.update(over)
    return lib.flce_shard_backward(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"],
                                   args["Vs"], args["vs0"], args["Vt"], args["dtype"], args["eps"], args["s"],
                                   args["ign"], args["red"], args["lse"], args["nv"], args["g"], args["dx"],
                                   args["acc"], args["dW"], args["db"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(Vs=0), 1), (dict(vs0=-1), 1), (dict(vs0=700), 1), (dict(Vt=0), 1), (dict(Vt=(1 << 30) + 1), 1),
    (dict(H=12), 2), (dict(eps=1.5), 1), (dict(stats=None), 1), (dict(stats=P2 + 4), 1), (dict(W=P + 2), 1),
    (dict(wsb=16), 3), (dict(ws=None), 1),
])
def test_shard_forward_validation(lib, over, code):
    assert _sfwd(lib, **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(p=0), 1), (dict(N=0), 1), (dict(Vt=0), 1), (dict(eps=-1.0), 1), (dict(red=5), 1),
    (dict(stats=None), 1), (dict(stats=P2 + 8), 1), (dict(targets=None), 1), (dict(loss=None), 1),
    (dict(wsb=64), 3), (dict(ws=None), 1),
])
def test_shard_merge_validation(lib, over, code):
    assert _smerge(lib, **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(Vs=0), 1), (dict(vs0=601), 1), (dict(Vt=500), 1), (dict(s=-1.0), 1), (dict(lse=None), 1),
    (dict(g=None), 1), (dict(dx=P2 + 4), 1), (dict(dW=P2 + 8), 1), (dict(wsb=100), 3),
])
def test_shard_backward_validation(lib, over, code):
    assert _sbwd(lib, **over) == code


def test_shard_workspace_sizes(lib):
    f, m, b = _lib.flce_shard_workspace_size(8192, 4096, 16032, _lib.FLCE_BF16, True)
    ff, bb = _lib.flce_workspace_size(8192, 4096, 16032, _lib.FLCE_BF16, True, 2)
    assert f == ff                                   # same forward partials
    assert m >= 8192 * 4                             # per-row losses of the merge
    assert b == bb                                   # 16032 rows fit one slab: no dx accumulator in either
    # several slabs: the plain backward holds the accumulator's low halves, the
    # shard backward none (it accumulates in the caller's fp32 buffer)
    _, _, b4 = _lib.flce_shard_workspace_size(8192, 4096, 64128, _lib.FLCE_BF16, True)
    _, bb4 = _lib.flce_workspace_size(8192, 4096, 64128, _lib.FLCE_BF16, True, 2)
    assert b4 == bb4 - 8192 * 4096 * 2
    assert _sbwd(lib, dx=None, dW=None, db=None) == 0   # nothing requested: no launch, OK


def test_ex_entry_points_validate_options(lib):
    import math as _m
    bad = _lib.options(logit_scale=float("inf"))
    assert lib.flce_forward_ex(P, P, None, P, 64, 128, 1000, 0, 0.0, 0.0, -100, 2, ctypes.byref(bad), P2, P2, P2,
                               P2, 1 << 30, None) == 1
    assert lib.flce_backward_ex(P, P, None, P, 64, 128, 1000, 0, 0.0, 0.0, -100, 2, ctypes.byref(bad), P2, P2, P2,
                                P2, P2, None, P2, 1 << 30, None) == 1
    nan = _lib.options(logit_scale=_m.nan)
    assert lib.flce_forward_ex(P, P, None, P, 64, 128, 1000, 0, 0.0, 0.0, -100, 2, ctypes.byref(nan), P2, P2, P2,
                               P2, 1 << 30, None) == 1
    misaligned = _lib.options(z_loss=P2 + 2)
    assert lib.flce_forward_ex(P, P, None, P, 64, 128, 1000, 0, 0.0, 0.0, -100, 2, ctypes.byref(misaligned), P2,
                               P2, P2, P2, 1 << 30, None) == 1
    # the usual argument checks still come first for the rest
    ok = _lib.options(logit_scale=0.5)
    assert lib.flce_forward_ex(P, P, None, P, 0, 128, 1000, 0, 0.0, 0.0, -100, 2, ctypes.byref(ok), P2, P2, P2,
                               P2, 1 << 30, None) == 1
    assert lib.flce_backward_ex(P, P, None, P, 64, 12, 1000, 0, 0.0, 0.0, -100, 2, ctypes.byref(ok), P2, P2, P2,
                                P2, P2, None, P2, 1 << 30, None) == 2


def _fna(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, V=1000, dtype=0, eps=0.0, s=0.0, ign=-100,
                red=2, opts=None, loss=P2, lse=P2, nv=P2, stream=None)
    args.update(over)
    return lib.flce_forward_noalloc(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"],
                                    args["V"], args["dtype"], args["eps"], args["s"], args["ign"], args["red"],
                                    args["opts"], args["loss"], args["lse"], args["nv"], args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(N=0), 1), (dict(H=12), 2), (dict(dtype=7), 2), (dict(eps=1.5), 1), (dict(s=-1.0), 1),
    (dict(red=3), 1), (dict(x=None), 1), (dict(W=P + 2), 1), (dict(targets=P + 4), 1), (dict(loss=None), 1),
    (dict(nv=P2 + 4), 1),
    # 8 phases x 2^20 tokens x 16 bytes of partials = 128 MiB: more than the static scratch
    (dict(N=1 << 20, V=4000), 5),
])
def test_noalloc_forward_validation(lib, over, code):
    # every case fails on the host, before the scratch address is looked up
    assert _fna(lib, **over) == code


def test_noalloc_forward_rejects_bad_options(lib):
    bad = _lib.options(logit_scale=float("inf"))
    assert _fna(lib, opts=ctypes.byref(bad)) == 1
    misaligned = _lib.options(z_loss=P2 + 2)
    assert _fna(lib, opts=ctypes.byref(misaligned)) == 1


def test_noalloc_scratch_bound(lib):
    # The header's constant is the binding's; every workload's forward fits,
    # and the first token count past the bound is rejected on the host.
    m = re.search(r"#define FLCE_FORWARD_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.FORWARD_SCRATCH_BYTES
    for N, H, V in ((64, 128, 1000), (4096, 2048, 32000), (8192, 4096, 128256), (32768, 2048, 128000),
                    (16384, 1024, 256000)):
        f, _ = _lib.flce_workspace_size(N, H, V, _lib.FLCE_BF16, True, 2)
        assert f <= _lib.FORWARD_SCRATCH_BYTES
    lo, hi = 8192, 1 << 20
    fits = lambda n: _lib.flce_workspace_size(n, 128, 4000, _lib.FLCE_BF16, False, 2)[0] <= \
        _lib.FORWARD_SCRATCH_BYTES
    assert fits(lo) and not fits(hi)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if fits(mid) else (lo, mid)
    assert _fna(lib, N=hi, V=4000, dtype=1) == _lib.FLCE_ERR_SCRATCH_TOO_SMALL
    assert 100_000 < lo < 130_000


def test_fused_workspace_and_default_chunk(lib):
    # Default chunk: the fewest chunks whose workspace fits in what the
    # recompute schedule takes for the same problem (equal extra memory),
    # balanced in multiples of 256 tokens.
    for N, H, V, bias in ((8192, 4096, 128256, True), (4096, 2048, 32000, False), (32768, 2048, 128000, True),
                          (16384, 1024, 256000, False)):
        f, b = _lib.flce_workspace_size(N, H, V, _lib.FLCE_BF16, bias, 2)
        fb, chunk = _lib.flce_fused_workspace_size(N, H, V, _lib.FLCE_BF16, bias, 0)
        assert chunk % 256 == 0 and fb <= f + b
        # one chunk of 256 more would not fit, or N is covered in fewer chunks
        nchunks = -(-N // chunk)
        bigger = -(-N // (nchunks - 1)) if nchunks > 1 else None
        if bigger is not None:
            bigger = -(-bigger // 256) * 256
            assert _lib.flce_fused_workspace_size(N, H, V, _lib.FLCE_BF16, bias, bigger)[0] > f + b
    assert _lib.flce_fused_workspace_size(8192, 4096, 128256, _lib.FLCE_BF16, True, 0)[1] == 1024
    # explicit chunk: the kept logits [chunk][V rounded up to 256] in bf16 dominate
    fb, chunk = _lib.flce_fused_workspace_size(8192, 4096, 128256, _lib.FLCE_BF16, True, 1024)
    assert chunk == 1024
    lde = 501 * 256
    kept = 1024 * lde * 2
    maxima = 1024 * 501 * 2 * 4
    dx_parts = 4 * 1024 * 4096 * 4            # 64 output tiles: the dx product splits K in four
    assert kept + maxima + dx_parts < fb < kept + maxima + dx_parts + 8 * (1 << 20)
    # fp16 adds the 256-byte slab-scale slot; fp32 keeps 4-byte values
    assert _lib.flce_fused_workspace_size(8192, 4096, 128256, _lib.FLCE_F16, True, 1024)[0] == fb + 256
    assert _lib.flce_fused_workspace_size(64, 128, 1000, _lib.FLCE_F32, True, 256) == \
        _lib.flce_fused_workspace_size(64, 128, 1000, _lib.FLCE_F32, True, 0)
    with pytest.raises(_lib.FlceError):
        _lib.flce_fused_workspace_size(8192, 4096, 128256, _lib.FLCE_BF16, True, 100)


def _ffb(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, V=1000, dtype=0, eps=0.0, s=0.0, ign=-100, red=2,
                opts=None, g=P2, chunk=0, loss=P2, lse=P2, nv=P2, dx=P2, dW=P2, db=None, ws=P2, wsb=1 << 30,
                stream=None)
    args.update(over)
    return lib.flce_fused_forward_backward(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"],
                                           args["V"], args["dtype"], args["eps"], args["s"], args["ign"],
                                           args["red"], args["opts"], args["g"], args["chunk"], args["loss"],
                                           args["lse"], args["nv"], args["dx"], args["dW"], args["db"], args["ws"],
                                           args["wsb"], args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(N=0), 1), (dict(H=12), 2), (dict(dtype=5), 2), (dict(eps=1.5), 1), (dict(s=-1.0), 1), (dict(red=4), 1),
    (dict(g=None), 1), (dict(g=P2 + 2), 1), (dict(chunk=100), 1), (dict(chunk=-256), 1),
    (dict(x=None), 1), (dict(loss=None), 1), (dict(dx=P2 + 8), 1), (dict(dW=P2 + 4), 1),
    (dict(wsb=16), 3), (dict(ws=None), 1),
])
def test_fused_validation(lib, over, code):
    assert _ffb(lib, **over) == code


def test_keep_workspace_sizes(lib):
    # keep: the first slab [N][slab] in the input dtype and its maxima
    # [N][slab / 256][2] fp32; the backward's workspace is the recompute's less
    # the slab; the forward's partials cover both of its launches' phases.
    for N, H, V, dt, bias in ((8192, 4096, 128256, 1, True), (4096, 2048, 32000, 1, False),
                              (16384, 1024, 256000, 1, False), (64, 128, 1000, 0, True), (600, 328, 2083, 2, True)):
        es = 4 if dt == 0 else 2
        slab = _lib.flce_backward_slab_cols(N, H, V, dt)
        f, b = _lib.flce_workspace_size(N, H, V, dt, bias, 2)
        fk, k, bk = _lib.flce_keep_workspace_size(N, H, V, dt, bias, 2)
        slab_bytes = -(-N * slab * es // 256) * 256
        assert bk == b - slab_bytes
        assert slab_bytes + N * (slab // 256) * 8 <= k <= slab_bytes + N * (slab // 256) * 8 + 256
        assert f <= fk <= f + 256 * 16 * N
    # the Llama-3-sized head: peak extra memory (keep + backward workspace) stays
    # under 10% of the fp32 logits
    fk, k, bk = _lib.flce_keep_workspace_size(8192, 4096, 128256, 1, True, 2)
    assert max(fk, bk) + k < 0.1 * 8192 * 128256 * 4


def _fk(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, V=1000, dtype=0, eps=0.0, s=0.0, ign=-100, red=2,
                opts=None, loss=P2, lse=P2, nv=P2, keep=P2, keepb=1 << 30, ws=P2, wsb=1 << 30, stream=None)
    args.update(over)
    return lib.flce_forward_keep(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"], args["V"],
                                 args["dtype"], args["eps"], args["s"], args["ign"], args["red"], args["opts"],
                                 args["loss"], args["lse"], args["nv"], args["keep"], args["keepb"], args["ws"],
                                 args["wsb"], args["stream"])


def _bk(lib, **over):
    args = dict(x=P, W=P, b=None, targets=P, N=64, H=128, V=1000, dtype=0, eps=0.0, s=0.0, ign=-100, red=2,
                opts=None, lse=P2, nv=P2, g=P2, keep=P2, keepb=1 << 30, dx=P2, dW=P2, db=None, ws=P2, wsb=1 << 30,
                stream=None)
    args.update(over)
    return lib.flce_backward_kept(args["x"], args["W"], args["b"], args["targets"], args["N"], args["H"],
                                  args["V"], args["dtype"], args["eps"], args["s"], args["ign"], args["red"],
                                  args["opts"], args["lse"], args["nv"], args["g"], args["keep"], args["keepb"],
                                  args["dx"], args["dW"], args["db"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(N=0), 1), (dict(H=12), 2), (dict(dtype=5), 2), (dict(eps=1.5), 1), (dict(s=-1.0), 1), (dict(red=4), 1),
    (dict(x=None), 1), (dict(x=P + 8), 1), (dict(loss=None), 1), (dict(lse=P2 + 2), 1),
    (dict(keep=None), 1), (dict(keep=P2 + 8), 1), (dict(keepb=1000), 3),
    (dict(wsb=16), 3), (dict(ws=None), 1),
])
def test_forward_keep_validation(lib, over, code):
    assert _fk(lib, **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(N=0), 1), (dict(H=20), 2), (dict(eps=2.0), 1), (dict(red=9), 1),
    (dict(lse=None), 1), (dict(nv=None), 1), (dict(g=None), 1), (dict(x=None), 1),
    (dict(dx=P2 + 4), 1), (dict(dW=P2 + 8), 1),
    (dict(keep=None), 1), (dict(keep=P2 + 8), 1), (dict(keepb=1000), 3),
    (dict(wsb=100), 3), (dict(ws=None), 1),
])
def test_backward_kept_validation(lib, over, code):
    assert _bk(lib, **over) == code


def test_backward_kept_with_nothing_requested_is_a_no_op(lib):
    assert _bk(lib, dx=None, dW=None, db=None) == 0


def test_timing_log_validation(lib):
    # no log yet on this thread: nothing to read; bad capacities are rejected
    # before any HIP call
    assert lib.flce_timing_count() == 0
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    assert lib.flce_timing_read(0, ctypes.byref(name), ctypes.byref(ms)) == 1
    assert lib.flce_timing_read(-1, ctypes.byref(name), ctypes.byref(ms)) == 1
    assert lib.flce_timing_start(1) == 1
    assert lib.flce_timing_start(-5) == 1
    assert lib.flce_timing_start(1 << 21) == 1
    assert lib.flce_timing_stop() == 0 and lib.flce_timing_clear() == 0
    assert _lib.kernel_family("(bwd_dx_kernel<T, kDxFirst, false>)") == "bwd_dx_kernel"
    assert _lib.kernel_family("fwd_combine_kernel") == "fwd_combine_kernel"
