"""The seeded input generator: determinism, rounding and distribution checks."""

import math

import numpy as np
import torch

from lm_head_cross_flce_amd import synth


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 0: first outputs as published with the algorithm
    # (Vigna's reference splitmix64.c, seed 0).
    z = synth.raw_u64(0, 0, 3)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_slices_match_whole_stream():
    key = synth.stream_key(42, "x")
    whole = synth.raw_u64(key, 0, 1000)
    np.testing.assert_array_equal(whole[300:700], synth.raw_u64(key, 300, 400))


def test_streams_differ_by_tag_and_seed():
    a = synth.raw_u64(synth.stream_key(42, "x"), 0, 8)
    b = synth.raw_u64(synth.stream_key(42, "W"), 0, 8)
    c = synth.raw_u64(synth.stream_key(43, "x"), 0, 8)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    bits = synth.f64_to_bf16_bits(v)
    got = synth.bf16_bits_to_f64(bits)
    # neighbours one bf16 ulp up and down
    up = synth.bf16_bits_to_f64((bits.astype(np.int32) + 1).astype(np.uint16))
    dn = synth.bf16_bits_to_f64((bits.astype(np.int32) - 1).astype(np.uint16))
    assert np.all(np.abs(v - got) <= np.abs(v - up))
    assert np.all(np.abs(v - got) <= np.abs(v - dn))
    # exact ties go to the even pattern
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)])
    tb = synth.f64_to_bf16_bits(ties)
    assert np.all(tb % 2 == 0)
    # agrees with torch's fp32 -> bf16 rounding on fp32-representable values
    v32 = v.astype(np.float32).astype(np.float64)
    tb32 = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f64_to_bf16_bits(v32), tb32)


def test_f16_draws_round_to_nearest_even():
    # the fp16 workloads round each fp64 draw once to half, nearest-even
    a = synth.normal(44, "x", 50001, 1.0, "f16")
    assert a.dtype == np.float16
    key = synth.stream_key(44, "x")
    v = synth._normals_chunk(key, 0, 25001).reshape(-1)[:50001]
    h = a.astype(np.float64)
    up = np.nextafter(a, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(a, np.float16(-np.inf)).astype(np.float64)
    assert np.all(np.abs(v - h) <= np.abs(v - up)) and np.all(np.abs(v - h) <= np.abs(v - dn))
    # agrees with torch's fp32 -> fp16 rounding on fp32-representable values (torch
    # converts fp64 through fp32, a double rounding, so it is not compared on v)
    v32 = v.astype(np.float32)
    np.testing.assert_array_equal(torch.from_numpy(v32).to(torch.float16).numpy(),
                                  v32.astype(np.float64).astype(np.float16))
    # and ties go to the even pattern
    ties = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -11)])
    assert np.all(ties.astype(np.float16).view(np.uint16) % 2 == 0)


def test_normal_moments_and_determinism():
    a = synth.normal(42, "x", 200001, 2.0, "bf16")
    b = synth.normal(42, "x", 200001, 2.0, "bf16")
    np.testing.assert_array_equal(a, b)
    f = synth.bf16_bits_to_f64(a)
    assert abs(f.mean()) < 0.02 and abs(f.std() - 2.0) < 0.02
    # parallel chunked draw equals a serial draw
    big = synth.normal(7, "W", 3 * (1 << 20) + 5, 1.0, "f32")
    small = synth.normal(7, "W", 1000, 1.0, "f32")
    np.testing.assert_array_equal(big[:1000], small)


def test_uniform_and_zipf_targets():
    u = synth.uniform_ints(1, "targets", 100000, 1000)
    assert u.min() >= 0 and u.max() < 1000
    counts = np.bincount(u, minlength=1000)
    assert counts.std() < 20  # ~ sqrt(100) for a uniform draw
    z = synth.zipf_ints(1, "targets", 200000, 5000, 1.1)
    k = np.arange(1, 5001.0)
    p = k ** -1.1 / np.sum(k ** -1.1)
    emp = np.bincount(z, minlength=5000) / z.size
    np.testing.assert_allclose(emp[:5], p[:5], rtol=0.05)


def test_choose_rows_exact_count():
    r = synth.choose_rows(44, "ignore", 8192, 410)
    assert r.size == 410 and np.unique(r).size == 410 and r.max() < 8192


def test_workload_shapes_and_ignores():
    w = synth.scaled(synth.WORKLOADS["n8192_h4096_v128256"], "c3_small", N=512, H=64, V=300, n_ignored=26)
    inp = synth.make_inputs(w)
    assert inp.x.shape == (512, 64) and inp.x.dtype == np.uint16
    assert inp.W.shape == (300, 64) and inp.b.shape == (300,)
    assert int(np.sum(inp.targets == -100)) == 26
    assert inp.grad.shape == (1,) and inp.grad[0] == 1.0
    wt = synth.WORKLOADS["tiny_f32"]
    ti = synth.make_inputs(wt)
    assert ti.x.dtype == np.float32 and int(np.sum(ti.targets == -100)) == 8
    assert abs(float(np.std(ti.b)) - math.sqrt(0.1)) < 0.1
    w5 = synth.scaled(synth.WORKLOADS["n16384_h1024_v256000"], "c5_small", N=256, H=32, V=2000)
    i5 = synth.make_inputs(w5)
    assert i5.grad.shape == (256,) and i5.b is None
