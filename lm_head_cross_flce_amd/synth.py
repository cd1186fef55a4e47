"""Seeded synthetic inputs for fused linear cross entropy (FLCE) workloads.

This module draws random numbers and nothing else: it holds none of the loss
arithmetic.  Both the GPU path's tests/benchmark and the CPU oracle's tests take
their inputs from here, so the two sides see bit-identical operands.

Generator
---------
* One SplitMix64 stream per (config seed, tensor tag).  SplitMix64 is Steele,
  Lea and Flood's "Fast splittable pseudorandom number generators" (OOPSLA
  2014): the state advances by the golden-ratio increment 0x9E3779B97F4A7C15 and
  each output is the state passed through a two-multiply xor-shift finaliser.
  Output ``i`` of a stream with key ``k`` is ``mix(k + (i + 1) * golden)``, so
  any slice of a stream can be produced independently (counter-based), which is
  what lets the large tensors be drawn in parallel chunks.
* Uniform doubles: the top 53 bits of an output, times 2**-53.
* Gaussians: Box-Muller in fp64 on consecutive output pairs, scaled by the
  standard deviation, then rounded to nearest-even into bf16 (or fp32).
* Uniform integers in [0, V): rejection sampling on full 64-bit outputs.
* Zipf(a): inverse CDF over ranks k = 1..V with p(k) proportional to k**-a;
  the token id is k - 1.
* Ignored rows: a partial Fisher-Yates shuffle that picks an exact count.

Noise notation N(0, v) in the workload descriptions is read with v as the
variance (so W ~ N(0, 1/H) gives unit-variance logits).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_TWO_POW_M53 = 2.0 ** -53

# One stream per tensor tag.
TAGS = {"x": 1, "W": 2, "b": 3, "targets": 4, "ignore": 5, "g": 6}

_CHUNK = 1 << 20


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser on a uint64 array (in place, returned)."""
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _mix_scalar(v: int) -> int:
    z = np.array([v & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return int(_mix(z)[0])


def stream_key(seed: int, tag: str) -> int:
    """Key of the stream for (seed, tag)."""
    return _mix_scalar((_mix_scalar(seed) + TAGS[tag] * 0x632BE59BD9B4E019) & 0xFFFFFFFFFFFFFFFF)


def raw_u64(key: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream with state ``key``."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(key) + idx * _GOLDEN
        return _mix(z)


def uniform01(key: int, start: int, count: int) -> np.ndarray:
    """Doubles in [0, 1) from the top 53 bits of each output."""
    return (raw_u64(key, start, count) >> np.uint64(11)).astype(np.float64) * _TWO_POW_M53


def _normals_chunk(key: int, pair_start: int, npairs: int) -> np.ndarray:
    z = raw_u64(key, 2 * pair_start, 2 * npairs).reshape(npairs, 2)
    # u1 in (0, 1] so log(u1) is finite; u2 in [0, 1).
    u1 = ((z[:, 0] >> np.uint64(11)).astype(np.float64) + 1.0) * _TWO_POW_M53
    u2 = (z[:, 1] >> np.uint64(11)).astype(np.float64) * _TWO_POW_M53
    r = np.sqrt(-2.0 * np.log(u1))
    t = (2.0 * math.pi) * u2
    out = np.empty((npairs, 2), dtype=np.float64)
    out[:, 0] = r * np.cos(t)
    out[:, 1] = r * np.sin(t)
    return out.reshape(-1)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to nearest-even bf16; returns the uint16 bit patterns.

    Rounds once, directly from fp64 (no intermediate fp32 rounding).  Values are
    assumed finite and inside bf16's normal range (true for the Gaussian draws
    used here; checked).
    """
    bits = v.view(np.uint64)
    # fp64 has 52 mantissa bits, bf16 has 7: drop 45 bits with round-half-even.
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f = rounded.view(np.float64)
    nz = f != 0.0
    if np.any(np.abs(f[nz]) < 2.0 ** -126) or not np.all(np.isfinite(f)):
        raise ValueError("value outside the normal bf16 range")
    f32 = f.astype(np.float32)  # exact: at most 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal(seed: int, tag: str, count: int, std: float, dtype: str, mean: float = 0.0) -> np.ndarray:
    """``count`` draws from N(mean, std**2) rounded to ``dtype``.

    dtype "bf16" returns uint16 bit patterns; "f16" returns float16 (numpy's
    fp64 -> half conversion rounds to nearest-even); "f32" returns float32.
    """
    key = stream_key(seed, tag)
    npairs = (count + 1) // 2
    out = np.empty(count, dtype={"bf16": np.uint16, "f16": np.float16}.get(dtype, np.float32))
    chunk_pairs = _CHUNK // 2

    def work(p0: int) -> None:
        n = min(chunk_pairs, npairs - p0)
        vals = _normals_chunk(key, p0, n) * std
        if mean != 0.0:
            vals = vals + mean
        lo, hi = 2 * p0, min(count, 2 * (p0 + n))
        vals = vals[: hi - lo]
        if dtype == "bf16":
            out[lo:hi] = f64_to_bf16_bits(vals)
        elif dtype == "f16":
            out[lo:hi] = vals.astype(np.float16)
        else:
            out[lo:hi] = vals.astype(np.float32)

    starts = range(0, npairs, chunk_pairs)
    if npairs > chunk_pairs:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, starts))
    else:
        for p0 in starts:
            work(p0)
    return out


def uniform_ints(seed: int, tag: str, count: int, n: int) -> np.ndarray:
    """``count`` integers uniform on [0, n) by rejection on 64-bit outputs."""
    key = stream_key(seed, tag)
    limit = (1 << 64) - ((1 << 64) % n)  # accept z < limit, then z mod n
    out = np.empty(count, dtype=np.int64)
    pending = np.arange(count, dtype=np.int64)
    attempt = 0
    while pending.size:
        # attempt a uses outputs a*count + i for element i
        z = raw_u64(key, attempt * count, count)[pending]
        if limit == 1 << 64:
            ok = np.ones(z.shape, dtype=bool)
        else:
            ok = z < np.uint64(limit)
        out[pending[ok]] = (z[ok] % np.uint64(n)).astype(np.int64)
        pending = pending[~ok]
        attempt += 1
    return out


def zipf_ints(seed: int, tag: str, count: int, n: int, a: float) -> np.ndarray:
    """``count`` ids in [0, n) with P(id = k-1) proportional to k**-a."""
    k = np.arange(1, n + 1, dtype=np.float64)
    cdf = np.cumsum(k ** -a)
    cdf /= cdf[-1]
    u = uniform01(stream_key(seed, tag), 0, count)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, n - 1).astype(np.int64)


def choose_rows(seed: int, tag: str, n: int, m: int) -> np.ndarray:
    """Exactly ``m`` distinct row indices out of ``n`` (partial Fisher-Yates)."""
    if m > n:
        raise ValueError("cannot choose more rows than exist")
    key = stream_key(seed, tag)
    z = raw_u64(key, 0, m)
    perm = np.arange(n, dtype=np.int64)
    for j in range(m):
        r = j + int(z[j] % np.uint64(n - j))
        perm[j], perm[r] = perm[r], perm[j]
    return np.sort(perm[:m])


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    """Shapes, distributions and loss options of one synthetic workload."""

    name: str
    N: int
    H: int
    V: int
    dtype: str                    # "bf16", "f16" or "f32": dtype of x, W and b
    x_std: float = 1.0
    w_std: Optional[float] = None  # None -> 1/sqrt(H)
    b_std: Optional[float] = None  # None -> no bias
    b_mean: float = 0.0           # mean of the bias draws
    targets: str = "uniform"      # "uniform" or "zipf"
    zipf_a: float = 1.1
    n_ignored: int = 0
    label_smoothing: float = 0.0
    z_loss_scale: float = 0.0
    reduction: str = "mean"       # "none" | "sum" | "mean"
    grad: str = "one"             # "one" | "scalar_normal" | "vector_normal"
    seed: int = 42
    ignore_index: int = -100
    notes: str = ""
    extra: dict = field(default_factory=dict)


# The five workloads (seeds 42 + index) and an fp16 variant of the Llama-3-sized head.
WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", N=64, H=128, V=1000, dtype="f32", b_std=math.sqrt(0.1),
        n_ignored=8, reduction="mean", grad="one", seed=42,
        notes="tiny fp32 case: b ~ N(0, 0.1), 8 rows ignored"),
    "n4096_h2048_v32000": Workload(
        "n4096_h2048_v32000", N=4096, H=2048, V=32000, dtype="bf16",
        reduction="mean", grad="scalar_normal", seed=43,
        notes="no bias, eps 0, s 0, mean, upstream grad one bf16 N(0,1) draw"),
    "n8192_h4096_v128256": Workload(
        "n8192_h4096_v128256", N=8192, H=4096, V=128256, dtype="bf16",
        b_std=math.sqrt(0.02), n_ignored=410, label_smoothing=0.1,
        z_loss_scale=1e-4, reduction="mean", grad="one", seed=44,
        notes="Llama-3-sized head: bias N(0, 0.02), 5% ignored, eps 0.1, s 1e-4"),
    "n32768_h2048_v128000": Workload(
        "n32768_h2048_v128000", N=32768, H=2048, V=128000, dtype="bf16",
        w_std=1.0, b_std=1.0, reduction="mean", grad="scalar_normal", seed=45,
        notes="large-magnitude logits (std ~45): x, W, b all N(0, 1)"),
    "n16384_h1024_v256000": Workload(
        "n16384_h1024_v256000", N=16384, H=1024, V=256000, dtype="bf16",
        targets="zipf", label_smoothing=0.05, z_loss_scale=1e-4,
        reduction="none", grad="vector_normal", seed=46,
        notes="small H / large V: Zipf(1.1) targets, eps 0.05, s 1e-4, none"),
    # The Llama-3-sized head with fp16 inputs: the same draws (seed 44) rounded to half.
    "n8192_h4096_v128256_f16": Workload(
        "n8192_h4096_v128256_f16", N=8192, H=4096, V=128256, dtype="f16",
        b_std=math.sqrt(0.02), n_ignored=410, label_smoothing=0.1,
        z_loss_scale=1e-4, reduction="mean", grad="one", seed=44,
        notes="Llama-3-sized head in fp16: bias N(0, 0.02), 5% ignored, eps 0.1, s 1e-4"),
}

BENCH_WORKLOAD = "n8192_h4096_v128256"


def scaled(w: Workload, name: str, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (used for reduced-size cases)."""
    d = dict(w.__dict__)
    d.pop("extra", None)
    d.update(kw)
    d["name"] = name
    return Workload(**d)


@dataclass
class Inputs:
    """Host-side arrays of one workload draw.

    x, W, b hold bf16 bit patterns (uint16) or float32 values, row-major:
    x [N, H], W [V, H], b [V] or None.  targets is int64 [N].  grad is float32:
    shape [1] for sum/mean, [N] for none.
    """

    w: Workload
    x: np.ndarray
    W: np.ndarray
    b: Optional[np.ndarray]
    targets: np.ndarray
    grad: np.ndarray

    def as_f64(self, name: str) -> Optional[np.ndarray]:
        """Exact fp64 copy of x, W or b."""
        a = getattr(self, name)
        if a is None:
            return None
        if self.w.dtype == "bf16":
            return bf16_bits_to_f64(a)
        return a.astype(np.float64)


def make_inputs(w: Workload, parts=("x", "W", "b", "targets", "grad")) -> Inputs:
    """Draw the inputs of workload ``w`` (only the requested parts)."""
    s = w.seed
    w_std = w.w_std if w.w_std is not None else 1.0 / math.sqrt(w.H)
    x = normal(s, "x", w.N * w.H, w.x_std, w.dtype).reshape(w.N, w.H) if "x" in parts else None
    W = normal(s, "W", w.V * w.H, w_std, w.dtype).reshape(w.V, w.H) if "W" in parts else None
    b = None
    if w.b_std is not None and "b" in parts:
        b = normal(s, "b", w.V, w.b_std, w.dtype, w.b_mean)
    targets = None
    if "targets" in parts:
        if w.targets == "zipf":
            targets = zipf_ints(s, "targets", w.N, w.V, w.zipf_a)
        else:
            targets = uniform_ints(s, "targets", w.N, w.V)
        if w.n_ignored:
            targets[choose_rows(s, "ignore", w.N, w.n_ignored)] = w.ignore_index
    grad = None
    if "grad" in parts:
        if w.grad == "one":
            grad = np.ones(1, dtype=np.float32)
        elif w.grad == "scalar_normal":
            grad = bf16_bits_to_f64(normal(s, "g", 1, 1.0, "bf16")).astype(np.float32)
        else:
            grad = bf16_bits_to_f64(normal(s, "g", w.N, 1.0, "bf16")).astype(np.float32)
        if w.reduction == "none" and grad.size == 1:
            grad = np.full(w.N, grad[0], dtype=np.float32)
        if w.reduction != "none" and grad.size != 1:
            raise ValueError("sum/mean take a scalar upstream gradient")
    return Inputs(w, x, W, b, targets, grad)
