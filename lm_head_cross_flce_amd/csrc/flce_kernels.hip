// FLCE kernels for gfx950.
//
// Forward (statistics only; logits recomputed in backward, the schedule of
// DeepSpeed PR 8792):
//   fwd_lse_kernel     logits tiles z = scale (W x^T + b) on MFMA; the
//                      epilogue folds each tile into per-token online max /
//                      sum-exp (the online softmax the fla kernel cites), the
//                      running sum of logits (label smoothing) and the target
//                      logit.  Persistent over (token tile, vocabulary phase).
//   fwd_combine_kernel merges the per-phase partials: lse = m + log d and the
//                      per-row loss of the label-smoothed CE plus z-loss (and
//                      the z-loss term alone when asked for).
//   fwd_stats_kernel   vocabulary shards: merges the phases into per-token
//                      statistics instead (the shard merge then runs
//                      fwd_combine over the shards).
//   fwd_finalize       fixed-order sums and non-ignored count (no host sync).
// Backward, one vocabulary slab at a time:
//   bwd_coef_kernel    per-token c_n (upstream grad, 1/T for mean, the logit
//                      scale) folded with the z-loss factor (1 + 2 s lse) of
//                      Liger PR 239.
//   bwd_dz_kernel      recomputes logits tiles (persistent) and turns them
//                      into dlogits dz = c [(1 + 2 s lse) p - eps/V
//                      - (1 - eps) [j = y]], written to the slab; optional db
//                      partial sums (fp32).
//   bwd_dx_kernel      dx += dz W[slab] into an fp32 accumulator; the last
//                      slab writes dx in x's dtype (optionally added to it).
//   bwd_dw_kernel      dW[slab] = dz^T x with K = all tokens, fp32 in
//                      registers, written once in W's dtype (optionally added);
//                      its first H-tile workgroups also finish db.
//   bwd_db_kernel      db alone, when dW is not requested.
#include "flce_device.hpp"
#include "flce_launch.hpp"

namespace flce {

// Cache policy of the dlogits slab's stores: sc0 | nt (non-temporal).  The
// slab is written once and read once, by the two gradient products.  With
// this policy the backward pass measured 0.5-2% faster at the bf16 workloads;
// the same policy on the dx accumulator's read-modify-write and on the dx and
// dW stores measured slower, so those keep the default policy.
constexpr int kSlabPolicy = 3;

// ---------------------------------------------------------------------------
// Epilogue helpers.  Accumulator layout (Acc): element r of block (i, j) in
// lane l is row 16 i + 4 g + r and column 16 j + l % 16 of the wave tile,
// with g = l / 16.  A lane thus holds, for each of its 8 columns, 32 rows:
// four consecutive ones in each of the 8 row blocks.
// ---------------------------------------------------------------------------

// acc += x as one v_add_f32 the compiler cannot reorder or merge, for sums
// whose adds the compiler otherwise restructured (and spilled).  x must not
// come straight from a transcendental: use add_pinned_after_trans for that.
__device__ __forceinline__ void add_pinned(float& acc, float x) {
  asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc) : "v"(x));
}
// The same for x straight from a transcendental (v_exp_f32): a VALU
// instruction that reads such a result needs one wait state first, which the
// compiler does not insert before inline assembly, so the s_nop supplies it.
__device__ __forceinline__ void add_pinned_after_trans(float& acc, float x) {
  asm volatile("s_nop 0\n\tv_add_f32 %0, %0, %1" : "+v"(acc) : "v"(x));
}

__device__ __forceinline__ void merge_md(float& m, float& d, float m2, float d2) {
  const float mn = fmaxf(m, m2);
  float r = 0.f;
  if (m != -INFINITY) r += d * fast_exp2((m - mn) * kLog2e);
  if (m2 != -INFINITY) r += d2 * fast_exp2((m2 - mn) * kLog2e);
  m = mn;
  d = r;
}

// Fold column j of a tile (this lane's 32 rows of one token) into the running
// (m, d) of that token, the running sum of logits, and the target logit.
// Logits are scale * acc + bias, the bias already multiplied by scale.
// rb: tile row index of the lane's row 0 (v0 + wave row offset + 4 g); t: the
// token's target minus rb (negative if ignored or elsewhere).
// RAGGED here: this tile is the vocabulary's partial last one (rows at or
// past V are masked), not the kernels' launch-wide flag of the same name.
// UNIT: no bias and a logit scale of 1, so the logits are the accumulators
// themselves (skips one fma per logit; bit-identical).
template <bool SMOOTH, bool RAGGED, bool UNIT = false>
__device__ __forceinline__ void lse_column(const Acc& acc, int j, const f32x4 (&bias)[8], float scale, float& m,
                                           float& d, float& sz, float& zy, int t, int rb, int V) {
  float z[32];
  float bmax = -INFINITY, zs = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 v = acc_read4(acc[i][j]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = UNIT ? v[r] : fmaf(v[r], scale, bias[i][r]);
      if (RAGGED) {
        const bool ok = rb + 16 * i + r < V;
        if (SMOOTH) zs += ok ? x : 0.f;
        x = ok ? x : -INFINITY;
      } else if (SMOOTH) {
        zs += x;
      }
      z[4 * i + r] = x;
      bmax = fmaxf(bmax, x);
    }
  }
  const float mn = fmaxf(m, bmax);
  if (!RAGGED || mn != -INFINITY) {
    const float nml = -mn * kLog2e;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) ps += fast_exp2(fmaf(z[e], kLog2e, nml));
    d = d * fast_exp2((m - mn) * kLog2e) + ps;  // m = -inf: the factor is 0
    m = mn;
  }
  if (SMOOTH) sz += zs;
  // Target row (t = 16 i + r for the owning lane): wave-uniform branch, rarely taken.
  const bool own = t >= 0 && t < 128 && ((t >> 2) & 3) == 0;
  if (__ballot(own)) {
    float val = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (t == 16 * (e >> 2) + (e & 3)) val = z[e];
    if (own) zy = val;
  }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------

// Workgroup w owns token tile nt and the vocabulary tiles ph, ph + P, ...
// When NT % 8 == 0 the 1/8 of the grid on one XCD covers NT/8 token tiles
// times all P phases, so each XCD streams W tiles that its neighbours reuse.
//
// XFIRST: each K block's x copies are issued before W's.  Same-box A/Bs of the
// forward: x first is 3.6% faster at N=8192, H=4096, V=128256 (8 phases),
// 4.4% at N=4096 (16 phases) and 3.1% at N=16384 (4 phases at the time), but
// was 0.7% slower with 2 phases (16 token tiles per XCD sharing each W tile).
// The launch takes x first with at least 4 phases, which the phase rule
// (at least 8 when the vocabulary has 8 tiles) makes the usual case.
//
// RAGGED: V or N may not be a multiple of 256, so some tile may be partial.
// Without it the partial-tile epilogue is not compiled in: the compiler
// computed its 32 row compares in every tile and held them in 64 scalar
// registers.
template <class T, bool BIAS, bool SMOOTH, bool XFIRST, bool RAGGED>
__global__ void __launch_bounds__(kThreads, 1) fwd_lse_kernel(FwdLaunch a) {
  FLCE_LDS(L, T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  const int w = blockIdx.x;
  int nt, ph;
  if ((a.NT & 7) == 0) {
    const int slot = w >> 3;
    ph = slot % a.P;
    nt = (w & 7) * (a.NT >> 3) + slot / a.P;
  } else {
    ph = w % a.P;
    nt = w / a.P;
  }
  const int n0 = nt * kTile;
  const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
  const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};

  // This lane's 8 tokens: n0 + wn * 128 + 16 j + lane % 16.
  int ycol[8];
  float m[8], d[8], sz[8], zy[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = n0 + wn * kWaveTile + 16 * j + (lane & 15);
    const int64_t t = n < a.N ? a.targets[n] : a.ignore_index;
    const int64_t lt = t - a.vocab_start;   // row of W holding the target, if any
    ycol[j] = (t == a.ignore_index || lt < 0 || lt >= a.V) ? -1 : (int)lt;
    m[j] = -INFINITY;
    d[j] = 0.f;
    sz[j] = 0.f;
    zy[j] = 0.f;
  }

  Acc acc;
  const int rloc = wm * kWaveTile + 4 * g;   // tile row of this lane's row 0
  // bf16: the next tile's first stages are copied while this tile's epilogue runs.
  TileCopy<true, true> tc;
  if constexpr (sizeof(T) == 2) {
    if (ph < a.VT) tc.start(A, ph * kTile, B, n0, L, tid);
  }
  for (int vt = ph; vt < a.VT; vt += a.P) {
    const int v0 = vt * kTile;
    BiasTile<T> bt;
    if (BIAS) bt.fetch((const T*)a.b, a.V, v0, tid);
    if constexpr (sizeof(T) == 2) {
      gemm_tile_bf16_run<true, true, BIAS ? 1 : 0, XFIRST>(acc, A, B, a.H, L, tid, tc);
      if (vt + a.P < a.VT) tc.start(A, v0 + a.P * kTile, B, n0, L, tid);
    } else {
      gemm_tile<T, true, true>(acc, A, v0, B, n0, a.H, L, tid);
    }
    f32x4 bias[8];
    if (BIAS) {
      bt.publish(L.bias, tid, a.logit_scale);
      lds_barrier();
#pragma unroll
      for (int i = 0; i < 8; ++i) bias[i] = read_bias4(L.bias, rloc + 16 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) bias[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int rb = v0 + rloc;
    const bool full = !RAGGED || v0 + kTile <= a.V;
    const bool unit = !BIAS && a.logit_scale == 1.f;   // logits are the accumulators themselves
    acc_drain();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (full && unit) lse_column<SMOOTH, false, true>(acc, j, bias, a.logit_scale, m[j], d[j], sz[j], zy[j], ycol[j] - rb, rb, a.V);
      else if (full) lse_column<SMOOTH, false>(acc, j, bias, a.logit_scale, m[j], d[j], sz[j], zy[j], ycol[j] - rb, rb, a.V);
      else lse_column<SMOOTH, true>(acc, j, bias, a.logit_scale, m[j], d[j], sz[j], zy[j], ycol[j] - rb, rb, a.V);
      // One column at a time keeps the live logits to 32 registers.
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The four lanes l % 16 + 16 g' hold the same tokens (different rows): merge them.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const float m2 = __shfl_xor(m[j], mask), d2 = __shfl_xor(d[j], mask);
      const float s2 = __shfl_xor(sz[j], mask), y2 = __shfl_xor(zy[j], mask);
      merge_md(m[j], d[j], m2, d2);
      sz[j] += s2;
      zy[j] += y2;
    }
  }
  // Then the two waves that share tokens (wm = 0, 1).
  lds_f32x4* red = (lds_f32x4*)L.a[0];
  if (wm == 1 && lane < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wn * kWaveTile + 16 * j + lane] = f32x4{m[j], d[j], sz[j], zy[j]};
  }
  __syncthreads();
  if (wm == 0 && lane < 16) {
    f32x4* part = (f32x4*)a.partials;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 o = red[wn * kWaveTile + 16 * j + lane];
      merge_md(m[j], d[j], o[0], o[1]);
      const int n = n0 + wn * kWaveTile + 16 * j + lane;
      if (n < a.N) part[(int64_t)ph * a.N + n] = f32x4{m[j], d[j], sz[j] + o[2], zy[j] + o[3]};
    }
  }
}

__global__ void __launch_bounds__(256) fwd_combine_kernel(FwdLaunch a) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  const f32x4* part = (const f32x4*)a.partials;
  float m = -INFINITY, d = 0.f, sz = 0.f, zy = 0.f;
  for (int p = 0; p < a.P; ++p) {
    const f32x4 q = part[(int64_t)p * a.N + n];
    merge_md(m, d, q[0], q[1]);
    sz += q[2];
    zy += q[3];
  }
  const float lse = m + logf(d);
  const bool valid = a.targets[n] != a.ignore_index;
  const float zl = valid ? a.s * lse * lse : 0.f;
  const float l = valid ? (lse - (1.f - a.eps) * zy - a.eps_over_v * sz) + zl : 0.f;
  a.lse[n] = lse;
  a.rowloss[n] = l;
  if (a.reduction == kNone) a.loss[n] = l;
  if (a.zloss) {
    a.rowzl[n] = zl;
    if (a.reduction == kNone) a.zloss[n] = zl;
  }
}

// Shard forward: the phases' partials of each token merged into one
// {m, d, sum z, z_y} over the shard's rows (z_y is 0 unless the target lies in
// the shard).
__global__ void __launch_bounds__(256) fwd_stats_kernel(FwdLaunch a) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  const f32x4* part = (const f32x4*)a.partials;
  float m = -INFINITY, d = 0.f, sz = 0.f, zy = 0.f;
  for (int p = 0; p < a.P; ++p) {
    const f32x4 q = part[(int64_t)p * a.N + n];
    merge_md(m, d, q[0], q[1]);
    sz += q[2];
    zy += q[3];
  }
  ((f32x4*)a.stats)[n] = f32x4{m, d, sz, zy};
}

__global__ void __launch_bounds__(1024) fwd_finalize_kernel(FwdLaunch a) {
  __shared__ double ssum[1024];
  __shared__ double zsum[1024];
  __shared__ long long scnt[1024];
  const int tid = threadIdx.x;
  double s = 0.0, z = 0.0;
  long long c = 0;
  for (int n = tid; n < a.N; n += 1024) {
    s += (double)a.rowloss[n];
    if (a.zloss) z += (double)a.rowzl[n];
    c += (a.targets[n] != a.ignore_index) ? 1 : 0;
  }
  ssum[tid] = s;
  zsum[tid] = z;
  scnt[tid] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) {
      ssum[tid] += ssum[tid + w];
      zsum[tid] += zsum[tid + w];
      scnt[tid] += scnt[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const long long T = scnt[0];
    a.n_valid[0] = T;
    if (a.reduction == kSum) a.loss[0] = (float)ssum[0];
    if (a.reduction == kMean) a.loss[0] = T > 0 ? (float)(ssum[0] / (double)T) : 0.f;
    if (a.zloss && a.reduction == kSum) a.zloss[0] = (float)zsum[0];
    if (a.zloss && a.reduction == kMean) a.zloss[0] = T > 0 ? (float)(zsum[0] / (double)T) : 0.f;
  }
}

// Launches without a bias whose tiles are all whole (V and N multiples of
// 256) take the instance without the partial-tile code.  With a bias that
// instance spilled 87-103 VGPRs (the branch had been bounding the compiler's
// scheduling), so biased launches, and fp32 inputs, keep the other one.
template <class T, bool XFIRST>
static void launch_fwd_lse_order(const FwdLaunch& a, hipStream_t st) {
  const int G = a.NT * a.P;
  const bool bias = a.b != nullptr, smooth = a.eps > 0.f;
  const bool whole = sizeof(T) == 2 && a.V % kTile == 0 && a.N % kTile == 0;
  constexpr bool kW = sizeof(T) != 2;   // RAGGED of the whole-tile instance (fp32: none)
  if (bias && smooth) FLCE_LAUNCH((fwd_lse_kernel<T, true, true, XFIRST, true>), dim3(G), dim3(kThreads), 0, st, a);
  else if (bias) FLCE_LAUNCH((fwd_lse_kernel<T, true, false, XFIRST, true>), dim3(G), dim3(kThreads), 0, st, a);
  else if (smooth && whole) FLCE_LAUNCH((fwd_lse_kernel<T, false, true, XFIRST, kW>), dim3(G), dim3(kThreads), 0, st, a);
  else if (smooth) FLCE_LAUNCH((fwd_lse_kernel<T, false, true, XFIRST, true>), dim3(G), dim3(kThreads), 0, st, a);
  else if (whole) FLCE_LAUNCH((fwd_lse_kernel<T, false, false, XFIRST, kW>), dim3(G), dim3(kThreads), 0, st, a);
  else FLCE_LAUNCH((fwd_lse_kernel<T, false, false, XFIRST, true>), dim3(G), dim3(kThreads), 0, st, a);
}

template <class T>
static void launch_fwd_lse(const FwdLaunch& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (a.P >= 4) launch_fwd_lse_order<T, true>(a, st);
    else launch_fwd_lse_order<T, false>(a, st);
  } else {
    launch_fwd_lse_order<T, false>(a, st);   // fp32 operands are staged through registers, not by block copies
  }
}

template <class T>
static hipError_t launch_forward_t(const FwdLaunch& a, hipStream_t st) {
  launch_fwd_lse<T>(a, st);
  FLCE_LAUNCH(fwd_combine_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  FLCE_LAUNCH(fwd_finalize_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdLaunch& a, int dtype, hipStream_t st) {
  if (dtype == 1) return launch_forward_t<uint16_t>(a, st);
  if (dtype == 2) return launch_forward_t<_Float16>(a, st);
  return launch_forward_t<float>(a, st);
}

template <class T>
static hipError_t launch_shard_forward_t(const FwdLaunch& a, hipStream_t st) {
  launch_fwd_lse<T>(a, st);
  FLCE_LAUNCH(fwd_stats_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_shard_forward(const FwdLaunch& a, int dtype, hipStream_t st) {
  if (dtype == 1) return launch_shard_forward_t<uint16_t>(a, st);
  if (dtype == 2) return launch_shard_forward_t<_Float16>(a, st);
  return launch_shard_forward_t<float>(a, st);
}

hipError_t launch_merge(const FwdLaunch& a, hipStream_t st) {
  FLCE_LAUNCH(fwd_combine_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  FLCE_LAUNCH(fwd_finalize_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------

// Per-token dlogits coefficient c_n: the upstream gradient (per token for
// reduction none), divided by the non-ignored count for mean, times the
// logits' scale (the gradient of the raw logits); 0 for ignored rows.
__device__ __forceinline__ float token_coef(const BwdLaunch& a, int n, bool valid) {
  const float g = a.reduction == kNone ? a.grad[n] : a.grad[0];
  const long long T = a.n_valid[0];
  float c = g;
  if (a.reduction == kMean) c = T > 0 ? g / (float)T : 0.f;
  if (!valid) c = 0.f;
  return c * a.logit_scale;
}

// fp16 inputs: the dlogits slab holds dz * S, with S a power of two chosen
// so that the largest possible |dz * S| is at most 2^14.  |dz_nj| <= |c_n|
// (|1 + 2 s lse_n| + eps / V + 1 - eps), and |c_n| is about g / T for the
// mean: at the Llama-3-sized head an unscaled dz of c_n p ~ 1e-9 would
// underflow fp16 (smallest subnormal 6e-8).  The slab's products are scaled
// back by 1/S (exact) in the dx, dW and db epilogues.  One block; writes
// gscale = {S, 1/S}.
__global__ void __launch_bounds__(1024) bwd_scale_kernel(BwdLaunch a) {
  __shared__ float smax[1024];
  const int tid = threadIdx.x;
  float mx = 0.f;
  for (int n = tid; n < a.N; n += 1024) {
    const bool valid = a.targets[n] != a.ignore_index;
    const float c = fabsf(token_coef(a, n, valid));
    const float bound = c * (fabsf(1.f + 2.f * a.s * a.lse[n]) + a.eps_over_v + (1.f - a.eps));
    if (valid && bound > mx) mx = bound;   // NaN bounds are skipped
  }
  smax[tid] = mx;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) smax[tid] = fmaxf(smax[tid], smax[tid + w]);
    __syncthreads();
  }
  if (tid == 0) {
    float S = 1.f;
    const float m = smax[0];
    if (m > 0.f && m <= 3.0e38f) {
      int e;
      (void)frexpf(m, &e);                 // m <= 2^e
      int k = 14 - e;
      k = k > 126 ? 126 : (k < -126 ? -126 : k);
      S = ldexpf(1.f, k);
    }
    a.gscale[0] = S;
    a.gscale[1] = 1.f / S;
  }
}

__global__ void __launch_bounds__(256) bwd_coef_kernel(BwdLaunch a) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  const int64_t t = a.targets[n];
  const bool valid = t != a.ignore_index;
  float c = token_coef(a, n, valid);
  if (a.gscale) c *= a.gscale[0];   // fp16: the slab holds dz * S
  const float lse = a.lse[n];
  ((f32x4*)a.coef)[n] = f32x4{c * (1.f + 2.f * a.s * lse), c * a.eps_over_v, c * (1.f - a.eps), lse * kLog2e};
  const int64_t lt = t - a.vocab_start;   // row of W holding the target, if any
  a.yv[n] = (valid && lt >= 0 && lt < a.V) ? (int)lt : -1;
}

// Sums over the 16 lanes of a lane group (lane / 16).  A step halves the
// values a lane holds: DPP control CTRL pairs every lane with one whose
// lane-id bit MASK differs and whose higher bits agree (row mirror for bit 3,
// half-row mirror for bit 2, quad permutations for bits 1 and 0), and the
// lane with the bit set keeps the upper half.
template <int COUNT, int MASK, int CTRL>
__device__ __forceinline__ void xreduce_step(float (&v)[8], int lane) {
  const bool up = (lane & MASK) != 0;
#pragma unroll
  for (int k = 0; k < COUNT / 2; ++k) {
    const float keep = up ? v[COUNT / 2 + k] : v[k];
    const float send = up ? v[k] : v[COUNT / 2 + k];
    v[k] = keep + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), CTRL,
                                                                       0xf, 0xf, false));
  }
}

// Group total of value q = (lane % 16) / 2 of 8 per-lane values, returned to
// lanes 2q and 2q + 1 of every group.
__device__ __forceinline__ float group_sum8(float (&v)[8], int lane) {
  xreduce_step<8, 8, 0x140>(v, lane);   // row_mirror: l <-> 15 - l
  xreduce_step<4, 4, 0x141>(v, lane);   // row_half_mirror: l <-> l ^ 7
  xreduce_step<2, 2, 0x4e>(v, lane);    // quad_perm [2, 3, 0, 1]: l <-> l ^ 2
  return v[0] + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[0]), 0xb1, 0xf,
                                                                      0xf, false));   // l <-> l ^ 1
}

// Per-token data of a tile's 256 tokens: thread t fetches token n0 + t
// before the mainloop (two loads; tokens past N get c = 0 and an infinite
// log-sum-exp so their dlogits are 0) and publishes it to LDS after it.
struct TokenTile {
  f32x4 cf;   // {c (1 + 2 s lse), c eps / V, c (1 - eps), lse log2 e}
  int y;      // target, -1 if ignored
  __device__ __forceinline__ void fetch(const BwdLaunch& a, int n0, int tid) {
    const bool ok = n0 + tid < a.N;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc((const f32x4*)a.coef + n0);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.yv + n0);
    const f32x4 c = __builtin_bit_cast(f32x4, buf_load16(rc, ok ? (uint32_t)tid * 16u : kOOB));
    const int t = (int)__builtin_amdgcn_raw_buffer_load_b32(ry, ok ? (uint32_t)tid * 4u : kOOB, 0, 0);
    cf = ok ? c : f32x4{0.f, 0.f, 0.f, INFINITY};
    y = ok ? t : -1;
  }
  __device__ __forceinline__ void publish(lds_f32x4* lc, __attribute__((address_space(3))) int* ly, int tid) const {
    lc[tid] = cf;
    ly[tid] = y;
  }
};

// First tile row of lane group g's four rows in MFMA block i, W's rows
// being the tile rows.  16-bit tiles copy W with permuted rows
// (tile_row_perm), so a lane's values in blocks 2s and 2s + 1 of a token
// column are eight consecutive vocabulary rows; fp32 tiles keep the MFMA row
// order (two runs of four rows, 16 apart).
template <class T>
__device__ __forceinline__ constexpr int dz_row(int i, int g) {
  return sizeof(T) == 2 ? 32 * (i >> 1) + 8 * g + 4 * (i & 1) : 16 * i + 4 * g;
}

// One tile of the recompute kernel for fp32 inputs, W's rows as the tile
// rows.  EXTRA is unused: fp32 tiles copy through registers.

template <class T, bool BIAS, bool DB, bool RAGGED, int EXTRA>
__device__ __forceinline__ void dz_tile(const BwdLaunch& a, int vs, int TM, int G, int t, TileCopy<true, true>& tc,
                                        const Lds& L, lds_f32* red, lds_f32x4* ltok, __attribute__((address_space(3))) int* lyv,
                                        int tid) {
  static_assert(sizeof(T) == 4, "16-bit inputs use dz_tile_t");
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
  const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};
  const int g = lane >> 4;
  int tm, tn;
  tile_coords(t, G, TM, a.NT, tm, tn);
  const int v0 = vs + tm * kTile, n0 = tn * kTile;
  TokenTile tt;
  tt.fetch(a, n0, tid);
  BiasTile<T> bt;
  if (BIAS) bt.fetch((const T*)a.b, a.V, v0, tid);
  Acc acc;
  (void)tc;
  gemm_tile<T, true, true>(acc, A, v0, B, n0, a.H, L, tid);
  tt.publish(ltok, lyv, tid);
  if (BIAS) bt.publish(L.bias, tid);
  lds_barrier();
  acc_drain();
  // Vocabulary rows past V read W and b as zeros; their dlogits are stored as
  // exact zeros.  The input-gradient product reads the slab up to the next
  // multiple of 8 columns (whole 16-byte copies), and the unmasked value of
  // such a row, c (1 + 2 s lse) e^(-lse), overflows to inf when lse is very
  // negative (a large negative bias; sooner with fp16's scaled slab), which
  // times W's zero rows would give NaN.  Only the vocabulary's last tile is
  // ragged (vleft < 256), so the mask is a wave-uniform branch.
  const int vleft = a.V - v0;
  const float sl2e = a.logit_scale * kLog2e;   // p = 2^((scale (z + b)) log2 e - lse log2 e)
  // Bands s of 32 wave rows (blocks 2s, 2s + 1), token blocks j within them:
  // dlogits of the lane's token (16 j + l % 16) at its rows r0 .. r0 + 3 and
  // r1 .. r1 + 3 (tile-relative), the band's db row sums, and the slab store.
  // A band's row sums are reduced over the lane group as soon as the band is
  // done, so few stay live.
  float dbs[4];
  const bool ragged = RAGGED && vleft < kTile;   // wave-uniform
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r0 = wm * kWaveTile + dz_row<T>(2 * s, g), r1 = wm * kWaveTile + dz_row<T>(2 * s + 1, g);
    const f32x4 bias0 = BIAS ? read_bias4(L.bias, r0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 bias1 = BIAS ? read_bias4(L.bias, r1) : f32x4{0.f, 0.f, 0.f, 0.f};
    float rs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rs[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int nl = wn * kWaveTile + 16 * j + (lane & 15);   // token within the tile
      const f32x4 cf = ltok[nl];
      const int y = lyv[nl];
      const f32x4 z0 = acc_read4(acc[2 * s][j]);
      const f32x4 z1 = acc_read4(acc[2 * s + 1][j]);
      float dz[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // Without a bias the accumulator is the logit (an added zero could
        // not be folded away: it would turn -0 into +0).
        const float a0 = BIAS ? z0[r] + bias0[r] : z0[r];
        const float a1 = BIAS ? z1[r] + bias1[r] : z1[r];
        dz[r] = fmaf(cf[0], fast_exp2(fmaf(a0, sl2e, -cf[3])), -cf[1]);
        dz[4 + r] = fmaf(cf[0], fast_exp2(fmaf(a1, sl2e, -cf[3])), -cf[1]);
      }
      {
        const int t0 = y - (v0 + r0), t1 = y - (v0 + r1);
        if (__ballot((unsigned)t0 < 4u || (unsigned)t1 < 4u)) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (t0 == r) dz[r] -= cf[2];
            if (t1 == r) dz[4 + r] -= cf[2];
          }
        }
      }
      if (ragged) {
        const int lim0 = vleft - r0, lim1 = vleft - r1;   // rows of each run inside the vocabulary
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (r >= lim0) dz[r] = 0.f;
          if (r >= lim1) dz[4 + r] = 0.f;
        }
      }
      if (DB) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rs[e] += dz[e];
      }
      if (n0 + nl < a.N) {
        T* row = (T*)a.slab + (int64_t)(n0 + nl) * a.ldS + (v0 - vs);
        store4<T>(row + r0, dz[0], dz[1], dz[2], dz[3]);
        store4<T>(row + r1, dz[4], dz[5], dz[6], dz[7]);
      }
    }
    if (DB) dbs[s] = group_sum8(rs, lane);
  }

  if (DB) {
    // Lanes 2q, 2q + 1 of group g hold band s's total of value q: tile row
    // r0 + q (q < 4) or r1 + q - 4.  The two waves that share rows (wn = 0, 1)
    // add through LDS; the next tile's mainloop barriers keep this tile's
    // reads of red ahead of the next tile's writes.
    const int q = (lane & 15) >> 1;
    const bool lead = (lane & 1) == 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = wm * kWaveTile + dz_row<T>(2 * s + (q >> 2), g) + (q & 3);
      if (wn == 1 && lead) red[row] = dbs[s];
    }
    lds_barrier();
    if (wn == 0 && lead) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rl = wm * kWaveTile + dz_row<T>(2 * s + (q >> 2), g) + (q & 3);
        if (v0 + rl < a.V) a.dbp[(int64_t)tn * a.ldS + (v0 - vs) + rl] = dbs[s] + red[rl];
      }
    }
  }
}

// One tile of the recompute kernel for 16-bit inputs, with the product's
// operands the other way round from the forward's: rows are tokens (A = x)
// and columns vocabulary rows (B = W, copied with permuted columns,
// tile_col_perm), so a lane holds, for each of its 32 tokens (blocks i, rows
// r), eight consecutive vocabulary rows 8 c .. 8 c + 7 of its wave's half
// (c = lane % 16) across the blocks j.  One 16-byte store then covers those
// rows of one token, and a wave instruction writes 4 tokens x 256 bytes
// (whole lines) instead of 16 tokens x 64 bytes.  The db row sums accumulate
// over the lane's tokens in fixed-order adds (as plain += the compiler
// restructured them and spilled about 50 VGPRs) and are reduced once per
// tile.  Same-box A/Bs against the forward's orientation: recompute -1.9%
// without db partials (N=8192, H=4096, V=128256, first slab kept), -0.7% to
// -1.9% at N=16384, H=1024 and N=4096, H=2048; with them (the same shapes
// with a bias) -1.3% to -1.6%, and -2.1% at N=32768, H=2048, V=128000;
// bit-identical dlogits.
//
// RAGGED: the launch holds a partial vocabulary tile (the slab's width not a
// multiple of 256) or partial token tiles (N not a multiple of 256).  Without
// it every tile is whole and the row masks and token checks compile away: the
// compiler hoisted the mask's eight compares per token row out of their
// wave-uniform branch, one VALU operation per dlogit in every tile.
template <class T, bool BIAS, bool DB, bool RAGGED, int EXTRA>
__device__ __forceinline__ void dz_tile_t(const BwdLaunch& a, int vs, int TM, int G, int t, TileCopy<true, true>& tc,
                                          const Lds& L, lds_f32* red, lds_f32x4* ltok,
                                          __attribute__((address_space(3))) int* lyv, int tid) {
  static_assert(sizeof(T) == 2, "16-bit inputs");
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const Opnd<T> A{(const T*)a.x, a.H, a.N, a.H};
  const Opnd<T> B{(const T*)a.W, a.H, a.V, a.H};
  const int g = lane >> 4, c = lane & 15;
  int tm, tn;
  tile_coords(t, G, TM, a.NT, tm, tn);
  const int v0 = vs + tm * kTile, n0 = tn * kTile;
  TokenTile tt;
  tt.fetch(a, n0, tid);
  BiasTile<T> bt;
  if (BIAS) bt.fetch((const T*)a.b, a.V, v0, tid);
  Acc acc;
  gemm_tile_bf16_run<true, true, EXTRA, true>(acc, A, B, a.H, L, tid, tc);
  const int tnext = t + gridDim.x;
  if (tnext < G) {
    int tm2, tn2;
    tile_coords(tnext, G, TM, a.NT, tm2, tn2);
    tc.start(A, tn2 * kTile, B, vs + tm2 * kTile, L, tid, false, true);
  }
  tt.publish(ltok, lyv, tid);
  if (BIAS) bt.publish(L.bias, tid);
  lds_barrier();
  acc_drain();
  const int vleft = a.V - v0;
  const bool ragged = RAGGED && vleft < kTile;   // wave-uniform
  const __amdgpu_buffer_rsrc_t rslab = make_rsrc((const T*)a.slab + (int64_t)n0 * a.ldS);
  const float sl2e = a.logit_scale * kLog2e;
  const int vl0 = wn * kWaveTile + 8 * c;   // this lane's vocabulary rows vl0 .. vl0 + 7 (tile-relative)
  // Store offset of token row lane_row + tr: the lane's part in the vector
  // offset, the row's (16 i + r, the same for every lane) in the scalar one.
  // The slab is at most 1 GiB, so rows before N stay below 2^30 bytes; rows
  // at or past N take kOOB (dropped) and a scalar offset of 0.
  const uint32_t rowbytes = (uint32_t)(a.ldS * (int64_t)sizeof(T));
  const int lane_row = wm * kWaveTile + 4 * g;
  const int rows_left = a.N - n0;
  const uint32_t vbase = (uint32_t)lane_row * rowbytes + (uint32_t)((v0 - vs + vl0) * (int)sizeof(T));
  f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = {0.f, 0.f, 0.f, 0.f};
  if (BIAS) {
    b0 = read_bias4(L.bias, vl0);
    b1 = read_bias4(L.bias, vl0 + 4);
  }
  float rs[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rs[j] = 0.f;
  auto row_dz = [&](int i, auto rr, float (&dz)[8], const f32x4& cf) {
    constexpr int R = decltype(rr)::value;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float bj = j < 4 ? b0[j] : b1[j - 4];
      const float z = acc_read1<R>(acc[i][j]);
      const float av = BIAS ? z + bj : z;
      dz[j] = fmaf(cf[0], fast_exp2(fmaf(av, sl2e, -cf[3])), -cf[1]);
    }
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nl = wm * kWaveTile + 16 * i + 4 * g + r;   // token within the tile
      const f32x4 cf = ltok[nl];
      const int y = lyv[nl];
      float dz[8];
      if (r == 0) row_dz(i, std::integral_constant<int, 0>{}, dz, cf);
      else if (r == 1) row_dz(i, std::integral_constant<int, 1>{}, dz, cf);
      else if (r == 2) row_dz(i, std::integral_constant<int, 2>{}, dz, cf);
      else row_dz(i, std::integral_constant<int, 3>{}, dz, cf);
      const int tg = y - (v0 + vl0);
      if (__ballot((unsigned)tg < 8u)) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (tg == k) dz[k] -= cf[2];
      }
      if (ragged) {
        const int lim = vleft - vl0;   // rows of this lane inside the vocabulary
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k >= lim) dz[k] = 0.f;
      }
      if (DB) {
#pragma unroll
        for (int k = 0; k < 8; ++k) add_pinned(rs[k], dz[k]);
      }
      const int tr = 16 * i + r;
      const uint32_t voff = !RAGGED || lane_row + tr < rows_left ? vbase : kOOB;
      const int soff = !RAGGED || tr < rows_left ? (int)((uint32_t)tr * rowbytes) : 0;
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{pack2<T>(dz[0], dz[1]), pack2<T>(dz[2], dz[3]), pack2<T>(dz[4], dz[5]), pack2<T>(dz[6], dz[7])},
          rslab, voff, soff, kSlabPolicy);

    }
  }
  if (DB) {
    // Lanes c, c + 16, c + 32, c + 48 hold the same rows; then the two waves
    // sharing rows (wm = 0, 1) add through LDS.  The next tile's mainloop
    // barriers keep this tile's reads of red ahead of the next tile's writes.
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      rs[k] += __shfl_xor(rs[k], 16);
      rs[k] += __shfl_xor(rs[k], 32);
    }
    if (wm == 1 && g == 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) red[vl0 + k] = rs[k];
    }
    lds_barrier();
    // Columns past V (inside the slab's padded width) get exact zeros, which
    // the db sums never read.
    if (wm == 0 && g == 0) {
      const __amdgpu_buffer_rsrc_t rdb = make_rsrc(a.dbp + (int64_t)tn * a.ldS + (v0 - vs));
      const f32x4 r0 = read_bias4(red, vl0), r1 = read_bias4(red, vl0 + 4);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, f32x4{rs[0] + r0[0], rs[1] + r0[1], rs[2] + r0[2], rs[3] + r0[3]}), rdb,
          (uint32_t)vl0 * 4u, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, f32x4{rs[4] + r1[0], rs[5] + r1[1], rs[6] + r1[2], rs[7] + r1[3]}), rdb,
          (uint32_t)(vl0 + 4) * 4u, 0, 0);
    }
  }
}

// Persistent over the slab's tiles (TM vocabulary tiles x NT token tiles): a
// workgroup takes logical tiles blockIdx.x, + gridDim.x, ..., so the tiles in
// flight together are the ones a one-tile-per-workgroup launch would run
// together (same XCD mapping), and each tile's first copies are issued while
// the previous tile's epilogue runs.  The first tile is peeled: only later
// tiles start with the previous tile's slab stores still in flight.
template <class T, bool BIAS, bool DB, bool RAGGED>
__global__ void __launch_bounds__(kThreads, 1) bwd_dz_kernel(BwdLaunch a, int vs, int TM) {
  FLCE_LDS(L, T);
  __shared__ __attribute__((aligned(16))) float red_s[kTile];       // db: the two waves sharing rows
  __shared__ __attribute__((aligned(16))) f32x4 tok_s[kTile];       // per-token coefficients
  __shared__ __attribute__((aligned(16))) int yv_s[kTile];          // per-token targets
  lds_f32* red = (lds_f32*)red_s;
  const int tid = threadIdx.x;
  const int G = TM * a.NT;
  TileCopy<true, true> tc;
  int t = blockIdx.x;
  if constexpr (sizeof(T) == 2) {   // dz_tile_t: x rows, W columns (permuted)
    const Opnd<T> A{(const T*)a.x, a.H, a.N, a.H};
    const Opnd<T> B{(const T*)a.W, a.H, a.V, a.H};
    int tm, tn;
    tile_coords(t, G, TM, a.NT, tm, tn);
    tc.start(A, tn * kTile, B, vs + tm * kTile, L, tid, false, true);
  }
  // Vector-memory instructions every wave issues between starting a tile's
  // copies and its mainloop: the per-token loads (2) and the bias fetch, plus,
  // after the first tile, the previous tile's slab stores (32).
  constexpr int kLoadsVm = 2 + (BIAS ? 1 : 0);
  constexpr int kStoresVm = 32;
  lds_f32x4* ltok = (lds_f32x4*)tok_s;
  __attribute__((address_space(3))) int* lyv = (__attribute__((address_space(3))) int*)yv_s;
  if constexpr (sizeof(T) == 2) {
    dz_tile_t<T, BIAS, DB, RAGGED, kLoadsVm>(a, vs, TM, G, t, tc, L, red, ltok, lyv, tid);
    for (t += gridDim.x; t < G; t += gridDim.x)
      dz_tile_t<T, BIAS, DB, RAGGED, kLoadsVm + kStoresVm>(a, vs, TM, G, t, tc, L, red, ltok, lyv, tid);
  } else {
    dz_tile<T, BIAS, DB, RAGGED, kLoadsVm>(a, vs, TM, G, t, tc, L, red, ltok, lyv, tid);
    for (t += gridDim.x; t < G; t += gridDim.x)
      dz_tile<T, BIAS, DB, RAGGED, kLoadsVm + kStoresVm>(a, vs, TM, G, t, tc, L, red, ltok, lyv, tid);
  }
}

// db[vs + c] = sum over token tiles of the slab's db partials (fixed order),
// for slab column c < width.
template <class T>
__device__ __forceinline__ void slab_db(const BwdLaunch& a, int vs, int width, int c) {
  if (c >= width) return;
  float s = 0.f;
  for (int t = 0; t < a.NT; ++t) s += a.dbp[(int64_t)t * a.ldS + c];
  if constexpr (IsF16<T>::value) s *= a.gscale[1];   // partials of dz * S
  if constexpr (sizeof(T) == 4) {
    float* p = (float*)a.db + vs + c;
    *p = a.accumulate ? *p + s : s;
  } else {
    uint16_t* p = (uint16_t*)a.db + vs + c;
    if (a.accumulate) s += h16_to_f32<T>(*p);
    *p = (uint16_t)(pack2<T>(s, 0.f) & 0xffffu);
  }
}

// Four consecutive output values added to what p holds (accumulate mode).
template <class T> __device__ __forceinline__ f32x4 load4(const T* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) { return *(const f32x4*)p; }
template <> __device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p) {
  const u32x2 v = *(const u32x2*)p;
  return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
               __uint_as_float(v[1] & 0xffff0000u)};
}
template <> __device__ __forceinline__ f32x4 load4<_Float16>(const _Float16* p) {
  const u32x2 v = *(const u32x2*)p;
  return f32x4{f16_bits_to_f32(v[0]), f16_bits_to_f32(v[0] >> 16), f16_bits_to_f32(v[1]), f16_bits_to_f32(v[1] >> 16)};
}

// dW[vs + v, h] for the slab: C[h][v] = sum_n x[n][h] dz[n][v].  ACC: added
// to what dW holds.
template <class T, bool ACC>
__global__ void __launch_bounds__(kThreads, 1) bwd_dw_kernel(BwdLaunch a, int vs, int width, int wpad, int TM,
                                                             int TN) {
  FLCE_LDS(L, T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, TM, TN, tm, tn);
  const int h0 = tm * kTile, v0 = tn * kTile;
  // The workgroups of the first H tile also finish db for their 256 columns.
  if (a.db != nullptr && tm == 0) slab_db<T>(a, vs, width, v0 + tid);
  const Opnd<T> A{(const T*)a.x, a.H, a.H, a.N};
  const Opnd<T> B{(const T*)a.slab, a.ldS, wpad, a.N};
  Acc acc;
  gemm_tile<T, false, false>(acc, A, h0, B, v0, a.N, L, tid);
  const float inv = IsF16<T>::value ? a.gscale[1] : 1.f;   // fp16: the slab holds dz * S
  acc_drain();
  T* dW = (T*)a.dW;
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int v = v0 + wn * kWaveTile + 16 * j + (lane & 15);
    T* rowp = dW + (int64_t)(vs + v) * a.H;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 z = acc_read4(acc[i][j]);
      if constexpr (IsF16<T>::value) z *= inv;
      const int h = h0 + wm * kWaveTile + 16 * i + 4 * g;
      if (v < width && h < a.H) {
        if (ACC) z += load4<T>(rowp + h);
        store4<T>(rowp + h, z[0], z[1], z[2], z[3]);
      }
    }
  }
}

// dx[n, h] += sum_{v in slab} dz[n][v] W[vs + v][h]: C[h][n].  MODE says
// whether the fp32 accumulator is written (first slab), read and written
// (middle slabs), read with dx written in its dtype (last slab), or skipped
// (a single slab).  The epilogue is branch-free (buffer accesses with
// out-of-range offsets for rows past N or columns past H) and reads the
// accumulator kAhead blocks ahead of adding and storing it, so the
// read-modify-write does not wait once per 16 bytes.
template <class T>
__device__ __forceinline__ void store4_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3])}, r, off, 0, 0);
  }
}

template <class T>
__device__ __forceinline__ f32x4 load4_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(f32x4, buf_load16(r, off));
  } else {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return f32x4{h16_to_f32<T>(v[0]), h16_to_f32<T>(v[0] >> 16), h16_to_f32<T>(v[1]), h16_to_f32<T>(v[1] >> 16)};
  }
}

// ACC (modes that write dx in its dtype): dx is added to what it holds; its
// old values are loaded ahead with the accumulator's.
//
// K split (a.dx_split parts, when the output has too few tiles to fill the
// CUs): workgroup b computes tile b % G over the slab columns
// [p kc, (p + 1) kc) of part p = b / G into accumulator p, in the First or
// Accum mode; a part past the slab's columns reads only zeros (its operands'
// valid K is 0), so it still writes or keeps its accumulator.
//
// SPLIT (16-bit T, one part): the accumulator is split as a.split_acc
// describes, high halves in dx, low halves in a.dx_acc; an fp32 value is
// exactly (high << 16) | low, so nothing is rounded before the last slab.
// With ACC, dx's old values are added in the First mode, before the first
// high halves overwrite them.
template <class T, int MODE, bool ACC, bool SPLIT = false>
__global__ void __launch_bounds__(kThreads, 1) bwd_dx_kernel(BwdLaunch a, int vs, int width, int wpad, int TM,
                                                             int kc) {
  static_assert(!SPLIT || sizeof(T) == 2, "split accumulators hold fp32 values in two 16-bit halves");
  FLCE_LDS(L, T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int G = TM * a.NT;
  const int part = blockIdx.x / G;
  int tm, tn;
  tile_coords(blockIdx.x - part * G, G, TM, a.NT, tm, tn);
  const int h0 = tm * kTile, n0 = tn * kTile;
  const int k0 = part * kc;
  const bool live = k0 < wpad;
  const int kw = live ? min(width - k0, kc) : 0;     // valid W rows of this part (may be <= 0)
  const int kp = live ? min(wpad - k0, kc) : 0;      // slab columns of this part
  const Opnd<T> A{(const T*)a.W + (int64_t)(vs + (live ? k0 : 0)) * a.H, a.H, a.H, kw > 0 ? kw : 0};
  const Opnd<T> B{(const T*)a.slab + (live ? k0 : 0), a.ldS, a.N, kp};
  Acc acc;
  gemm_tile<T, false, true>(acc, A, h0, B, n0, kp > 0 ? kp : 1, L, tid);   // K >= 1: an empty part sums zeros

  constexpr bool kRead = MODE == kDxAccum || MODE == kDxLast;
  constexpr bool kAcc = MODE == kDxFirst || MODE == kDxAccum;   // write the fp32 accumulator
  // Descriptors start at token row n0, so offsets stay below 256 * H * 4 bytes.
  const __amdgpu_buffer_rsrc_t racc =
      SPLIT ? make_rsrc((const uint16_t*)a.dx_acc + (int64_t)n0 * a.H)
            : make_rsrc(a.dx_acc + (int64_t)part * a.N * a.H + (int64_t)n0 * a.H);
  const __amdgpu_buffer_rsrc_t rdx = make_rsrc((const T*)a.dx + (int64_t)n0 * a.H);
  const int g = lane >> 4;
  // Byte offset of block b = 8 j + i (row n = n0 + nl, columns h .. h + 3)
  // for elements of es bytes; kOOB past N or H.
  auto boff = [&](int b, uint32_t es) -> uint32_t {
    const int i = b & 7, j = b >> 3;
    const int nl = wn * kWaveTile + 16 * j + (lane & 15);
    const int h = h0 + wm * kWaveTile + 16 * i + 4 * g;
    return (n0 + nl < a.N && h < a.H) ? (uint32_t)(nl * a.H + h) * es : kOOB;
  };
  const float inv = IsF16<T>::value ? a.gscale[1] : 1.f;   // fp16: the slab holds dz * S
  acc_drain();
  // Loads run kAhead blocks ahead (12 x 1 KB in flight per wave), about what
  // one CU's share of HBM bandwidth needs while every CU makes its
  // read-modify-write at the same moment.
  constexpr int kAhead = 12;
  if constexpr (SPLIT) {
    // Pairs of blocks 2q, 2q + 1 (columns h and h + 16 of one token).
    // v_permlane16_swap trades value r of block 2q held by lane groups
    // g = 1, 3 for value r of block 2q + 1 held by groups g = 0, 2 (lanes 16
    // apart, same token), after which a lane holds eight consecutive columns:
    // block 2q's from 4g (g even) or block 2q + 1's from 16 + 4(g - 1) (g odd).
    // Each half of the accumulator then moves in one 16-byte access.
    constexpr int kAheadP = kAhead / 2;
    constexpr bool kOld = ACC && MODE == kDxFirst;   // dx's old values, before its first overwrite
    auto poff = [&](int q) -> uint32_t {
      const int i = (2 * q) & 7, j = (2 * q) >> 3;
      const int nl = wn * kWaveTile + 16 * j + (lane & 15);
      const int h = h0 + wm * kWaveTile + 16 * i + 4 * (g & 2) + 16 * (g & 1);
      return (n0 + nl < a.N && h < a.H) ? (uint32_t)(nl * a.H + h) * 2u : kOOB;   // H % 8 == 0: all 8 or none
    };
    u32x4 hi[kAheadP + 1], lo[kAheadP + 1], ox[kAheadP + 1];
    auto fetch = [&](int q) {
      const uint32_t off = poff(q);
      if (kRead) {
        hi[q % (kAheadP + 1)] = __builtin_bit_cast(u32x4, buf_load16(rdx, off));
        lo[q % (kAheadP + 1)] = __builtin_bit_cast(u32x4, buf_load16(racc, off));
      }
      if (kOld) ox[q % (kAheadP + 1)] = __builtin_bit_cast(u32x4, buf_load16(rdx, off));
    };
#pragma unroll
    for (int q = 0; q < kAheadP; ++q) fetch(q);
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      if (q + kAheadP < 32) fetch(q + kAheadP);
      const int i = (2 * q) & 7, j = (2 * q) >> 3;
      f32x4 v0 = acc_read4(acc[i][j]), v1 = acc_read4(acc[i + 1][j]);
      if constexpr (IsF16<T>::value) {
        v0 *= inv;
        v1 *= inv;
      }
      float w[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0[r]), __float_as_uint(v1[r]), false, false);
        w[r] = __uint_as_float(sw[0]);
        w[4 + r] = __uint_as_float(sw[1]);
      }
      if (kRead) {
        // element 2k's bits: the low halves of word k of each part; 2k + 1's: the high halves
        const u32x4 h = hi[q % (kAheadP + 1)], l = lo[q % (kAheadP + 1)];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          w[2 * k] += __uint_as_float((h[k] << 16) | (l[k] & 0xffffu));
          w[2 * k + 1] += __uint_as_float((h[k] & 0xffff0000u) | (l[k] >> 16));
        }
      }
      if (kOld) {
        const u32x4 o = ox[q % (kAheadP + 1)];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          w[2 * k] += h16_to_f32<T>(o[k]);
          w[2 * k + 1] += h16_to_f32<T>(o[k] >> 16);
        }
      }
      const uint32_t off = poff(q);
      if (kAcc) {
        u32x4 hw, lw;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t u0 = __float_as_uint(w[2 * k]), u1 = __float_as_uint(w[2 * k + 1]);
          hw[k] = (u0 >> 16) | (u1 & 0xffff0000u);
          lw[k] = (u0 & 0xffffu) | (u1 << 16);
        }
        __builtin_amdgcn_raw_buffer_store_b128(hw, rdx, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(lw, racc, off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack2<T>(w[0], w[1]), pack2<T>(w[2], w[3]), pack2<T>(w[4], w[5]), pack2<T>(w[6], w[7])}, rdx, off,
            0, 0);
      }
    }
  } else {
    constexpr bool kOld = ACC && !kAcc;   // read the dx being added to
    f32x4 old[kAhead + 1], oldx[kAhead + 1];
#pragma unroll
    for (int b = 0; b < kAhead; ++b) {
      if (kRead) old[b] = __builtin_bit_cast(f32x4, buf_load16(racc, boff(b, 4u)));
      if (kOld) oldx[b] = load4_buf<T>(rdx, boff(b, (uint32_t)sizeof(T)));
    }
#pragma unroll
    for (int b = 0; b < 64; ++b) {
      const int bn = b + kAhead;
      if (kRead && bn < 64) old[bn % (kAhead + 1)] = __builtin_bit_cast(f32x4, buf_load16(racc, boff(bn, 4u)));
      if (kOld && bn < 64) oldx[bn % (kAhead + 1)] = load4_buf<T>(rdx, boff(bn, (uint32_t)sizeof(T)));
      f32x4 v = acc_read4(acc[b & 7][b >> 3]);
      if constexpr (IsF16<T>::value) v *= inv;
      if (kRead) v += old[b % (kAhead + 1)];
      if (kOld) v += oldx[b % (kAhead + 1)];
      if (kAcc) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), racc, boff(b, 4u), 0, 0);
      } else {
        store4_buf<T>(rdx, boff(b, (uint32_t)sizeof(T)), v);
      }
    }
  }
}

// dx from the K-split accumulators: thread i sums four consecutive elements
// of every part in part order (plus dx's old values when accumulating).
template <class T, bool ACC>
__global__ void __launch_bounds__(256) bwd_dx_finalize_kernel(BwdLaunch a) {
  const int64_t n4 = (int64_t)a.N * a.H / 4;
  const int64_t stride = (int64_t)a.N * a.H;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 v = ((const f32x4*)a.dx_acc)[i];
    for (int p = 1; p < a.dx_split; ++p) v += ((const f32x4*)(a.dx_acc + p * stride))[i];
    T* d = (T*)a.dx + 4 * i;
    if (ACC) v += load4<T>(d);
    store4<T>(d, v[0], v[1], v[2], v[3]);
  }
}

hipError_t launch_bwd_dx_finalize(const BwdLaunch& a, int dtype, hipStream_t st) {
  const int64_t n4 = (int64_t)a.N * a.H / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4 * kPersistGrid) blocks = 4 * kPersistGrid;
  const dim3 grid((unsigned)blocks), blk(256);
  if (dtype == 1) {
    if (a.accumulate) FLCE_LAUNCH((bwd_dx_finalize_kernel<uint16_t, true>), grid, blk, 0, st, a);
    else FLCE_LAUNCH((bwd_dx_finalize_kernel<uint16_t, false>), grid, blk, 0, st, a);
  } else if (dtype == 2) {
    if (a.accumulate) FLCE_LAUNCH((bwd_dx_finalize_kernel<_Float16, true>), grid, blk, 0, st, a);
    else FLCE_LAUNCH((bwd_dx_finalize_kernel<_Float16, false>), grid, blk, 0, st, a);
  } else {
    if (a.accumulate) FLCE_LAUNCH((bwd_dx_finalize_kernel<float, true>), grid, blk, 0, st, a);
    else FLCE_LAUNCH((bwd_dx_finalize_kernel<float, false>), grid, blk, 0, st, a);
  }
  return hipGetLastError();
}

// db of one slab when no dW launch does it (frozen weight).
template <class T>
__global__ void __launch_bounds__(256) bwd_db_kernel(BwdLaunch a, int vs, int width) {
  slab_db<T>(a, vs, width, blockIdx.x * 256 + threadIdx.x);
}

hipError_t launch_bwd_prepare(const BwdLaunch& a, hipStream_t st) {
  if (a.gscale) FLCE_LAUNCH(bwd_scale_kernel, dim3(1), dim3(1024), 0, st, a);
  FLCE_LAUNCH(bwd_coef_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The dx product of one slab.  K split: each part takes kc slab columns (a
// multiple of the 64-deep copy block).  A split accumulator (several slabs,
// one part) runs the First, Accum and Last modes only; false for any other.
template <class T>
static bool launch_dx(const BwdLaunch& a, int vs, int width, int wpad, int TH, int dx_mode, hipStream_t st) {
  const int parts = a.dx_split > 1 ? a.dx_split : 1;
  const int kc = parts > 1 ? (((wpad + parts - 1) / parts + 63) / 64) * 64 : wpad;
  const dim3 gdx(TH * a.NT * parts), blk(kThreads);
  const bool acc = a.accumulate != 0;
  if constexpr (sizeof(T) == 2) {
    if (a.split_acc) {
      if (dx_mode == kDxFirst && acc) FLCE_LAUNCH((bwd_dx_kernel<T, kDxFirst, true, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
      else if (dx_mode == kDxFirst) FLCE_LAUNCH((bwd_dx_kernel<T, kDxFirst, false, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
      else if (dx_mode == kDxAccum) FLCE_LAUNCH((bwd_dx_kernel<T, kDxAccum, false, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
      else if (dx_mode == kDxLast) FLCE_LAUNCH((bwd_dx_kernel<T, kDxLast, false, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
      else return false;
      return true;
    }
  }
  if (dx_mode == kDxFirst) FLCE_LAUNCH((bwd_dx_kernel<T, kDxFirst, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
  else if (dx_mode == kDxAccum) FLCE_LAUNCH((bwd_dx_kernel<T, kDxAccum, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
  else if (dx_mode == kDxLast && !acc) FLCE_LAUNCH((bwd_dx_kernel<T, kDxLast, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
  else if (dx_mode == kDxLast) FLCE_LAUNCH((bwd_dx_kernel<T, kDxLast, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
  else if (!acc) FLCE_LAUNCH((bwd_dx_kernel<T, kDxOnly, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
  else FLCE_LAUNCH((bwd_dx_kernel<T, kDxOnly, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
  return true;
}

template <class T>
static hipError_t launch_bwd_slab_t(const BwdLaunch& a, int vs, int width, int dx_mode, bool want_db,
                                    bool dz_ready, hipStream_t st) {
  const int wpad = (width + 7) & ~7;
  const int TV = (width + kTile - 1) / kTile;
  const int TH = (a.H + kTile - 1) / kTile;
  const bool bias = a.b != nullptr;
  const dim3 blk(kThreads);
  const dim3 gdz(TV * a.NT < kPersistGrid ? TV * a.NT : kPersistGrid);
  // A partial vocabulary tile (only in the last slab) or partial token tiles.
  const bool ragged = width % kTile != 0 || a.N % kTile != 0;
  if (dz_ready) {
    // the slab already holds the dlogits (and the db partials are written)
  } else if (bias && want_db) {
    if (ragged) FLCE_LAUNCH((bwd_dz_kernel<T, true, true, true>), gdz, blk, 0, st, a, vs, TV);
    else FLCE_LAUNCH((bwd_dz_kernel<T, true, true, false>), gdz, blk, 0, st, a, vs, TV);
  } else if (bias) {
    if (ragged) FLCE_LAUNCH((bwd_dz_kernel<T, true, false, true>), gdz, blk, 0, st, a, vs, TV);
    else FLCE_LAUNCH((bwd_dz_kernel<T, true, false, false>), gdz, blk, 0, st, a, vs, TV);
  } else {
    if (ragged) FLCE_LAUNCH((bwd_dz_kernel<T, false, false, true>), gdz, blk, 0, st, a, vs, TV);
    else FLCE_LAUNCH((bwd_dz_kernel<T, false, false, false>), gdz, blk, 0, st, a, vs, TV);
  }
  if (a.dx && !launch_dx<T>(a, vs, width, wpad, TH, dx_mode, st)) return hipErrorInvalidValue;
  if (a.dW && a.accumulate) FLCE_LAUNCH((bwd_dw_kernel<T, true>), dim3(TH * TV), blk, 0, st, a, vs, width, wpad, TH, TV);
  else if (a.dW) FLCE_LAUNCH((bwd_dw_kernel<T, false>), dim3(TH * TV), blk, 0, st, a, vs, width, wpad, TH, TV);
  else if (want_db) FLCE_LAUNCH((bwd_db_kernel<T>), dim3(TV), blk, 0, st, a, vs, width);
  return hipGetLastError();
}

hipError_t launch_bwd_slab(const BwdLaunch& a, int dtype, int vs, int width, int dx_mode, bool want_db,
                           bool dz_ready, hipStream_t st) {
  if (dtype == 1) return launch_bwd_slab_t<uint16_t>(a, vs, width, dx_mode, want_db, dz_ready, st);
  if (dtype == 2) return launch_bwd_slab_t<_Float16>(a, vs, width, dx_mode, want_db, dz_ready, st);
  return launch_bwd_slab_t<float>(a, vs, width, dx_mode, want_db, dz_ready, st);
}


// ---------------------------------------------------------------------------
// Fused schedule: the gradients are formed during the forward pass, one token
// chunk at a time, as fla's fused_linear_cross_entropy_forward does (logits of
// a chunk, its dlogits, dx = dz W and dW += dz^T x; three products, 6NHV
// flops, instead of the recompute schedule's four).  Each chunk's logits are
// kept between its forward product and its dlogits pass.
// ---------------------------------------------------------------------------

// Stores per wave and chunk tile: 32 pieces of kept e values (16-bit
// inputs) and 8 of m_h.
constexpr int kFusedStoresVm = 40;

// One tile of the chunk forward: the logits product, then an epilogue that
// (pass 1) takes each token's max m_h over the 128 rows this wave holds,
// (pass 2) keeps e = exp(z - m_h) for every row, in T, and folds the tile
// into the running (m, d), sum z and z_y exactly as the forward does
// (d gains sum e exp(m_h - m')).  e lies in (0, 1], so a 16-bit copy has a
// relative error of at most 2^-9 however large the logits (a 16-bit copy of z
// itself would put |z| 2^-9 into the exponent).  16-bit tiles copy W with
// permuted rows (tile_row_perm), so a lane's values in blocks 2s and 2s + 1
// of a token column are eight consecutive vocabulary rows: one 16-byte store.
template <class T, bool BIAS, bool SMOOTH, bool XFIRST, bool RAGGED, bool UNIT, int EXTRA>
__device__ __forceinline__ void fused_fwd_tile(const FwdLaunch& a, int vt, int n0, TileCopy<true, true>& tc,
                                               const Lds& L, const int (&ycol)[8], float (&m)[8], float (&d)[8],
                                               float (&sz)[8], float (&zy)[8], __amdgpu_buffer_rsrc_t re,
                                               __amdgpu_buffer_rsrc_t rm, int tid) {
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
  const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};
  const int v0 = vt * kTile;
  BiasTile<T> bt;
  if (BIAS) bt.fetch((const T*)a.b, a.V, v0, tid);
  Acc acc;
  if constexpr (sizeof(T) == 2) {
    gemm_tile_bf16_run<true, true, EXTRA, XFIRST>(acc, A, B, a.H, L, tid, tc);
    if (vt + a.P < a.VT) tc.start(A, v0 + a.P * kTile, B, n0, L, tid, true);
  } else {
    gemm_tile<T, true, true>(acc, A, v0, B, n0, a.H, L, tid);
  }
  if (BIAS) {
    bt.publish(L.bias, tid, a.logit_scale);
    lds_barrier();
  }
  acc_drain();
  const int rw = wm * kWaveTile;
  const int vleft = a.V - v0;          // rows of this tile inside the vocabulary
  const bool ragged = RAGGED && vleft < kTile;   // the vocabulary's last tile (wave-uniform)
  const float sc = a.logit_scale;
  auto logit = [&](float v, float bv, int row) -> float {
    const float z = UNIT ? v : fmaf(v, sc, bv);   // UNIT: no bias, scale 1 (bit-identical)
    return (!ragged || row < vleft) ? z : -INFINITY;
  };
  // Pass 1: m_h of each token column.
  float mh[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mh[j] = -INFINITY;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r0 = rw + dz_row<T>(2 * s, g), r1 = rw + dz_row<T>(2 * s + 1, g);
    const f32x4 b0 = BIAS ? read_bias4(L.bias, r0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 b1 = BIAS ? read_bias4(L.bias, r1) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 z0 = acc_read4(acc[2 * s][j]);
      const f32x4 z1 = acc_read4(acc[2 * s + 1][j]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mh[j] = fmaxf(mh[j], logit(z0[r], b0[r], r0 + r));
        mh[j] = fmaxf(mh[j], logit(z1[r], b1[r], r1 + r));
      }
      __builtin_amdgcn_sched_barrier(0);   // one column at a time keeps few values live
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mh[j] = fmaxf(mh[j], __shfl_xor(mh[j], 16));
    mh[j] = fmaxf(mh[j], __shfl_xor(mh[j], 32));
  }
  // m_h of token column j: lanes of group 0 store it (the other lanes' stores
  // are dropped by an out-of-range offset, so every wave issues all 8).
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int nl = wn * kWaveTile + 16 * j + (lane & 15);
    const uint32_t off =
        (g == 0 && (!RAGGED || n0 + nl < a.N)) ? (uint32_t)(((int64_t)nl * 2 * a.VT + 2 * vt + wm) * 4) : kOOB;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mh[j]), rm, off, 0, 0);
  }
  // Pass 2: kept values, sums and the target logit.
  float se[8], zs[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    se[j] = 0.f;
    zs[j] = 0.f;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int r0 = rw + dz_row<T>(2 * s, g), r1 = rw + dz_row<T>(2 * s + 1, g);
    const f32x4 b0 = BIAS ? read_bias4(L.bias, r0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 b1 = BIAS ? read_bias4(L.bias, r1) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int nl = wn * kWaveTile + 16 * j + (lane & 15);
      const f32x4 z0 = acc_read4(acc[2 * s][j]);
      const f32x4 z1 = acc_read4(acc[2 * s + 1][j]);
      float z[8], e[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = logit(z0[r], b0[r], r0 + r);
        z[4 + r] = logit(z1[r], b1[r], r1 + r);
      }
      const float nml = -mh[j] * kLog2e;
      const bool live = !ragged || mh[j] != -INFINITY;   // a half tile wholly past V keeps zeros
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        e[k] = live ? fast_exp2(fmaf(z[k], kLog2e, nml)) : 0.f;
        if (RAGGED) {
          se[j] += e[k];
          if (SMOOTH) zs[j] += (!ragged || z[k] != -INFINITY) ? z[k] : 0.f;
        } else {
          // The same adds in the same order, pinned: as plain += the compiler
          // restructured the sums and spilled.
          add_pinned_after_trans(se[j], e[k]);
          if (SMOOTH) add_pinned(zs[j], z[k]);
        }
      }
      // Target logit by selects: a branch here (as in the other epilogues)
      // made the shared instance keep this pass's values live across it and
      // spill.  The whole-tile instance takes the branch, rarely entered.
      const int t0 = ycol[j] - (v0 + r0), t1 = ycol[j] - (v0 + r1);
      if (RAGGED) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          zy[j] = t0 == r ? z[r] : zy[j];
          zy[j] = t1 == r ? z[4 + r] : zy[j];
        }
      } else if (__ballot((unsigned)t0 < 4u || (unsigned)t1 < 4u)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (t0 == r) zy[j] = z[r];
          if (t1 == r) zy[j] = z[4 + r];
        }
      }
      if constexpr (sizeof(T) == 2) {
        const uint32_t off = !RAGGED || n0 + nl < a.N ? (uint32_t)(((int64_t)nl * a.lde + v0 + r0) * 2) : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack2<T>(e[0], e[1]), pack2<T>(e[2], e[3]), pack2<T>(e[4], e[5]), pack2<T>(e[6], e[7])}, re,
            off, 0, 0);
      } else {
        const bool ok = n0 + nl < a.N;
        const uint32_t o0 = ok ? (uint32_t)(((int64_t)nl * a.lde + v0 + r0) * 4) : kOOB;
        const uint32_t o1 = ok ? (uint32_t)(((int64_t)nl * a.lde + v0 + r1) * 4) : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{e[0], e[1], e[2], e[3]}), re, o0,
                                               0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{e[4], e[5], e[6], e[7]}), re, o1,
                                               0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float mn = fmaxf(m[j], mh[j]);
    if (!ragged || mn != -INFINITY) {
      d[j] = d[j] * fast_exp2((m[j] - mn) * kLog2e) + se[j] * fast_exp2((mh[j] - mn) * kLog2e);
      m[j] = mn;
    }
    if (SMOOTH) sz[j] += zs[j];
  }
}

// Chunk forward: the forward kernel's schedule (persistent over token tile and
// vocabulary phase, one workgroup per CU) with fused_fwd_tile's epilogue;
// writes the same per-phase partials, which fwd_combine_kernel merges.
// RAGGED as for fwd_lse_kernel.  UNIT (whole-tile launches without a bias and
// with a logit scale of 1): the logits are the accumulators themselves.
template <class T, bool BIAS, bool SMOOTH, bool XFIRST, bool RAGGED, bool UNIT>
__global__ void __launch_bounds__(kThreads, 1) fused_fwd_kernel(FwdLaunch a) {
  FLCE_LDS(L, T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int w = blockIdx.x;
  int nt, ph;
  if ((a.NT & 7) == 0) {
    const int slot = w >> 3;
    ph = slot % a.P;
    nt = (w & 7) * (a.NT >> 3) + slot / a.P;
  } else {
    ph = w % a.P;
    nt = w / a.P;
  }
  const int n0 = nt * kTile;
  int ycol[8];
  float m[8], d[8], sz[8], zy[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = n0 + wn * kWaveTile + 16 * j + (lane & 15);
    const int64_t t = n < a.N ? a.targets[n] : a.ignore_index;
    ycol[j] = (t == a.ignore_index || t < 0 || t >= a.V) ? -1 : (int)t;
    m[j] = -INFINITY;
    d[j] = 0.f;
    sz[j] = 0.f;
    zy[j] = 0.f;
  }
  // Descriptors start at the tile's first token, so offsets stay below 2^31.
  const __amdgpu_buffer_rsrc_t re = make_rsrc((const T*)a.ebuf + (int64_t)n0 * a.lde);
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.mref + (int64_t)n0 * 2 * a.VT);
  TileCopy<true, true> tc;
  if constexpr (sizeof(T) == 2) {
    const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
    const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};
    if (ph < a.VT) tc.start(A, ph * kTile, B, n0, L, tid, true);
  }
  int vt = ph;
  // The first tile is peeled: later tiles start with the previous tile's
  // kept-value stores still in flight (counted in the mainloop's first wait).
  if (vt < a.VT) {
    fused_fwd_tile<T, BIAS, SMOOTH, XFIRST, RAGGED, UNIT, BIAS ? 1 : 0>(a, vt, n0, tc, L, ycol, m, d, sz, zy, re, rm,
                                                                        tid);
    vt += a.P;
  }
  for (; vt < a.VT; vt += a.P)
    fused_fwd_tile<T, BIAS, SMOOTH, XFIRST, RAGGED, UNIT, (BIAS ? 1 : 0) + kFusedStoresVm>(a, vt, n0, tc, L, ycol, m, d, sz, zy,
                                                                             re, rm, tid);
  // Merge the four lanes of a token, then the two waves, as the forward does.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const float m2 = __shfl_xor(m[j], mask), d2 = __shfl_xor(d[j], mask);
      const float s2 = __shfl_xor(sz[j], mask), y2 = __shfl_xor(zy[j], mask);
      merge_md(m[j], d[j], m2, d2);
      sz[j] += s2;
      zy[j] += y2;
    }
  }
  lds_f32x4* red = (lds_f32x4*)L.a[0];
  __syncthreads();   // every wave's last LDS read of the final tile is done
  if (wm == 1 && lane < 16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wn * kWaveTile + 16 * j + lane] = f32x4{m[j], d[j], sz[j], zy[j]};
  }
  __syncthreads();
  if (wm == 0 && lane < 16) {
    f32x4* part = (f32x4*)a.partials;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 o = red[wn * kWaveTile + 16 * j + lane];
      merge_md(m[j], d[j], o[0], o[1]);
      const int n = n0 + wn * kWaveTile + 16 * j + lane;
      if (n < a.N) part[(int64_t)ph * a.N + n] = f32x4{m[j], d[j], sz[j] + o[2], zy[j] + o[3]};
    }
  }
}

__global__ void __launch_bounds__(1024) fused_count_kernel(FwdLaunch a) {
  __shared__ long long scnt[1024];
  const int tid = threadIdx.x;
  long long c = 0;
  for (int n = tid; n < a.N; n += 1024) c += (a.targets[n] != a.ignore_index) ? 1 : 0;
  scnt[tid] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) scnt[tid] += scnt[tid + w];
    __syncthreads();
  }
  if (tid == 0) a.n_valid[0] = scnt[0];
}

// Dlogits of a chunk, in place over the kept values:
//   dz = c (1 + 2 s lse) e exp(m_h - lse) - c eps / V - c (1 - eps) [j = y]
// (Liger-Kernel PR 239's total gradient, with p = e exp(m_h - lse)), zero
// past V, stored in T, and with DB the fp32 column sums of dz over each block
// of 256 tokens.  For fp16 the coefficients carry the slab scale S (as in the
// recompute schedule), so the stored values are dz S and the column sums are
// multiplied by 1/S (exact: a power of two).  Block bx + CB by (CB = the
// column blocks; one grid dimension, so any N fits) has 1024 threads
// (16 waves per CU keep enough loads in flight for this HBM-bound pass):
// thread t takes the 8 columns 2048 bx + 8 (t % 256) .. + 7 (one half tile:
// one m_h per token) of the 64 tokens 256 by + 64 (t / 256) .. + 63, eight
// rows at a time (four for fp32).  With DB the four quarters' column sums are added in LDS,
// in quarter order.
template <class T, bool DB>
__global__ void __launch_bounds__(1024) fused_dz_kernel(FusedDz f) {
  __shared__ float qsum[DB ? 3 : 1][256][8];
  const int tx = threadIdx.x & 255, qr = threadIdx.x >> 8;
  const unsigned CB = (unsigned)((f.VT * kTile + 2047) / 2048);
  const unsigned bx = blockIdx.x % CB, by = blockIdx.x / CB;
  const int c = (bx * 256 + tx) * 8;
  const bool active = c < f.VT * kTile;   // no early return: the DB sum below has a barrier
  const int vt = c >> 8, h = (c >> 7) & 1;
  const int n0 = (int)by * kTile + 64 * qr;
  const int n1 = min(n0 + 64, f.N);
  const float inv_s = (IsF16<T>::value && f.gscale) ? f.gscale[1] : 1.f;
  const f32x4* coef = (const f32x4*)f.coef;
  float cs[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) cs[k] = 0.f;
  constexpr int kRows = sizeof(T) == 2 ? 8 : 4;   // fp32: half the rows per batch fits 128 VGPRs
  for (int nb = n0; active && nb < n1; nb += kRows) {
    float v[kRows][8];
    float mr[kRows];
#pragma unroll
    for (int q = 0; q < kRows; ++q) {
      const int n = min(nb + q, n1 - 1);   // rows past the quarter repeat the last (not stored, not summed)
      const int64_t base = (int64_t)n * f.lde + c;
      if constexpr (sizeof(T) == 2) {
        const u32x4 u = *(const u32x4*)((const T*)f.ebuf + base);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[q][2 * k] = h16_to_f32<T>(u[k]);
          v[q][2 * k + 1] = h16_to_f32<T>(u[k] >> 16);
        }
      } else {
        const f32x4 u0 = *(const f32x4*)((const float*)f.ebuf + base);
        const f32x4 u1 = *(const f32x4*)((const float*)f.ebuf + base + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[q][k] = u0[k];
          v[q][4 + k] = u1[k];
        }
      }
      mr[q] = f.mref[(int64_t)n * 2 * f.VT + 2 * vt + h];
    }
#pragma unroll
    for (int q = 0; q < kRows; ++q) {
      const int n = nb + q;
      if (n >= n1) break;
      const f32x4 cf = coef[n];
      const int y = f.yv[n];
      const float p_scale = cf[0] * fast_exp2(fmaf(mr[q], kLog2e, -cf[3]));   // c (1 + 2 s lse) e^(m_h - lse)
      float dz[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float z = fmaf(p_scale, v[q][k], -cf[1]);
        if (c + k == y) z -= cf[2];
        z = c + k < f.V ? z : 0.f;
        if (DB) cs[k] += z;
        dz[k] = z;
      }
      const int64_t base = (int64_t)n * f.lde + c;
      if constexpr (sizeof(T) == 2) {
        *(u32x4*)((T*)f.ebuf + base) =
            u32x4{pack2<T>(dz[0], dz[1]), pack2<T>(dz[2], dz[3]), pack2<T>(dz[4], dz[5]), pack2<T>(dz[6], dz[7])};
      } else {
        *(f32x4*)((float*)f.ebuf + base) = f32x4{dz[0], dz[1], dz[2], dz[3]};
        *(f32x4*)((float*)f.ebuf + base + 4) = f32x4{dz[4], dz[5], dz[6], dz[7]};
      }
    }
  }
  if (DB) {
    if (qr > 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qsum[qr - 1][tx][k] = cs[k];
    }
    __syncthreads();
    if (qr == 0 && active) {
#pragma unroll
      for (int k = 0; k < 8; ++k) cs[k] = ((cs[k] + qsum[0][tx][k]) + qsum[1][tx][k]) + qsum[2][tx][k];
      float* o = f.dbp + (int64_t)by * f.lde + c;
      *(f32x4*)o = f32x4{cs[0], cs[1], cs[2], cs[3]} * inv_s;
      *(f32x4*)(o + 4) = f32x4{cs[4], cs[5], cs[6], cs[7]} * inv_s;
    }
  }
}

// db over the chunks: dbacc[v] (+)= the chunk's block sums in block order;
// after the last chunk, db[v] = dbacc[v] (plus db's old value when
// accumulating), rounded once to T.
template <class T>
__global__ void __launch_bounds__(256) fused_db_kernel(const float* dbp, int rows, int64_t lde, float* dbacc, int V,
                                                       int first, int last, void* db, int accumulate) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  float s = first ? 0.f : dbacc[v];
  for (int t = 0; t < rows; ++t) s += dbp[(int64_t)t * lde + v];
  dbacc[v] = s;
  if (!last) return;
  if constexpr (sizeof(T) == 4) {
    float* p = (float*)db + v;
    *p = accumulate ? *p + s : s;
  } else {
    uint16_t* p = (uint16_t*)db + v;
    if (accumulate) s += h16_to_f32<T>(*p);
    *p = (uint16_t)(pack2<T>(s, 0.f) & 0xffffu);
  }
}

hipError_t launch_fused_count(const FwdLaunch& a, hipStream_t st) {
  FLCE_LAUNCH(fused_count_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

template <class T, bool XFIRST, bool RAGGED>
static void launch_fused_fwd_inst(const FwdLaunch& a, hipStream_t st) {
  const int G = a.NT * a.P;
  const bool bias = a.b != nullptr, smooth = a.eps > 0.f;
  const bool unit = !RAGGED && !bias && a.logit_scale == 1.f;
  constexpr bool kU = !RAGGED;   // UNIT of the unit instances (whole tiles only)
  if (bias && smooth) FLCE_LAUNCH((fused_fwd_kernel<T, true, true, XFIRST, RAGGED, false>), dim3(G), dim3(kThreads), 0, st, a);
  else if (bias) FLCE_LAUNCH((fused_fwd_kernel<T, true, false, XFIRST, RAGGED, false>), dim3(G), dim3(kThreads), 0, st, a);
  else if (smooth && unit) FLCE_LAUNCH((fused_fwd_kernel<T, false, true, XFIRST, RAGGED, kU>), dim3(G), dim3(kThreads), 0, st, a);
  else if (smooth) FLCE_LAUNCH((fused_fwd_kernel<T, false, true, XFIRST, RAGGED, false>), dim3(G), dim3(kThreads), 0, st, a);
  else if (unit) FLCE_LAUNCH((fused_fwd_kernel<T, false, false, XFIRST, RAGGED, kU>), dim3(G), dim3(kThreads), 0, st, a);
  else FLCE_LAUNCH((fused_fwd_kernel<T, false, false, XFIRST, RAGGED, false>), dim3(G), dim3(kThreads), 0, st, a);
}

// Whole tiles only (V and N multiples of 256, 16-bit inputs): the instance
// without the partial-tile masks and token checks.
template <class T, bool XFIRST>
static void launch_fused_fwd_order(const FwdLaunch& a, hipStream_t st) {
  if (sizeof(T) == 2 && a.V % kTile == 0 && a.N % kTile == 0) launch_fused_fwd_inst<T, XFIRST, sizeof(T) != 2>(a, st);
  else launch_fused_fwd_inst<T, XFIRST, true>(a, st);
}

template <class T>
static hipError_t launch_fused_forward_t(const FwdLaunch& a, hipStream_t st) {
  if (sizeof(T) == 2 && a.P >= 4) launch_fused_fwd_order<T, true>(a, st);
  else launch_fused_fwd_order<T, false>(a, st);
  FLCE_LAUNCH(fwd_combine_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fused_forward(const FwdLaunch& a, int dtype, hipStream_t st) {
  if (dtype == 1) return launch_fused_forward_t<uint16_t>(a, st);
  if (dtype == 2) return launch_fused_forward_t<_Float16>(a, st);
  return launch_fused_forward_t<float>(a, st);
}

// Forward that keeps the first vocabulary slab's logits: the kept-value
// schedule on W's rows [0, head.V), the plain forward on the rest (rest.V
// rows from vocab_start head.V; none when rest.V is 0), each writing its own
// phases' partials, then one merge of all head.P + rest.P phases.
template <class T>
static hipError_t launch_forward_keep_t(const FwdLaunch& head, const FwdLaunch& rest, hipStream_t st) {
  if (sizeof(T) == 2 && head.P >= 4) launch_fused_fwd_order<T, true>(head, st);
  else launch_fused_fwd_order<T, false>(head, st);
  if (rest.V > 0) launch_fwd_lse<T>(rest, st);
  FwdLaunch all = head;
  all.P = head.P + (rest.V > 0 ? rest.P : 0);
  FLCE_LAUNCH(fwd_combine_kernel, dim3((all.N + 255) / 256), dim3(256), 0, st, all);
  FLCE_LAUNCH(fwd_finalize_kernel, dim3(1), dim3(1024), 0, st, all);
  return hipGetLastError();
}

hipError_t launch_forward_keep(const FwdLaunch& head, const FwdLaunch& rest, int dtype, hipStream_t st) {
  if (dtype == 1) return launch_forward_keep_t<uint16_t>(head, rest, st);
  if (dtype == 2) return launch_forward_keep_t<_Float16>(head, rest, st);
  return launch_forward_keep_t<float>(head, rest, st);
}

template <class T>
static hipError_t launch_fused_dz_t(const FusedDz& f, hipStream_t st) {
  const dim3 grid((unsigned)((f.VT * kTile + 2047) / 2048) * (unsigned)((f.N + kTile - 1) / kTile));
  if (f.dbp) FLCE_LAUNCH((fused_dz_kernel<T, true>), grid, dim3(1024), 0, st, f);
  else FLCE_LAUNCH((fused_dz_kernel<T, false>), grid, dim3(1024), 0, st, f);
  return hipGetLastError();
}

hipError_t launch_fused_dz(const FusedDz& f, int dtype, hipStream_t st) {
  if (dtype == 1) return launch_fused_dz_t<uint16_t>(f, st);
  if (dtype == 2) return launch_fused_dz_t<_Float16>(f, st);
  return launch_fused_dz_t<float>(f, st);
}

// The chunk's products: dx rows (K = all V columns of the dlogits, one slab;
// split along K into a.dx_split parts when its tiles cannot fill the CUs) and
// dW += dz^T x over the chunk's tokens.
template <class T>
static hipError_t launch_fused_products_t(const BwdLaunch& a, bool first, hipStream_t st) {
  const int width = a.V, wpad = (width + 7) & ~7;
  const int TV = (width + kTile - 1) / kTile;
  const int TH = (a.H + kTile - 1) / kTile;
  const dim3 blk(kThreads);
  const bool acc = a.accumulate != 0;
  if (a.dx) {
    const int parts = a.dx_split > 1 ? a.dx_split : 1;
    const int kc = parts > 1 ? (((wpad + parts - 1) / parts + 63) / 64) * 64 : wpad;
    const dim3 gdx(TH * a.NT * parts);
    if (parts > 1) {
      FLCE_LAUNCH((bwd_dx_kernel<T, kDxFirst, false>), gdx, blk, 0, st, a, 0, width, wpad, TH, kc);
      if (launch_bwd_dx_finalize(a, sizeof(T) == 4 ? 0 : (IsF16<T>::value ? 2 : 1), st) != hipSuccess)
        return hipGetLastError();
    } else if (acc) {
      FLCE_LAUNCH((bwd_dx_kernel<T, kDxOnly, true>), gdx, blk, 0, st, a, 0, width, wpad, TH, kc);
    } else {
      FLCE_LAUNCH((bwd_dx_kernel<T, kDxOnly, false>), gdx, blk, 0, st, a, 0, width, wpad, TH, kc);
    }
  }
  if (a.dW) {
    if (first && !acc) FLCE_LAUNCH((bwd_dw_kernel<T, false>), dim3(TH * TV), blk, 0, st, a, 0, width, wpad, TH, TV);
    else FLCE_LAUNCH((bwd_dw_kernel<T, true>), dim3(TH * TV), blk, 0, st, a, 0, width, wpad, TH, TV);
  }
  return hipGetLastError();
}

hipError_t launch_fused_products(const BwdLaunch& a, int dtype, bool first, hipStream_t st) {
  if (dtype == 1) return launch_fused_products_t<uint16_t>(a, first, st);
  if (dtype == 2) return launch_fused_products_t<_Float16>(a, first, st);
  return launch_fused_products_t<float>(a, first, st);
}

hipError_t launch_fused_db(const float* dbp, int rows, int64_t lde, float* dbacc, int V, bool first, bool last,
                           void* db, int dtype, bool accumulate, hipStream_t st) {
  const dim3 grid((unsigned)((V + 255) / 256)), blk(256);
  if (dtype == 1)
    FLCE_LAUNCH((fused_db_kernel<uint16_t>), grid, blk, 0, st, dbp, rows, lde, dbacc, V, (int)first, (int)last, db, (int)accumulate);
  else if (dtype == 2)
    FLCE_LAUNCH((fused_db_kernel<_Float16>), grid, blk, 0, st, dbp, rows, lde, dbacc, V, (int)first, (int)last, db, (int)accumulate);
  else
    FLCE_LAUNCH((fused_db_kernel<float>), grid, blk, 0, st, dbp, rows, lde, dbacc, V, (int)first, (int)last, db, (int)accumulate);
  return hipGetLastError();
}

hipError_t launch_finalize(const FwdLaunch& a, hipStream_t st) {
  FLCE_LAUNCH(fwd_finalize_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace flce
