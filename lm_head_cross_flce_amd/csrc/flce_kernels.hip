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

// ---------------------------------------------------------------------------
// Epilogue helpers.  Accumulator layout (Acc): element r of block (i, j) in
// lane l is row 16 i + 4 g + r and column 16 j + l % 16 of the wave tile,
// with g = l / 16.  A lane thus holds, for each of its 8 columns, 32 rows:
// four consecutive ones in each of the 8 row blocks.
// ---------------------------------------------------------------------------

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
template <class T, bool BIAS, bool SMOOTH, bool XFIRST>
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
    const bool full = v0 + kTile <= a.V;
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

template <class T, bool XFIRST>
static void launch_fwd_lse_order(const FwdLaunch& a, hipStream_t st) {
  const int G = a.NT * a.P;
  const bool bias = a.b != nullptr, smooth = a.eps > 0.f;
  if (bias && smooth) hipLaunchKernelGGL((fwd_lse_kernel<T, true, true, XFIRST>), dim3(G), dim3(kThreads), 0, st, a);
  else if (bias) hipLaunchKernelGGL((fwd_lse_kernel<T, true, false, XFIRST>), dim3(G), dim3(kThreads), 0, st, a);
  else if (smooth) hipLaunchKernelGGL((fwd_lse_kernel<T, false, true, XFIRST>), dim3(G), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((fwd_lse_kernel<T, false, false, XFIRST>), dim3(G), dim3(kThreads), 0, st, a);
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
  hipLaunchKernelGGL(fwd_combine_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(fwd_finalize_kernel, dim3(1), dim3(1024), 0, st, a);
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
  hipLaunchKernelGGL(fwd_stats_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_shard_forward(const FwdLaunch& a, int dtype, hipStream_t st) {
  if (dtype == 1) return launch_shard_forward_t<uint16_t>(a, st);
  if (dtype == 2) return launch_shard_forward_t<_Float16>(a, st);
  return launch_shard_forward_t<float>(a, st);
}

hipError_t launch_merge(const FwdLaunch& a, hipStream_t st) {
  hipLaunchKernelGGL(fwd_combine_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(fwd_finalize_kernel, dim3(1), dim3(1024), 0, st, a);
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

// One tile of the recompute kernel.  EXTRA: the vector-memory instructions
// every wave has issued since this tile's copies started (see
// gemm_tile_bf16_run).  bf16 tiles copy W with permuted rows
// (tile_row_perm), so a lane's values in blocks 2s and 2s + 1 of a token
// column are eight consecutive vocabulary rows; fp32 tiles keep the MFMA row
// order (two runs of four rows, 16 apart).
template <class T>
__device__ __forceinline__ constexpr int dz_row(int i, int g) {
  return sizeof(T) == 2 ? 32 * (i >> 1) + 8 * g + 4 * (i & 1) : 16 * i + 4 * g;
}

template <class T, bool BIAS, bool DB, int EXTRA>
__device__ __forceinline__ void dz_tile(const BwdLaunch& a, int vs, int TM, int G, int t, TileCopy<true, true>& tc,
                                        const Lds& L, lds_f32* red, lds_f32x4* ltok, __attribute__((address_space(3))) int* lyv,
                                        int tid) {
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
  if constexpr (sizeof(T) == 2) {
    gemm_tile_bf16_run<true, true, EXTRA>(acc, A, B, a.H, L, tid, tc);
    const int tnext = t + gridDim.x;
    if (tnext < G) {
      int tm2, tn2;
      tile_coords(tnext, G, TM, a.NT, tm2, tn2);
      tc.start(A, vs + tm2 * kTile, B, tn2 * kTile, L, tid, true);
    }
  } else {
    gemm_tile<T, true, true>(acc, A, v0, B, n0, a.H, L, tid);
  }
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
  // Slab rows of this tile's tokens, from token n0 on.
  const __amdgpu_buffer_rsrc_t rslab = make_rsrc((const T*)a.slab + (int64_t)n0 * a.ldS);
  const float sl2e = a.logit_scale * kLog2e;   // p = 2^((scale (z + b)) log2 e - lse log2 e)
  // Bands s of 32 wave rows (blocks 2s, 2s + 1), token blocks j within them:
  // dlogits of the lane's token (16 j + l % 16) at its rows r0 .. r0 + 3 and
  // r1 .. r1 + 3 (tile-relative), the band's db row sums, and the slab store.
  // A band's row sums are reduced over the lane group as soon as the band is
  // done, so few stay live.
  float dbs[4];
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
        dz[r] = fmaf(cf[0], fast_exp2(fmaf(z0[r] + bias0[r], sl2e, -cf[3])), -cf[1]);
        dz[4 + r] = fmaf(cf[0], fast_exp2(fmaf(z1[r] + bias1[r], sl2e, -cf[3])), -cf[1]);
      }
      const int t0 = y - (v0 + r0), t1 = y - (v0 + r1);
      if (__ballot((t0 >= 0 && t0 < 4) || (t1 >= 0 && t1 < 4))) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (t0 == r) dz[r] -= cf[2];
          if (t1 == r) dz[4 + r] -= cf[2];
        }
      }
      if (vleft < kTile) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (r0 + r >= vleft) dz[r] = 0.f;
          if (r1 + r >= vleft) dz[4 + r] = 0.f;
        }
      }
      if (DB) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rs[e] += dz[e];
      }
      if constexpr (sizeof(T) == 2) {
        // r1 = r0 + 4: sixteen contiguous bytes; a wave instruction writes 16
        // tokens x 64 bytes.
        const uint32_t off =
            n0 + nl < a.N ? (uint32_t)(((int64_t)nl * a.ldS + (v0 - vs) + r0) * 2) : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack2<T>(dz[0], dz[1]), pack2<T>(dz[2], dz[3]), pack2<T>(dz[4], dz[5]),
                  pack2<T>(dz[6], dz[7])},
            rslab, off, 0, 0);
      } else {
        if (n0 + nl < a.N) {
          T* row = (T*)a.slab + (int64_t)(n0 + nl) * a.ldS + (v0 - vs);
          store4<T>(row + r0, dz[0], dz[1], dz[2], dz[3]);
          store4<T>(row + r1, dz[4], dz[5], dz[6], dz[7]);
        }
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

// Persistent over the slab's tiles (TM vocabulary tiles x NT token tiles): a
// workgroup takes logical tiles blockIdx.x, + gridDim.x, ..., so the tiles in
// flight together are the ones a one-tile-per-workgroup launch would run
// together (same XCD mapping), and each tile's first copies are issued while
// the previous tile's epilogue runs.  The first tile is peeled: only later
// tiles start with the previous tile's slab stores still in flight.
template <class T, bool BIAS, bool DB>
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
  if constexpr (sizeof(T) == 2) {
    const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
    const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};
    int tm, tn;
    tile_coords(t, G, TM, a.NT, tm, tn);
    tc.start(A, vs + tm * kTile, B, tn * kTile, L, tid, true);
  }
  // Vector-memory instructions every wave issues between starting a tile's
  // copies and its mainloop: the per-token loads (2) and the bias fetch, plus,
  // after the first tile, the previous tile's slab stores (32).
  constexpr int kLoadsVm = 2 + (BIAS ? 1 : 0);
  constexpr int kStoresVm = 32;
  lds_f32x4* ltok = (lds_f32x4*)tok_s;
  __attribute__((address_space(3))) int* lyv = (__attribute__((address_space(3))) int*)yv_s;
  dz_tile<T, BIAS, DB, kLoadsVm>(a, vs, TM, G, t, tc, L, red, ltok, lyv, tid);
  for (t += gridDim.x; t < G; t += gridDim.x)
    dz_tile<T, BIAS, DB, kLoadsVm + kStoresVm>(a, vs, TM, G, t, tc, L, red, ltok, lyv, tid);
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
template <class T, int MODE, bool ACC>
__global__ void __launch_bounds__(kThreads, 1) bwd_dx_kernel(BwdLaunch a, int vs, int width, int wpad, int TM,
                                                             int kc) {
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
  const __amdgpu_buffer_rsrc_t racc = make_rsrc(a.dx_acc + (int64_t)part * a.N * a.H + (int64_t)n0 * a.H);
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
    if (a.accumulate) hipLaunchKernelGGL((bwd_dx_finalize_kernel<uint16_t, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((bwd_dx_finalize_kernel<uint16_t, false>), grid, blk, 0, st, a);
  } else if (dtype == 2) {
    if (a.accumulate) hipLaunchKernelGGL((bwd_dx_finalize_kernel<_Float16, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((bwd_dx_finalize_kernel<_Float16, false>), grid, blk, 0, st, a);
  } else {
    if (a.accumulate) hipLaunchKernelGGL((bwd_dx_finalize_kernel<float, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((bwd_dx_finalize_kernel<float, false>), grid, blk, 0, st, a);
  }
  return hipGetLastError();
}

// db of one slab when no dW launch does it (frozen weight).
template <class T>
__global__ void __launch_bounds__(256) bwd_db_kernel(BwdLaunch a, int vs, int width) {
  slab_db<T>(a, vs, width, blockIdx.x * 256 + threadIdx.x);
}

hipError_t launch_bwd_prepare(const BwdLaunch& a, hipStream_t st) {
  if (a.gscale) hipLaunchKernelGGL(bwd_scale_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(bwd_coef_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_bwd_slab_t(const BwdLaunch& a, int vs, int width, int dx_mode, bool want_db,
                                    hipStream_t st) {
  const int wpad = (width + 7) & ~7;
  const int TV = (width + kTile - 1) / kTile;
  const int TH = (a.H + kTile - 1) / kTile;
  const bool bias = a.b != nullptr;
  const dim3 blk(kThreads);
  const dim3 gdz(TV * a.NT < kPersistGrid ? TV * a.NT : kPersistGrid);
  if (bias && want_db) hipLaunchKernelGGL((bwd_dz_kernel<T, true, true>), gdz, blk, 0, st, a, vs, TV);
  else if (bias) hipLaunchKernelGGL((bwd_dz_kernel<T, true, false>), gdz, blk, 0, st, a, vs, TV);
  else hipLaunchKernelGGL((bwd_dz_kernel<T, false, false>), gdz, blk, 0, st, a, vs, TV);
  if (a.dx) {
    // K split: each part takes kc slab columns (a multiple of the 64-deep copy block).
    const int parts = a.dx_split > 1 ? a.dx_split : 1;
    const int kc = parts > 1 ? (((wpad + parts - 1) / parts + 63) / 64) * 64 : wpad;
    const dim3 gdx(TH * a.NT * parts);
    const bool acc = a.accumulate != 0;
    if (dx_mode == kDxFirst) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxFirst, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
    else if (dx_mode == kDxAccum) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxAccum, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
    else if (dx_mode == kDxLast && !acc) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxLast, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
    else if (dx_mode == kDxLast) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxLast, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
    else if (!acc) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxOnly, false>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
    else hipLaunchKernelGGL((bwd_dx_kernel<T, kDxOnly, true>), gdx, blk, 0, st, a, vs, width, wpad, TH, kc);
  }
  if (a.dW && a.accumulate) hipLaunchKernelGGL((bwd_dw_kernel<T, true>), dim3(TH * TV), blk, 0, st, a, vs, width, wpad, TH, TV);
  else if (a.dW) hipLaunchKernelGGL((bwd_dw_kernel<T, false>), dim3(TH * TV), blk, 0, st, a, vs, width, wpad, TH, TV);
  else if (want_db) hipLaunchKernelGGL((bwd_db_kernel<T>), dim3(TV), blk, 0, st, a, vs, width);
  return hipGetLastError();
}

hipError_t launch_bwd_slab(const BwdLaunch& a, int dtype, int vs, int width, int dx_mode, bool want_db,
                           hipStream_t st) {
  if (dtype == 1) return launch_bwd_slab_t<uint16_t>(a, vs, width, dx_mode, want_db, st);
  if (dtype == 2) return launch_bwd_slab_t<_Float16>(a, vs, width, dx_mode, want_db, st);
  return launch_bwd_slab_t<float>(a, vs, width, dx_mode, want_db, st);
}


}  // namespace flce
