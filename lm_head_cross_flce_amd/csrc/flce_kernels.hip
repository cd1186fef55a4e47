// FLCE kernels for gfx950.
//
// Forward (statistics only; logits recomputed in backward, the schedule of
// DeepSpeed PR 8792):
//   fwd_lse_kernel     logits tiles z = W x^T (+ b) on MFMA; the epilogue folds
//                      each tile into per-token online max / sum-exp (the
//                      online softmax the fla kernel cites), the running sum of
//                      logits (label smoothing) and the target logit.
//   fwd_combine_kernel merges the per-phase partials: lse = m + log d and the
//                      per-row loss of the label-smoothed CE plus z-loss.
//   fwd_finalize       fixed-order sum and non-ignored count (no host sync).
// Backward, one vocabulary slab at a time:
//   bwd_coef_kernel    per-token c_n (upstream grad, 1/T for mean) folded with
//                      the z-loss factor (1 + 2 s lse) of Liger PR 239.
//   bwd_dz_kernel      recomputes a logits tile and turns it into dlogits
//                      dz = c [(1 + 2 s lse) p - eps/V - (1 - eps) [j = y]],
//                      written to the slab; optional db partial sums (fp32).
//   bwd_dw_kernel      dW[slab] = dz^T x with K = all tokens, fp32 in
//                      registers, written once in W's dtype.
//   bwd_dx_kernel      dx += dz W[slab] into an fp32 accumulator; the last
//                      slab writes dx in x's dtype.
//   bwd_db_kernel      fixed-order sum of the db partials.
#include "flce_device.hpp"
#include "flce_launch.hpp"

namespace flce {

// ---------------------------------------------------------------------------
// Epilogue helpers.  Lane half g = lane / 32; for accumulator element e of
// block (i, j) the row inside the wave tile is 32 i + 8 (e / 4) + 4 g + e % 4
// and the column is 32 j + lane % 32.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int row_off(int i, int e) { return 32 * i + 8 * (e >> 2) + (e & 3); }

// Copy one 32 x 32 accumulator block to VGPRs where the epilogue needs it.
// Left to itself the register allocator copies all 256 accumulators at the end
// of the mainloop, which overflows the VGPRs and spills; volatile reads keep
// each block's copies in program order.  The caller has let the MFMA pipeline
// drain (acc_drain) before the first read.
__device__ __forceinline__ void read_acc16(float (&z)[16], const f32x16& blk) {
#pragma unroll
  for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[e]) : "a"(blk[e]));
}

// Wait states between the last MFMA and a read of its accumulators (more than
// the longest MFMA used here needs).  The scheduling barrier keeps every MFMA
// of the mainloop ahead of the wait.
__device__ __forceinline__ void acc_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Fold one 32 x 32 block (16 values of one column per lane, already in
// VGPRs) into the running (m, d) of that column, the running sum of logits,
// and the target logit.
template <bool SMOOTH, bool RAGGED>
__device__ __forceinline__ void lse_block(const float (&acc)[16], const float (&bv)[16], int i, float& m, float& d,
                                          float& sz, float& zy, int t, int rb, int V) {
  float z[16];
  float bmax = -INFINITY, zs = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    z[e] = acc[e] + bv[e];
    if (RAGGED) {
      const bool ok = rb + row_off(i, e) < V;
      if (SMOOTH) zs += ok ? z[e] : 0.f;
      z[e] = ok ? z[e] : -INFINITY;
    } else if (SMOOTH) {
      zs += z[e];
    }
    bmax = fmaxf(bmax, z[e]);
  }
  const float mn = fmaxf(m, bmax);
  if (!RAGGED || mn != -INFINITY) {
    const float nml = -mn * kLog2e;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ps += fast_exp2(fmaf(z[e], kLog2e, nml));
    d = d * fast_exp2((m - mn) * kLog2e) + ps;  // m = -inf: the factor is 0
    m = mn;
  }
  if (SMOOTH) sz += zs;
  // Target row: wave-uniform branch, rarely taken.
  const int tb = t - 32 * i;
  const bool own = (tb >= 0) && (tb < 32) && ((tb & 4) == 0);
  if (__ballot(own)) {
    float val = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (tb == row_off(0, e)) val = z[e];
    if (own) zy = val;
  }
}

__device__ __forceinline__ void merge_md(float& m, float& d, float m2, float d2) {
  const float mn = fmaxf(m, m2);
  float r = 0.f;
  if (m != -INFINITY) r += d * fast_exp2((m - mn) * kLog2e);
  if (m2 != -INFINITY) r += d2 * fast_exp2((m2 - mn) * kLog2e);
  m = mn;
  d = r;
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------

// Workgroup w owns token tile nt and the vocabulary tiles ph, ph + P, ...
// When NT % 8 == 0 the 1/8 of the grid on one XCD covers NT/8 token tiles
// times all P phases, so each XCD streams W tiles that its neighbours reuse.
template <class T, bool BIAS, bool SMOOTH>
__global__ void __launch_bounds__(kThreads, 1) fwd_lse_kernel(FwdLaunch a) {
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
  const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
  const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};

  int ycol[4];
  float m[4], d[4], sz[4], zy[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * kWaveTile + 32 * j + (lane & 31);
    const int64_t t = n < a.N ? a.targets[n] : a.ignore_index;
    ycol[j] = (t == a.ignore_index) ? -1 : (int)t;
    m[j] = -INFINITY;
    d[j] = 0.f;
    sz[j] = 0.f;
    zy[j] = 0.f;
  }

  f32x16 acc[4][4];
  const int rloc = wm * kWaveTile + 4 * (lane >> 5);   // first tile row of this lane's row block 0
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
      gemm_tile_bf16_run<true, true>(acc, A, B, a.H, L, tid, tc);
      if (vt + a.P < a.VT) tc.start(A, v0 + a.P * kTile, B, n0, L, tid);
    } else {
      gemm_tile<T, true, true>(acc, A, v0, B, n0, a.H, L, tid);
    }
    if (BIAS) {
      bt.publish(L.bias, tid);
      lds_barrier();
    }
    const int rb = v0 + rloc;
    const bool full = v0 + kTile <= a.V;
    acc_drain();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float bv[16];
      if (BIAS) {
        read_bias16(bv, L.bias, rloc, i);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) bv[e] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float z[16];
        read_acc16(z, acc[i][j]);
        if (full) lse_block<SMOOTH, false>(z, bv, i, m[j], d[j], sz[j], zy[j], ycol[j] - rb, rb, a.V);
        else lse_block<SMOOTH, true>(z, bv, i, m[j], d[j], sz[j], zy[j], ycol[j] - rb, rb, a.V);
        // One block at a time: interleaving blocks buys little and spills.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Lanes l and l + 32 hold the same columns (different rows): merge them.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float m2 = __shfl_xor(m[j], 32), d2 = __shfl_xor(d[j], 32);
    const float s2 = __shfl_xor(sz[j], 32), y2 = __shfl_xor(zy[j], 32);
    merge_md(m[j], d[j], m2, d2);
    sz[j] += s2;
    zy[j] += y2;
  }
  // Then the two waves that share columns (wm = 0, 1).
  lds_f32x4* red = (lds_f32x4*)L.a[0];
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wn * kWaveTile + 32 * j + lane] = f32x4{m[j], d[j], sz[j], zy[j]};
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
    f32x4* part = (f32x4*)a.partials;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 o = red[wn * kWaveTile + 32 * j + lane];
      merge_md(m[j], d[j], o[0], o[1]);
      const int n = n0 + wn * kWaveTile + 32 * j + lane;
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
  const float l = valid ? (lse - (1.f - a.eps) * zy - a.eps_over_v * sz + a.s * lse * lse) : 0.f;
  a.lse[n] = lse;
  a.rowloss[n] = l;
  if (a.reduction == kNone) a.loss[n] = l;
}

__global__ void __launch_bounds__(1024) fwd_finalize_kernel(FwdLaunch a) {
  __shared__ double ssum[1024];
  __shared__ long long scnt[1024];
  const int tid = threadIdx.x;
  double s = 0.0;
  long long c = 0;
  for (int n = tid; n < a.N; n += 1024) {
    s += (double)a.rowloss[n];
    c += (a.targets[n] != a.ignore_index) ? 1 : 0;
  }
  ssum[tid] = s;
  scnt[tid] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) {
      ssum[tid] += ssum[tid + w];
      scnt[tid] += scnt[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.n_valid[0] = scnt[0];
    if (a.reduction == kSum) a.loss[0] = (float)ssum[0];
    if (a.reduction == kMean) a.loss[0] = scnt[0] > 0 ? (float)(ssum[0] / (double)scnt[0]) : 0.f;
  }
}

template <class T>
static hipError_t launch_forward_t(const FwdLaunch& a, hipStream_t st) {
  const int G = a.NT * a.P;
  const bool bias = a.b != nullptr, smooth = a.eps > 0.f;
  if (bias && smooth) hipLaunchKernelGGL((fwd_lse_kernel<T, true, true>), dim3(G), dim3(kThreads), 0, st, a);
  else if (bias) hipLaunchKernelGGL((fwd_lse_kernel<T, true, false>), dim3(G), dim3(kThreads), 0, st, a);
  else if (smooth) hipLaunchKernelGGL((fwd_lse_kernel<T, false, true>), dim3(G), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((fwd_lse_kernel<T, false, false>), dim3(G), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL(fwd_combine_kernel, dim3((a.N + 255) / 256), dim3(256), 0, st, a);
  hipLaunchKernelGGL(fwd_finalize_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdLaunch& a, int dtype, hipStream_t st) {
  return dtype == 1 ? launch_forward_t<uint16_t>(a, st) : launch_forward_t<float>(a, st);
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) bwd_coef_kernel(BwdLaunch a) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  const int64_t t = a.targets[n];
  const bool valid = t != a.ignore_index;
  const float g = a.reduction == kNone ? a.grad[n] : a.grad[0];
  const long long T = a.n_valid[0];
  float c = g;
  if (a.reduction == kMean) c = T > 0 ? g / (float)T : 0.f;
  if (!valid) c = 0.f;
  const float lse = a.lse[n];
  ((f32x4*)a.coef)[n] = f32x4{c * (1.f + 2.f * a.s * lse), c * a.eps_over_v, c * (1.f - a.eps), lse * kLog2e};
  a.yv[n] = valid ? (int)t : -1;
}

// Sum 16 per-lane values over the 32 lanes of each wave half, halving the
// values held per lane at every step (masks 16, 8, 4, 2), then adding the
// neighbour (mask 1).  Afterwards lanes l and l ^ 1 hold the total of value
// e = (l % 32) / 2 (bits 1..4 of the lane index).
template <int HALF>
__device__ __forceinline__ void xreduce_step(float (&v)[16], int lane) {
  constexpr int mask = HALF;   // lane bit that selects the kept half
  const bool up = (lane & mask) != 0;
#pragma unroll
  for (int k = 0; k < HALF / 2; ++k) {
    const float keep = up ? v[HALF / 2 + k] : v[k];
    const float send = up ? v[k] : v[HALF / 2 + k];
    v[k] = keep + __shfl_xor(send, mask);
  }
}

__device__ __forceinline__ float row_sum16(float (&v)[16], int lane) {
  xreduce_step<16>(v, lane);
  xreduce_step<8>(v, lane);
  xreduce_step<4>(v, lane);
  xreduce_step<2>(v, lane);
  return v[0] + __shfl_xor(v[0], 1);
}

// Store one 32 x 32 block of dlogits (a lane's column n = lane % 32 and rows
// 8 q + 4 (lane / 32) + r) into the slab, whose rows are tokens with the
// vocabulary contiguous.  Written directly, every lane would store 8 bytes
// into a different token row; instead the block goes through a 2 KB LDS
// buffer of this wave ([token][64 bytes], 16-byte chunk c of row n at
// c ^ (n & 3)) and comes back as 16 contiguous bytes per lane, four lanes
// per 64-byte row segment.  Rows nrow + row at or past nlimit are not
// stored.  Two buffer stores per block, issued by every lane whatever the
// rows.  The buffer is private to the wave, whose LDS operations complete in
// order, so no barrier is needed.
__device__ __forceinline__ void store_block_bf16(lds_t* sb, const float (&dz)[16], __amdgpu_buffer_rsrc_t rslab,
                                                 int64_t ldS, int nrow, int nlimit, int vcol, int lane) {
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(lds_u32x2*)(sb + n * 64 + 16 * (q ^ (n & 3)) + 8 * g) =
        u32x2{pack_bf16x2(dz[4 * q], dz[4 * q + 1]), pack_bf16x2(dz[4 * q + 2], dz[4 * q + 3])};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = 16 * k + (lane >> 2), c = lane & 3;
    const u32x4 v = lds_load16(sb + row * 64 + 16 * (c ^ (row & 3)));
    const uint32_t off = nrow + row < nlimit ? (uint32_t)(((int64_t)(nrow + row) * ldS + vcol + 8 * c) * 2) : kOOB;
    __builtin_amdgcn_raw_buffer_store_b128(v, rslab, off, 0, 0);
  }
}

// One tile of the recompute kernel.  EXTRA: the vector-memory instructions
// every wave has issued since this tile's copies started (see
// gemm_tile_bf16_run).
template <class T, bool BIAS, bool DB, int EXTRA>
__device__ __forceinline__ void dz_tile(const BwdLaunch& a, int vs, int TM, int G, int t, TileCopy<true, true>& tc,
                                        const Lds& L, lds_f32* red, lds_t* stage, int tid) {
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
  const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};
  const int g = lane >> 5;
  const int rloc = wm * kWaveTile + 4 * g;
  const f32x4* coef = (const f32x4*)a.coef;
  int tm, tn;
  tile_coords(t, G, TM, a.NT, tm, tn);
  const int v0 = vs + tm * kTile, n0 = tn * kTile;
  const int rb = v0 + rloc;
  const bool full = v0 + kTile <= a.V;
  // Per-token coefficients and targets are fetched before the mainloop,
  // through descriptors that start at token n0 (rows past N read zero).
  const __amdgpu_buffer_rsrc_t rcoef = make_rsrc(coef + n0);
  const __amdgpu_buffer_rsrc_t ryv = make_rsrc(a.yv + n0);
  f32x4 cf[4];
  int tcol[4];
  T* rowp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nl = wn * kWaveTile + 32 * j + (lane & 31);
    const bool ok = n0 + nl < a.N;
    const f32x4 c = __builtin_bit_cast(f32x4, buf_load16(rcoef, ok ? (uint32_t)nl * 16u : kOOB));
    const int y = (int)__builtin_amdgcn_raw_buffer_load_b32(ryv, ok ? (uint32_t)nl * 4u : kOOB, 0, 0);
    cf[j] = ok ? c : f32x4{0.f, 0.f, 0.f, INFINITY};
    tcol[j] = (ok ? y : -1) - rb;
    rowp[j] = ok ? (T*)a.slab + (int64_t)(n0 + nl) * a.ldS + (v0 - vs) + wm * kWaveTile + 4 * g : nullptr;
  }
  f32x16 acc[4][4];
  BiasTile<T> bt;
  if (BIAS) bt.fetch((const T*)a.b, a.V, v0, tid);
  if constexpr (sizeof(T) == 2) {
    gemm_tile_bf16_run<true, true, EXTRA>(acc, A, B, a.H, L, tid, tc);
    const int tnext = t + gridDim.x;
    if (tnext < G) {
      int tm2, tn2;
      tile_coords(tnext, G, TM, a.NT, tm2, tn2);
      tc.start(A, vs + tm2 * kTile, B, tn2 * kTile, L, tid);
    }
  } else {
    gemm_tile<T, true, true>(acc, A, v0, B, n0, a.H, L, tid);
  }
  if (BIAS) {
    bt.publish(L.bias, tid);
    lds_barrier();
  }
  acc_drain();
  // Slab rows of this tile's tokens, from token n0 on.
  const __amdgpu_buffer_rsrc_t rslab = make_rsrc((const T*)a.slab + (int64_t)n0 * a.ldS);
  float dbsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float bv[16];
    if (BIAS) {
      read_bias16(bv, L.bias, rloc, i);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) bv[e] = 0.f;
    }
    float rs[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) rs[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float z[16];
      read_acc16(z, acc[i][j]);
      float dz[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(fmaf(z[e] + bv[e], kLog2e, -cf[j][3]));
        dz[e] = fmaf(cf[j][0], p, -cf[j][1]);
        if (!full && rb + row_off(i, e) >= a.V) dz[e] = 0.f;
      }
      const int tb = tcol[j] - 32 * i;
      const bool own = (tb >= 0) && (tb < 32) && ((tb & 4) == 0);
      if (__ballot(own)) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (own && tb == row_off(0, e)) dz[e] -= cf[j][2];
      }
      if constexpr (sizeof(T) == 2) {
        store_block_bf16(stage, dz, rslab, a.ldS, wn * kWaveTile + 32 * j, a.N - n0,
                         (v0 - vs) + wm * kWaveTile + 32 * i, lane);
      } else if (rowp[j] != nullptr) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          store4<T>(rowp[j] + 32 * i + 8 * q, dz[4 * q], dz[4 * q + 1], dz[4 * q + 2], dz[4 * q + 3]);
      }
      if (DB) {
#pragma unroll
        for (int e = 0; e < 16; ++e) rs[e] += dz[e];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (DB) dbsum[i] = row_sum16(rs, lane);
  }

  if (DB) {
    // Lane l (even) holds the column sums of row e = (l % 32) / 2 of each row
    // block i; add the two waves that share rows (wn = 0, 1).  The next
    // tile's mainloop barriers keep this tile's reads of red ahead of the
    // next tile's writes.
    const int e = (lane & 31) >> 1;
    if (wn == 1 && (lane & 1) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wm * kWaveTile + row_off(i, e) + 4 * g] = dbsum[i];
    }
    lds_barrier();
    if (wn == 0 && (lane & 1) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = row_off(i, e) + 4 * g;
        const int row = v0 + wm * kWaveTile + rl;
        if (row < a.V) a.dbp[(int64_t)tn * a.ldS + (row - vs)] = dbsum[i] + red[wm * kWaveTile + rl];
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
  __shared__ __attribute__((aligned(16))) float red_s[kTile];   // db: the two waves sharing rows
  __shared__ __attribute__((aligned(16))) char stage_s[4][2048];  // bf16 store staging, one 32 x 32 block per wave
  lds_f32* red = (lds_f32*)red_s;
  const int tid = threadIdx.x, wave = tid >> 6;
  lds_t* stage = (lds_t*)stage_s[wave];
  const int G = TM * a.NT;
  TileCopy<true, true> tc;
  int t = blockIdx.x;
  if constexpr (sizeof(T) == 2) {
    const Opnd<T> A{(const T*)a.W, a.H, a.V, a.H};
    const Opnd<T> B{(const T*)a.x, a.H, a.N, a.H};
    int tm, tn;
    tile_coords(t, G, TM, a.NT, tm, tn);
    tc.start(A, vs + tm * kTile, B, tn * kTile, L, tid);
  }
  // Vector-memory instructions every wave issues between starting a tile's
  // copies and its mainloop: the per-token loads (8) and the bias fetch, plus,
  // after the first tile, the previous tile's slab stores (32).
  constexpr int kLoadsVm = 8 + (BIAS ? 1 : 0);
  constexpr int kStoresVm = 32;
  dz_tile<T, BIAS, DB, kLoadsVm>(a, vs, TM, G, t, tc, L, red, stage, tid);
  for (t += gridDim.x; t < G; t += gridDim.x)
    dz_tile<T, BIAS, DB, kLoadsVm + kStoresVm>(a, vs, TM, G, t, tc, L, red, stage, tid);
}

// db[vs + c] = sum over token tiles of the slab's db partials (fixed order),
// for slab column c < width.
template <class T>
__device__ __forceinline__ void slab_db(const BwdLaunch& a, int vs, int width, int c) {
  if (c >= width) return;
  float s = 0.f;
  for (int t = 0; t < a.NT; ++t) s += a.dbp[(int64_t)t * a.ldS + c];
  if constexpr (sizeof(T) == 4) ((float*)a.db)[vs + c] = s;
  else ((uint16_t*)a.db)[vs + c] = (uint16_t)(pack_bf16x2(s, 0.f) & 0xffffu);
}

// dW[vs + v, h] for the slab: C[h][v] = sum_n x[n][h] dz[n][v].
template <class T>
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
  f32x16 acc[4][4];
  gemm_tile<T, false, false>(acc, A, h0, B, v0, a.N, L, tid);
  T* dW = (T*)a.dW;
  const int g = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = v0 + wn * kWaveTile + 32 * j + (lane & 31);
    if (v >= width) continue;
    T* rowp = dW + (int64_t)(vs + v) * a.H;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int h = h0 + wm * kWaveTile + 32 * i + 8 * q + 4 * g;
        if (h < a.H)
          store4<T>(rowp + h, acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
  }
}

// dx[n, h] += sum_{v in slab} dz[n][v] W[vs + v][h]: C[h][n].  MODE says
// whether the fp32 accumulator is written (first slab), read and written
// (middle slabs), read with dx written in its dtype (last slab), or skipped
// (a single slab).  The epilogue is branch-free (buffer accesses with
// out-of-range offsets for rows past N or columns past H) and reads each
// accumulator block one block ahead of adding and storing it, so the
// read-modify-write does not wait once per 16 bytes.
template <class T>
__device__ __forceinline__ void store4_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, r, off, 0, 0);
  }
}

template <class T, int MODE>
__global__ void __launch_bounds__(kThreads, 1) bwd_dx_kernel(BwdLaunch a, int vs, int width, int wpad, int TM) {
  FLCE_LDS(L, T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, TM, a.NT, tm, tn);
  const int h0 = tm * kTile, n0 = tn * kTile;
  const Opnd<T> A{(const T*)a.W + (int64_t)vs * a.H, a.H, a.H, width};
  const Opnd<T> B{(const T*)a.slab, a.ldS, a.N, wpad};
  f32x16 acc[4][4];
  gemm_tile<T, false, true>(acc, A, h0, B, n0, wpad, L, tid);

  constexpr bool kRead = MODE == kDxAccum || MODE == kDxLast;
  constexpr bool kAcc = MODE == kDxFirst || MODE == kDxAccum;   // write the fp32 accumulator
  // Descriptors start at token row n0, so offsets stay below 256 * H * 4 bytes.
  const __amdgpu_buffer_rsrc_t racc = make_rsrc(a.dx_acc + (int64_t)n0 * a.H);
  const __amdgpu_buffer_rsrc_t rdx = make_rsrc((const T*)a.dx + (int64_t)n0 * a.H);
  const int g = lane >> 5;
  // Byte offset of block (i, j), group q (row n = n0 + nl, column h) for
  // elements of es bytes; kOOB past N or H.
  auto boff = [&](int i, int j, int q, uint32_t es) -> uint32_t {
    const int nl = wn * kWaveTile + 32 * j + (lane & 31);
    const int h = h0 + wm * kWaveTile + 32 * i + 8 * q + 4 * g;
    return (n0 + nl < a.N && h < a.H) ? (uint32_t)(nl * a.H + h) * es : kOOB;
  };
  acc_drain();
  // Loads run kAhead blocks ahead (12 x 1 KB in flight per wave), about what
  // one CU's share of HBM bandwidth needs while every CU makes its
  // read-modify-write at the same moment.
  constexpr int kAhead = 3;
  f32x4 old[kAhead + 1][4];
  if (kRead) {
#pragma unroll
    for (int b = 0; b < kAhead; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) old[b][q] = __builtin_bit_cast(f32x4, buf_load16(racc, boff(b & 3, b >> 2, q, 4u)));
  }
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const int i = b & 3, j = b >> 2;
    const int bn = b + kAhead;
    if (kRead && bn < 16) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        old[bn % (kAhead + 1)][q] = __builtin_bit_cast(f32x4, buf_load16(racc, boff(bn & 3, bn >> 2, q, 4u)));
    }
    float z[16];
    read_acc16(z, acc[i][j]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v = {z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]};
      if (kRead) v += old[b % (kAhead + 1)][q];
      if (kAcc) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), racc, boff(i, j, q, 4u), 0, 0);
      } else {
        store4_buf<T>(rdx, boff(i, j, q, (uint32_t)sizeof(T)), v);
      }
    }
  }
}

// db of one slab when no dW launch does it (frozen weight).
template <class T>
__global__ void __launch_bounds__(256) bwd_db_kernel(BwdLaunch a, int vs, int width) {
  slab_db<T>(a, vs, width, blockIdx.x * 256 + threadIdx.x);
}

hipError_t launch_bwd_prepare(const BwdLaunch& a, hipStream_t st) {
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
  if (a.dW) hipLaunchKernelGGL((bwd_dw_kernel<T>), dim3(TH * TV), blk, 0, st, a, vs, width, wpad, TH, TV);
  else if (want_db) hipLaunchKernelGGL((bwd_db_kernel<T>), dim3(TV), blk, 0, st, a, vs, width);
  if (a.dx) {
    const dim3 gdx(TH * a.NT);
    if (dx_mode == kDxFirst) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxFirst>), gdx, blk, 0, st, a, vs, width, wpad, TH);
    else if (dx_mode == kDxAccum) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxAccum>), gdx, blk, 0, st, a, vs, width, wpad, TH);
    else if (dx_mode == kDxLast) hipLaunchKernelGGL((bwd_dx_kernel<T, kDxLast>), gdx, blk, 0, st, a, vs, width, wpad, TH);
    else hipLaunchKernelGGL((bwd_dx_kernel<T, kDxOnly>), gdx, blk, 0, st, a, vs, width, wpad, TH);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_slab(const BwdLaunch& a, int dtype, int vs, int width, int dx_mode, bool want_db,
                           hipStream_t st) {
  return dtype == 1 ? launch_bwd_slab_t<uint16_t>(a, vs, width, dx_mode, want_db, st)
                    : launch_bwd_slab_t<float>(a, vs, width, dx_mode, want_db, st);
}


}  // namespace flce
