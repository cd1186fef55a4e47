// Device building blocks for the FLCE kernels on gfx950 (CDNA4, wave64).
//
// Every contraction of the method is computed by one tile routine: a 256 x 256
// output tile per 256-thread workgroup (4 waves in a 2 x 2 grid, 128 x 128 per
// wave as 4 x 4 blocks of 32 x 32 MFMA accumulators).
//
//   C[m, n] = sum_k A[m, k] * B[n, k]
//
// Each operand is read from global memory either "K-contiguous" (element
// (m, k) at p[m * ld + k]) or "M-contiguous" (element (m, k) at p[k * ld + m]).
// bf16 operands are copied global -> LDS by the buffer unit in their global
// layout (32-wide K stages, a ring of four LDS slots per operand) and read with
// 16-byte LDS loads (K-contiguous) or transposing 8-byte loads (M-contiguous).
// fp32 operands go through registers into two padded LDS buffers.
//
// MFMA output layout (32 x 32 blocks): accumulator element r of lane l holds
// row 8 * (r / 4) + 4 * (l / 32) + (r % 4) and column l % 32 of its block, so
// one lane owns one column and 16 rows, four of them consecutive.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kPersistGrid = 256;              // one workgroup per CU (MI355X: 256 CUs)
constexpr int kTile = 256;                  // BM = BN
constexpr int kWaveTile = 128;
constexpr int kRowBytes = 144;              // fp32 LDS rows: 128 B of K + 16 B pad (bank spread)
constexpr int kBufBytes = kTile * kRowBytes;
constexpr float kLog2e = 1.4426950408889634f;

// Storage type tags: bf16 values are carried as uint16_t bit patterns.
template <class T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int kVec = 8;    // elements per 16-byte chunk
  static constexpr int kBK = 64;    // K per LDS stage
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  static constexpr int kBK = 32;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

template <class T> __device__ __forceinline__ float load_as_f32(const T* p);
template <> __device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) {
  return bf16_bits_to_f32(*p);
}

// Round-to-nearest-even pack of two floats into bf16x2 (hardware convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Store four consecutive output values (one lane's run of four rows) as T.
template <class T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(f32x4*)p = f32x4{a, b, c, d};
}
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  *(u32x2*)p = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS and buffer-load primitives
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

__device__ __forceinline__ u32x4 lds_load16(const lds_t* p) { return *(const lds_u32x4*)p; }

__device__ __forceinline__ void lds_store16(lds_t* p, u32x4 v) { *(lds_u32x4*)p = v; }

// Operand buffers: bf16 tiles use a ring of four 16 KB stages per operand; fp32
// tiles use two 36 KB stages per operand (a[0..1], b[0..1]).  Each buffer is its
// own __shared__ object (declared by FLCE_LDS in every kernel) so the compiler
// can tell that reads of one buffer never overlap a copy into another and need
// not wait for it.
typedef __attribute__((address_space(3))) float lds_f32;

struct Lds {
  lds_t* a[4];
  lds_t* b[4];
  lds_f32* bias;   // 256 fp32: the bias of the current tile's rows
};
template <class T> struct LdsSize {
  static constexpr int kBig = sizeof(T) == 2 ? 16384 : kBufBytes;  // stages 0, 1
  static constexpr int kSmall = sizeof(T) == 2 ? 16384 : 16;       // stages 2, 3 (bf16 only)
};
#define FLCE_LDS(name, T)                                                                          \
  __shared__ __attribute__((aligned(16))) char name##_a0[LdsSize<T>::kBig];                        \
  __shared__ __attribute__((aligned(16))) char name##_a1[LdsSize<T>::kBig];                        \
  __shared__ __attribute__((aligned(16))) char name##_a2[LdsSize<T>::kSmall];                      \
  __shared__ __attribute__((aligned(16))) char name##_a3[LdsSize<T>::kSmall];                      \
  __shared__ __attribute__((aligned(16))) char name##_b0[LdsSize<T>::kBig];                        \
  __shared__ __attribute__((aligned(16))) char name##_b1[LdsSize<T>::kBig];                        \
  __shared__ __attribute__((aligned(16))) char name##_b2[LdsSize<T>::kSmall];                      \
  __shared__ __attribute__((aligned(16))) char name##_b3[LdsSize<T>::kSmall];                      \
  __shared__ __attribute__((aligned(16))) float name##_bias[kTile];                                \
  const Lds name {                                                                                 \
    {(lds_t*)name##_a0, (lds_t*)name##_a1, (lds_t*)name##_a2, (lds_t*)name##_a3},                  \
    {(lds_t*)name##_b0, (lds_t*)name##_b1, (lds_t*)name##_b2, (lds_t*)name##_b3},                  \
    (lds_f32*)name##_bias                                                                          \
  }

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its vector-memory copies (which may be the next tile's, still in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Buffer loads return zero for an offset past the descriptor's range, which
// masks out-of-range rows and columns without branches.
constexpr uint32_t kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Bias of the 256 rows r0 .. r0 + 255 of a tile (r0 < V).  fetch() has thread
// t read row r0 + t through a descriptor that ends at row V, so rows past V
// read zero with no branch; it is issued before the mainloop and lands in a
// register.  publish() stores it to LDS after the mainloop (followed by an
// lds_barrier), and read_bias16() gives a lane the 16 rows it holds in row block i.
template <class T> struct BiasTile {
  float v;
  __device__ __forceinline__ void fetch(const T* b, int64_t V, int64_t r0, int tid) {
    const int64_t left = V - r0;
    const int nrec = (int)((left < kTile ? left : kTile) * (int64_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(b + r0), (short)0, nrec, 0x00020000);
    if constexpr (sizeof(T) == 2) {
      v = bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (uint32_t)tid * 2u, 0, 0));
    } else {
      v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)tid * 4u, 0, 0));
    }
  }
  __device__ __forceinline__ void publish(lds_f32* dst, int tid) const { dst[tid] = v; }
};

// bv[e] = bias of row rloc + 32 i + 8 (e / 4) + e % 4 of the tile (rloc a multiple of 4).
__device__ __forceinline__ void read_bias16(float (&bv)[16], const lds_f32* src, int rloc, int i) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 t = *(const __attribute__((address_space(3))) f32x4*)(src + rloc + 32 * i + 8 * q);
    bv[4 * q] = t[0];
    bv[4 * q + 1] = t[1];
    bv[4 * q + 2] = t[2];
    bv[4 * q + 3] = t[3];
  }
}

// ---------------------------------------------------------------------------
// Operands and global -> LDS staging
// ---------------------------------------------------------------------------

template <class T> struct Opnd {
  const T* p;
  int64_t ld;    // leading dimension in elements
  int mext;      // valid extent along the tile's M (row) dimension
  int kext;      // valid extent along K
};

// One stage of one operand: 256 rows x kBK, 8 x 16 bytes per thread.  The
// descriptor is rebased on every stage (scalar arithmetic), so the per-lane
// byte offsets are fixed for the whole tile and stay small.
template <class T, bool KCONTIG> struct Stager;

// K-contiguous: thread (kc = tid % 8, rr = tid / 8) loads 16 bytes of K at
// column chunk kc of rows rr + 32 q.  Requires kext % kVec == 0.
template <class T> struct Stager<T, true> {
  u32x4 r[8];
  uint32_t off[8];
  const T* base;
  int kc_elem;
  __device__ __forceinline__ void init(const Opnd<T>& o, int m0, int tid) {
    const int kc = tid & 7, rr = tid >> 3;
    kc_elem = kc * Elem<T>::kVec;
    base = o.p + (int64_t)m0 * o.ld;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = rr + 32 * q;
      off[q] = (m0 + row < o.mext) ? (uint32_t)(((int64_t)row * o.ld + kc_elem) * sizeof(T)) : kOOB;
    }
  }
  __device__ __forceinline__ void load(const Opnd<T>& o, int k0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0);
    const bool kok = k0 + kc_elem < o.kext;
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = buf_load16(rs, kok ? off[q] : kOOB);
  }
  __device__ __forceinline__ void store(lds_t* buf, int tid) const {
    store_half<0>(buf, tid);
    store_half<1>(buf, tid);
  }
  template <int HALF>
  __device__ __forceinline__ void store_half(lds_t* buf, int tid) const {
    const int kc = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int q = 4 * HALF; q < 4 * HALF + 4; ++q) lds_store16(buf + (rr + 32 * q) * kRowBytes + kc * 16, r[q]);
  }
};

// M-contiguous bf16: thread (kc = tid % 8, mc = tid / 8) loads rows
// k0 + 8 kc + e (e < 8) at columns m0 + 8 mc .. + 7, then writes the
// transposed 8 x 8 block.  Requires mext % 8 == 0.
template <> struct Stager<uint16_t, false> {
  u32x4 r[8];
  uint32_t off[8];
  const uint16_t* base;
  int krow;
  __device__ __forceinline__ void init(const Opnd<uint16_t>& o, int m0, int tid) {
    const int kc = tid & 7, mc = tid >> 3;
    krow = kc * 8;
    base = o.p + m0;
    const bool mok = m0 + mc * 8 < o.mext;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      off[e] = mok ? (uint32_t)(((int64_t)(krow + e) * o.ld + mc * 8) * 2) : kOOB;
  }
  __device__ __forceinline__ void load(const Opnd<uint16_t>& o, int k0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * o.ld);
    const int kleft = o.kext - k0 - krow;   // rows e < kleft are valid
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = buf_load16(rs, e < kleft ? off[e] : kOOB);
  }
  __device__ __forceinline__ void store(lds_t* buf, int tid) const {
    store_half<0>(buf, tid);
    store_half<1>(buf, tid);
  }
  template <int HALF>
  __device__ __forceinline__ void store_half(lds_t* buf, int tid) const {
    const int kc = tid & 7, mc = tid >> 3;
#pragma unroll
    for (int p = 2 * HALF; p < 2 * HALF + 2; ++p) {
      u32x4 ev, od;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = r[2 * w][p], b = r[2 * w + 1][p];
        ev[w] = (a & 0xffffu) | (b << 16);
        od[w] = (a >> 16) | (b & 0xffff0000u);
      }
      lds_store16(buf + (mc * 8 + 2 * p) * kRowBytes + kc * 16, ev);
      lds_store16(buf + (mc * 8 + 2 * p + 1) * kRowBytes + kc * 16, od);
    }
  }
};

// M-contiguous fp32: 4 x 4 blocks, two per thread (mc = tid / 8 + 32 p).
template <> struct Stager<float, false> {
  u32x4 r[8];
  uint32_t off[8];
  const float* base;
  int krow;
  __device__ __forceinline__ void init(const Opnd<float>& o, int m0, int tid) {
    const int kc = tid & 7;
    krow = kc * 4;
    base = o.p + m0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int mc = (tid >> 3) + 32 * p;
      const bool mok = m0 + mc * 4 < o.mext;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        off[4 * p + e] = mok ? (uint32_t)(((int64_t)(krow + e) * o.ld + mc * 4) * 4) : kOOB;
    }
  }
  __device__ __forceinline__ void load(const Opnd<float>& o, int k0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * o.ld);
    const int kleft = o.kext - k0 - krow;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = buf_load16(rs, (i & 3) < kleft ? off[i] : kOOB);
  }
  __device__ __forceinline__ void store(lds_t* buf, int tid) const {
    const int kc = tid & 7;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int mc = (tid >> 3) + 32 * p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 t = {r[4 * p][i], r[4 * p + 1][i], r[4 * p + 2][i], r[4 * p + 3][i]};
        lds_store16(buf + (mc * 4 + i) * kRowBytes + kc * 16, t);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one LDS stage
// ---------------------------------------------------------------------------

template <class T> struct Mma;

template <> struct Mma<uint16_t> {
  // 4 sub-steps of K = 16: v_mfma_f32_32x32x16_bf16.
  static __device__ __forceinline__ void stage(f32x16 (&acc)[4][4], const lds_t* bA, const lds_t* bB,
                                               int wm, int wn, int lane) {
    const int rl = lane & 31, kh = lane >> 5;
    const lds_t* pa = bA + (wm * 128 + rl) * kRowBytes + kh * 16;
    const lds_t* pb = bB + (wn * 128 + rl) * kRowBytes + kh * 16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = lds_load16(pa + 32 * i * kRowBytes + s * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lds_load16(pb + 32 * j * kRowBytes + s * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
    }
  }
};

template <> struct Mma<float> {
  // 2 sub-steps of K = 16, each 8 x v_mfma_f32_32x32x2_f32.  Lane half kh holds
  // logical k = 16 s + 8 kh + e for register e; instruction e pairs k and k + 8.
  static __device__ __forceinline__ void stage(f32x16 (&acc)[4][4], const lds_t* bA, const lds_t* bB,
                                               int wm, int wn, int lane) {
    const int rl = lane & 31, kh = lane >> 5;
    const lds_t* pa = bA + (wm * 128 + rl) * kRowBytes + kh * 32;
    const lds_t* pb = bB + (wn * 128 + rl) * kRowBytes + kh * 32;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      f32x4 a[4][2], b[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i][0] = __builtin_bit_cast(f32x4, lds_load16(pa + 32 * i * kRowBytes + s * 64));
        a[i][1] = __builtin_bit_cast(f32x4, lds_load16(pa + 32 * i * kRowBytes + s * 64 + 16));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j][0] = __builtin_bit_cast(f32x4, lds_load16(pb + 32 * j * kRowBytes + s * 64));
        b[j][1] = __builtin_bit_cast(f32x4, lds_load16(pb + 32 * j * kRowBytes + s * 64 + 16));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e >> 2][e & 3], b[j][e >> 2][e & 3],
                                                             acc[i][j], 0, 0, 0);
    }
  }
};

// ---------------------------------------------------------------------------
// Tile mainloops
// ---------------------------------------------------------------------------

// fp32 operands (correctness-oriented; no fine-grained interleave).
template <bool AK, bool BK>
__device__ __forceinline__ void gemm_tile_f32(f32x16 (&acc)[4][4], const Opnd<float>& A, int m0,
                                              const Opnd<float>& B, int n0, int K, const Lds& L, int tid) {
  constexpr int kBK = Elem<float>::kBK;
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  Stager<float, AK> sa;
  Stager<float, BK> sb;
  sa.init(A, m0, tid);
  sb.init(B, n0, tid);
  const int KT = (K + kBK - 1) / kBK;
  sa.load(A, 0);
  sb.load(B, 0);
  sa.store(L.a[0], tid);
  sb.store(L.b[0], tid);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      sa.load(A, (kt + 1) * kBK);
      sb.load(B, (kt + 1) * kBK);
    }
    Mma<float>::stage(acc, cur ? L.a[1] : L.a[0], cur ? L.b[1] : L.b[0], wm, wn, lane);
    if (more) {
      sa.store(cur ? L.a[0] : L.a[1], tid);
      sb.store(cur ? L.b[0] : L.b[1], tid);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 mainloop.  K advances in stages of 32 through a ring of four LDS
// buffers per operand; each stage is copied three stages ahead by the buffer
// unit (buffer_load ... lds, 16 bytes per lane, each wave instruction filling
// 1 KB of LDS contiguously), so no registers or LDS-write instructions carry
// operands and about three stages of MFMA work cover the copy latency.
//
// K-contiguous operand, one stage = 256 rows x 32 k: LDS rows of 64 bytes;
// 16-byte chunk p of row r holds logical K chunk p ^ ((r >> 2) & 3).  A
// fragment read (16 lanes = 16 consecutive rows, one logical chunk) then
// touches each of the 64 banks once.
//
// M-contiguous operand, one stage = 32 k x 256 m in its global layout: LDS
// rows (one per k) of 512 bytes; chunk p of row k holds logical chunk
// p ^ (4 (k & 3)).  Fragments are read with ds_read_b64_tr_b16, which within
// each 16-lane group hands lane l element l % 4 of the 8-byte pieces addressed
// by lanes 4 e + l / 4 (e = 0..3): lane j of a group addresses row
// k = 8 kh + 4 r + j / 4 at columns m .. m + 3 with m = 16 (group & 1) +
// 4 (j % 4), so lane l receives column l % 32 at k = 8 kh + 4 r + e, the same
// K order as a 16-byte read of a K-contiguous row.  The 32 lanes read together
// cover 4 rows x 4 chunks, again all 64 banks.
// ---------------------------------------------------------------------------

constexpr int kStageK = 32;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_t* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]): wait until at most N vector-memory operations are
// outstanding and all LDS operations are done.
template <int N> constexpr int waitcnt_vm_lgkm0() { return (N & 15) | ((N >> 4) << 14) | (7 << 4); }

template <bool KCONTIG> struct Dma;

// 16 wave instructions per stage (4 per wave): instruction idx fills rows
// 16 idx .. 16 idx + 15.
template <> struct Dma<true> {
  uint32_t off[4];
  const uint16_t* base;
  int wave;
  __device__ __forceinline__ void init(const Opnd<uint16_t>& o, int m0, int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    base = o.p + (int64_t)m0 * o.ld;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * (4 * q + wave) + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      off[q] = (m0 + row < o.mext) ? (uint32_t)(((int64_t)row * o.ld + 8 * c) * 2) : kOOB;
    }
  }
  // Branch-free so that a stage body stays one basic block.
  __device__ __forceinline__ void issue(const Opnd<uint16_t>& o, int k0, lds_t* buf, int tid) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0);
    const int kleft = o.kext - k0;
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * (4 * q + wave) + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      dma16(rs, buf + (4 * q + wave) * 1024, 8 * c < kleft ? off[q] : kOOB);
    }
  }
};

// 16 wave instructions per stage (4 per wave): instruction idx fills k rows
// 2 idx and 2 idx + 1.
template <> struct Dma<false> {
  uint32_t off[4];
  const uint16_t* base;
  int64_t ld;
  int wave;
  __device__ __forceinline__ void init(const Opnd<uint16_t>& o, int m0, int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    base = o.p + m0;
    ld = o.ld;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 2 * (4 * q + wave) + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (row & 3));
      off[q] = (m0 + 8 * c < o.mext) ? (uint32_t)(((int64_t)row * o.ld + 8 * c) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ void issue(const Opnd<uint16_t>& o, int k0, lds_t* buf, int tid) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)k0 * ld);
    const int kleft = o.kext - k0;
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 2 * (4 * q + wave) + (lane >> 5);
      dma16(rs, buf + (4 * q + wave) * 1024, row < kleft ? off[q] : kOOB);
    }
  }
};

// Per-lane LDS addresses of one operand's fragments.
template <bool KCONTIG> struct FragAddr;

template <> struct FragAddr<true> {
  int a[2];   // per sub-step s; block i adds 32 * 64 * i
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int rl = lane & 31, kh = lane >> 5, f = (rl >> 2) & 3;
#pragma unroll
    for (int s = 0; s < 2; ++s) a[s] = (wbase + rl) * 64 + 16 * ((2 * s + kh) ^ f);
  }
  __device__ __forceinline__ u32x4 read(const lds_t* buf, int i, int s) const {
    return lds_load16(buf + a[s] + 2048 * i);
  }
};

template <> struct FragAddr<false> {
  int a[4];   // per block i; sub-step s and half r add (16 s + 4 r) * 512
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int j = lane & 15, kh = lane >> 5, g = (lane >> 4) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wbase + 32 * i + 16 * g + 4 * (j & 3);
      const int c = (m >> 3) ^ (4 * (j >> 2));
      a[i] = (8 * kh + (j >> 2)) * 512 + 16 * c + 8 * (j & 1);
    }
  }
  __device__ __forceinline__ u32x4 read(const lds_t* buf, int i, int s) const {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const lds_t* p = buf + a[i] + 16 * 512 * s;
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * 512)));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
};

// bf16 fragments of one K = 16 sub-step for this wave: 4 A blocks, 4 B blocks.
struct FragBF16 {
  u32x4 a[4], b[4];
};

template <bool AK, bool BK>
__device__ __forceinline__ void load_frag(FragBF16& f, const FragAddr<AK>& fa, const FragAddr<BK>& fb,
                                          const lds_t* bA, const lds_t* bB, int s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = fa.read(bA, i, s);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = fb.read(bB, j, s);
}

__device__ __forceinline__ void mma_frag(f32x16 (&acc)[4][4], const FragBF16& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[i]),
                                                           __builtin_bit_cast(bf16x8, f.b[j]), acc[i][j], 0, 0, 0);
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgVmem = 0x010, kSgDsRead = 0x100;

// One stage of the bf16 pipeline, for the stage held in ring slot CUR.  The
// barrier sits between the stage's two K sub-steps' worth of MFMAs, so each
// body starts with the previous stage's second sub-step (registers f1) while
// this stage's first fragments are read and the stage three ahead is copied:
//   [mma f1 (previous s1) | read f0 <- s0 | copy stage + 3 -> slot CUR + 3]
//   [mma f0 (s0) | read f1 <- s1]   wait for the copy of the next stage, barrier
template <int CUR, bool FIRST, bool AK, bool BK, int VMW = 16>
__device__ __forceinline__ void stage_bf16(f32x16 (&acc)[4][4], FragBF16& f0, FragBF16& f1,
                                           const FragAddr<AK>& fa, const FragAddr<BK>& fb, const Lds& L, int tid,
                                           const Opnd<uint16_t>& A, const Opnd<uint16_t>& B, const Dma<AK>& da,
                                           const Dma<BK>& db, int k_copy) {
  constexpr int kReads = (AK ? 4 : 8) + (BK ? 4 : 8);   // LDS read instructions per sub-step
  constexpr int NXT = (CUR + 3) & 3;
  const lds_t* bA = L.a[CUR];
  const lds_t* bB = L.b[CUR];
  load_frag<AK, BK>(f0, fa, fb, bA, bB, 0);
  if (!FIRST) mma_frag(acc, f1);
  da.issue(A, k_copy, L.a[NXT], tid);
  db.issue(B, k_copy, L.b[NXT], tid);
  load_frag<AK, BK>(f1, fa, fb, bA, bB, 1);
  mma_frag(acc, f0);
  if (FIRST) {
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, kReads, 0);
    __builtin_amdgcn_sched_group_barrier(kSgVmem, 8, 0);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, kReads / 8, 0);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, kReads / 8, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSgMfma, 8, 0);
  // Keep the trailing MFMAs ahead of the barrier: they cover the latency of
  // the last fragment reads, which the barrier waits for.
  __builtin_amdgcn_sched_barrier(0);
  // The next stage's copies were issued two bodies ago; the 16 newer copy
  // instructions (the next two stages) may stay in flight, and VMW - 16 more
  // where the caller issued other memory operations in between.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<VMW>());
  __builtin_amdgcn_s_barrier();
}

// Copy state of one bf16 tile.  start() issues the copies of the first three
// stages; it may run while the previous tile's epilogue is still working, as
// long as every wave has finished that tile's mainloop (whose last barrier
// follows the last fragment read of every slot).
template <bool AK, bool BK> struct TileCopy {
  Dma<AK> da;
  Dma<BK> db;
  __device__ __forceinline__ void start(const Opnd<uint16_t>& A, int m0, const Opnd<uint16_t>& B, int n0,
                                        const Lds& L, int tid) {
    da.init(A, m0, tid);
    db.init(B, n0, tid);
    // Copies past K read zeros (out-of-range offsets), so the stage bodies
    // need no branches; the ones still in flight are drained at the end.
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      da.issue(A, st * kStageK, L.a[st], tid);
      db.issue(B, st * kStageK, L.b[st], tid);
    }
  }
};

// Mainloop of a tile whose copies TileCopy::start has issued.  EXTRA is a
// lower bound on the vector-memory instructions each wave issued after
// start() and before this call (an epilogue's stores and loads): vmcnt counts
// stores too, in issue order, so the waits for stages 0-2, whose copies are
// older than those instructions, allow EXTRA more to stay in flight instead
// of draining the epilogue's stores.  Counting too few only costs a stall;
// every counted instruction must be issued unconditionally by every wave.
template <bool AK, bool BK, int EXTRA = 0>
__device__ __forceinline__ void gemm_tile_bf16_run(f32x16 (&acc)[4][4], const Opnd<uint16_t>& A,
                                                   const Opnd<uint16_t>& B, int K, const Lds& L, int tid,
                                                   const TileCopy<AK, BK>& tc) {
  static_assert(EXTRA >= 0 && 16 + EXTRA <= 63, "vmcnt holds at most 63");
  constexpr int W0 = 16 + EXTRA;
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const Dma<AK>& da = tc.da;
  const Dma<BK>& db = tc.db;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  FragAddr<AK> fa;
  FragAddr<BK> fb;
  fa.init(wm * 128, lane);
  fb.init(wn * 128, lane);
  const int KT = (K + kStageK - 1) / kStageK;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<W0>());
  __builtin_amdgcn_s_barrier();
  FragBF16 f0, f1;
  // Stages 0 and 1 end by waiting for the copies of stages 1 and 2, which
  // start() issued; from stage 2 on, the waited-for copies are the body's own.
  stage_bf16<0, true, AK, BK, W0>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, 3 * kStageK);
  if (KT > 1) stage_bf16<1, false, AK, BK, W0>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, 4 * kStageK);
  int kt = 2;
  for (; kt + 3 < KT; kt += 4) {
    stage_bf16<2, false, AK, BK>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, (kt + 3) * kStageK);
    stage_bf16<3, false, AK, BK>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, (kt + 4) * kStageK);
    stage_bf16<0, false, AK, BK>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, (kt + 5) * kStageK);
    stage_bf16<1, false, AK, BK>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, (kt + 6) * kStageK);
  }
  if (kt < KT) stage_bf16<2, false, AK, BK>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, (kt + 3) * kStageK);
  if (kt + 1 < KT) stage_bf16<3, false, AK, BK>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, (kt + 4) * kStageK);
  if (kt + 2 < KT) stage_bf16<0, false, AK, BK>(acc, f0, f1, fa, fb, L, tid, A, B, da, db, (kt + 5) * kStageK);
  mma_frag(acc, f1);  // second sub-step of the last stage
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
}

template <bool AK, bool BK>
__device__ __forceinline__ void gemm_tile_bf16(f32x16 (&acc)[4][4], const Opnd<uint16_t>& A, int m0,
                                               const Opnd<uint16_t>& B, int n0, int K, const Lds& L, int tid) {
  TileCopy<AK, BK> tc;
  tc.start(A, m0, B, n0, L, tid);
  gemm_tile_bf16_run<AK, BK>(acc, A, B, K, L, tid, tc);
}

// One 256 x 256 output tile: acc = A[m0:m0+256, :K] * B[n0:n0+256, :K]^T.
// Every wave's last LDS read precedes the mainloop's last barrier, so LDS may
// be reused right after it returns.
template <class T, bool AK, bool BK>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[4][4], const Opnd<T>& A, int m0,
                                          const Opnd<T>& B, int n0, int K, const Lds& L, int tid) {
  if constexpr (sizeof(T) == 2) gemm_tile_bf16<AK, BK>(acc, A, m0, B, n0, K, L, tid);
  else gemm_tile_f32<AK, BK>(acc, A, m0, B, n0, K, L, tid);
}

// ---------------------------------------------------------------------------
// Tile scheduling
// ---------------------------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Renumber so that 1/8 of the grid of consecutive logical tiles lands on
// one XCD, then raster the logical tiles in groups of 8 M-tiles so those
// neighbours share A and B panels in that L2.
__device__ __forceinline__ void tile_coords(int w, int G, int TM, int TN, int& tm, int& tn) {
  int t = w;
  if ((G & 7) == 0) t = (w & 7) * (G >> 3) + (w >> 3);
  constexpr int GM = 8;
  const int per_group = GM * TN;
  const int group = t / per_group;
  const int fm = group * GM;
  const int gm = min(GM, TM - fm);
  const int within = t - group * per_group;
  tm = fm + within % gm;
  tn = within / gm;
}

}  // namespace flce
