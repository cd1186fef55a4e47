// Device building blocks for the FLCE kernels on gfx950 (CDNA4, wave64).
//
// Every contraction of the method is computed by one tile routine: a 256 x 256
// output tile per 256-thread workgroup (4 waves in a 2 x 2 grid, 128 x 128 per
// wave as 8 x 8 blocks of 16 x 16 MFMA accumulators).
//
//   C[m, n] = sum_k A[m, k] * B[n, k]
//
// Each operand is read from global memory either "K-contiguous" (element
// (m, k) at p[m * ld + k]) or "M-contiguous" (element (m, k) at p[k * ld + m]).
// bf16 operands are copied global -> LDS by the buffer unit in 64-deep K
// blocks (two LDS buffers per operand) and read with 16-byte LDS loads
// (K-contiguous) or transposing 8-byte loads (M-contiguous).  fp32 operands go
// through registers into two padded LDS buffers.
//
// MFMA output layout (16 x 16 blocks): accumulator element r of lane l holds
// row 4 * (l / 16) + r and column l % 16 of its block, so one lane owns one
// column and four consecutive rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kPersistGrid = 256;              // one workgroup per CU (MI355X: 256 CUs)
constexpr int kTile = 256;                  // BM = BN
constexpr int kWaveTile = 128;
constexpr int kRowBytes = 144;              // fp32 LDS rows: 128 B of K + 16 B pad (bank spread)
constexpr int kBufBytes = kTile * kRowBytes;
constexpr int kStageK = 32;                 // bf16: K per MFMA stage
constexpr int kBlockK = 64;                 // bf16: K per copy block (two stages)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// 16-bit element types: uint16_t holds bfloat16 bits, _Float16 is IEEE half.
// Both travel through the same copies and LDS layouts; they differ in the
// MFMA instruction and in the conversions to and from fp32.
template <class T> struct IsF16 { static constexpr bool value = false; };
template <> struct IsF16<_Float16> { static constexpr bool value = true; };

__device__ __forceinline__ float f16_bits_to_f32(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
// fp32 of one 16-bit element's bits (bf16 or fp16).
template <class T> __device__ __forceinline__ float h16_to_f32(uint32_t v) {
  if constexpr (IsF16<T>::value) return f16_bits_to_f32(v);
  else return bf16_bits_to_f32(v & 0xffffu);
}

// Round-to-nearest-even pack of two floats into bf16x2 (hardware convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Round-to-nearest-even pack of two floats into IEEE half x 2.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (_Float16)lo), b = __builtin_bit_cast(uint16_t, (_Float16)hi);
  return a | (b << 16);
}
template <class T> __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (IsF16<T>::value) return pack_f16x2(lo, hi);
  else return pack_bf16x2(lo, hi);
}

// Store four consecutive output values (one lane's run of four rows) as T.
template <class T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(f32x4*)p = f32x4{a, b, c, d};
}
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  *(u32x2*)p = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
template <> __device__ __forceinline__ void store4<_Float16>(_Float16* p, float a, float b, float c, float d) {
  *(u32x2*)p = u32x2{pack_f16x2(a, b), pack_f16x2(c, d)};
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

// Operand buffers: two per operand, 32 KB for bf16 (one 64-deep K block) and
// 36 KB for fp32 (one padded 32-deep stage).  Each buffer is its own
// __shared__ object (declared by FLCE_LDS in every kernel) so the compiler can
// tell that reads of one buffer never overlap a copy into another and need
// not wait for it.
typedef __attribute__((address_space(3))) float lds_f32;

struct Lds {
  lds_t* a[2];
  lds_t* b[2];
  lds_f32* bias;   // 256 fp32: the bias of the current tile's rows
};
template <class T> struct LdsSize {
  static constexpr int kBuf = sizeof(T) == 2 ? kTile * kBlockK * 2 : kBufBytes;
};
#define FLCE_LDS(name, T)                                                                          \
  __shared__ __attribute__((aligned(16))) char name##_a0[LdsSize<T>::kBuf];                        \
  __shared__ __attribute__((aligned(16))) char name##_a1[LdsSize<T>::kBuf];                        \
  __shared__ __attribute__((aligned(16))) char name##_b0[LdsSize<T>::kBuf];                        \
  __shared__ __attribute__((aligned(16))) char name##_b1[LdsSize<T>::kBuf];                        \
  __shared__ __attribute__((aligned(16))) float name##_bias[kTile];                                \
  const Lds name {                                                                                 \
    {(lds_t*)name##_a0, (lds_t*)name##_a1}, {(lds_t*)name##_b0, (lds_t*)name##_b1}, (lds_f32*)name##_bias \
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
// lds_barrier), and read_bias4() gives a lane the bias of four consecutive rows.
template <class T> struct BiasTile {
  float v;
  __device__ __forceinline__ void fetch(const T* b, int64_t V, int64_t r0, int tid) {
    const int64_t left = V - r0;
    const int nrec = (int)((left < kTile ? left : kTile) * (int64_t)sizeof(T));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(b + r0), (short)0, nrec, 0x00020000);
    if constexpr (sizeof(T) == 2) {
      v = h16_to_f32<T>(__builtin_amdgcn_raw_buffer_load_b16(r, (uint32_t)tid * 2u, 0, 0));
    } else {
      v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)tid * 4u, 0, 0));
    }
  }
  __device__ __forceinline__ void publish(lds_f32* dst, int tid, float scale = 1.f) const { dst[tid] = v * scale; }
};

// Bias of tile rows row .. row + 3 (row a multiple of 4).
__device__ __forceinline__ f32x4 read_bias4(const lds_f32* src, int row) {
  return *(const __attribute__((address_space(3))) f32x4*)(src + row);
}

// ---------------------------------------------------------------------------
// Operands, accumulators and the MFMA
// ---------------------------------------------------------------------------

template <class T> struct Opnd {
  const T* p;
  int64_t ld;    // leading dimension in elements
  int mext;      // valid extent along the tile's M (row) dimension
  int kext;      // valid extent along K
};

// A wave's 128 x 128 tile as 8 x 8 blocks of 16 x 16.  Element r of block
// (i, j) in lane l is row 16 i + 4 (l / 16) + r, column 16 j + l % 16.
typedef f32x4 Acc[8][8];

// One v_mfma_f32_16x16x32_bf16 (F16: _f16) into an accumulator kept in AGPRs.  The
// accumulator is tied to the destination in inline asm: the compiler's own
// register choice for this instruction moves accumulators between registers
// on every step.  ZERO starts the accumulator at zero.  The compiler does not
// see the instruction's latency: acc_drain() must precede any read of the
// accumulators (acc_read4).
template <bool ZERO, bool F16 = false>
__device__ __forceinline__ void mfma16(f32x4& c, const u32x4& a, const u32x4& b) {
  if constexpr (F16) {
    if (ZERO) asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
    else asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  } else {
    if (ZERO) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
    else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
}
template <bool ZERO>
__device__ __forceinline__ void mfma16_f32(f32x4& c, float a, float b) {
  if (ZERO) asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Wait states between the last MFMA of a tile and reads of its accumulators
// (more than the longest MFMA used here needs).  The scheduling barrier keeps
// every MFMA ahead of the wait.
__device__ __forceinline__ void acc_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// One block's accumulators in VGPRs.  Volatile reads keep each block's copies
// where the epilogue uses them; left to itself the register allocator copies
// all 256 accumulators at once and spills.
__device__ __forceinline__ f32x4 acc_read4(const f32x4& blk) {
  f32x4 z;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[0]) : "a"(blk[0]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[1]) : "a"(blk[1]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[2]) : "a"(blk[2]));
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z[3]) : "a"(blk[3]));
  return z;
}
// Value R of one block's accumulators (an epilogue that walks output rows
// takes one value from each of eight blocks at a time).
template <int R>
__device__ __forceinline__ float acc_read1(const f32x4& blk) {
  float z;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(z) : "a"(blk[R]));
  return z;
}

// ---------------------------------------------------------------------------
// fp32 operands: register-staged copies and v_mfma_f32_16x16x4_f32
// (correctness-oriented; no fine-grained interleave)
// ---------------------------------------------------------------------------

// One stage of one operand: 256 rows x 32 fp32, 8 x 16 bytes per thread,
// stored to LDS rows of kRowBytes with K contiguous.
template <class T, bool KCONTIG> struct Stager;

// K-contiguous: thread (kc = tid % 8, rr = tid / 8) loads 16 bytes of K at
// column chunk kc of rows rr + 32 q.
template <> struct Stager<float, true> {
  u32x4 r[8];
  uint32_t off[8];
  const float* base;
  int kc_elem;
  __device__ __forceinline__ void init(const Opnd<float>& o, int m0, int tid) {
    const int kc = tid & 7, rr = tid >> 3;
    kc_elem = kc * 4;
    base = o.p + (int64_t)m0 * o.ld;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = rr + 32 * q;
      off[q] = (m0 + row < o.mext) ? (uint32_t)(((int64_t)row * o.ld + kc_elem) * 4) : kOOB;
    }
  }
  __device__ __forceinline__ void load(const Opnd<float>& o, int k0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0);
    const bool kok = k0 + kc_elem < o.kext;
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = buf_load16(rs, kok ? off[q] : kOOB);
  }
  __device__ __forceinline__ void store(lds_t* buf, int tid) const {
    const int kc = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int q = 0; q < 8; ++q) lds_store16(buf + (rr + 32 * q) * kRowBytes + kc * 16, r[q]);
  }
};

// M-contiguous fp32: 4 x 4 blocks transposed in registers, two per thread
// (mc = tid / 8 + 32 p).
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

// One 32-deep fp32 stage: per 16 x 16 block, 8 x v_mfma_f32_16x16x4_f32.  A
// 16-byte read gives lane l four consecutive k at 4 (l / 16) (+ 16 for the
// second half of the stage); instruction e uses element e, so lane group g
// supplies k = 4 g + e: over e = 0..3 the four groups cover k = 0..15 in a
// permuted order, the same for A and B.
template <bool FIRST>
__device__ __forceinline__ void mma_stage_f32(Acc& acc, const lds_t* bA, const lds_t* bB, int wm, int wn, int lane) {
  const int rl = lane & 15, g = lane >> 4;
  const lds_t* pa = bA + (wm * 128 + rl) * kRowBytes + g * 16;
  const lds_t* pb = bB + (wn * 128 + rl) * kRowBytes + g * 16;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_bit_cast(f32x4, lds_load16(pa + 16 * i * kRowBytes + 64 * h));
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = __builtin_bit_cast(f32x4, lds_load16(pb + 16 * j * kRowBytes + 64 * h));
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (FIRST && h == 0 && e == 0) mfma16_f32<true>(acc[i][j], a[i][e], b[j][e]);
          else mfma16_f32<false>(acc[i][j], a[i][e], b[j][e]);
        }
  }
}

// fp32 tile mainloop: two padded LDS buffers per operand, register staging.
// Ends with a barrier; the accumulators need acc_drain() before they are read.
template <bool AK, bool BK>
__device__ __forceinline__ void gemm_tile_f32(Acc& acc, const Opnd<float>& A, int m0, const Opnd<float>& B, int n0,
                                              int K, const Lds& L, int tid) {
  constexpr int kBK = 32;
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
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
    if (kt == 0) mma_stage_f32<true>(acc, L.a[0], L.b[0], wm, wn, lane);
    else mma_stage_f32<false>(acc, cur ? L.a[1] : L.a[0], cur ? L.b[1] : L.b[0], wm, wn, lane);
    if (more) {
      sa.store(cur ? L.a[0] : L.a[1], tid);
      sb.store(cur ? L.b[0] : L.b[1], tid);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 mainloop.  The MFMAs consume K in stages of 32; the buffer unit copies
// K in blocks of 64 (two stages) into two LDS buffers per operand
// (buffer_load ... lds, 16 bytes per lane, each wave instruction filling 1 KB
// of LDS contiguously), so no registers or LDS-write instructions carry
// operands.  Block b + 1 is copied while block b is computed, and one wait
// plus one barrier per block (after its second stage) both publishes block
// b + 1 and frees block b's buffer for block b + 2.
//
// K-contiguous operand, one block = 256 rows x 64 k: LDS rows of 128 bytes,
// so every copy instruction fetches whole 128-byte lines (8 rows x 8 chunks);
// 16-byte chunk p of row r holds logical K chunk p ^ (r & 7).  A fragment (16
// rows, lane l: row l % 16, K chunk 4 h + l / 16 in stage half h) is one
// 16-byte read per lane, and every 8 consecutive lanes cover the 8 chunk
// positions of a 128-byte bank cycle, so the reads are free of bank conflicts.
//
// M-contiguous operand, one block = 64 k x 256 m in its global layout: LDS
// rows (one per k) of 512 bytes; chunk p of row k holds logical chunk
// p ^ mswz(k).  Fragments are read with ds_read_b64_tr_b16, which within
// each 16-lane group hands lane l element l % 4 of the 8-byte pieces
// addressed by lanes 4 e + l / 4 (e = 0..3): lane j of group G addresses row
// k = 8 G + 4 h + j / 4 (plus 32 in a block's second stage) at columns
// m0 + 4 (j % 4) .. + 3, so lane l receives column m0 + l % 16 at
// k = 8 G + 4 h + e, the K order of a 16-byte read of a K-contiguous row; two
// reads (h = 0, 1) give the lane its 8 values.  The LDS serves such a read
// 32 lanes (two groups, 256 bytes over its 64 banks) per cycle: within a
// group, 4 (k & 3) spreads the four rows' 32-byte runs over the 256 bytes;
// 2 ((k >> 3) & 1) moves the odd group's runs to the other 16-byte chunks, so
// the two groups of a cycle do not share banks.  (With 4 (k & 3) alone they
// did: every such read took two extra cycles, which the LDS bank-conflict
// counter showed as one per MFMA in the weight-gradient product.)
// ---------------------------------------------------------------------------

// Chunk swizzle of row k of an M-contiguous operand's LDS block.
__device__ __forceinline__ constexpr int mswz(int k) { return (4 * (k & 3)) | (2 * ((k >> 3) & 1)); }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_t* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]): wait until at most N vector-memory operations are
// outstanding and all LDS operations are done.
template <int N> constexpr int waitcnt_vm_lgkm0() { return (N & 15) | ((N >> 4) << 14) | (7 << 4); }

// Copies of one operand: 32 wave instructions per block, 8 per wave (q =
// 0..7, instruction index 4 q + wave).  issue(q) fills them one at a time so
// a stage body can spread them between MFMAs; TAIL masks K chunks past the
// operand's valid K (blocks that are not wholly inside it).
template <bool KCONTIG> struct Dma;

// Tile row t of an operand copied with permuted rows holds global row
// m0 + tile_row_perm(t): bits 3..2 of t move to bits 4..3 and bit 4 to bit 2.
// An accumulator lane then owns, in blocks 2s and 2s + 1 of a wave, the eight
// consecutive rows 32 s + 8 (l / 16) .. + 7 of its 128 (instead of two runs
// of four 16 rows apart), so it can store them as one 16-byte piece.
__device__ __forceinline__ constexpr int tile_row_perm(int t) {
  return (t & 0xE3) | ((t & 0x0C) << 1) | ((t & 0x10) >> 2);
}

// Tile row t of an operand copied with permuted columns holds global row
// m0 + tile_col_perm(t): within each half of 128 rows, row 16 j + c (the
// MFMA output column c of block j) holds row 8 c + j, so a lane's values in
// the eight blocks of one output row are eight consecutive global rows.
__device__ __forceinline__ constexpr int tile_col_perm(int t) {
  return (t & 0x80) | ((t & 0x0F) << 3) | ((t & 0x70) >> 4);
}

// K-contiguous: instruction idx fills rows 8 idx .. 8 idx + 7; lane l takes
// row 8 idx + l / 8 and LDS chunk l % 8, which holds global chunk
// (l % 8) ^ (l / 8).  perm: tile rows hold permuted global rows, 1 by
// tile_row_perm, 2 by tile_col_perm.
template <> struct Dma<true> {
  uint32_t off[8];
  const uint16_t* base;
  int wave;
  template <class E>
  __device__ __forceinline__ void init(const Opnd<E>& o, int m0, int tid, int perm = 0) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    base = (const uint16_t*)o.p + (int64_t)m0 * o.ld;
    const int c = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int t = 8 * (4 * q + wave) + (lane >> 3);
      const int row = perm == 1 ? tile_row_perm(t) : perm == 2 ? tile_col_perm(t) : t;
      off[q] = (m0 + row < o.mext) ? (uint32_t)(((int64_t)row * o.ld + 8 * c) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int k0) const { return make_rsrc(base + k0); }
  template <bool TAIL>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int kleft, lds_t* buf, int lane, int q) const {
    const int c = (lane & 7) ^ (lane >> 3);
    dma16(rs, buf + (4 * q + wave) * 1024, (!TAIL || 8 * c < kleft) ? off[q] : kOOB);
  }
};

// M-contiguous: instruction idx fills k rows 2 idx and 2 idx + 1.
template <> struct Dma<false> {
  uint32_t off[8];
  const uint16_t* base;
  int64_t ld;
  int wave;
  template <class E>
  __device__ __forceinline__ void init(const Opnd<E>& o, int m0, int tid, int = 0) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    base = (const uint16_t*)o.p + m0;
    ld = o.ld;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = 2 * (4 * q + wave) + (lane >> 5);
      const int c = (lane & 31) ^ mswz(row);
      off[q] = (m0 + 8 * c < o.mext) ? (uint32_t)(((int64_t)row * o.ld + 8 * c) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int k0) const { return make_rsrc(base + (int64_t)k0 * ld); }
  template <bool TAIL>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int kleft, lds_t* buf, int lane, int q) const {
    const int row = 2 * (4 * q + wave) + (lane >> 5);
    dma16(rs, buf + (4 * q + wave) * 1024, (!TAIL || row < kleft) ? off[q] : kOOB);
  }
};

// Per-lane LDS addresses of one operand's fragments; PAR is the stage's half
// of its K block.
template <bool KCONTIG> struct FragAddr;

template <> struct FragAddr<true> {
  static constexpr int kReads = 1;   // LDS read instructions per 16-row block
  int base[2];                       // per block half; block i adds 16 * 128 * i
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int rl = lane & 15, c = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) base[h] = (wbase + rl) * 128 + 16 * ((4 * h + c) ^ (rl & 7));
  }
  template <int PAR, int H>
  __device__ __forceinline__ void read(u32x4& f, const lds_t* buf, int i) const {
    f = lds_load16(buf + base[PAR] + 2048 * i);
  }
};

template <> struct FragAddr<false> {
  static constexpr int kReads = 2;
  int a[2][8];   // per read h and block i, for the block's first stage
  __device__ __forceinline__ void init(int wbase, int lane) {
    const int j = lane & 15, G = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 8 * G + 4 * h + (j >> 2);
        const int m = wbase + 16 * i + 4 * (j & 3);
        a[h][i] = k * 512 + 16 * ((m >> 3) ^ mswz(k)) + 2 * (m & 7);
      }
  }
  // Read H of block i: elements 2H, 2H + 1 of the fragment's dwords.  The
  // block's second stage lies 32 rows (16 KB) further; k & 3 is unchanged.
  template <int PAR, int H>
  __device__ __forceinline__ void read(u32x4& f, const lds_t* buf, int i) const {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const u32x2 v = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + 16384 * PAR + a[H][i])));
    f[2 * H] = v[0];
    f[2 * H + 1] = v[1];
  }
};

// bf16 fragments of one stage for this wave: 8 A blocks, 8 B blocks.
struct Frag {
  u32x4 a[8], b[8];
};

// One read instruction of a stage's fragments, by index: A blocks 0..3 come
// first (kReads each), then B blocks 0..7, then A blocks 4..7.
template <bool AK, bool BK, int PAR>
__device__ __forceinline__ void frag_read(Frag& f, const FragAddr<AK>& fa, const FragAddr<BK>& fb, const lds_t* bA,
                                          const lds_t* bB, int idx) {
  constexpr int RA = FragAddr<AK>::kReads, RB = FragAddr<BK>::kReads;
  if (idx < 4 * RA) {
    const int i = idx / RA;
    if (RA == 1 || (idx % RA) == 0) fa.template read<PAR, 0>(f.a[i], bA, i);
    else fa.template read<PAR, 1>(f.a[i], bA, i);
  } else if (idx < 4 * RA + 8 * RB) {
    const int t = idx - 4 * RA, j = t / RB;
    if (RB == 1 || (t % RB) == 0) fb.template read<PAR, 0>(f.b[j], bB, j);
    else fb.template read<PAR, 1>(f.b[j], bB, j);
  } else {
    const int t = idx - 4 * RA - 8 * RB, i = 4 + t / RA;
    if (RA == 1 || (t % RA) == 0) fa.template read<PAR, 0>(f.a[i], bA, i);
    else fa.template read<PAR, 1>(f.a[i], bA, i);
  }
}

// Instruction plan of one stage body: 32 + 32 MFMA slots per wave.  The first
// 32 run the previous stage's blocks i = 4..7 while this stage's A 0..3 and
// B 0..7 fragments are read (kR1 reads); the next 32 run this stage's blocks
// i = 0..3 while A 4..7 are read (kR2 reads).  A block's first stage (PAR 0)
// also issues the 16 copies of the next block, as early as it can: copies
// and first reads alternate from slot 0, and copies that do not fit in the
// first half follow the second half's reads.  Slot kinds: 0 none, 1 read,
// 2 copy; idx*() gives the read or copy index.
template <int RA, int RB, int PAR> struct StagePlan {
  static constexpr int kR1 = 4 * RA + 8 * RB, kR2 = 4 * RA;
  static constexpr int kC = PAR == 0 ? 16 : 0;
  // copies every fourth slot of both halves; reads in the other slots, in order
  static constexpr bool copy_slot(int k) { return kC > 0 && (k & 3) == 0; }
  static constexpr int nonc_before(int k) { return kC > 0 ? k - (k + 3) / 4 : k; }   // non-copy slots before k
  static constexpr int kind1(int k) { return copy_slot(k) ? 2 : (nonc_before(k) < kR1 ? 1 : 0); }
  static constexpr int idx1(int k) { return copy_slot(k) ? k / 4 : nonc_before(k); }
  static constexpr int kind2(int k) { return copy_slot(k) ? 2 : (nonc_before(k) < kR2 ? 1 : 0); }
  static constexpr int idx2(int k) { return copy_slot(k) ? 8 + k / 4 : kR1 + nonc_before(k); }
  // Every read and every copy is placed exactly once.
  static constexpr bool complete() {
    int reads = 0, copies = 0, rsum = 0, csum = 0;
    for (int k = 0; k < 32; ++k) {
      if (kind1(k) == 1) { ++reads; rsum += idx1(k); }
      if (kind1(k) == 2) { ++copies; csum += idx1(k); }
      if (kind2(k) == 1) { ++reads; rsum += idx2(k); }
      if (kind2(k) == 2) { ++copies; csum += idx2(k); }
    }
    const int nr = kR1 + kR2;
    return reads == nr && copies == kC && rsum == nr * (nr - 1) / 2 && csum == kC * (kC - 1) / 2;
  }
  static_assert(complete(), "stage plan must place every read and copy once");
};

// One stage body: half PAR of the K block in buffer BUF.  A PAR 0 stage
// copies the block at k_copy into the other buffer, A's eight copies before
// B's (BFIRST: B's first); a PAR 1 stage ends with
// the block's wait (the next block's copies done; VMW newer memory
// operations may stay in flight) and barrier.  FIRST: the tile's first stage
// (no previous MFMAs; blocks 0..3 start from zero); SECOND: blocks 4..7
// start from zero.  Every instruction slot ends in a scheduling barrier,
// which pins this order.
template <int PAR, int BUF, bool FIRST, bool SECOND, bool AK, bool BK, int VMW, bool TAIL, bool BFIRST, class E>
__device__ __forceinline__ void stage_bf16(Acc& acc, Frag& P, Frag& C, const FragAddr<AK>& fa,
                                           const FragAddr<BK>& fb, const Lds& L, int lane, const Opnd<E>& A,
                                           const Opnd<E>& B, const Dma<AK>& da, const Dma<BK>& db,
                                           int k_copy) {
  constexpr bool F16 = IsF16<E>::value;
  typedef StagePlan<FragAddr<AK>::kReads, FragAddr<BK>::kReads, PAR> Plan;
  const lds_t* bA = L.a[BUF];
  const lds_t* bB = L.b[BUF];
  const __amdgpu_buffer_rsrc_t rsa = da.rsrc(k_copy);
  const __amdgpu_buffer_rsrc_t rsb = db.rsrc(k_copy);
  const int kla = A.kext - k_copy, klb = B.kext - k_copy;
  auto copy = [&](int q) {
    if (BFIRST ? q >= 8 : q < 8) da.template issue<TAIL>(rsa, kla, L.a[BUF ^ 1], lane, q & 7);
    else db.template issue<TAIL>(rsb, klb, L.b[BUF ^ 1], lane, q & 7);
  };
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (!FIRST) mfma16<SECOND, F16>(acc[4 + k / 8][k % 8], P.a[4 + k / 8], P.b[k % 8]);
    if (Plan::kind1(k) == 1) frag_read<AK, BK, PAR>(C, fa, fb, bA, bB, Plan::idx1(k));
    else if (Plan::kind1(k) == 2) copy(Plan::idx1(k));
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    mfma16<FIRST, F16>(acc[k / 8][k % 8], C.a[k / 8], C.b[k % 8]);
    if (Plan::kind2(k) == 1) frag_read<AK, BK, PAR>(C, fa, fb, bA, bB, Plan::idx2(k));
    else if (Plan::kind2(k) == 2) copy(Plan::idx2(k));
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (PAR == 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<VMW>());
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The upper half (blocks 4..7) of a tile's last stage.
template <bool ZERO, bool F16 = false>
__device__ __forceinline__ void stage_last_half(Acc& acc, const Frag& P) {
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    mfma16<ZERO, F16>(acc[4 + k / 8][k % 8], P.a[4 + k / 8], P.b[k % 8]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Copy state of one bf16 tile.  start() issues the copies of the first K
// block into buffer 0; it may run while the previous tile's epilogue is still
// working, as long as every wave has finished that tile's mainloop (whose
// last barrier follows its last fragment read and the completion of its
// copies).  perm_a: A's tile rows hold permuted rows (tile_row_perm); perm_b:
// B's hold permuted columns (tile_col_perm).  A permuted operand must be
// K-contiguous.
template <bool AK, bool BK> struct TileCopy {
  Dma<AK> da;
  Dma<BK> db;
  template <class E>
  __device__ __forceinline__ void start(const Opnd<E>& A, int m0, const Opnd<E>& B, int n0,
                                        const Lds& L, int tid, bool perm_a = false, bool perm_b = false) {
    da.init(A, m0, tid, perm_a ? 1 : 0);
    db.init(B, n0, tid, perm_b ? 2 : 0);
    const int lane = tid & 63;
    // Copies past K read zeros (out-of-range offsets), so the stage bodies
    // need no branches.
#pragma unroll
    for (int q = 0; q < 8; ++q) da.template issue<true>(da.rsrc(0), A.kext, L.a[0], lane, q);
#pragma unroll
    for (int q = 0; q < 8; ++q) db.template issue<true>(db.rsrc(0), B.kext, L.b[0], lane, q);
  }
};

// Mainloop of a tile whose first block TileCopy::start has issued.  EXTRA is
// a lower bound on the vector-memory instructions each wave issued after
// start() and before this call (an epilogue's stores and loads): vmcnt counts
// stores too, in issue order, so the wait for the first block, whose copies
// are older than those instructions, allows EXTRA more to stay in flight
// instead of draining the epilogue's stores.  Counting too few only costs a
// stall; every counted instruction must be issued unconditionally by every
// wave.  Returns with all copies complete; the accumulators need acc_drain()
// before they are read.
//
// BFIRST issues each block's B copies ahead of its A copies.  The better order
// depends on the kernel, from same-box A/Bs at the Llama-3-sized head: B first
// makes the forward 3.8% faster and the recompute slower; dW and dx are
// indifferent or slower.
template <bool AK, bool BK, int EXTRA = 0, bool BFIRST = false, class E>
__device__ __forceinline__ void gemm_tile_bf16_run(Acc& acc, const Opnd<E>& A, const Opnd<E>& B, int K,
                                                   const Lds& L, int tid, const TileCopy<AK, BK>& tc) {
  static_assert(EXTRA >= 0 && EXTRA <= 63, "vmcnt holds at most 63");
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const Dma<AK>& da = tc.da;
  const Dma<BK>& db = tc.db;
  FragAddr<AK> fa;
  FragAddr<BK> fb;
  fa.init(wm * 128, lane);
  fb.init(wn * 128, lane);
  // Stages run in groups of four (two blocks, one per buffer); the count is
  // rounded up to a multiple of four, the extra stages reading zeros (their
  // copies lie past K).  The loops then hold whole groups and no stage body
  // is conditional: the register allocator keeps the tied accumulators in
  // place only along straight-line paths.  Stage s keeps its fragments in X
  // (s even) or Y (s odd).
  const int KT = (K + kStageK - 1) / kStageK;
  const int KTp = KT <= 4 ? 4 : (KT + 3) & ~3;
  // Blocks wholly inside both operands' valid K: their copies skip the
  // bounds check.  An operand's valid K can be shorter than the loop's K (the
  // input-gradient product runs K to a whole tile past the last vocabulary
  // row); blocks past it take the checked path, which reads zeros.
  const int KBF = min(K, min(A.kext, B.kext)) / kBlockK;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<EXTRA>());
  __builtin_amdgcn_s_barrier();
  Frag X, Y;
  stage_bf16<0, 0, true, false, AK, BK, 0, true, BFIRST>(acc, Y, X, fa, fb, L, lane, A, B, da, db, 1 * kBlockK);
  stage_bf16<1, 0, false, true, AK, BK, 0, true, BFIRST>(acc, X, Y, fa, fb, L, lane, A, B, da, db, 0);
  stage_bf16<0, 1, false, false, AK, BK, 0, true, BFIRST>(acc, Y, X, fa, fb, L, lane, A, B, da, db, 2 * kBlockK);
  stage_bf16<1, 1, false, false, AK, BK, 0, true, BFIRST>(acc, X, Y, fa, fb, L, lane, A, B, da, db, 0);
  int kt = 4;
  // copies of blocks kt / 2 + 1 and kt / 2 + 2 wholly inside K: no masking
  for (; kt + 6 <= 2 * KBF; kt += 4) {
    stage_bf16<0, 0, false, false, AK, BK, 0, false, BFIRST>(acc, Y, X, fa, fb, L, lane, A, B, da, db,
                                                      (kt / 2 + 1) * kBlockK);
    stage_bf16<1, 0, false, false, AK, BK, 0, false, BFIRST>(acc, X, Y, fa, fb, L, lane, A, B, da, db, 0);
    stage_bf16<0, 1, false, false, AK, BK, 0, false, BFIRST>(acc, Y, X, fa, fb, L, lane, A, B, da, db,
                                                      (kt / 2 + 2) * kBlockK);
    stage_bf16<1, 1, false, false, AK, BK, 0, false, BFIRST>(acc, X, Y, fa, fb, L, lane, A, B, da, db, 0);
  }
  for (; kt < KTp; kt += 4) {
    stage_bf16<0, 0, false, false, AK, BK, 0, true, BFIRST>(acc, Y, X, fa, fb, L, lane, A, B, da, db, (kt / 2 + 1) * kBlockK);
    stage_bf16<1, 0, false, false, AK, BK, 0, true, BFIRST>(acc, X, Y, fa, fb, L, lane, A, B, da, db, 0);
    stage_bf16<0, 1, false, false, AK, BK, 0, true, BFIRST>(acc, Y, X, fa, fb, L, lane, A, B, da, db, (kt / 2 + 2) * kBlockK);
    stage_bf16<1, 1, false, false, AK, BK, 0, true, BFIRST>(acc, X, Y, fa, fb, L, lane, A, B, da, db, 0);
  }
  stage_last_half<false, IsF16<E>::value>(acc, Y);   // upper half of stage KTp - 1 (odd)
}

template <bool AK, bool BK, class E>
__device__ __forceinline__ void gemm_tile_bf16(Acc& acc, const Opnd<E>& A, int m0, const Opnd<E>& B,
                                               int n0, int K, const Lds& L, int tid) {
  TileCopy<AK, BK> tc;
  tc.start(A, m0, B, n0, L, tid);
  gemm_tile_bf16_run<AK, BK>(acc, A, B, K, L, tid, tc);
}

// One 256 x 256 output tile: acc = A[m0:m0+256, :K] * B[n0:n0+256, :K]^T.
// Every wave's last LDS read precedes the mainloop's last barrier, so LDS may
// be reused right after it returns.  Call acc_drain() before reading acc.
template <class T, bool AK, bool BK>
__device__ __forceinline__ void gemm_tile(Acc& acc, const Opnd<T>& A, int m0, const Opnd<T>& B, int n0, int K,
                                          const Lds& L, int tid) {
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
