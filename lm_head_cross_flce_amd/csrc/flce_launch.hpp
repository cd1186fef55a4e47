// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

// Launch timing: while the calling thread's timing log is on (the C-ABI's
// flce_timing_start), records a HIP event on st and tags it with `kernel`,
// the kernel just launched (null: the start of an entry point's launches).
// Does nothing otherwise.
void mark_launch(hipStream_t st, const char* kernel);

// Every kernel launch of the library: the launch, then its timing mark.
#define FLCE_LAUNCH(kernel, grid, block, shmem, stream, ...)                 \
  do {                                                                      \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);    \
    ::flce::mark_launch(stream, #kernel);                                   \
  } while (0)

enum Reduction { kNone = 0, kSum = 1, kMean = 2 };
enum DxMode { kDxFirst = 0, kDxAccum = 1, kDxLast = 2, kDxOnly = 3 };

struct FwdLaunch {
  const void* x; const void* W; const void* b; const int64_t* targets;
  int N, H, V;            // V: rows of W (a shard's rows for the shard forward)
  int NT, P, VT;          // token tiles, vocabulary phases, vocabulary tiles
  int64_t vocab_start;    // global index of W's row 0; targets are global indices
  int64_t ignore_index;
  float eps, eps_over_v, s;
  float logit_scale;      // logits are logit_scale * (x W^T + b)
  int reduction;
  void* partials;         // float4 [P][N]
  float* rowloss;         // [N]
  float* loss;            // [1] or [N]
  float* lse;             // [N]
  int64_t* n_valid;       // [1]
  float* stats;           // shard forward: float4 [N] {m, d, sum z, z_y} over the shard's rows
  float* zloss;           // optional: the z-loss term alone, [1] or [N] like loss; null if not wanted
  float* rowzl;           // [N] per-row z-loss terms (workspace), used when zloss is set
  // Fused schedule, chunk forward only: every logit of the chunk is kept as
  // e = exp(z - m_h) in the input dtype, m_h the max over the token's 128
  // rows of the tile that one wave holds.
  void* ebuf;             // [N][lde]
  int64_t lde;            // row stride of ebuf in elements (VT * 256)
  float* mref;            // [N][VT][2]: m_h per token, vocabulary tile and half tile
};

struct BwdLaunch {
  const void* x; const void* W; const void* b; const int64_t* targets;
  int N, H, V;            // V: rows of W (a shard's rows for the shard backward)
  int NT;
  int64_t vocab_start;    // global index of W's row 0; targets are global indices
  int64_t ignore_index;
  float eps, eps_over_v, s;
  float logit_scale;      // logits are logit_scale * (x W^T + b)
  int reduction;
  int accumulate;         // add dx, dW, db to what the outputs hold
  const float* lse; const int64_t* n_valid; const float* grad;
  void* coef;             // float4 [N]
  int* yv;                // [N]
  void* slab; int64_t ldS;
  float* dx_acc;          // [dx_split][N][H] fp32; with split_acc, uint16 [N][H]
  int dx_split;           // input-gradient K split: parts of each slab's columns, one accumulator each
  // 16-bit inputs, one part, several slabs: each fp32 accumulator value is
  // held as its high 16 bits in dx itself and its low 16 bits in dx_acc (the
  // last slab writes the rounded result over the high halves).
  int split_acc;
  float* dbp;             // [NT][ldS]: per token tile db partials of the current slab; null if no db
  float* gscale;          // fp16 inputs: {S, 1/S}, the dlogits slab's power-of-two scale; null otherwise
  void* dx; void* dW; void* db;
};

// Fused schedule, one chunk: the kept e values turned into dlogits in place.
struct FusedDz {
  void* ebuf; int64_t lde;
  const float* mref;      // [N][VT][2]
  const void* coef;       // float4 [N] from bwd_coef_kernel (with the fp16 slab scale)
  const int* yv;          // [N] target rows, -1 if ignored
  int N, V, VT;           // the chunk's tokens, vocabulary rows, vocabulary tiles
  float* dbp;             // [ceil(N / 256)][lde]: fp32 column sums per 256 tokens; null if no db
  const float* gscale;    // fp16: {S, 1/S}; the coefficients, so the stored dlogits, carry S; null otherwise
};

// dtype: 0 = fp32, 1 = bf16, 2 = fp16.  Each returns the launch error code.
hipError_t launch_forward(const FwdLaunch& a, int dtype, hipStream_t st);
// Shard forward: logits statistics of W's rows only, merged over phases into a.stats.
hipError_t launch_shard_forward(const FwdLaunch& a, int dtype, hipStream_t st);
// Merge of a.P shards' statistics (a.partials = float4 [P][N]) into lse, loss and the count.
hipError_t launch_merge(const FwdLaunch& a, hipStream_t st);
hipError_t launch_bwd_prepare(const BwdLaunch& a, hipStream_t st);
// dz_ready: the slab already holds the slab's dlogits (and, with want_db,
// the db partials in a.dbp), so the recompute is skipped.
hipError_t launch_bwd_slab(const BwdLaunch& a, int dtype, int vs, int width, int dx_mode, bool want_db,
                           bool dz_ready, hipStream_t st);
// dx = the sum of the a.dx_split fp32 accumulators (plus dx's old values when
// a.accumulate), written in dx's dtype.
hipError_t launch_bwd_dx_finalize(const BwdLaunch& a, int dtype, hipStream_t st);

// Fused schedule (gradients formed in the forward pass, one token chunk at a
// time).  launch_fused_count: the non-ignored count into a.n_valid before the
// first chunk.  launch_fused_forward: the chunk's logits tiles, statistics
// and kept e values, then the per-row lse and loss (a.* point at the chunk's
// rows).  launch_fused_dz: dlogits in place (and db column sums).
// launch_fused_products: the chunk's dx rows (K = the whole vocabulary) and
// its dW contribution, added to dW unless first (or a.accumulate) says to
// overwrite.  launch_fused_db: db accumulated in fp32 over the chunks
// (first: overwrite), and, with last, written to db in its dtype (added to
// it when accumulate).  launch_finalize: the reduced loss over all rows.
hipError_t launch_fused_count(const FwdLaunch& a, hipStream_t st);
hipError_t launch_fused_forward(const FwdLaunch& a, int dtype, hipStream_t st);
hipError_t launch_fused_dz(const FusedDz& f, int dtype, hipStream_t st);
hipError_t launch_fused_products(const BwdLaunch& a, int dtype, bool first, hipStream_t st);
hipError_t launch_fused_db(const float* dbp, int rows, int64_t lde, float* dbacc, int V, bool first, bool last,
                           void* db, int dtype, bool accumulate, hipStream_t st);
hipError_t launch_finalize(const FwdLaunch& a, hipStream_t st);
// Forward keeping the first slab's logits (e values in head.ebuf, maxima in
// head.mref) for the backward: head covers W's rows [0, head.V) with head.P
// phases, rest the remaining rest.V rows (vocab_start = head.V) with rest.P
// phases whose partials follow head's; then the merge and the final loss.
hipError_t launch_forward_keep(const FwdLaunch& head, const FwdLaunch& rest, int dtype, hipStream_t st);

}  // namespace flce
