// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

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
  float* dx_acc;          // [dx_split][N][H]
  int dx_split;           // input-gradient K split: parts of each slab's columns, one accumulator each
  float* dbp;             // [NT][ldS]: per token tile db partials of the current slab; null if no db
  float* gscale;          // fp16 inputs: {S, 1/S}, the dlogits slab's power-of-two scale; null otherwise
  void* dx; void* dW; void* db;
};

// dtype: 0 = fp32, 1 = bf16, 2 = fp16.  Each returns the launch error code.
hipError_t launch_forward(const FwdLaunch& a, int dtype, hipStream_t st);
// Shard forward: logits statistics of W's rows only, merged over phases into a.stats.
hipError_t launch_shard_forward(const FwdLaunch& a, int dtype, hipStream_t st);
// Merge of a.P shards' statistics (a.partials = float4 [P][N]) into lse, loss and the count.
hipError_t launch_merge(const FwdLaunch& a, hipStream_t st);
hipError_t launch_bwd_prepare(const BwdLaunch& a, hipStream_t st);
hipError_t launch_bwd_slab(const BwdLaunch& a, int dtype, int vs, int width, int dx_mode, bool want_db,
                           hipStream_t st);
// dx = the sum of the a.dx_split fp32 accumulators (plus dx's old values when
// a.accumulate), written in dx's dtype.
hipError_t launch_bwd_dx_finalize(const BwdLaunch& a, int dtype, hipStream_t st);

}  // namespace flce
