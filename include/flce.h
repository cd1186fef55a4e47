/*
 * flce.h - fused linear cross entropy (FLCE) for AMD Instinct MI355X (gfx950).
 *
 * The operation.  For hidden states x [N, H], an LM-head weight W [V, H]
 * (nn.Linear layout: row j is the weight of vocabulary entry j), an optional
 * bias b [V] and integer targets y [N]:
 *
 *   z[n, j]  = sum_h x[n, h] W[j, h] + b[j]                    (the logits)
 *   lse[n]   = m + log d,  m = max_j z[n, j],  d = sum_j exp(z[n, j] - m)
 *   l[n]     = lse[n] - (1 - eps) z[n, y_n] - (eps / V) sum_j z[n, j]
 *              + s * lse[n]^2                        (0 when y_n == ignore_index)
 *   loss     = sum_n l[n] / T (mean) | sum_n l[n] (sum) | l (none),
 *              T = #{n : y_n != ignore_index};  all rows ignored gives loss 0.
 *
 * Sources: fla-org flash-linear-attention, fla/modules/
 * fused_linear_cross_entropy.py (the F.linear logits, the cross_entropy_kernel
 * loss with label smoothing, the mean over non-ignored rows); Liger-Kernel PR
 * 239 "Support Z Loss in CE" (z-loss s * lse^2, the online max / sum-exp form
 * of lse, and the gradient below); DeepSpeed PR 8792 (reduction "none", logits
 * produced straight into fp32, statistics-only forward with the logits
 * recomputed one vocabulary block at a time in backward).
 *
 * The backward returns, with c_n = g / T (mean), g (sum) or g_n (none), and
 * c_n = 0 for ignored rows,
 *   dz[n, j] = c_n [ (1 + 2 s lse[n]) softmax(z[n])_j - eps / V - (1 - eps) [j == y_n] ]
 *   dx = dz W,   dW = dz^T x,   db = sum_n dz[n, :]
 * accumulated in fp32 and written once in the input dtype.
 *
 * The [N, V] logits are never stored: the forward keeps only per-token
 * statistics (lse), the backward recomputes the logits one vocabulary slab at
 * a time.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and never synchronises the host.  Work is enqueued on
 *    `stream` (NULL means the default stream) and completes asynchronously in
 *    stream order.
 *  - Tensors are dense and row-major: x [N, H] and W [V, H] with H contiguous,
 *    b [V], targets [N] int64.  x, W and b share one dtype (flce_dtype).
 *  - x, W, dx, dW and the workspaces must be 16-byte aligned, targets and
 *    n_valid 8-byte, every float32 buffer 4-byte and b, db element-aligned;
 *    H must be a multiple of 8 (FLCE_ERR_UNSUPPORTED otherwise).  Both
 *    follow from the kernels' copies, which move 16 bytes (8 bf16/fp16
 *    elements) of a row at a time; the pages set no such limit.  Callers
 *    with other H pad x and W with zero columns up to a multiple of 8 (the
 *    logits, the loss and dx's first H columns are unchanged) or use the
 *    PyTorch binding, which does so.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failed validation returns an error code and enqueues nothing.
 *  - Targets outside [0, V) that are not ignore_index are a precondition
 *    violation: the results for such rows are unspecified (no memory outside
 *    the given buffers is touched).  An ignore_index inside [0, V) is honoured
 *    (the row is ignored).
 *  - Entry points are thread-safe; calls that share a workspace must be
 *    ordered by the caller (same stream, or events).
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>   /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* The enums have int as their underlying type (C++ states it; C's enums of
 * these values are int-sized), so a caller may pass any int and the library
 * reports the values it does not know instead of the call being undefined. */
#ifdef __cplusplus
#define FLCE_ENUM(name) enum name : int
#else
#define FLCE_ENUM(name) enum name
#endif

typedef FLCE_ENUM(flce_status) {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARGUMENT = 1, /* bad size, null pointer, misalignment, eps/s out of range */
  FLCE_ERR_UNSUPPORTED = 2,      /* dtype or shape the library does not handle (e.g. H % 8 != 0) */
  FLCE_ERR_WORKSPACE_TOO_SMALL = 3,
  FLCE_ERR_HIP = 4,              /* a HIP launch failed; see hipGetLastError on the caller side */
  FLCE_ERR_SCRATCH_TOO_SMALL = 5 /* flce_forward_noalloc: the problem needs more than
                                    FLCE_FORWARD_SCRATCH_BYTES of forward scratch */
} flce_status;

typedef FLCE_ENUM(flce_reduction) {
  FLCE_REDUCTION_NONE = 0,
  FLCE_REDUCTION_SUM = 1,
  FLCE_REDUCTION_MEAN = 2
} flce_reduction;

typedef FLCE_ENUM(flce_dtype) {
  FLCE_F32 = 0,  /* x, W, b are float32; gradients are float32 */
  FLCE_BF16 = 1, /* x, W, b are bfloat16; gradients are bfloat16 (fp32 accumulation) */
  FLCE_F16 = 2   /* x, W, b are IEEE half; gradients are half (fp32 accumulation).  The dlogits
                    slab holds dz times a power of two S = 2^(14 - e), where 2^e bounds
                    max_n |c_n| (|1 + 2 s lse_n| + eps/V + 1 - eps) over non-ignored rows, so
                    that values near c_n / V stay in half's normal range; S cancels exactly
                    in dx, dW and db.  Logits and their statistics are fp32 as for bf16. */
} flce_dtype;

/*
 * Workspace bytes that flce_forward (*fwd_bytes) and flce_backward
 * (*bwd_bytes) need for this problem.  Pure host arithmetic: no HIP call.
 * Either output pointer may be NULL.  The forward figure holds per-token
 * partial statistics for each of P vocabulary phases (P x N x 16 bytes, P =
 * min(V/256 rounded up, max(8, 256 / (N/256 rounded up)))) and per-row losses.
 * The backward figure includes one
 * vocabulary slab of dlogits [N, slab] in the input dtype, plus O(N) and
 * O(N/256 * V) fp32 scratch (and, for fp16, 256 bytes for the slab's scale),
 * and what dx accumulates in over the slabs.  dx sums in fp32: with several
 * slabs, fp32 inputs accumulate in dx itself, and 16-bit inputs keep each
 * fp32 value's high 16 bits in dx (so dx holds no result until the call's
 * launches complete, and its contents are unspecified after an error return,
 * old values included when accumulating) and its low 16 bits in an [N, H]
 * 16-bit workspace array; one slab
 * needs neither.  When the dx product has too few 256 x 256 output tiles to
 * fill the GPU (at most half of its 256 CUs), each slab's columns are split
 * into P <= 8 parts instead, each with its own fp32 [N, H] accumulator in the
 * workspace (P x N x H x 4 bytes, at most about 64 MB).
 */
flce_status flce_workspace_size(int64_t N, int64_t H, int64_t V, flce_dtype dtype, int has_bias,
                                flce_reduction reduction, size_t* fwd_bytes, size_t* bwd_bytes);
/* (The figures also cover the _ex entry points.) */

/*
 * Forward (the logits product with an online log-sum-exp epilogue, then the
 * loss and its reduction): writes
 *   loss    float32, [1] for sum/mean, [N] for none
 *   lse     float32 [N]   (kept by the caller for flce_backward)
 *   n_valid int64 [1]     T, the non-ignored count (kept for flce_backward)
 * b may be NULL (no bias).  eps = label_smoothing in [0, 1]; s = z_loss_scale
 * >= 0; reduction is a flce_reduction.  workspace must hold at least
 * *fwd_bytes from flce_workspace_size for the same arguments.
 * Passages: fla fused_linear_cross_entropy.py, the forward driver (the
 * F.linear logits; total = the non-ignored count) and cross_entropy_kernel
 * (lse - z_y with the label-smoothing blend, the ignore_index early exit);
 * Liger-Kernel PR 239 "Details" (lse from the running max m and
 * d = sum exp(z - m); the z-loss s lse^2 added to the CE); DeepSpeed PR 8792
 * "What" (per-token statistics in forward, reduction none).
 */
flce_status flce_forward(const void* x, const void* W, const void* b, const int64_t* targets,
                         int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                         float label_smoothing, float z_loss_scale, int64_t ignore_index,
                         flce_reduction reduction,
                         float* loss, float* lse, int64_t* n_valid,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward: given the forward's lse and n_valid and the upstream gradient
 * grad_loss (float32: [1] for sum/mean, [N] for none), overwrites
 *   dx [N, H]  (may be NULL: not needed)
 *   dW [V, H]  (may be NULL: frozen weight)
 *   db [V]     (may be NULL: no bias, or not needed; ignored when b is NULL)
 * in the input dtype.  The other arguments must equal the forward's.
 * workspace must hold at least *bwd_bytes from flce_workspace_size.
 * Passages: Liger-Kernel PR 239 "Details" (the total gradient of the
 * smoothed CE plus z-loss with respect to the logits, dz above); fla forward
 * driver (dx = dz W, dW = dz^T x, db = the column sums of dz, the 1/total
 * scaling of mean); DeepSpeed PR 8792 "What" and "Memory and time" (logits
 * recomputed block by block in backward; dx summed in fp32 and cast once).
 */
flce_status flce_backward(const void* x, const void* W, const void* b, const int64_t* targets,
                          int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                          float label_smoothing, float z_loss_scale, int64_t ignore_index,
                          flce_reduction reduction, const float* lse, const int64_t* n_valid,
                          const float* grad_loss,
                          void* dx, void* dW, void* db,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Options of the _ex entry points (a NULL options pointer means the
 * defaults, which make them equal to flce_forward / flce_backward):
 *  logit_scale  the logits are logit_scale * (x W^T + b), as fla's
 *               fused_linear_cross_entropy_loss scales them (its
 *               cross_entropy_kernel multiplies the loaded logits by
 *               logit_scale before the softmax and the gradient of the raw
 *               logits by logit_scale); lse, the loss and the z-loss are those
 *               of the scaled logits.  Any finite value; default 1.
 *  accumulate   backward: add dx, dW and db to what those buffers hold
 *               (summed in fp32, rounded once to the input dtype) instead of
 *               overwriting them, as Liger-Kernel commit 95b01e9 adds each
 *               chunk's weight gradient into grad_weight.  Default 0.
 *  z_loss       forward: if non-NULL, also receives the z-loss term
 *               s * lse^2 alone, float32 [1] (sum/mean, reduced like loss) or
 *               [N] (none; 0 for ignored rows).  Default NULL.
 */
typedef struct flce_options {
  float logit_scale;
  int accumulate;
  float* z_loss;
} flce_options;

flce_status flce_forward_ex(const void* x, const void* W, const void* b, const int64_t* targets,
                            int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                            float label_smoothing, float z_loss_scale, int64_t ignore_index,
                            flce_reduction reduction, const flce_options* opts,
                            float* loss, float* lse, int64_t* n_valid,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

flce_status flce_backward_ex(const void* x, const void* W, const void* b, const int64_t* targets,
                             int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                             float label_smoothing, float z_loss_scale, int64_t ignore_index,
                             flce_reduction reduction, const flce_options* opts,
                             const float* lse, const int64_t* n_valid, const float* grad_loss,
                             void* dx, void* dW, void* db,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Recompute schedule with the first vocabulary slab kept.  flce_forward_keep
 * computes what flce_forward_ex computes and also leaves, in `keep`, the
 * logits of W's first slab rows (the first flce_backward_slab_cols rows, or
 * all V when the vocabulary fits in one slab) as e = exp(z - m_h) in the
 * input dtype with their fp32 maxima m_h, the form the fused schedule below
 * keeps them in.  flce_backward_kept takes that buffer and forms the first
 * slab's dlogits from it instead of recomputing its logits product: the
 * backward does 2NH(V - slab) fewer flops (none of the recompute when V fits
 * in one slab).  It uses `keep` as its dlogits slab, so its own workspace
 * holds no slab: the peak extra memory of the pair is about that of
 * flce_forward + flce_backward (plus the maxima, N x slab/256 x 8 bytes), but
 * `keep` is held from the forward to the backward.  Passages: fla
 * fused_linear_cross_entropy.py, the FusedLinearCrossEntropyFunction forward
 * docstring (the gradient formed during the forward pass, so the logits are
 * not recomputed) combined with DeepSpeed PR 8792 "What" (the logits of the
 * other vocabulary blocks recomputed in backward).
 *
 * flce_keep_workspace_size: the forward's workspace (*fwd_bytes), the keep
 * buffer (*keep_bytes) and the backward's workspace (*bwd_bytes); pure host
 * arithmetic, any output may be NULL.  flce_forward_keep: as
 * flce_forward_ex, plus keep (16-byte aligned, at least *keep_bytes).
 * flce_backward_kept: as flce_backward_ex, plus the keep buffer the forward
 * filled, with the same problem arguments and opts->logit_scale; it consumes
 * it (the buffer holds the last slab's dlogits afterwards), so a second
 * backward needs a new flce_forward_keep (or flce_backward_ex, which
 * recomputes every slab).  Results equal flce_backward_ex's up to the
 * rounding of the kept e values (relative 2^-9 in bf16; 2^-11 in fp16, absolute
 * 2^-25 below its normal range).
 */
flce_status flce_keep_workspace_size(int64_t N, int64_t H, int64_t V, flce_dtype dtype, int has_bias,
                                     flce_reduction reduction, size_t* fwd_bytes, size_t* keep_bytes,
                                     size_t* bwd_bytes);

flce_status flce_forward_keep(const void* x, const void* W, const void* b, const int64_t* targets,
                              int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                              float label_smoothing, float z_loss_scale, int64_t ignore_index,
                              flce_reduction reduction, const flce_options* opts,
                              float* loss, float* lse, int64_t* n_valid, void* keep, size_t keep_bytes,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

flce_status flce_backward_kept(const void* x, const void* W, const void* b, const int64_t* targets,
                               int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                               float label_smoothing, float z_loss_scale, int64_t ignore_index,
                               flce_reduction reduction, const flce_options* opts,
                               const float* lse, const int64_t* n_valid, const float* grad_loss,
                               void* keep, size_t keep_bytes, void* dx, void* dW, void* db,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fused schedule: loss and gradients in one pass, the gradients formed while
 * the forward runs, as fla's fused_linear_cross_entropy_forward and
 * Liger-Kernel commit 95b01e9 ("Summary"; the production-defaults table)
 * compute them.  Tokens are taken chunk_tokens at a time.  Each chunk's
 * logits are formed once: the logits product, then dx = dz W and
 * dW += dz^T x (three products, 6NHV flops, against four for
 * flce_forward + flce_backward).  Between the logits product and the
 * dlogits the chunk's logits are kept as e = exp(z - m_h) in the input
 * dtype, m_h (fp32) being the token's max over each half of a 256-row
 * vocabulary tile: e lies in (0, 1], so 16 bits keep a relative error of at
 * most 2^-9 however large the logits.  grad_loss must be known before the
 * pass (float32, [1] for sum/mean, [N] for none); a caller that learns it
 * later passes 1 and scales the gradients, which are linear in it.  dW is
 * accumulated over the chunks in its own dtype, as the pages' schedule adds
 * each chunk into grad_weight: one rounding per chunk, where the recompute
 * schedule rounds once.  db is summed in fp32 over all chunks and rounded
 * once.
 *
 * Writes loss, lse and n_valid as flce_forward does and dx, dW, db (each may
 * be NULL) as flce_backward does; opts as for the _ex entry points.
 * chunk_tokens is a multiple of 256, or 0 for the default: the fewest chunks
 * whose workspace fits in what flce_forward plus flce_backward take for the
 * same problem (the two schedules then use equal extra memory), balanced.
 * flce_fused_workspace_size gives the workspace bytes (*bytes) and the chunk
 * used (*chunk_used); pure host arithmetic, either output may be NULL.
 */
flce_status flce_fused_workspace_size(int64_t N, int64_t H, int64_t V, flce_dtype dtype, int has_bias,
                                      int64_t chunk_tokens, int64_t* chunk_used, size_t* bytes);

flce_status flce_fused_forward_backward(const void* x, const void* W, const void* b, const int64_t* targets,
                                        int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                                        float label_smoothing, float z_loss_scale, int64_t ignore_index,
                                        flce_reduction reduction, const flce_options* opts,
                                        const float* grad_loss, int64_t chunk_tokens,
                                        float* loss, float* lse, int64_t* n_valid,
                                        void* dx, void* dW, void* db,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * flce_forward_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The forward's per-phase partials and
 * per-row losses live in a static device array of FLCE_FORWARD_SCRATCH_BYTES
 * that each GPU holds (at its own address) from the library's first use on
 * it until the process ends; nothing is allocated or freed.  The problem must
 * fit: *fwd_bytes of flce_workspace_size <= FLCE_FORWARD_SCRATCH_BYTES (about
 * N <= 120k tokens at 8 vocabulary phases; N = 8192 needs 1.1 MB), else
 * FLCE_ERR_SCRATCH_TOO_SMALL with nothing enqueued.  `stream` must belong to
 * the current device (FLCE_ERR_INVALID_ARGUMENT otherwise); the first call
 * on a device looks up its array's address with that device current.  Every
 * call on one GPU shares that GPU's array: calls whose work overlaps on one
 * GPU (different streams, or threads) race and must be ordered by the caller.
 * Results are identical to flce_forward_ex's for the same arguments.
 */
#define FLCE_FORWARD_SCRATCH_BYTES ((size_t)16 << 20)
flce_status flce_forward_noalloc(const void* x, const void* W, const void* b, const int64_t* targets,
                                 int64_t N, int64_t H, int64_t V, flce_dtype dtype,
                                 float label_smoothing, float z_loss_scale, int64_t ignore_index,
                                 flce_reduction reduction, const flce_options* opts,
                                 float* loss, float* lse, int64_t* n_valid, hipStream_t stream);

/*
 * Vocabulary shards.  DeepSpeed PR 8792 ("What"; "Memory and time") splits W's
 * rows across ranks: each rank reduces its rows to per-token statistics in
 * forward, the statistics are merged across ranks (a max and sums), and in
 * backward each rank recomputes its own logits against the global lse and
 * produces dW and db for its rows and an fp32 partial of dx, summed across
 * ranks and cast once at the end (the PR's fp32 hidden-gradient review).  A
 * shard is W's rows [vocab_start, vocab_start + V_shard) of a head with
 * V_total rows; W_shard points at row vocab_start (and b_shard at
 * b[vocab_start]); targets stay global indices.  On one GPU the shards can
 * simply run one after another.
 *
 * flce_shard_workspace_size: workspace bytes for flce_shard_forward
 * (*fwd_bytes), flce_shard_merge (*merge_bytes) and flce_shard_backward
 * (*bwd_bytes); pure host arithmetic; outputs may be NULL.
 */
flce_status flce_shard_workspace_size(int64_t N, int64_t H, int64_t V_shard, flce_dtype dtype, int has_bias,
                                      size_t* fwd_bytes, size_t* merge_bytes, size_t* bwd_bytes);

/*
 * Shard forward: writes stats, float32 [N][4]: per token, over the shard's
 * rows only, {m = max_j z, d = sum_j exp(z - m), sum_j z (0 unless eps > 0),
 * z[y_n] if y_n lies in the shard, else 0}.  Every token gets statistics,
 * ignored ones included (the merge drops them).  eps = label_smoothing only
 * decides whether sum_j z is formed.
 */
flce_status flce_shard_forward(const void* x, const void* W_shard, const void* b_shard, const int64_t* targets,
                               int64_t N, int64_t H, int64_t V_shard, int64_t vocab_start, int64_t V_total,
                               flce_dtype dtype, float label_smoothing, int64_t ignore_index, float* stats,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Merge of num_shards shards' statistics, stacked as float32
 * [num_shards][N][4] (any order of shards), into loss, lse and n_valid exactly
 * as flce_forward writes them for the whole head (eps / V_total in the loss).
 * On several GPUs the stack is what an all-gather of the statistics gives; a
 * max all-reduce of m followed by sum all-reduces of the rescaled d, sum z and
 * z_y is the same merge.
 */
flce_status flce_shard_merge(const float* stats, int64_t num_shards, const int64_t* targets, int64_t N,
                             int64_t V_total, float label_smoothing, float z_loss_scale, int64_t ignore_index,
                             flce_reduction reduction, float* loss, float* lse, int64_t* n_valid, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Shard backward: with the merged lse and n_valid, overwrites
 *   dW_shard [V_shard, H]  (may be NULL)   and   db_shard [V_shard] (may be NULL)
 * in the input dtype, and writes the shard's contribution to dx, float32
 * [N, H], into dx_partial (may be NULL): overwritten, or added to what it
 * holds when accumulate_dx != 0 (so shards run in sequence can sum into one
 * buffer).  dx itself is the sum over all shards, cast once to the input
 * dtype by the caller.
 */
flce_status flce_shard_backward(const void* x, const void* W_shard, const void* b_shard, const int64_t* targets,
                                int64_t N, int64_t H, int64_t V_shard, int64_t vocab_start, int64_t V_total,
                                flce_dtype dtype, float label_smoothing, float z_loss_scale, int64_t ignore_index,
                                flce_reduction reduction, const float* lse, const int64_t* n_valid, const float* grad_loss,
                                float* dx_partial, int accumulate_dx, void* dW_shard, void* db_shard,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* A static, human-readable name for a status code. */
const char* flce_status_string(flce_status status);

/*
 * Launch timing, for measurement (the per-kernel figures a benchmark reports
 * beside a profiler's trace).  flce_timing_start(capacity) discards the
 * calling thread's previous log, creates `capacity` HIP events (2 to 2^20)
 * and turns logging on: from then on the thread's entry-point calls record an
 * event on their stream before their first kernel and after each kernel
 * launch (hipEventRecord only: no synchronisation, no device memory), until
 * the events are used up or flce_timing_stop.  The events skip the
 * system-scope fence (hipEventDisableSystemFence), so a record writes back no
 * caches between kernels.  flce_timing_count gives the
 * number of kernel launches logged; flce_timing_read(i, &kernel, &ms) waits
 * for launch i's closing event and gives the launch's kernel (a static
 * string: the kernel and its template arguments as the source names them)
 * and the time from the event before it to the one after it.
 * flce_timing_clear destroys the events.  With logging off (the default) the
 * entry points record nothing.  Not one of the pages' operations.
 */
flce_status flce_timing_start(int capacity);
flce_status flce_timing_stop(void);
int64_t flce_timing_count(void);
flce_status flce_timing_read(int64_t index, const char** kernel, float* ms);
flce_status flce_timing_clear(void);

/* Vocabulary slab width (columns of dlogits held at once) the backward uses
 * for this problem; pure host arithmetic.  Returns 0 on invalid arguments.
 * The environment variable FLCE_SLAB_COLS, a positive multiple of 256 (other
 * values are ignored), overrides the automatic width (capped at V rounded up
 * to 256): narrower slabs take less workspace and keep buffer, and more
 * recompute launches.  At N=8192, H=4096, V=128256, 8192 columns hold all
 * extra memory under 10% of the bf16 logits (206.8 MB with the first slab
 * kept) for about 3% more time per step.  Below 256 x 256 / ceil(H / 256)
 * columns a slab's dW product has fewer output tiles than the GPU's 256 CUs:
 * at N=16384, H=1024, V=256000, 8192 columns cost 17%.  It is read on every
 * call, so it must not change between a workspace query and the calls that
 * use its answer. */
int64_t flce_backward_slab_cols(int64_t N, int64_t H, int64_t V, flce_dtype dtype);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
