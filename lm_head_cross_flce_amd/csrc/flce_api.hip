// C-ABI entry points of the FLCE library: argument validation, workspace
// layout and the launch sequence.  No allocation and no host synchronisation:
// everything is enqueued on the caller's stream.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <numeric>
#include <vector>

#include "flce.h"
#include "flce_launch.hpp"

namespace {

constexpr int kCUs = 256;                      // MI355X compute units
constexpr int kTile = 256;
constexpr size_t kAlign = 256;
constexpr size_t kSlabCapBytes = size_t(1) << 30;
constexpr size_t kSlabTargetBytes = size_t(256) << 20;
constexpr size_t kScratchBytes = FLCE_FORWARD_SCRATCH_BYTES;   // flce_forward_noalloc's static scratch

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Geometry {
  int NT, VT, P;
  int64_t slab_cols;
  int dx_split;
  size_t off_partials, off_rowloss, off_rowzl, fwd_total;
  size_t off_slab, off_dxacc, off_dbp, off_coef, off_yv, off_gscale, bwd_total;
  // Kept first slab (flce_forward_keep / flce_backward_kept): the forward's
  // kept-value schedule covers W's rows [0, width0) (VT0 tiles, P0 phases),
  // the plain forward the other VT - VT0 tiles (P1 phases); the keep buffer
  // holds the slab [N][slab_cols] in the input dtype at 0 and the maxima
  // [N][VT0][2] fp32 at off_kmref.
  int64_t width0;
  int VT0, P0, P1;
  size_t off_kmref, keep_total;
};

flce_status check_shape(int64_t N, int64_t H, int64_t V, int dtype) {
  if (N < 1 || H < 1 || V < 1) return FLCE_ERR_INVALID_ARGUMENT;
  if (dtype != FLCE_F32 && dtype != FLCE_BF16 && dtype != FLCE_F16) return FLCE_ERR_UNSUPPORTED;
  if (N > (int64_t(1) << 30) || V > (int64_t(1) << 30) || H > (int64_t(1) << 20)) return FLCE_ERR_UNSUPPORTED;
  if (H % 8 != 0) return FLCE_ERR_UNSUPPORTED;
  return FLCE_OK;
}

// Vocabulary slab width for the backward: the wider of (a) enough vocabulary
// tiles that the dW contraction of one slab (H/256 x slab/256 output tiles)
// fills every CU twice (once when the fp32 dx accumulator is under 128 MiB)
// and (b) the widest slab within 256 MiB whose dW tiles fill whole rounds of
// 256 CUs; capped at 1 GiB.  Every slab after the first costs one
// read-modify-write pass over the fp32 dx accumulator (N x H x 8 bytes),
// which all CUs make at the same moment, so wider slabs save HBM time when
// the accumulator is large; when it is small, a narrower slab is faster (at
// N=16384, H=1024, V=256000: 16384 columns instead of 32768, backward -1.7%,
// as more of the slab is still cached when dx and dW read it).  (b) gives the
// Llama-3-sized head (N=8192, H=4096, V=128256) 16384 columns, with all extra
// memory at 9.7% of its fp32 logits.
// FLCE_SLAB_COLS (a positive multiple of 256; the caller's memory knob) or
// else FLCE_DEBUG_SLAB_COLS (the tests force many slabs with it) overrides it.
int64_t slab_cols(int64_t N, int64_t H, int64_t V, int dtype) {
  const int64_t es = dtype == FLCE_F32 ? 4 : 2;
  const int64_t vmax = cdiv(V, kTile) * kTile;
  for (const char* name : {"FLCE_SLAB_COLS", "FLCE_DEBUG_SLAB_COLS"}) {
    if (const char* env = std::getenv(name)) {
      const long long c = std::atoll(env);
      if (c > 0 && c % kTile == 0) return c < vmax ? c : vmax;
    }
  }
  const int64_t th = cdiv(H, kTile);
  const bool small_acc = (size_t)N * (size_t)H * 4 < (size_t(128) << 20);
  int64_t want = cdiv((small_acc ? 1 : 2) * kCUs, th) * kTile;
  const int64_t round_cols = kTile * (kCUs / std::gcd((int64_t)kCUs, th));   // whole dW rounds
  const int64_t by_bytes = (int64_t)(kSlabTargetBytes / (size_t)(N * es)) / round_cols * round_cols;
  if (by_bytes > want) want = by_bytes;
  int64_t cap = (int64_t)(kSlabCapBytes / (size_t)(N * es)) / kTile * kTile;
  if (cap < kTile) cap = kTile;
  int64_t c = want < cap ? want : cap;
  return c < vmax ? c : vmax;
}

// Input-gradient K split.  The dx product has cdiv(N, 256) x cdiv(H, 256)
// output tiles, one workgroup each; when that is at most half the CUs, each
// slab's columns are split into parts that run side by side, each adding into
// its own fp32 accumulator, and the parts are summed once after the last slab.
// At most 8 parts of at least 512 columns.  The Llama-3-sized head (512
// tiles) never splits; N=4096, H=2048 (128 tiles) splits in two.
int dx_split(int64_t N, int64_t H, int64_t slab_cols) {
  const int64_t tiles = cdiv(N, kTile) * cdiv(H, kTile);
  if (2 * tiles > kCUs) return 1;
  int64_t p = kCUs / tiles;
  if (p > slab_cols / 512) p = slab_cols / 512;
  if (p > 8) p = 8;
  return p < 2 ? 1 : (int)p;
}

// Where the backward accumulates dx over the slabs.  Several K parts: one
// fp32 [N][H] accumulator each, summed once at the end.  One part and several
// slabs: fp32 inputs accumulate in dx itself; 16-bit inputs keep each fp32
// value's high half in dx and its low half in an [N][H] 16-bit array (exact:
// the value is the two halves' bits).  One slab: no accumulator.
bool dx_in_place(int64_t V, int64_t slab_cols, int parts) { return parts <= 1 && cdiv(V, slab_cols) > 1; }

size_t dx_acc_bytes(int64_t N, int64_t H, int64_t V, int dtype, int64_t slab_cols, int parts) {
  if (parts > 1) return (size_t)parts * N * H * 4;
  if (!dx_in_place(V, slab_cols, parts) || dtype == FLCE_F32) return 0;
  return (size_t)N * H * 2;
}

// Forward phases for NT token tiles: enough that the grid (token tiles x
// phases) fills the CUs, and at least 8 (see geometry), at most VT.
int fwd_phases(int NT, int VT) {
  int P = kCUs / NT;
  if (P < 8) P = 8;
  if (P > VT) P = VT;
  return P;
}

// with_dx_acc: the backward keeps its own fp32 dx accumulator (the shard
// backward accumulates into the caller's buffer instead).  kept: the layouts
// of flce_forward_keep and flce_backward_kept (the forward's partials cover
// both of its launches' phases; the backward's slab is the keep buffer).
Geometry geometry(int64_t N, int64_t H, int64_t V, int dtype, int has_bias, bool with_dx_acc = true,
                  bool kept = false) {
  Geometry g{};
  const int64_t es = dtype == FLCE_F32 ? 4 : 2;
  g.NT = (int)cdiv(N, kTile);
  g.VT = (int)cdiv(V, kTile);
  g.slab_cols = slab_cols(N, H, V, dtype);
  g.width0 = g.slab_cols < V ? g.slab_cols : V;
  g.VT0 = (int)cdiv(g.width0, kTile);
  g.P0 = fwd_phases(g.NT, g.VT0);
  g.P1 = g.VT > g.VT0 ? fwd_phases(g.NT, g.VT - g.VT0) : 0;
  // Forward phases: enough that the grid (token tiles x phases) fills the CUs,
  // and at least 8, so that each XCD's 32 concurrent tiles are 4 token tiles
  // x 8 vocabulary tiles (12 operand panels per round; 16 x 2 at N=32768
  // would stream 18) and take x's copies first.  Past 256 workgroups the grid
  // runs in rounds.  N=32768, H=2048, V=128000: 8 phases instead of 2, forward
  // -3.7% (same-box A/B).
  const int P = fwd_phases(g.NT, g.VT);
  g.P = P;
  size_t off = 0;
  g.off_partials = off;
  off = align_up(off + (size_t)(kept ? g.P0 + g.P1 : P) * N * 16);
  g.off_rowloss = off;
  off = align_up(off + (size_t)N * 4);
  g.off_rowzl = off;
  off = align_up(off + (size_t)N * 4);
  g.fwd_total = off;

  g.dx_split = with_dx_acc ? dx_split(N, H, g.slab_cols) : 1;
  off = 0;
  g.off_slab = off;
  if (!kept) off = align_up(off + (size_t)N * g.slab_cols * es);
  g.off_dxacc = off;
  if (with_dx_acc) off = align_up(off + dx_acc_bytes(N, H, V, dtype, g.slab_cols, g.dx_split));
  g.off_dbp = off;
  if (has_bias) off = align_up(off + (size_t)g.NT * g.slab_cols * 4);
  g.off_coef = off;
  off = align_up(off + (size_t)N * 16);
  g.off_yv = off;
  off = align_up(off + (size_t)N * 4);
  g.off_gscale = off;   // fp16: the dlogits slab's scale {S, 1/S}
  if (dtype == FLCE_F16) off = align_up(off + 8);
  g.bwd_total = off;

  g.off_kmref = align_up((size_t)N * g.slab_cols * es);
  g.keep_total = align_up(g.off_kmref + (size_t)N * g.VT0 * 2 * 4);
  return g;
}

// Fused schedule (gradients formed in the forward pass, one token chunk at a
// time).  Workspace: the chunk's kept logits [chunk][VT * 256] in the input
// dtype (turned into dlogits in place), their per-(token, tile, half) maxima,
// the chunk forward's per-phase partials, per-row losses of all N tokens,
// per-token coefficients, the dx product's K-split accumulators, and db's
// per-256-token column sums and fp32 running total.  Sized for the largest
// chunk and for the shorter last chunk, whichever needs more.
struct FusedGeometry {
  int64_t chunk;
  int VT;
  int64_t lde;
  size_t off_partials, off_rowloss, off_rowzl, off_e, off_mref, off_coef, off_yv, off_dxacc, off_dbp, off_dbacc,
      off_gscale, total;
};

FusedGeometry fused_geometry(int64_t N, int64_t H, int64_t V, int dtype, int has_bias, int64_t chunk) {
  FusedGeometry g{};
  const int64_t es = dtype == FLCE_F32 ? 4 : 2;
  g.chunk = chunk < N ? chunk : N;
  g.VT = (int)cdiv(V, kTile);
  g.lde = (int64_t)g.VT * kTile;
  const int64_t nchunks = cdiv(N, g.chunk);
  const int64_t sizes[2] = {g.chunk, N - (nchunks - 1) * g.chunk};
  size_t part = 0, dxacc = 0;
  for (int64_t c : sizes) {
    const int NTc = (int)cdiv(c, kTile);
    const size_t p = (size_t)fwd_phases(NTc, g.VT) * c * 16;
    const int split = dx_split(c, H, g.lde);
    const size_t a = split > 1 ? (size_t)split * c * H * 4 : 0;
    if (p > part) part = p;
    if (a > dxacc) dxacc = a;
  }
  size_t off = 0;
  g.off_partials = off;
  off = align_up(off + part);
  g.off_rowloss = off;
  off = align_up(off + (size_t)N * 4);
  g.off_rowzl = off;
  off = align_up(off + (size_t)N * 4);
  g.off_e = off;
  off = align_up(off + (size_t)g.chunk * g.lde * es);
  g.off_mref = off;
  off = align_up(off + (size_t)g.chunk * g.VT * 2 * 4);
  g.off_coef = off;
  off = align_up(off + (size_t)g.chunk * 16);
  g.off_yv = off;
  off = align_up(off + (size_t)g.chunk * 4);
  g.off_dxacc = off;
  off = align_up(off + dxacc);
  g.off_dbp = off;
  if (has_bias) off = align_up(off + (size_t)cdiv(g.chunk, kTile) * g.lde * 4);
  g.off_dbacc = off;
  if (has_bias) off = align_up(off + (size_t)V * 4);
  g.off_gscale = off;
  if (dtype == FLCE_F16) off = align_up(off + 8);
  g.total = off;
  return g;
}

// Default chunk: the fewest chunks whose workspace fits in what the recompute
// schedule uses for the same problem (forward plus backward workspace: the
// two schedules then compare at equal extra memory), then balanced, in
// multiples of 256 tokens.  At least 256 tokens.
int64_t fused_default_chunk(int64_t N, int64_t H, int64_t V, int dtype, int has_bias) {
  const Geometry r = geometry(N, H, V, dtype, has_bias);
  const size_t budget = r.fwd_total + r.bwd_total;
  int64_t best = kTile;
  for (int64_t c = cdiv(N, kTile) * kTile; c >= kTile; c -= kTile) {
    if (fused_geometry(N, H, V, dtype, has_bias, c).total <= budget) {
      best = c;
      break;
    }
  }
  const int64_t nchunks = cdiv(N, best);
  return cdiv(cdiv(N, nchunks), kTile) * kTile;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

flce_status check_options(float eps, float s, int reduction) {
  if (!(eps >= 0.f && eps <= 1.f)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!(s >= 0.f) || !std::isfinite(s)) return FLCE_ERR_INVALID_ARGUMENT;
  if (reduction != FLCE_REDUCTION_NONE && reduction != FLCE_REDUCTION_SUM && reduction != FLCE_REDUCTION_MEAN)
    return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

flce_status check_shard(int64_t V_shard, int64_t vocab_start, int64_t V_total) {
  if (vocab_start < 0 || V_total < 1 || V_total > (int64_t(1) << 30)) return FLCE_ERR_INVALID_ARGUMENT;
  if (vocab_start + V_shard > V_total) return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

flce_status check_inputs(const void* x, const void* W, const void* b, const int64_t* targets, int dtype) {
  if (!x || !W || !targets) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(targets, 8)) return FLCE_ERR_INVALID_ARGUMENT;
  if (b && !aligned(b, dtype == FLCE_F32 ? 4 : 2)) return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

// Backward launch sequence shared by the full and the shard entry points:
// per-token coefficients, then per slab the recompute, dx and dW (+ db)
// launches.  dx_out_fp32: dx is the fp32 accumulator itself (a.dx_acc),
// never cast; accumulate: it already holds a partial sum to add to.
// kmref (flce_backward_kept): the slab buffer a.slab already holds slab 0's
// kept values e and kmref their maxima; slab 0's dlogits are made from them in
// place (and its db partials written) instead of being recomputed.
flce_status run_backward(flce::BwdLaunch& a, const Geometry& g, int64_t V, int dtype, bool want_db,
                         bool dx_out_fp32, bool accumulate, hipStream_t s, const float* kmref = nullptr) {
  (void)hipGetLastError();
  flce::mark_launch(s, nullptr);
  if (flce::launch_bwd_prepare(a, s) != hipSuccess) return FLCE_ERR_HIP;
  if (kmref) {
    flce::FusedDz fd{};
    fd.ebuf = a.slab; fd.lde = a.ldS;
    fd.mref = kmref;
    fd.coef = a.coef; fd.yv = a.yv;
    fd.N = a.N; fd.V = (int)g.width0; fd.VT = g.VT0;
    fd.dbp = want_db ? a.dbp : nullptr;
    fd.gscale = nullptr;   // db partials of dz * S, as the recompute writes them (1/S is applied in their sum)
    if (flce::launch_fused_dz(fd, dtype, s) != hipSuccess) return FLCE_ERR_HIP;
  }
  const int64_t cols = g.slab_cols;
  const int64_t nslab = cdiv(V, cols);
  // dx accumulated in place (see dx_acc_bytes): fp32 dx is its own
  // accumulator, which the caller's-buffer modes below handle.
  const bool in_place = !dx_out_fp32 && a.dx && dx_in_place(V, cols, a.dx_split);
  const bool fp32_in_place = in_place && dtype == FLCE_F32;
  if (fp32_in_place) a.dx_acc = (float*)a.dx;
  a.split_acc = in_place && dtype != FLCE_F32;
  for (int64_t k = 0; k < nslab; ++k) {
    const int64_t vs = k * cols;
    const int64_t width = (V - vs) < cols ? (V - vs) : cols;
    int mode = flce::kDxAccum;
    if (dx_out_fp32 || fp32_in_place) {
      if (k == 0 && !(accumulate || (fp32_in_place && a.accumulate))) mode = flce::kDxFirst;
    } else if (a.dx_split > 1) {
      mode = k == 0 ? flce::kDxFirst : flce::kDxAccum;   // the parts' sum is written below
    } else if (nslab == 1) {
      mode = flce::kDxOnly;
    } else if (k == 0) {
      mode = flce::kDxFirst;
    } else if (k == nslab - 1) {
      mode = flce::kDxLast;
    }
    if (flce::launch_bwd_slab(a, dtype, (int)vs, (int)width, mode, want_db, kmref && k == 0, s) != hipSuccess)
      return FLCE_ERR_HIP;
  }
  if (a.dx && !dx_out_fp32 && a.dx_split > 1 && flce::launch_bwd_dx_finalize(a, dtype, s) != hipSuccess)
    return FLCE_ERR_HIP;
  return FLCE_OK;
}

flce_options default_options() {
  flce_options o{};
  o.logit_scale = 1.f;
  o.accumulate = 0;
  o.z_loss = nullptr;
  return o;
}

// Host-side checks of a forward call (no HIP call).
flce_status check_forward(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                          int64_t H, int64_t V, int dtype, float eps, float s, int reduction, const flce_options& o,
                          const float* loss, const float* lse, const int64_t* n_valid) {
  if (!std::isfinite(o.logit_scale)) return FLCE_ERR_INVALID_ARGUMENT;
  if (o.z_loss && !aligned(o.z_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  flce_status st = check_shape(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  if ((st = check_options(eps, s, reduction)) != FLCE_OK) return st;
  if ((st = check_inputs(x, W, b, targets, dtype)) != FLCE_OK) return st;
  if (!loss || !lse || !n_valid || !aligned(loss, 4) || !aligned(lse, 4) || !aligned(n_valid, 8))
    return FLCE_ERR_INVALID_ARGUMENT;
  return FLCE_OK;
}

// The forward's launches, with its per-phase partials and per-row losses in
// ws (g.fwd_total bytes, laid out by geometry()).
flce_status forward_into(const Geometry& g, const void* x, const void* W, const void* b, const int64_t* targets,
                         int64_t N, int64_t H, int64_t V, int dtype, float eps, float s, int64_t ignore_index,
                         int reduction, const flce_options& o, float* loss, float* lse, int64_t* n_valid, char* ws,
                         hipStream_t stream) {
  flce::FwdLaunch a{};
  a.x = x; a.W = W; a.b = b; a.targets = targets;
  a.N = (int)N; a.H = (int)H; a.V = (int)V;
  a.NT = g.NT; a.P = g.P; a.VT = g.VT;
  a.ignore_index = ignore_index;
  a.eps = eps;
  a.eps_over_v = (float)((double)eps / (double)V);
  a.s = s;
  a.reduction = reduction;
  a.logit_scale = o.logit_scale;
  a.partials = ws + g.off_partials;
  a.rowloss = (float*)(ws + g.off_rowloss);
  a.rowzl = (float*)(ws + g.off_rowzl);
  a.zloss = o.z_loss;
  a.loss = loss; a.lse = lse; a.n_valid = n_valid;
  (void)hipGetLastError();
  flce::mark_launch(stream, nullptr);
  if (flce::launch_forward(a, dtype, stream) != hipSuccess) return FLCE_ERR_HIP;
  return FLCE_OK;
}

// flce_forward_keep's launches: the kept-value forward over W's first
// g.width0 rows, writing e and its maxima into keep, and the plain forward
// over the rest, then one merge.
flce_status forward_keep_into(const Geometry& g, const void* x, const void* W, const void* b,
                              const int64_t* targets, int64_t N, int64_t H, int64_t V, int dtype, float eps, float s,
                              int64_t ignore_index, int reduction, const flce_options& o, float* loss, float* lse,
                              int64_t* n_valid, char* keep, char* ws, hipStream_t stream) {
  const int64_t es = dtype == FLCE_F32 ? 4 : 2;
  flce::FwdLaunch head{};
  head.x = x; head.W = W; head.b = b; head.targets = targets;
  head.N = (int)N; head.H = (int)H; head.V = (int)g.width0;
  head.NT = g.NT; head.P = g.P0; head.VT = g.VT0;
  head.ignore_index = ignore_index;
  head.eps = eps;
  head.eps_over_v = (float)((double)eps / (double)V);
  head.s = s;
  head.reduction = reduction;
  head.logit_scale = o.logit_scale;
  head.partials = ws + g.off_partials;
  head.rowloss = (float*)(ws + g.off_rowloss);
  head.rowzl = (float*)(ws + g.off_rowzl);
  head.zloss = o.z_loss;
  head.loss = loss; head.lse = lse; head.n_valid = n_valid;
  head.ebuf = keep;
  head.lde = g.slab_cols;
  head.mref = (float*)(keep + g.off_kmref);
  flce::FwdLaunch rest = head;
  rest.V = (int)(V - g.width0);
  if (rest.V > 0) {
    rest.W = (const char*)W + g.width0 * H * es;
    rest.b = b ? (const char*)b + g.width0 * es : nullptr;
    rest.VT = g.VT - g.VT0;
    rest.P = g.P1;
    rest.vocab_start = g.width0;
    rest.partials = ws + g.off_partials + (size_t)g.P0 * N * 16;
    rest.ebuf = nullptr;
    rest.mref = nullptr;
  }
  (void)hipGetLastError();
  flce::mark_launch(stream, nullptr);
  if (flce::launch_forward_keep(head, rest, dtype, stream) != hipSuccess) return FLCE_ERR_HIP;
  return FLCE_OK;
}

// ---------------------------------------------------------------------------
// Launch timing log (flce_timing_*).  Per host thread: a fixed set of events
// created by flce_timing_start, recorded in order by mark_launch until the
// set is used up.
// ---------------------------------------------------------------------------
struct TimingLog {
  bool on = false;
  size_t used = 0;
  std::vector<hipEvent_t> ev;
  std::vector<const char*> tag;
  std::vector<int> launch_mark;   // mark index that ends each logged launch
};
thread_local TimingLog g_tlog;

void timing_clear(TimingLog& t) {
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.clear();
  t.tag.clear();
  t.launch_mark.clear();
  t.used = 0;
  t.on = false;
}

// ---------------------------------------------------------------------------
// Static forward scratch (flce_forward_noalloc).  Each GPU holds its own copy
// of this array at its own address for the life of the process; host code
// uses only the address hipGetSymbolAddress returns for a device (the array's
// name on the host is a stand-in, not a device address).  The address is
// looked up once per device, with that device current, and cached.  The
// forward writes every byte it later reads (each phase's partials for every
// token, each row's loss), so nothing needs clearing between calls.
// ---------------------------------------------------------------------------

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The scratch array of the device that `stream` belongs to, which must be the
// current device (the symbol lookup is made with that device current).
flce_status scratch_on_stream_device(hipStream_t stream, char** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur < 0 || cur >= kMaxDevices) return FLCE_ERR_HIP;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return FLCE_ERR_HIP;
    if (sd != cur) return FLCE_ERR_INVALID_ARGUMENT;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FLCE_ERR_HIP;
    g_scratch_ptr[cur] = (char*)p;
  }
  *out = g_scratch_ptr[cur];
  return FLCE_OK;
}

flce_status backward_impl(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N, int64_t H,
                          int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale, int64_t ignore_index,
                          flce_reduction reduction, const flce_options* opts, const float* lse, const int64_t* n_valid,
                          const float* grad_loss, void* dx, void* dW, void* db, void* keep, size_t keep_bytes,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace

namespace flce {
void mark_launch(hipStream_t st, const char* kernel) {
  TimingLog& t = g_tlog;
  if (!t.on || t.used >= t.ev.size()) return;
  if (hipEventRecord(t.ev[t.used], st) != hipSuccess) {
    t.on = false;
    return;
  }
  t.tag[t.used] = kernel;
  if (kernel && t.used > 0) t.launch_mark.push_back((int)t.used);
  ++t.used;
}
}  // namespace flce

extern "C" {

flce_status flce_timing_start(int capacity) {
  if (capacity < 2 || capacity > (1 << 20)) return FLCE_ERR_INVALID_ARGUMENT;
  TimingLog& t = g_tlog;
  timing_clear(t);
  t.ev.resize((size_t)capacity, nullptr);
  t.tag.assign((size_t)capacity, nullptr);
  for (int i = 0; i < capacity; ++i) {
    // timing only: no system-scope fence (cache writeback) at each record
    if (hipEventCreateWithFlags(&t.ev[(size_t)i], hipEventDisableSystemFence) != hipSuccess) {
      t.ev.resize((size_t)i);
      timing_clear(t);
      return FLCE_ERR_HIP;
    }
  }
  t.on = true;
  return FLCE_OK;
}

flce_status flce_timing_stop(void) {
  g_tlog.on = false;
  return FLCE_OK;
}

int64_t flce_timing_count(void) { return (int64_t)g_tlog.launch_mark.size(); }

flce_status flce_timing_read(int64_t index, const char** kernel, float* ms) {
  const TimingLog& t = g_tlog;
  if (index < 0 || index >= (int64_t)t.launch_mark.size() || !kernel || !ms) return FLCE_ERR_INVALID_ARGUMENT;
  const int j = t.launch_mark[(size_t)index];
  if (hipEventSynchronize(t.ev[(size_t)j]) != hipSuccess) return FLCE_ERR_HIP;
  if (hipEventElapsedTime(ms, t.ev[(size_t)j - 1], t.ev[(size_t)j]) != hipSuccess) return FLCE_ERR_HIP;
  *kernel = t.tag[(size_t)j];
  return FLCE_OK;
}

flce_status flce_timing_clear(void) {
  timing_clear(g_tlog);
  return FLCE_OK;
}

const char* flce_status_string(flce_status status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case FLCE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FLCE_ERR_HIP: return "HIP launch failed";
    case FLCE_ERR_SCRATCH_TOO_SMALL: return "problem needs more forward scratch than the static buffer holds";
    default: return "unknown status";
  }
}

int64_t flce_backward_slab_cols(int64_t N, int64_t H, int64_t V, flce_dtype dtype) {
  if (check_shape(N, H, V, dtype) != FLCE_OK) return 0;
  return slab_cols(N, H, V, dtype);
}

flce_status flce_workspace_size(int64_t N, int64_t H, int64_t V, flce_dtype dtype, int has_bias, flce_reduction reduction,
                                size_t* fwd_bytes, size_t* bwd_bytes) {
  flce_status st = check_shape(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  st = check_options(0.f, 0.f, reduction);
  if (st != FLCE_OK) return st;
  const Geometry g = geometry(N, H, V, dtype, has_bias);
  if (fwd_bytes) *fwd_bytes = g.fwd_total;
  if (bwd_bytes) *bwd_bytes = g.bwd_total;
  return FLCE_OK;
}

flce_status flce_forward(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                         int64_t H, int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale,
                         int64_t ignore_index, flce_reduction reduction, float* loss, float* lse, int64_t* n_valid,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return flce_forward_ex(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index, reduction,
                         nullptr, loss, lse, n_valid, workspace, workspace_bytes, stream);
}

flce_status flce_forward_ex(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                            int64_t H, int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale,
                            int64_t ignore_index, flce_reduction reduction, const flce_options* opts, float* loss, float* lse,
                            int64_t* n_valid, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const flce_options o = opts ? *opts : default_options();
  flce_status st = check_forward(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, reduction, o,
                                 loss, lse, n_valid);
  if (st != FLCE_OK) return st;
  const Geometry g = geometry(N, H, V, dtype, b != nullptr);
  if (workspace_bytes < g.fwd_total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  return forward_into(g, x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index, reduction,
                      o, loss, lse, n_valid, (char*)workspace, (hipStream_t)stream);
}

flce_status flce_forward_noalloc(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                                 int64_t H, int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale,
                                 int64_t ignore_index, flce_reduction reduction, const flce_options* opts, float* loss,
                                 float* lse, int64_t* n_valid, hipStream_t stream) {
  const flce_options o = opts ? *opts : default_options();
  flce_status st = check_forward(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, reduction, o,
                                 loss, lse, n_valid);
  if (st != FLCE_OK) return st;
  const Geometry g = geometry(N, H, V, dtype, b != nullptr);
  if (g.fwd_total > kScratchBytes) return FLCE_ERR_SCRATCH_TOO_SMALL;
  char* ws = nullptr;
  if ((st = scratch_on_stream_device((hipStream_t)stream, &ws)) != FLCE_OK) return st;
  return forward_into(g, x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index, reduction,
                      o, loss, lse, n_valid, ws, (hipStream_t)stream);
}

flce_status flce_backward(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                          int64_t H, int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale,
                          int64_t ignore_index, flce_reduction reduction, const float* lse, const int64_t* n_valid,
                          const float* grad_loss, void* dx, void* dW, void* db, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return flce_backward_ex(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index, reduction,
                          nullptr, lse, n_valid, grad_loss, dx, dW, db, workspace, workspace_bytes, stream);
}

flce_status flce_backward_ex(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                             int64_t H, int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale,
                             int64_t ignore_index, flce_reduction reduction, const flce_options* opts, const float* lse,
                             const int64_t* n_valid, const float* grad_loss, void* dx, void* dW, void* db,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return backward_impl(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index, reduction, opts,
                       lse, n_valid, grad_loss, dx, dW, db, nullptr, 0, workspace, workspace_bytes, stream);
}

flce_status flce_keep_workspace_size(int64_t N, int64_t H, int64_t V, flce_dtype dtype, int has_bias,
                                     flce_reduction reduction, size_t* fwd_bytes, size_t* keep_bytes,
                                     size_t* bwd_bytes) {
  flce_status st = check_shape(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  st = check_options(0.f, 0.f, reduction);
  if (st != FLCE_OK) return st;
  const Geometry g = geometry(N, H, V, dtype, has_bias, true, true);
  if (fwd_bytes) *fwd_bytes = g.fwd_total;
  if (keep_bytes) *keep_bytes = g.keep_total;
  if (bwd_bytes) *bwd_bytes = g.bwd_total;
  return FLCE_OK;
}

flce_status flce_forward_keep(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                              int64_t H, int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale,
                              int64_t ignore_index, flce_reduction reduction, const flce_options* opts, float* loss,
                              float* lse, int64_t* n_valid, void* keep, size_t keep_bytes, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  const flce_options o = opts ? *opts : default_options();
  flce_status st = check_forward(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, reduction, o,
                                 loss, lse, n_valid);
  if (st != FLCE_OK) return st;
  const Geometry g = geometry(N, H, V, dtype, b != nullptr, true, true);
  if (workspace_bytes < g.fwd_total || keep_bytes < g.keep_total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 16) || !keep || !aligned(keep, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  return forward_keep_into(g, x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index,
                           reduction, o, loss, lse, n_valid, (char*)keep, (char*)workspace, (hipStream_t)stream);
}

flce_status flce_backward_kept(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N,
                               int64_t H, int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale,
                               int64_t ignore_index, flce_reduction reduction, const flce_options* opts,
                               const float* lse, const int64_t* n_valid, const float* grad_loss, void* keep,
                               size_t keep_bytes, void* dx, void* dW, void* db, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  if (!keep) return FLCE_ERR_INVALID_ARGUMENT;
  return backward_impl(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, ignore_index, reduction, opts,
                       lse, n_valid, grad_loss, dx, dW, db, keep, keep_bytes, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// flce_backward_ex, and with keep != NULL flce_backward_kept.
flce_status backward_impl(const void* x, const void* W, const void* b, const int64_t* targets, int64_t N, int64_t H,
                          int64_t V, flce_dtype dtype, float label_smoothing, float z_loss_scale, int64_t ignore_index,
                          flce_reduction reduction, const flce_options* opts, const float* lse, const int64_t* n_valid,
                          const float* grad_loss, void* dx, void* dW, void* db, void* keep, size_t keep_bytes,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const flce_options o = opts ? *opts : default_options();
  if (!std::isfinite(o.logit_scale)) return FLCE_ERR_INVALID_ARGUMENT;
  flce_status st = check_shape(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  if ((st = check_options(label_smoothing, z_loss_scale, reduction)) != FLCE_OK) return st;
  if ((st = check_inputs(x, W, b, targets, dtype)) != FLCE_OK) return st;
  if (!lse || !n_valid || !grad_loss) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned(lse, 4) || !aligned(n_valid, 8) || !aligned(grad_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if ((dx && !aligned(dx, 16)) || (dW && !aligned(dW, 16))) return FLCE_ERR_INVALID_ARGUMENT;
  if (db && !aligned(db, dtype == FLCE_F32 ? 4 : 2)) return FLCE_ERR_INVALID_ARGUMENT;
  const bool kept = keep != nullptr;
  const Geometry g = geometry(N, H, V, dtype, b != nullptr, true, kept);
  if (workspace_bytes < g.bwd_total || (kept && keep_bytes < g.keep_total)) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 16) || (kept && !aligned(keep, 16))) return FLCE_ERR_INVALID_ARGUMENT;
  const bool want_db = b != nullptr && db != nullptr;
  if (!dx && !dW && !want_db) return FLCE_OK;

  char* ws = (char*)workspace;
  flce::BwdLaunch a{};
  a.x = x; a.W = W; a.b = b; a.targets = targets;
  a.N = (int)N; a.H = (int)H; a.V = (int)V;
  a.NT = g.NT;
  a.ignore_index = ignore_index;
  a.eps = label_smoothing;
  a.eps_over_v = (float)((double)label_smoothing / (double)V);
  a.s = z_loss_scale;
  a.logit_scale = o.logit_scale;
  a.reduction = reduction;
  a.accumulate = o.accumulate != 0;
  a.lse = lse; a.n_valid = n_valid; a.grad = grad_loss;
  a.coef = ws + g.off_coef;
  a.yv = (int*)(ws + g.off_yv);
  a.slab = kept ? (char*)keep : ws + g.off_slab;
  a.ldS = g.slab_cols;
  a.dx_acc = (float*)(ws + g.off_dxacc);
  a.dx_split = g.dx_split;
  a.dbp = want_db ? (float*)(ws + g.off_dbp) : nullptr;
  a.gscale = dtype == FLCE_F16 ? (float*)(ws + g.off_gscale) : nullptr;
  a.dx = dx; a.dW = dW; a.db = want_db ? db : nullptr;

  return run_backward(a, g, V, dtype, want_db, false, false, (hipStream_t)stream,
                      kept ? (const float*)((char*)keep + g.off_kmref) : nullptr);
}

}  // namespace

extern "C" {

flce_status flce_fused_workspace_size(int64_t N, int64_t H, int64_t V, flce_dtype dtype, int has_bias,
                                      int64_t chunk_tokens, int64_t* chunk_used, size_t* bytes) {
  flce_status st = check_shape(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  if (chunk_tokens < 0 || chunk_tokens % kTile != 0) return FLCE_ERR_INVALID_ARGUMENT;
  const int64_t chunk = chunk_tokens ? chunk_tokens : fused_default_chunk(N, H, V, dtype, has_bias);
  const FusedGeometry g = fused_geometry(N, H, V, dtype, has_bias, chunk);
  if (chunk_used) *chunk_used = g.chunk;
  if (bytes) *bytes = g.total;
  return FLCE_OK;
}

flce_status flce_fused_forward_backward(const void* x, const void* W, const void* b, const int64_t* targets,
                                        int64_t N, int64_t H, int64_t V, flce_dtype dtype, float label_smoothing,
                                        float z_loss_scale, int64_t ignore_index, flce_reduction reduction,
                                        const flce_options* opts, const float* grad_loss, int64_t chunk_tokens,
                                        float* loss, float* lse, int64_t* n_valid, void* dx, void* dW, void* db,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const flce_options o = opts ? *opts : default_options();
  flce_status st = check_forward(x, W, b, targets, N, H, V, dtype, label_smoothing, z_loss_scale, reduction, o,
                                 loss, lse, n_valid);
  if (st != FLCE_OK) return st;
  if (!grad_loss || !aligned(grad_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if ((dx && !aligned(dx, 16)) || (dW && !aligned(dW, 16))) return FLCE_ERR_INVALID_ARGUMENT;
  if (db && !aligned(db, dtype == FLCE_F32 ? 4 : 2)) return FLCE_ERR_INVALID_ARGUMENT;
  if (chunk_tokens < 0 || chunk_tokens % kTile != 0) return FLCE_ERR_INVALID_ARGUMENT;
  const int64_t chunk = chunk_tokens ? chunk_tokens : fused_default_chunk(N, H, V, dtype, b != nullptr);
  const FusedGeometry g = fused_geometry(N, H, V, dtype, b != nullptr, chunk);
  if (workspace_bytes < g.total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  const bool want_db = b != nullptr && db != nullptr;
  const bool grads = dx || dW || want_db;
  const int64_t es = dtype == FLCE_F32 ? 4 : 2;
  const bool none = reduction == FLCE_REDUCTION_NONE;
  char* ws = (char*)workspace;
  float* gscale = dtype == FLCE_F16 ? (float*)(ws + g.off_gscale) : nullptr;

  flce::FwdLaunch base{};
  base.W = W; base.b = b;
  base.H = (int)H; base.V = (int)V; base.VT = g.VT;
  base.ignore_index = ignore_index;
  base.eps = label_smoothing;
  base.eps_over_v = (float)((double)label_smoothing / (double)V);
  base.s = z_loss_scale;
  base.reduction = reduction;
  base.logit_scale = o.logit_scale;
  base.n_valid = n_valid;
  (void)hipGetLastError();
  flce::mark_launch(stream, nullptr);
  // The mean's count is needed by the first chunk's dlogits.
  flce::FwdLaunch cnt = base;
  cnt.targets = targets;
  cnt.N = (int)N;
  if (grads && flce::launch_fused_count(cnt, stream) != hipSuccess) return FLCE_ERR_HIP;
  for (int64_t c0 = 0; c0 < N; c0 += g.chunk) {
    const int nc = (int)((N - c0) < g.chunk ? (N - c0) : g.chunk);
    const int NTc = (int)cdiv(nc, kTile);
    const bool first = c0 == 0, last = c0 + nc >= N;
    flce::FwdLaunch fa = base;
    fa.x = (const char*)x + c0 * H * es;
    fa.targets = targets + c0;
    fa.N = nc;
    fa.NT = NTc;
    fa.P = fwd_phases(NTc, g.VT);
    fa.partials = ws + g.off_partials;
    fa.rowloss = (float*)(ws + g.off_rowloss) + c0;
    fa.rowzl = (float*)(ws + g.off_rowzl) + c0;
    fa.zloss = o.z_loss ? (none ? o.z_loss + c0 : o.z_loss) : nullptr;
    fa.loss = none ? loss + c0 : loss;
    fa.lse = lse + c0;
    fa.ebuf = ws + g.off_e;
    fa.lde = g.lde;
    fa.mref = (float*)(ws + g.off_mref);
    if (flce::launch_fused_forward(fa, dtype, stream) != hipSuccess) return FLCE_ERR_HIP;
    if (!grads) continue;
    flce::BwdLaunch ba{};
    ba.x = fa.x; ba.W = W; ba.b = b; ba.targets = targets + c0;
    ba.N = nc; ba.H = (int)H; ba.V = (int)V; ba.NT = NTc;
    ba.ignore_index = ignore_index;
    ba.eps = label_smoothing;
    ba.eps_over_v = base.eps_over_v;
    ba.s = z_loss_scale;
    ba.logit_scale = o.logit_scale;
    ba.reduction = reduction;
    ba.accumulate = o.accumulate != 0;
    ba.lse = lse + c0; ba.n_valid = n_valid;
    ba.grad = none ? grad_loss + c0 : grad_loss;
    ba.coef = ws + g.off_coef;
    ba.yv = (int*)(ws + g.off_yv);
    ba.slab = ws + g.off_e;
    ba.ldS = g.lde;
    ba.dx_acc = (float*)(ws + g.off_dxacc);
    ba.dx_split = dx_split(nc, H, g.lde);
    ba.gscale = gscale;
    ba.dx = dx ? (char*)dx + c0 * H * es : nullptr;
    ba.dW = dW;
    ba.db = nullptr;
    if (flce::launch_bwd_prepare(ba, stream) != hipSuccess) return FLCE_ERR_HIP;
    flce::FusedDz fd{};
    fd.ebuf = ws + g.off_e; fd.lde = g.lde;
    fd.mref = (const float*)(ws + g.off_mref);
    fd.coef = ba.coef; fd.yv = ba.yv;
    fd.N = nc; fd.V = (int)V; fd.VT = g.VT;
    fd.dbp = want_db ? (float*)(ws + g.off_dbp) : nullptr;
    fd.gscale = gscale;
    if (flce::launch_fused_dz(fd, dtype, stream) != hipSuccess) return FLCE_ERR_HIP;
    if (want_db && flce::launch_fused_db(fd.dbp, NTc, g.lde, (float*)(ws + g.off_dbacc), (int)V, first, last, db,
                                         dtype, o.accumulate != 0, stream) != hipSuccess)
      return FLCE_ERR_HIP;
    if ((dx || dW) && flce::launch_fused_products(ba, dtype, first, stream) != hipSuccess) return FLCE_ERR_HIP;
  }
  flce::FwdLaunch fin = base;
  fin.targets = targets;
  fin.N = (int)N;
  fin.rowloss = (float*)(ws + g.off_rowloss);
  fin.rowzl = (float*)(ws + g.off_rowzl);
  fin.zloss = o.z_loss;
  fin.loss = loss;
  if (flce::launch_finalize(fin, stream) != hipSuccess) return FLCE_ERR_HIP;
  return FLCE_OK;
}

flce_status flce_shard_workspace_size(int64_t N, int64_t H, int64_t V_shard, flce_dtype dtype, int has_bias,
                                      size_t* fwd_bytes, size_t* merge_bytes, size_t* bwd_bytes) {
  flce_status st = check_shape(N, H, V_shard, dtype);
  if (st != FLCE_OK) return st;
  const Geometry g = geometry(N, H, V_shard, dtype, has_bias, false);
  if (fwd_bytes) *fwd_bytes = g.fwd_total;
  if (merge_bytes) *merge_bytes = align_up((size_t)N * 4);
  if (bwd_bytes) *bwd_bytes = g.bwd_total;
  return FLCE_OK;
}

flce_status flce_shard_forward(const void* x, const void* W_shard, const void* b_shard, const int64_t* targets,
                               int64_t N, int64_t H, int64_t V_shard, int64_t vocab_start, int64_t V_total,
                               flce_dtype dtype, float label_smoothing, int64_t ignore_index, float* stats,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  flce_status st = check_shape(N, H, V_shard, dtype);
  if (st != FLCE_OK) return st;
  if ((st = check_shard(V_shard, vocab_start, V_total)) != FLCE_OK) return st;
  if ((st = check_options(label_smoothing, 0.f, FLCE_REDUCTION_MEAN)) != FLCE_OK) return st;
  if ((st = check_inputs(x, W_shard, b_shard, targets, dtype)) != FLCE_OK) return st;
  if (!stats || !aligned(stats, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  const Geometry g = geometry(N, H, V_shard, dtype, b_shard != nullptr, false);
  if (workspace_bytes < g.fwd_total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 16)) return FLCE_ERR_INVALID_ARGUMENT;

  char* ws = (char*)workspace;
  flce::FwdLaunch a{};
  a.x = x; a.W = W_shard; a.b = b_shard; a.targets = targets;
  a.N = (int)N; a.H = (int)H; a.V = (int)V_shard;
  a.NT = g.NT; a.P = g.P; a.VT = g.VT;
  a.vocab_start = vocab_start;
  a.ignore_index = ignore_index;
  a.eps = label_smoothing;
  a.logit_scale = 1.f;
  a.partials = ws + g.off_partials;
  a.stats = stats;
  (void)hipGetLastError();
  flce::mark_launch((hipStream_t)stream, nullptr);
  if (flce::launch_shard_forward(a, dtype, (hipStream_t)stream) != hipSuccess) return FLCE_ERR_HIP;
  return FLCE_OK;
}

flce_status flce_shard_merge(const float* stats, int64_t num_shards, const int64_t* targets, int64_t N,
                             int64_t V_total, float label_smoothing, float z_loss_scale, int64_t ignore_index,
                             flce_reduction reduction, float* loss, float* lse, int64_t* n_valid, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (N < 1 || N > (int64_t(1) << 30) || V_total < 1 || V_total > (int64_t(1) << 30)) return FLCE_ERR_INVALID_ARGUMENT;
  if (num_shards < 1 || num_shards > (int64_t(1) << 20)) return FLCE_ERR_INVALID_ARGUMENT;
  flce_status st = check_options(label_smoothing, z_loss_scale, reduction);
  if (st != FLCE_OK) return st;
  if (!stats || !aligned(stats, 16) || !targets || !aligned(targets, 8)) return FLCE_ERR_INVALID_ARGUMENT;
  if (!loss || !lse || !n_valid || !aligned(loss, 4) || !aligned(lse, 4) || !aligned(n_valid, 8))
    return FLCE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < align_up((size_t)N * 4)) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 16)) return FLCE_ERR_INVALID_ARGUMENT;

  flce::FwdLaunch a{};
  a.targets = targets;
  a.N = (int)N;
  a.P = (int)num_shards;
  a.ignore_index = ignore_index;
  a.eps = label_smoothing;
  a.eps_over_v = (float)((double)label_smoothing / (double)V_total);
  a.s = z_loss_scale;
  a.logit_scale = 1.f;
  a.reduction = reduction;
  a.partials = const_cast<float*>(stats);
  a.rowloss = (float*)workspace;
  a.loss = loss; a.lse = lse; a.n_valid = n_valid;
  (void)hipGetLastError();
  flce::mark_launch((hipStream_t)stream, nullptr);
  if (flce::launch_merge(a, (hipStream_t)stream) != hipSuccess) return FLCE_ERR_HIP;
  return FLCE_OK;
}

flce_status flce_shard_backward(const void* x, const void* W_shard, const void* b_shard, const int64_t* targets,
                                int64_t N, int64_t H, int64_t V_shard, int64_t vocab_start, int64_t V_total,
                                flce_dtype dtype, float label_smoothing, float z_loss_scale, int64_t ignore_index,
                                flce_reduction reduction, const float* lse, const int64_t* n_valid, const float* grad_loss,
                                float* dx_partial, int accumulate_dx, void* dW_shard, void* db_shard,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  flce_status st = check_shape(N, H, V_shard, dtype);
  if (st != FLCE_OK) return st;
  if ((st = check_shard(V_shard, vocab_start, V_total)) != FLCE_OK) return st;
  if ((st = check_options(label_smoothing, z_loss_scale, reduction)) != FLCE_OK) return st;
  if ((st = check_inputs(x, W_shard, b_shard, targets, dtype)) != FLCE_OK) return st;
  if (!lse || !n_valid || !grad_loss) return FLCE_ERR_INVALID_ARGUMENT;
  if (!aligned(lse, 4) || !aligned(n_valid, 8) || !aligned(grad_loss, 4)) return FLCE_ERR_INVALID_ARGUMENT;
  if ((dx_partial && !aligned(dx_partial, 16)) || (dW_shard && !aligned(dW_shard, 16))) return FLCE_ERR_INVALID_ARGUMENT;
  if (db_shard && !aligned(db_shard, dtype == FLCE_F32 ? 4 : 2)) return FLCE_ERR_INVALID_ARGUMENT;
  const Geometry g = geometry(N, H, V_shard, dtype, b_shard != nullptr, false);
  if (workspace_bytes < g.bwd_total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned(workspace, 16)) return FLCE_ERR_INVALID_ARGUMENT;
  const bool want_db = b_shard != nullptr && db_shard != nullptr;
  if (!dx_partial && !dW_shard && !want_db) return FLCE_OK;

  char* ws = (char*)workspace;
  flce::BwdLaunch a{};
  a.x = x; a.W = W_shard; a.b = b_shard; a.targets = targets;
  a.N = (int)N; a.H = (int)H; a.V = (int)V_shard;
  a.NT = g.NT;
  a.vocab_start = vocab_start;
  a.ignore_index = ignore_index;
  a.eps = label_smoothing;
  a.eps_over_v = (float)((double)label_smoothing / (double)V_total);
  a.s = z_loss_scale;
  a.logit_scale = 1.f;
  a.reduction = reduction;
  a.lse = lse; a.n_valid = n_valid; a.grad = grad_loss;
  a.coef = ws + g.off_coef;
  a.yv = (int*)(ws + g.off_yv);
  a.slab = ws + g.off_slab;
  a.ldS = g.slab_cols;
  a.dx_acc = dx_partial;
  a.dbp = want_db ? (float*)(ws + g.off_dbp) : nullptr;
  a.gscale = dtype == FLCE_F16 ? (float*)(ws + g.off_gscale) : nullptr;
  a.dx = dx_partial; a.dW = dW_shard; a.db = want_db ? db_shard : nullptr;
  return run_backward(a, g, V_shard, dtype, want_db, true, accumulate_dx != 0, (hipStream_t)stream);
}

}  // extern "C"
