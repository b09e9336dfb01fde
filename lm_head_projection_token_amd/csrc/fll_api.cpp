// C ABI of the fused lm_head loss: planner, argument checks, dispatch of the
// per-chunk kernel sequence, and event-based kernel timing.
//
// The chunk loop follows the chunked gradient-in-forward structure
// [FusedLinearKLDivLoss page, Summary]: for each token chunk the logits, the
// row statistics, the loss terms and the dlogits are formed, then dX (and dW,
// db only when asked for [frozen lm_head GRPO page, Summary; LoRA
// normalization page, Key Changes]) are produced before the next chunk.
#include "../../include/fll.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "fll_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

constexpr int64_t kMaxChunkRows = 8192;
constexpr size_t kDefaultBudget = size_t(64) << 30;  // 64 GiB of 288 GB

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline size_t align256(size_t a) { return (a + 255) & ~size_t(255); }
inline bool ratio_head(int h) { return h == FLL_HEAD_PPO_CLIP || h == FLL_HEAD_CISPO; }
// heads whose per-row term is a function of log p(y_r) of a label
inline bool label_head(int h) {
  return h == FLL_HEAD_SELECTIVE_LOGPROB || h == FLL_HEAD_CROSS_ENTROPY || ratio_head(h);
}

int check_problem(const fll_problem *p) {
  if (!p) return fail(FLL_ERR_INVALID_ARG, "problem is NULL");
  if (p->reduction == FLL_RED_NONE)
    return fail(FLL_ERR_UNSUPPORTED,
                "reduction 'none' is unsupported: gradient-in-forward needs a "
                "scalar loss (use an unfused per-element KL instead)");
  if (p->reduction < FLL_RED_BATCHMEAN || p->reduction > FLL_RED_SUM)
    return fail(FLL_ERR_INVALID_ARG, "unknown reduction %d", p->reduction);
  if (p->dtype != FLL_BF16 && p->dtype != FLL_FP32)
    return fail(FLL_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (p->head < FLL_HEAD_KL || p->head > FLL_HEAD_CISPO)
    return fail(FLL_ERR_INVALID_ARG, "unknown head %d", p->head);
  if (ratio_head(p->head)) {
    if (!(p->clip_low >= 0.0f && p->clip_low <= 1.0f))
      return fail(FLL_ERR_INVALID_ARG, "clip_low must lie in [0, 1]");
    if (!(p->clip_high >= 0.0f))  // +inf allowed: no upper clip
      return fail(FLL_ERR_INVALID_ARG, "clip_high must be >= 0");
  } else if (p->clip_low != 0.0f || p->clip_high != 0.0f) {
    return fail(FLL_ERR_INVALID_ARG, "clip_low and clip_high are for the ratio heads");
  }
  if (p->head == FLL_HEAD_JSD) {
    if (p->H_teacher < 8 || p->H_teacher % 8 != 0 || p->H_teacher > (int64_t(1) << 20))
      return fail(FLL_ERR_INVALID_ARG,
                  "the JSD head needs H_teacher, a multiple of 8 in [8, 2^20] (got %lld)",
                  (long long)p->H_teacher);
    if (p->teacher_has_bias != 0 && p->teacher_has_bias != 1)
      return fail(FLL_ERR_INVALID_ARG, "flags must be 0 or 1");
  } else if (p->H_teacher != 0 || p->teacher_has_bias != 0) {
    return fail(FLL_ERR_INVALID_ARG, "H_teacher and teacher_has_bias are for the JSD head");
  }
  if (p->logits_bf16 != 0 && p->logits_bf16 != 1)
    return fail(FLL_ERR_INVALID_ARG, "flags must be 0 or 1");
  if (p->logits_bf16 && p->dtype != FLL_BF16)
    return fail(FLL_ERR_INVALID_ARG, "logits_bf16 is for bf16 problems");
  if (p->BT < 0) return fail(FLL_ERR_INVALID_ARG, "BT < 0");
  if (p->V < 1) return fail(FLL_ERR_INVALID_ARG, "V must be >= 1");
  if (p->H < 8 || p->H % 8 != 0)
    return fail(FLL_ERR_INVALID_ARG, "H must be a positive multiple of 8 (got %lld)",
                (long long)p->H);
  if (p->V > (int64_t(1) << 21) - 64 || p->H > (int64_t(1) << 20))
    return fail(FLL_ERR_INVALID_ARG, "V (max 2^21 - 64) or H (max 2^20) too large");
  for (int f : {p->has_bias, p->compute_dW, p->compute_db})
    if (f != 0 && f != 1) return fail(FLL_ERR_INVALID_ARG, "flags must be 0 or 1");
  if (p->compute_db && !p->has_bias)
    return fail(FLL_ERR_INVALID_ARG, "compute_db needs has_bias");
  if (!(p->temperature > 0.0f) || !std::isfinite(p->temperature))
    return fail(FLL_ERR_INVALID_ARG, "temperature must be positive and finite");
  if (!(p->eps >= 0.0f) || !std::isfinite(p->eps))
    return fail(FLL_ERR_INVALID_ARG, "eps must be >= 0 and finite");
  return FLL_OK;
}

// Lay out the workspace for a given chunk size.
void layout(fll_plan_t *pl, int64_t C) {
  const fll_problem &p = pl->p;
  pl->chunk_rows = C;
  pl->n_chunks = p.BT > 0 ? cdiv(p.BT, C) : 0;
  pl->s_pitch = rup(p.V, 64);
  // The dX GEMM has only C/tile x H/tile output tiles, so its vocabulary
  // (K) range is split until one workgroup per CU fills the 256 CUs of an
  // MI355X (measured ahead of two per CU: 1.2 % at C = 4096 and 2048 with
  // H = 4096, V = 128256; 22 % at C = 512, V = 32000), each split keeping
  // at least 2048 vocabulary entries. The split depends on the chunk size
  // but never on the dW/db flags, so dX is bit-identical with and without
  // them.
  const int64_t tile = p.dtype == FLL_BF16 ? 256 : 64;
  const int64_t out_tiles = cdiv(C, tile) * cdiv(p.H, tile);
  const int64_t max_splits = std::max<int64_t>(1, std::min<int64_t>(16, p.V / 2048));
  int64_t splits = std::min(max_splits, std::max<int64_t>(1, cdiv(256, out_tiles)));
  pl->dx_split_len = rup(cdiv(p.V, splits), 64);
  pl->dx_splits = cdiv(p.V, pl->dx_split_len);
  // per-row (max, sum exp) of every 128-column block, from the bf16 logits GEMM
  pl->stat_tiles = p.dtype == FLL_BF16 ? cdiv(p.V, 128) : 0;
  size_t off = 0;
  const size_t s_elem = p.logits_bf16 ? 2 : 4;  // bytes per chunk logit
  pl->off_logits = off;
  off = align256(off + size_t(C) * size_t(pl->s_pitch) * s_elem);
  pl->off_rowval = off;
  off = align256(off + size_t(std::max<int64_t>(p.BT, 1)) * 4);
  pl->off_stats = off;
  off = align256(off + size_t(C) * size_t(pl->stat_tiles) * 8);
  // fp32 partial sums of the dX splits; after dX is reduced the same bytes
  // hold the db column sums over kDbSplits row ranges (db without dW) or the
  // chunk's X transposed for the bf16 dW GEMM. Sized for all three whatever
  // the flags, so C does not depend on them.
  pl->off_dx_partial = off;
  {
    const size_t dx_part = pl->dx_splits > 1 ? size_t(pl->dx_splits) * C * p.H * 4 : 0;
    const size_t db_part = size_t(fll::kDbSplits) * size_t(p.V) * 4;
    const size_t xt_part = p.dtype == FLL_BF16 ? size_t(p.H) * size_t(rup(C, 64)) * 2 : 0;
    off = align256(off + std::max(std::max(dx_part, db_part), xt_part));
  }
  pl->off_scalars = off;
  off = align256(off + sizeof(fll::DevScalars));
  // JSD: the teacher's logits of the chunk and their row statistics
  pl->off_teacher = off;
  pl->off_teacher_stats = off;
  if (p.head == FLL_HEAD_JSD) {
    off = align256(off + size_t(C) * size_t(pl->s_pitch) * s_elem);
    pl->off_teacher_stats = off;
    off = align256(off + size_t(C) * size_t(pl->stat_tiles) * 8);
  }
  pl->workspace_bytes = off;
}

int make_plan(const fll_problem *problem, size_t budget, int64_t chunk_rows,
              fll_plan_t *plan) {
  int st = check_problem(problem);
  if (st) return st;
  if (!plan) return fail(FLL_ERR_INVALID_ARG, "plan is NULL");
  if (chunk_rows < 0) return fail(FLL_ERR_INVALID_ARG, "chunk_rows < 0");
  if (budget == 0) budget = kDefaultBudget;
  fll_plan_t pl;
  memset(&pl, 0, sizeof(pl));
  pl.p = *problem;
  const int64_t BT = problem->BT;
  const int64_t tile = problem->dtype == FLL_BF16 ? 256 : 64;
  int64_t C;
  if (chunk_rows > 0) {
    C = std::min<int64_t>(chunk_rows, std::max<int64_t>(BT, 1));
  } else if (BT <= tile) {
    C = std::max<int64_t>(BT, 1);
  } else {
    // at least two chunks: the BT x V logits are never formed at once
    C = std::min(rup(cdiv(BT, 2), tile), kMaxChunkRows);
  }
  layout(&pl, C);
  while (pl.workspace_bytes > budget && chunk_rows == 0 && C > tile) {
    C -= tile;
    layout(&pl, C);
  }
  if (pl.workspace_bytes > budget)
    return fail(FLL_ERR_WORKSPACE, "workspace of %zu bytes exceeds the budget of %zu",
                pl.workspace_bytes, budget);
  *plan = pl;
  return FLL_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_args(const fll_plan_t *pl, const fll_args *a) {
  if (!pl || !a) return fail(FLL_ERR_INVALID_ARG, "plan or args is NULL");
  int st = check_problem(&pl->p);
  if (st) return st;
  if (pl->chunk_rows < 1) return fail(FLL_ERR_INVALID_ARG, "plan has no chunk size");
  fll_plan_t re;
  memset(&re, 0, sizeof(re));
  re.p = pl->p;
  layout(&re, pl->chunk_rows);
  if (memcmp(&re, pl, sizeof(re)) != 0)
    return fail(FLL_ERR_INVALID_ARG, "plan was modified or is not from fll_plan");
  const fll_problem &p = pl->p;
  const size_t esz = p.dtype == FLL_BF16 ? 2 : 4;
  if (!a->loss) return fail(FLL_ERR_INVALID_ARG, "loss is NULL");
  if (!aligned(a->loss, 4)) return fail(FLL_ERR_INVALID_ARG, "loss misaligned");
  if (p.compute_dW && !a->dW) return fail(FLL_ERR_INVALID_ARG, "compute_dW but dW is NULL");
  if (p.compute_db && !a->db) return fail(FLL_ERR_INVALID_ARG, "compute_db but db is NULL");
  if (p.compute_dW && !aligned(a->dW, 16)) return fail(FLL_ERR_INVALID_ARG, "dW not 16-byte aligned");
  if (p.compute_db && !aligned(a->db, 4)) return fail(FLL_ERR_INVALID_ARG, "db misaligned");
  if (p.has_bias && !a->b) return fail(FLL_ERR_INVALID_ARG, "has_bias but b is NULL");
  if (!p.has_bias && a->b) return fail(FLL_ERR_INVALID_ARG, "b given but has_bias is 0");
  if (p.has_bias && !aligned(a->b, esz)) return fail(FLL_ERR_INVALID_ARG, "b misaligned");
  if (!a->workspace || a->workspace_bytes < pl->workspace_bytes)
    return fail(FLL_ERR_WORKSPACE, "workspace NULL or smaller than plan.workspace_bytes (%zu)",
                pl->workspace_bytes);
  if (!aligned(a->workspace, 256)) return fail(FLL_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (p.BT == 0) return FLL_OK;
  if (!a->X || !a->W || !a->dX) return fail(FLL_ERR_INVALID_ARG, "X, W and dX are required");
  if (!aligned(a->X, 16) || !aligned(a->W, 16) || !aligned(a->dX, 16))
    return fail(FLL_ERR_INVALID_ARG, "X, W and dX must be 16-byte aligned");
  if (label_head(p.head)) {
    if (!a->labels) return fail(FLL_ERR_INVALID_ARG, "the label heads need labels");
    if (a->target)
      return fail(FLL_ERR_INVALID_ARG, "target given for a label head");
    if (ratio_head(p.head) && !a->old_logprobs)
      return fail(FLL_ERR_INVALID_ARG, "the ratio heads need old_logprobs");
  } else if (p.head == FLL_HEAD_KL) {
    if (!a->target) return fail(FLL_ERR_INVALID_ARG, "the KL head needs a target");
    if (a->weights) return fail(FLL_ERR_INVALID_ARG, "weights given for the KL head");
    if (!aligned(a->target, 4)) return fail(FLL_ERR_INVALID_ARG, "target misaligned");
  } else {
    if (a->target || a->weights)
      return fail(FLL_ERR_INVALID_ARG, "the JSD head takes no target and no weights");
    if (!a->X_teacher || !a->W_teacher)
      return fail(FLL_ERR_INVALID_ARG, "the JSD head needs X_teacher and W_teacher");
    if (!aligned(a->X_teacher, 16) || !aligned(a->W_teacher, 16))
      return fail(FLL_ERR_INVALID_ARG, "X_teacher and W_teacher must be 16-byte aligned");
    if (p.teacher_has_bias && !a->b_teacher)
      return fail(FLL_ERR_INVALID_ARG, "teacher_has_bias but b_teacher is NULL");
    if (p.teacher_has_bias && !aligned(a->b_teacher, esz))
      return fail(FLL_ERR_INVALID_ARG, "b_teacher misaligned");
  }
  if (!ratio_head(p.head) && a->old_logprobs)
    return fail(FLL_ERR_INVALID_ARG, "old_logprobs is for the ratio heads");
  if (a->old_logprobs && !aligned(a->old_logprobs, 4))
    return fail(FLL_ERR_INVALID_ARG, "old_logprobs misaligned");
  if (p.head != FLL_HEAD_JSD && (a->X_teacher || a->W_teacher || a->b_teacher))
    return fail(FLL_ERR_INVALID_ARG, "teacher inputs are for the JSD head");
  if (p.head == FLL_HEAD_JSD && !p.teacher_has_bias && a->b_teacher)
    return fail(FLL_ERR_INVALID_ARG, "b_teacher given but teacher_has_bias is 0");
  if (a->labels && !aligned(a->labels, 8)) return fail(FLL_ERR_INVALID_ARG, "labels misaligned");
  if (a->weights && !aligned(a->weights, 4)) return fail(FLL_ERR_INVALID_ARG, "weights misaligned");
  if (a->per_row && !aligned(a->per_row, 4)) return fail(FLL_ERR_INVALID_ARG, "per_row misaligned");
  return FLL_OK;
}

// ---- kernel timing ----------------------------------------------------------

struct Timed {
  int kind;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<Timed> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with an event pair when timing is on.
struct Probe {
  int kind;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  Probe(int k, hipStream_t s, bool timed) : kind(k), st(s) {
    if (!timed || !g_prof_on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    a = pooled_event();
    b = pooled_event();
    if (a) (void)hipEventRecord(a, st);
  }
  ~Probe() {
    if (!a || !b) return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({kind, a, b});
  }
};

// ---- the allocation-free entry point's scratch --------------------------
// One array per device, in the library's device code; its address on a
// device comes from hipGetSymbolAddress, once per device (the array's name
// in host code is only a host-side handle, not a device address). Every
// fll_fwd_bwd_static call on a device shares it, so overlapping calls on one
// device race; the call writes every region it reads before reading it, so
// nothing needs clearing between calls.
static __device__ __align__(256) char scratch[FLL_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FLL_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FLL_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FLL_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLL_OK;
}

int hip_check(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(FLL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return FLL_OK;
}

// Enqueue one checked call: the per-chunk kernel sequence over the
// workspace args->workspace. timed: record the profiling events (when on).
int enqueue(const fll_plan_t *plan, const fll_args *args, hipStream_t s, bool timed) {
  int st = FLL_OK;
  // hipGetLastError reports the last failure of any HIP caller on this
  // thread; drop a stale one left by another library so only this call's
  // launches are checked below.
  (void)hipGetLastError();
  const fll_problem &p = plan->p;
  const fll_args &a = *args;
  char *ws = static_cast<char *>(a.workspace);
  float *S = reinterpret_cast<float *>(ws + plan->off_logits);
  float *rowval = a.per_row ? a.per_row : reinterpret_cast<float *>(ws + plan->off_rowval);
  float *partial = reinterpret_cast<float *>(ws + plan->off_dx_partial);
  float2 *stats = plan->stat_tiles ? reinterpret_cast<float2 *>(ws + plan->off_stats) : nullptr;
  auto *sc = reinterpret_cast<fll::DevScalars *>(ws + plan->off_scalars);
  const bool jsd = p.head == FLL_HEAD_JSD;
  float *T = jsd ? reinterpret_cast<float *>(ws + plan->off_teacher) : nullptr;
  float2 *stats_t = jsd && plan->stat_tiles
                        ? reinterpret_cast<float2 *>(ws + plan->off_teacher_stats)
                        : nullptr;
  const bool bf16 = p.dtype == FLL_BF16;
  const size_t esz = bf16 ? 2 : 4;
  // bf16 chunk logits: the label heads take the label's logit in fp32 from
  // the logits GEMM, through the per-row buffer the row kernel then fills
  float *label_logit = bf16 && p.logits_bf16 && label_head(p.head) && a.labels ? rowval : nullptr;
  const float inv_tau = 1.0f / p.temperature;

  if (p.BT == 0) {
    fll::launch_fill(a.loss, 1, 0.0f, s);
    if (p.compute_dW) fll::launch_fill(a.dW, p.V * p.H, 0.0f, s);
    if (p.compute_db) fll::launch_fill(a.db, p.V, 0.0f, s);
    return hip_check("empty-call fill");
  }

  {
    Probe pr(FLL_K_PREP, s, timed);
    fll::launch_prep(a.labels, p.BT, p.ignore_index, p.head, p.reduction, p.V, sc, s);
  }
  if ((st = hip_check("prep"))) return st;

  const int64_t C = plan->chunk_rows;
  for (int64_t c = 0; c < plan->n_chunks; ++c) {
    const int64_t r0 = c * C;
    const int64_t rows = std::min<int64_t>(C, p.BT - r0);
    const char *Xc = static_cast<const char *>(a.X) + size_t(r0) * p.H * esz;
    char *dXc = static_cast<char *>(a.dX) + size_t(r0) * p.H * esz;
    if (jsd) {
      // the teacher's own projection: T = (X_t W_t^T + b_t) / tau, with its
      // row statistics [FusedLinearKLDivLoss page, Summary]
      const char *Xtc = static_cast<const char *>(a.X_teacher) + size_t(r0) * p.H_teacher * esz;
      Probe pr(FLL_K_TEACHER, s, timed);
      if (bf16)
        fll::launch_logits_bf16(Xtc, p.H_teacher, a.W_teacher, p.H_teacher, a.b_teacher,
                                inv_tau, T, plan->s_pitch, p.logits_bf16, stats_t,
                                plan->stat_tiles, rows, p.V, p.H_teacher, nullptr, 0,
                                nullptr, s);
      else
        fll::launch_logits_f32(reinterpret_cast<const float *>(Xtc), p.H_teacher,
                               static_cast<const float *>(a.W_teacher), p.H_teacher,
                               static_cast<const float *>(a.b_teacher), inv_tau, T,
                               plan->s_pitch, rows, p.V, p.H_teacher, s);
    }
    if ((st = hip_check("teacher logits GEMM"))) return st;
    {
      Probe pr(FLL_K_LOGITS, s, timed);
      if (bf16)
        fll::launch_logits_bf16(Xc, p.H, a.W, p.H, a.b, inv_tau, S, plan->s_pitch,
                                p.logits_bf16, stats, plan->stat_tiles, rows, p.V, p.H,
                                a.labels, r0, label_logit, s);
      else
        fll::launch_logits_f32(reinterpret_cast<const float *>(Xc), p.H,
                               static_cast<const float *>(a.W), p.H,
                               static_cast<const float *>(a.b), inv_tau, S,
                               plan->s_pitch, rows, p.V, p.H, s);
    }
    if ((st = hip_check("logits GEMM"))) return st;
    {
      fll::RowArgs ra;
      ra.S = S;
      ra.s_pitch = plan->s_pitch;
      ra.rows = rows;
      ra.row0 = r0;
      ra.V = p.V;
      ra.head = p.head;
      ra.dz_bf16 = bf16 ? 1 : 0;
      ra.s_bf16 = p.logits_bf16;
      ra.labels = a.labels;
      ra.ignore_index = p.ignore_index;
      ra.target = a.target;
      ra.weights = a.weights;
      ra.inv_tau = inv_tau;
      ra.eps = p.eps;
      ra.sc = sc;
      ra.rowval = rowval;
      ra.stats = stats;
      ra.n_stat = plan->stat_tiles;
      ra.T = T;
      ra.stats_t = stats_t;
      ra.label_logit = label_logit;
      ra.old_logprobs = a.old_logprobs;
      ra.clip_low = p.clip_low;
      ra.clip_high = p.clip_high;
      Probe pr(FLL_K_ROW, s, timed);
      fll::launch_row(ra, s);
    }
    if ((st = hip_check("row kernel"))) return st;
    // dZ: bf16 packed at the start of each fp32 logits row (pitch
    // 2 * s_pitch elements), bf16 over bf16 logits (pitch s_pitch), or fp32
    // in place (pitch s_pitch).
    const int64_t ldz = bf16 && !p.logits_bf16 ? 2 * plan->s_pitch : plan->s_pitch;
    {
      Probe pr(FLL_K_DX, s, timed);
      if (bf16)
        fll::launch_dx_bf16(S, ldz, a.W, p.H, dXc, p.H, partial, rows, p.H, p.V,
                            plan->dx_splits, plan->dx_split_len, s);
      else
        fll::launch_dx_f32(S, ldz, static_cast<const float *>(a.W), p.H,
                           reinterpret_cast<float *>(dXc), p.H, partial, rows, p.H,
                           p.V, plan->dx_splits, plan->dx_split_len, s);
    }
    if ((st = hip_check("dX GEMM"))) return st;
    if (plan->dx_splits > 1) {
      Probe pr(FLL_K_DX_REDUCE, s, timed);
      fll::launch_dx_reduce(partial, plan->dx_splits, rows, p.H, dXc, p.H, bf16 ? 1 : 0, s);
      if ((st = hip_check("dX reduce"))) return st;
    }
    // bf16: db is formed inside the dW GEMM when both are asked for
    const bool db_in_dw = bf16 && p.compute_dW && p.compute_db;
    if (p.compute_dW && bf16) {
      // the chunk's X transposed (H x C, pitch a multiple of 64 tokens), so
      // that the dW GEMM reads both operands along its token dimension in
      // whole cache lines; the dX partials are reduced by now
      Probe pr(FLL_K_TRANSPOSE, s, timed);
      fll::launch_transpose_bf16(Xc, p.H, rows, p.H, partial, rup(C, 64), s);
      if ((st = hip_check("X transpose"))) return st;
    }
    if (p.compute_dW) {
      Probe pr(FLL_K_DW, s, timed);
      if (bf16)
        fll::launch_dw_bf16(S, ldz, partial, rup(C, 64), a.dW, db_in_dw ? a.db : nullptr, p.V,
                            p.H, rows, c > 0, s);
      else
        fll::launch_dw_f32(S, ldz, reinterpret_cast<const float *>(Xc), p.H, a.dW,
                           p.V, p.H, rows, c > 0, s);
      if ((st = hip_check("dW GEMM"))) return st;
    }
    if (p.compute_db && !db_in_dw) {
      Probe pr(FLL_K_DB, s, timed);
      fll::launch_colsum(S, bf16 ? 1 : 0, ldz, rows, p.V, partial, a.db, c > 0, s);
      if ((st = hip_check("db column sums"))) return st;
    }
  }
  {
    Probe pr(FLL_K_FINAL, s, timed);
    // the ratio heads' advantages are inside their per-row terms already
    const bool weighted = p.head == FLL_HEAD_SELECTIVE_LOGPROB || p.head == FLL_HEAD_CROSS_ENTROPY;
    fll::launch_finalize(rowval, weighted ? a.weights : nullptr, p.BT, sc, a.loss, s);
  }
  return hip_check("loss reduction");
}

}  // namespace

extern "C" {

int fll_version(void) { return FLL_VERSION; }

const char *fll_strerror(int status) {
  switch (status) {
    case FLL_OK: return "ok";
    case FLL_ERR_INVALID_ARG: return "invalid argument";
    case FLL_ERR_UNSUPPORTED: return "unsupported request";
    case FLL_ERR_WORKSPACE: return "workspace missing, too small or over budget";
    case FLL_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *fll_last_error(void) { return g_err; }

int fll_fwd_bwd(const fll_plan_t *plan, const fll_args *args, fll_stream stream) {
  g_err[0] = 0;
  int st = check_args(plan, args);
  if (st) return st;
  return enqueue(plan, args, reinterpret_cast<hipStream_t>(stream), true);
}

int fll_fwd_bwd_static(const fll_plan_t *plan, const fll_args *args, fll_stream stream) {
  g_err[0] = 0;
  if (!plan || !args) return fail(FLL_ERR_INVALID_ARG, "plan or args is NULL");
  if (args->workspace || args->workspace_bytes)
    return fail(FLL_ERR_INVALID_ARG,
                "fll_fwd_bwd_static uses the library's scratch: workspace must be NULL "
                "and workspace_bytes 0");
  if (plan->workspace_bytes > FLL_STATIC_SCRATCH_BYTES)
    return fail(FLL_ERR_WORKSPACE,
                "the plan needs %zu workspace bytes, more than the %zu of the static "
                "scratch: plan with max_workspace_bytes = FLL_STATIC_SCRATCH_BYTES",
                plan->workspace_bytes, size_t(FLL_STATIC_SCRATCH_BYTES));
  void *ptr = nullptr;
  int st = scratch_on_current_device(&ptr);
  if (st) return st;
  fll_args a = *args;
  a.workspace = ptr;
  a.workspace_bytes = FLL_STATIC_SCRATCH_BYTES;
  st = check_args(plan, &a);
  if (st) return st;
  return enqueue(plan, &a, reinterpret_cast<hipStream_t>(stream), false);
}

int fll_plan(const fll_problem *problem, size_t max_workspace_bytes, int64_t chunk_rows,
             fll_plan_t *plan) {
  g_err[0] = 0;
  return make_plan(problem, max_workspace_bytes, chunk_rows, plan);
}

int fll_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto &t : g_prof) {
    g_event_pool.push_back(t.start);
    g_event_pool.push_back(t.stop);
  }
  g_prof.clear();
  g_prof_on = enable != 0;
  return FLL_OK;
}

int fll_profile_read(fll_profile_t *out, int reset) {
  if (!out) return fail(FLL_ERR_INVALID_ARG, "out is NULL");
  memset(out, 0, sizeof(*out));
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto &t : g_prof) {
    if (hipEventSynchronize(t.stop) != hipSuccess)
      return fail(FLL_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess)
      return fail(FLL_ERR_HIP, "hipEventElapsedTime failed");
    out->launches[t.kind] += 1;
    out->total_ms[t.kind] += ms;
  }
  if (reset) {
    for (auto &t : g_prof) {
      g_event_pool.push_back(t.start);
      g_event_pool.push_back(t.stop);
    }
    g_prof.clear();
  }
  return FLL_OK;
}

}  // extern "C"
