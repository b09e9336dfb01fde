/*
 * fll.h -- fused lm_head loss with gradient-in-forward, for MI355X (gfx950).
 *
 * One call computes, for token rows X [BT x H] against a vocabulary head
 * W [V x H] (+ bias b [V]):
 *
 *   S      = (X W^T + b) / temperature           (logits, tempered)
 *   logP   = S - logsumexp_v(S)                  (row log-softmax over V)
 *   loss   = g * sum_r w_r * L_r                 (scalar, on the device)
 *   dX     = dZ W,  dW = dZ^T X,  db = sum_r dZ_r (dZ = d loss / d(X W^T + b))
 *
 * with one of six per-row heads:
 *
 *   FLL_HEAD_KL:                L_r = sum_v q_rv log(max(q_rv, eps)) - q_rv logP_rv
 *       KL(target || model) against an explicit target distribution q
 *       [FusedLinearKLDivLoss page, Summary and Details].
 *   FLL_HEAD_SELECTIVE_LOGPROB: L_r = logP_{r, y_r}, weighted by w_r
 *       the per-token selective log-prob of the GRPO family
 *       [frozen lm_head GRPO page, Summary].
 *   FLL_HEAD_CROSS_ENTROPY:     L_r = -logP_{r, y_r}, weighted by w_r
 *   FLL_HEAD_JSD:               L_r = 1/2 KL(Pt_r || M_r) + 1/2 KL(P_r || M_r),
 *       M = (Pt + P) / 2, the Jensen-Shannon divergence between the model and
 *       a teacher whose distribution Pt comes from its own projection
 *       Pt = softmax((X_t W_t^T + b_t) / temperature), which takes no gradient
 *       [FusedLinearKLDivLoss page, Summary: the fused JSD loss whose teacher
 *       side needs its own projection]
 *   FLL_HEAD_PPO_CLIP:          L_r = -min(rho_r A_r, clip(rho_r, 1 - clip_low,
 *                                          1 + clip_high) A_r),
 *       rho_r = exp(logP_{r, y_r} - old_r): the clipped surrogate of the GRPO
 *       family built on the selective log-prob [frozen lm_head GRPO page,
 *       Summary]; the published PPO objective, with DAPO's separate widths
 *   FLL_HEAD_CISPO:             L_r = -sg(clip(rho_r, 1 - clip_low, 1 + clip_high))
 *                                     A_r logP_{r, y_r},
 *       the clipped ratio as a weight with no gradient through it (CISPO,
 *       of the same family)
 *
 * The work runs in token chunks, and each chunk's gradient is formed inside
 * the same call (gradient-in-forward), so the BT x V logits are never
 * materialised: only one chunk of C x V logits lives in the caller's
 * workspace, and the bf16 dlogits are written in place over it
 * [FusedLinearKLDivLoss page, Summary and Details]. dW and db are formed
 * only when asked for, and skipping them skips their kernels entirely
 * [frozen lm_head GRPO page, Summary; LoRA normalization page, Key Changes].
 *
 * Conventions for every entry point:
 *  - Plain C types only. Device pointers point to memory on the current HIP
 *    device; host pointers are marked "host".
 *  - The caller owns every buffer (inputs, outputs, workspace). The library
 *    allocates no device memory and keeps no pointer after a call returns
 *    (fll_fwd_bwd_static takes its workspace from a fixed device array the
 *    library holds instead of the caller's).
 *  - All matrices are row-major and densely packed (row pitch = row length).
 *  - Status codes are fll_status values. Every argument is checked on the
 *    host before anything is enqueued, so an argument, support or workspace
 *    error leaves every output untouched. FLL_ERR_HIP (a launch that failed)
 *    can come after earlier kernels of the call were enqueued: the outputs
 *    are then undefined. fll_last_error() gives a thread-local message.
 */
#ifndef FLL_H
#define FLL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLL_VERSION 4

/* A hipStream_t, passed opaquely. NULL means the null (default) stream. */
typedef void *fll_stream;

typedef enum {
  FLL_OK = 0,
  FLL_ERR_INVALID_ARG = -1, /* a null/misaligned pointer, a bad size or flag */
  FLL_ERR_UNSUPPORTED = -2, /* a well-formed request the method refuses     */
  FLL_ERR_WORKSPACE = -3,   /* workspace missing, too small, or over budget */
  FLL_ERR_HIP = -4          /* a HIP launch or runtime call failed          */
} fll_status;

/* FLL_HEAD_CROSS_ENTROPY: L_r = -log p(y_r), optionally weighted by w_r --
 * the KL head against a one-hot target, i.e. the fused linear cross-entropy
 * loss whose chunk geometry the FusedLinearKLDivLoss page (Summary) reuses.
 * FLL_HEAD_PPO_CLIP and FLL_HEAD_CISPO (the ratio heads): the advantages A
 * are `weights` (NULL = 1) and the old log-probs `old_logprobs`; the loss is
 * g * sum_r L_r (A enters L_r, not as an outer weight). A tie of the PPO
 * minimum (rho inside the clip range) takes the unclipped branch, whose
 * gradient is -rho A (times d logP_y); the clipped branch has none.
 * GRPO's per-sequence mean and Dr. GRPO's constant normaliser are positive
 * per-token factors: fold them into A and use FLL_RED_SUM. */
typedef enum {
  FLL_HEAD_KL = 0,
  FLL_HEAD_SELECTIVE_LOGPROB = 1,
  FLL_HEAD_CROSS_ENTROPY = 2,
  FLL_HEAD_JSD = 3,
  FLL_HEAD_PPO_CLIP = 4,
  FLL_HEAD_CISPO = 5
} fll_head;

/* Reductions with the semantics of torch.nn.KLDivLoss
 * [FusedLinearKLDivLoss page, Details]. With n = the number of rows whose
 * label is not ignore_index (all rows when labels is NULL):
 *   BATCHMEAN: g = 1/n;  MEAN: g = 1/(n V) for KL and JSD, 1/n for the
 *   label heads (selective, cross-entropy, ratio: their tokens are the
 *   batch; the token mean of DAPO and BNPO);  SUM: g = 1;  n = 0 gives g = 0.
 * NONE is refused with FLL_ERR_UNSUPPORTED: gradient-in-forward needs a
 * scalar loss [FusedLinearKLDivLoss page, Details]. */
typedef enum {
  FLL_RED_BATCHMEAN = 0,
  FLL_RED_MEAN = 1,
  FLL_RED_SUM = 2,
  FLL_RED_NONE = 3
} fll_reduction;

/* Element type of X, W, b and dX. bf16 is the MFMA path; fp32 is exact
 * fp32 arithmetic (fp32 MFMA), meant for small problems. */
typedef enum { FLL_BF16 = 0, FLL_FP32 = 1 } fll_dtype;

/* The problem. Host struct, passed by pointer, read only during the call. */
typedef struct {
  int64_t BT;           /* token rows, >= 0 (0 is a valid empty call)        */
  int64_t H;            /* hidden size, >= 8 and a multiple of 8             */
  int64_t V;            /* vocabulary size, >= 1                             */
  int32_t dtype;        /* fll_dtype                                         */
  int32_t head;         /* fll_head                                          */
  int32_t has_bias;     /* 0/1: b is given                                   */
  int32_t compute_dW;   /* 0/1: form dW (fp32). 0 skips the dW GEMM          */
  int32_t compute_db;   /* 0/1: form db (fp32); needs has_bias               */
  int32_t reduction;    /* fll_reduction                                     */
  int64_t ignore_index; /* label value marking a row as ignored (e.g. -100)  */
  float temperature;    /* > 0, finite; divides the model logits (and, for
                           JSD, the teacher's logits)                         */
  float eps;            /* >= 0, finite; KL clamps q inside log(q) only; an
                           entry with q = 0 adds exactly 0 (eps = 0 too)      */
  int64_t H_teacher;    /* JSD: the teacher's hidden size, >= 8 and a multiple
                           of 8; every other head: 0                          */
  int32_t teacher_has_bias; /* JSD: 0/1, b_teacher is given; otherwise 0      */
  int32_t logits_bf16;  /* bf16 problems, 0/1: keep each chunk's logits (and
                           the JSD teacher's) in bf16, rounded to nearest even,
                           instead of fp32. Halves the chunk buffer and the
                           bytes its logits GEMM writes and its row kernel
                           reads; the per-row log-sum-exp is still formed from
                           the fp32 accumulators, so only each p_v and the
                           label's logit see the rounding. The dlogits then
                           overwrite the logits element for element. 0 keeps
                           the fp32 chunk temporaries the method describes
                           [FusedLinearKLDivLoss page, Details] and is the
                           default. fp32 problems: 0.                        */
  float clip_low;       /* ratio heads: the ratio is clipped to
                           [1 - clip_low, 1 + clip_high]; 0 <= clip_low <= 1  */
  float clip_high;      /* ratio heads: >= 0, +inf allowed (no upper clip).
                           Every other head: both 0.                          */
} fll_problem;

/* The plan: a value type (nothing to free). Its fields after `p` are the
 * library's own layout decisions; callers read workspace_bytes and may read
 * the rest, but must not edit them (fll_fwd_bwd re-derives and checks them). */
typedef struct {
  fll_problem p;
  int64_t chunk_rows;     /* C: token rows per chunk                        */
  int64_t n_chunks;       /* ceil(BT / C)                                   */
  int64_t s_pitch;        /* elements per row of the chunk's logits buffer
                             (fp32, or bf16 with logits_bf16)               */
  int64_t dx_splits;      /* dX split over the vocabulary: depends on V, H and
                             the chunk size, never on compute_dW/compute_db */
  int64_t dx_split_len;   /* vocabulary columns per dX split                */
  int64_t stat_tiles;     /* per-row statistics tiles (logits GEMM columns) */
  size_t off_logits;      /* workspace byte offsets                         */
  size_t off_rowval;
  size_t off_stats;
  size_t off_dx_partial;
  size_t off_scalars;
  size_t off_teacher;     /* JSD: teacher logits and statistics of a chunk  */
  size_t off_teacher_stats;
  size_t workspace_bytes; /* bytes the caller must provide                  */
} fll_plan_t;

/* Buffers of one call. Every pointer is a device pointer. */
typedef struct {
  const void *X;       /* [BT x H], dtype                                     */
  const void *W;       /* [V x H], dtype                                      */
  const void *b;       /* [V], dtype; NULL iff has_bias == 0                  */
  const int64_t *labels; /* [BT]. SELECTIVE, CROSS_ENTROPY, ratio heads:
                            required, values in [0, V) or ignore_index. KL,
                            JSD: optional row mask (a row is ignored iff its
                            label == ignore_index).                           */
  const float *target; /* KL: [BT x V] fp32 target probabilities, required.
                          Rows of ignored tokens are never read. Other heads:
                          NULL.                                               */
  const float *weights; /* SELECTIVE, CROSS_ENTROPY: [BT] fp32 per-token
                           weights (advantages); ratio heads: the advantages
                           A; NULL means all 1. KL, JSD: NULL.                */
  void *dX;            /* [BT x H], dtype: written (every row, ignored = 0)    */
  float *dW;           /* [V x H] fp32: written iff compute_dW, else untouched
                          and may be NULL                                     */
  float *db;           /* [V] fp32: written iff compute_db, else untouched    */
  float *loss;         /* [1] fp32: written                                   */
  float *per_row;      /* optional [BT] fp32: KL_r (KL), log p(y_r)
                          (SELECTIVE), -log p(y_r) (CROSS_ENTROPY), JS_r
                          (JSD) before weighting, or the ratio heads' L_r;
                          0 on ignored rows                                  */
  void *workspace;     /* >= plan.workspace_bytes, 256-byte aligned; contents
                          are scratch and need no initialisation              */
  size_t workspace_bytes;
  const void *X_teacher; /* JSD: [BT x H_teacher], dtype, 16-byte aligned; else NULL */
  const void *W_teacher; /* JSD: [V x H_teacher], dtype, 16-byte aligned; else NULL  */
  const void *b_teacher; /* JSD: [V], dtype, iff teacher_has_bias; else NULL          */
  const float *old_logprobs; /* ratio heads: [BT] fp32 log-probs of the labels
                                under the policy that sampled them (read on
                                non-ignored rows only); else NULL            */
} fll_args;

/* Plan a problem: choose the token-chunk size and the workspace layout.
 *
 * Host only; makes no HIP call, so it runs without a GPU. The chunk size C
 * keeps at least two chunks whenever BT exceeds one 256-row tile, so the
 * BT x V logits are never formed at once [FusedLinearKLDivLoss page,
 * Summary: chunked, the full BT x V logits never materialised], caps C at
 * 8192 rows, and shrinks it until the workspace fits the budget. C never
 * depends on compute_dW / compute_db, so dX is bit-identical with and
 * without them.
 *
 *   problem             host, read only.
 *   max_workspace_bytes budget for the workspace; 0 = 64 GiB (a share of
 *                       the 288 GB of one MI355X).
 *   chunk_rows          0 = choose; > 0 forces C (testing, tuning).
 *   plan                host, written on success.
 * Returns FLL_OK, FLL_ERR_INVALID_ARG, FLL_ERR_UNSUPPORTED (reduction NONE)
 * or FLL_ERR_WORKSPACE (no chunk size fits the budget). */
int fll_plan(const fll_problem *problem, size_t max_workspace_bytes,
             int64_t chunk_rows, fll_plan_t *plan);

/* Run the fused forward + backward on `stream`.
 *
 * Enqueues every kernel on `stream` and returns without synchronising; the
 * results are valid once the stream reaches them. dX, dW, db, loss and
 * per_row are outputs of this call: they are overwritten, never accumulated
 * across calls. The loss is formed as if the upstream gradient were 1; a
 * caller with another upstream scale multiplies the gradients by it. The
 * dW / db kernels are launched only when compute_dW / compute_db are set
 * [frozen lm_head GRPO page, Summary; LoRA normalization page, Key Changes].
 *
 * A non-ignored label outside [0, V) (a label head) is not a
 * memory error: that row's per_row value and the loss become NaN and its
 * dlogits are zero. Calls that share a workspace must be ordered on one
 * stream.
 *
 *   plan    host, from fll_plan, read only.
 *   args    host struct of device pointers, read only.
 * Returns FLL_OK, FLL_ERR_INVALID_ARG, FLL_ERR_UNSUPPORTED,
 * FLL_ERR_WORKSPACE, or FLL_ERR_HIP (launch failure; see fll_last_error). */
int fll_fwd_bwd(const fll_plan_t *plan, const fll_args *args, fll_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as fll_fwd_bwd, with the workspace taken from a fixed array that the
 * library keeps on each device it runs on (FLL_STATIC_SCRATCH_BYTES, held
 * from the first call on a device until the process ends) instead of the
 * caller's. It allocates nothing and records no profiling events.
 *
 *   plan    from fll_plan(problem, FLL_STATIC_SCRATCH_BYTES, ..., &plan), so
 *           the chunk size fits the array; a plan needing more workspace is
 *           refused with FLL_ERR_WORKSPACE.
 *   args    as for fll_fwd_bwd, but workspace must be NULL and
 *           workspace_bytes 0 (else FLL_ERR_INVALID_ARG).
 * Every call on one device shares that device's array: calls that overlap
 * on one device (other streams, other threads) race and must be ordered by
 * the caller. Nothing in the array needs clearing between calls. Returns the
 * codes of fll_fwd_bwd. */
#define FLL_STATIC_SCRATCH_BYTES ((size_t)512 << 20)
int fll_fwd_bwd_static(const fll_plan_t *plan, const fll_args *args, fll_stream stream);

/* Static text for a status code. */
const char *fll_strerror(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char *fll_last_error(void);

/* FLL_VERSION of the built library. */
int fll_version(void);

/* Kernel timing, for measurement. When enabled, every fll_fwd_bwd call
 * records a HIP event pair around each kernel launch on its stream. */
enum {
  FLL_K_PREP = 0,     /* valid-row count and reduction scale            */
  FLL_K_LOGITS = 1,   /* logits GEMM                                    */
  FLL_K_ROW = 2,      /* fused row kernel (softmax, loss, dlogits)      */
  FLL_K_DX = 3,       /* dX GEMM                                        */
  FLL_K_DX_REDUCE = 4,/* dX split reduction                             */
  FLL_K_DW = 5,       /* dW GEMM (bf16: with db when both are asked for)*/
  FLL_K_DB = 6,       /* db column sums (db without dW, or fp32)        */
  FLL_K_FINAL = 7,    /* loss reduction                                 */
  FLL_K_TEACHER = 8,  /* JSD: teacher logits GEMM                       */
  FLL_K_TRANSPOSE = 9,/* bf16 dW: the chunk's X transposed              */
  FLL_K_COUNT = 10
};

typedef struct {
  int64_t launches[FLL_K_COUNT]; /* launches timed since the last reset    */
  double total_ms[FLL_K_COUNT];  /* summed event-measured durations (ms)   */
} fll_profile_t;

/* Turn timing on (1) or off (0); turning it on clears what was recorded. */
int fll_profile_enable(int enable);

/* Synchronise the recorded events and report the totals (host struct).
 * reset = 1 clears them afterwards. */
int fll_profile_read(fll_profile_t *out, int reset);

#ifdef __cplusplus
}
#endif

#endif /* FLL_H */
