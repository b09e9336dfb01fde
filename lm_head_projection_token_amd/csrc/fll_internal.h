// Internal launcher interface between the host dispatch (fll_api.cpp) and the
// HIP kernels. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fll {

// Scalars the device computes once per call, kept in the workspace.
struct DevScalars {
  long long n_valid;  // rows whose label is not ignore_index
  float g;            // reduction scale
  float pad;
};

// ---- bf16 MFMA GEMMs (gemm_bf16.hip) --------------------------------------

// S[m, n] = (sum_k X[m, k] W[n, k] + b[n]) * inv_tau for m < M, n < N.
// X: [M x K] row pitch ldx; W: [N x K] row pitch ldw; S row pitch lds
// elements, fp32, or bf16 (round to nearest even) when s_bf16.
// If stats != nullptr, also writes for every row m and 128-column block t
// the block's max and sum of exp(S - max) of the fp32 values:
// stats[m * n_stat + t] = (max, sum), n_stat = ceil(N / 128).
// label_logit (or null): for each row m with a label y = labels[label_row0
// + m] inside [0, N), the fp32 logit S[m, y] is written to
// label_logit[label_row0 + m] (bf16 chunk logits keep the label's logit
// exact for the label heads: selective, cross-entropy and ratio).
void launch_logits_bf16(const void *X, int64_t ldx, const void *W, int64_t ldw,
                        const void *b, float inv_tau, void *S, int64_t lds, int s_bf16,
                        float2 *stats, int64_t n_stat, int64_t M, int64_t N, int64_t K,
                        const int64_t *labels, int64_t label_row0, float *label_logit,
                        hipStream_t st);

// dX = dZ W. dZ: bf16 [M x K] row pitch ldz (elements); W: [K x N] pitch ldw.
// splits == 1: writes bf16 dX [M x N] (pitch ldo). splits > 1: writes fp32
// partials P[s][M x N] (pitch N) for s < splits, each over vocabulary columns
// [s * split_len, min(K, (s + 1) * split_len)).
void launch_dx_bf16(const void *dZ, int64_t ldz, const void *W, int64_t ldw,
                    void *dX, int64_t ldo, float *partial, int64_t M, int64_t N,
                    int64_t K, int64_t splits, int64_t split_len, hipStream_t st);

// dW[m, n] (+)= sum_k dZ[k, m] X[k, n]: dZ bf16 [K x M] pitch ldz, the
// chunk's X transposed, XT bf16 [N x K] pitch ldxt (16-byte aligned rows),
// dW fp32 [M x N] pitch N. accumulate = 0 stores.
// db (or null): db[m] (+)= sum_k dZ[k, m] for m < M, in the same launch.
void launch_dw_bf16(const void *dZ, int64_t ldz, const void *XT, int64_t ldxt,
                    float *dW, float *db, int64_t M, int64_t N, int64_t K,
                    int accumulate, hipStream_t st);

// XT[c, r] = X[r, c] for r < rows, c < cols (bf16): X pitch ldx, XT pitch
// ldt >= rows rounded up to 8; XT[c, r] = 0 for rows <= r < that multiple.
void launch_transpose_bf16(const void *X, int64_t ldx, int64_t rows, int64_t cols, void *XT,
                           int64_t ldt, hipStream_t st);

// ---- fp32 MFMA GEMMs (gemm_fp32.hip), same contracts in fp32 --------------

void launch_logits_f32(const float *X, int64_t ldx, const float *W, int64_t ldw,
                       const float *b, float inv_tau, float *S, int64_t lds,
                       int64_t M, int64_t N, int64_t K, hipStream_t st);
void launch_dx_f32(const float *dZ, int64_t ldz, const float *W, int64_t ldw,
                   float *dX, int64_t ldo, float *partial, int64_t M, int64_t N,
                   int64_t K, int64_t splits, int64_t split_len, hipStream_t st);
void launch_dw_f32(const float *dZ, int64_t ldz, const float *X, int64_t ldx,
                   float *dW, int64_t M, int64_t N, int64_t K, int accumulate,
                   hipStream_t st);

// ---- row and reduction kernels (row_kernels.hip) ---------------------------

// Count valid rows and form the reduction scale into *sc.
void launch_prep(const int64_t *labels, int64_t BT, int64_t ignore_index,
                 int head, int reduction, int64_t V, DevScalars *sc,
                 hipStream_t st);

// The fused row kernel over the rows [row0, row0 + rows) of one chunk. With
// stats it forms log-sum-exp from the logits GEMM's block statistics and
// streams the logits once; without, it takes a first pass for max / sum exp.
// S: the chunk's tempered logits, pitch s_pitch elements, fp32 or (s_bf16)
// bf16. On return the first V entries of each row hold dZ = dS / tau: over
// bf16 logits element for element; over fp32 logits bf16 packed at the start
// of the row (bf16 pitch 2 * s_pitch) when dz_bf16, else fp32 in place.
// rowval[r] receives the row's term: KL_r, log p(y_r), -log p(y_r), JS_r or
// the ratio heads' L_r (0 when ignored). T (JSD) has S's
// element type and pitch.
struct RowArgs {
  float *S;
  int64_t s_pitch;
  int s_bf16;     // S and T hold bf16 (then dz_bf16 is 1)
  int64_t rows;
  int64_t row0;   // global index of the chunk's first row
  int64_t V;
  int head;
  int dz_bf16;
  const int64_t *labels;  // global [BT] or null
  int64_t ignore_index;
  const float *target;    // global [BT x V] or null
  const float *weights;   // global [BT] or null
  float inv_tau;
  float eps;
  const DevScalars *sc;
  float *rowval;          // global [BT]
  const float2 *stats;    // per-(row, 128-column block) (max, sum exp) or null
  int64_t n_stat;         // blocks per row
  const float *T;         // JSD: the chunk's teacher logits (pitch s_pitch) or null
  const float2 *stats_t;  // JSD: the teacher's block statistics or null
  const float *label_logit;  // global [BT]: fp32 S[r, y_r] from the logits GEMM, or null
  const float *old_logprobs; // ratio heads: global [BT] old log-probs of the labels
  float clip_low, clip_high; // ratio heads: the ratio is clipped to [1 - low, 1 + high]
};
void launch_row(const RowArgs &a, hipStream_t st);

// db[v] (+)= sum over rows of dZ[r, v] for v < V: kDbSplits row ranges are
// summed into P [kDbSplits x V] fp32, then added in a fixed order.
constexpr int kDbSplits = 16;
void launch_colsum(const void *dZ, int dz_bf16, int64_t ldz, int64_t rows,
                   int64_t V, float *P, float *db, int accumulate, hipStream_t st);

// dX[m, n] = sum_s P[s][m, n] in order s = 0, 1, ...; dX in bf16 or fp32.
void launch_dx_reduce(const float *P, int64_t splits, int64_t M, int64_t N,
                      void *dX, int64_t ldo, int out_bf16, hipStream_t st);

// *loss = g * sum_r w_r rowval[r], summed in a fixed order in fp64.
void launch_finalize(const float *rowval, const float *weights, int64_t BT,
                     const DevScalars *sc, float *loss, hipStream_t st);

// Fill n floats with a value (no memset nodes, so graph capture is safe).
void launch_fill(float *p, int64_t n, float v, hipStream_t st);

}  // namespace fll
