// fp32 GEMMs of the fused lm_head loss for gfx950, on the fp32 MFMA
// (v_mfma_f32_16x16x4_f32: true fp32 products, fp32 accumulation; gfx950 has
// no reduced-precision xf32 variant). Meant for small fp32 problems where
// the loss must match to about 1e-5 relative, so the kernel is a plain
// LDS-tiled one: a 64 x 64 tile per workgroup of four wavefronts, each
// owning 32 x 32 as 2 x 2 blocks of 16 x 16, K staged 16 at a time.
// Operand roles and epilogues are those of the bf16 kernels.
#include <hip/hip_runtime.h>

#include "fll_internal.h"

namespace fll {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 64, TN = 64, TK = 16;

// K-contiguous operand: element (row, k) at p[row * ld + k].
struct F32K {
  __device__ static float get(const float *p, int64_t ld, int64_t row, int64_t k) {
    return p[row * ld + k];
  }
  // thread t loads k = t % 16, rows t / 16 + 16 i
  __device__ static void coords(int t, int i, int &r, int &k) {
    k = t & 15;
    r = (t >> 4) + 16 * i;
  }
};
// Row-contiguous operand: element (row, k) at p[k * ld + row].
struct F32MN {
  __device__ static float get(const float *p, int64_t ld, int64_t row, int64_t k) {
    return p[k * ld + row];
  }
  // thread t loads row t % 64, k = t / 64 + 4 i
  __device__ static void coords(int t, int i, int &r, int &k) {
    r = t & 63;
    k = (t >> 6) + 4 * i;
  }
};

struct EpiLogits32 {
  float *S;
  int64_t lds;
  const float *bias;
  float inv_tau;
  __device__ void put(int64_t m, int64_t n, float v, int) const {
    S[m * lds + n] = (v + (bias ? bias[n] : 0.0f)) * inv_tau;
  }
};
struct EpiDx32 {
  float *out;
  int64_t ldo;
  float *partial;
  int64_t M, N;
  __device__ void put(int64_t m, int64_t n, float v, int split) const {
    if (partial)
      partial[(int64_t(split) * M + m) * N + n] = v;
    else
      out[m * ldo + n] = v;
  }
};
struct EpiDw32 {
  float *dW;
  int64_t ld;
  int accumulate;
  __device__ void put(int64_t m, int64_t n, float v, int) const {
    float *p = dW + m * ld + n;
    *p = accumulate ? *p + v : v;
  }
};

template <class SA, class SB, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *A, int64_t lda,
                                                       const float *B, int64_t ldb,
                                                       int64_t M, int64_t N, int64_t K,
                                                       int64_t split_len, int tiles_m,
                                                       Epi epi) {
  __shared__ float la[TM][TK + 1];
  __shared__ float lb[TN][TK + 1];
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int split = blockIdx.y;
  const int64_t m0 = int64_t(tm) * TM, n0 = int64_t(tn) * TN;
  const int64_t kbeg = int64_t(split) * split_len;
  const int64_t kend = min(K, kbeg + split_len);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kbeg; k0 < kend; k0 += TK) {
    for (int i = 0; i < 4; ++i) {
      int r, k;
      SA::coords(t, i, r, k);
      const int64_t gm = m0 + r, gk = k0 + k;
      la[r][k] = (gm < M && gk < kend) ? SA::get(A, lda, gm, gk) : 0.0f;
      SB::coords(t, i, r, k);
      const int64_t gn = n0 + r, gk2 = k0 + k;
      lb[r][k] = (gn < N && gk2 < kend) ? SB::get(B, ldb, gn, gk2) : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < TK; kk += 4) {
      for (int i = 0; i < 2; ++i) {
        const float a = la[wm * 32 + i * 16 + (lane & 15)][kk + (lane >> 4)];
        for (int j = 0; j < 2; ++j) {
          const float b = lb[wn * 32 + j * 16 + (lane & 15)][kk + (lane >> 4)];
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  // 16 x 16 block layout: lane l holds column l % 16, rows 4 (l / 16) + r.
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j)
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
        const int64_t n = n0 + wn * 32 + j * 16 + (lane & 15);
        if (m < M && n < N) epi.put(m, n, acc[i][j][r], split);
      }
}

template <class SA, class SB, class Epi>
void launch32(const float *A, int64_t lda, const float *B, int64_t ldb, int64_t M,
              int64_t N, int64_t K, int64_t splits, int64_t split_len, const Epi &e,
              hipStream_t st) {
  const int tiles_m = int((M + TM - 1) / TM), tiles_n = int((N + TN - 1) / TN);
  if (tiles_m <= 0 || tiles_n <= 0 || splits <= 0) return;
  hipLaunchKernelGGL((gemm_f32_kernel<SA, SB, Epi>), dim3(tiles_m * tiles_n, unsigned(splits)),
                     dim3(256), 0, st, A, lda, B, ldb, M, N, K, split_len, tiles_m, e);
}

}  // namespace

void launch_logits_f32(const float *X, int64_t ldx, const float *W, int64_t ldw,
                       const float *b, float inv_tau, float *S, int64_t lds, int64_t M,
                       int64_t N, int64_t K, hipStream_t st) {
  launch32<F32K, F32K>(X, ldx, W, ldw, M, N, K, 1, K, EpiLogits32{S, lds, b, inv_tau}, st);
}

void launch_dx_f32(const float *dZ, int64_t ldz, const float *W, int64_t ldw, float *dX,
                   int64_t ldo, float *partial, int64_t M, int64_t N, int64_t K,
                   int64_t splits, int64_t split_len, hipStream_t st) {
  const int64_t sl = splits > 1 ? split_len : K;
  launch32<F32K, F32MN>(dZ, ldz, W, ldw, M, N, K, splits, sl,
                        EpiDx32{dX, ldo, splits > 1 ? partial : nullptr, M, N}, st);
}

void launch_dw_f32(const float *dZ, int64_t ldz, const float *X, int64_t ldx, float *dW,
                   int64_t M, int64_t N, int64_t K, int accumulate, hipStream_t st) {
  launch32<F32MN, F32MN>(dZ, ldz, X, ldx, M, N, K, 1, K, EpiDw32{dW, N, accumulate}, st);
}

}  // namespace fll
