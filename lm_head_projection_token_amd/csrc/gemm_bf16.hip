// bf16 MFMA GEMMs of the fused lm_head loss for gfx950 (CDNA4, wave64).
//
// The three products of one token chunk [frozen lm_head GRPO page, Summary:
// the forward logits and the grad_logits^T @ hidden weight gradient;
// FusedLinearKLDivLoss page, Details: fp32 weight-gradient accumulation]:
//
//   logits  S  = (X W^T + b) / tau     A = X   [C x H]  K-contiguous
//                                      B = W   [V x H]  K-contiguous
//   dX      dX = dZ W                  A = dZ  [C x V]  K-contiguous
//                                      B = W   (K = V)  N-contiguous
//   dW      dW (+)= dZ^T X             A = dZ^T (K = C) M-contiguous
//                                      B = X   (K = C)  N-contiguous
//
// One kernel template serves all three. A workgroup of 256 threads (four
// wavefronts in a 2 x 2 grid) computes a 256 x 256 tile; each wavefront owns
// 128 x 128 of it as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 with fp32
// accumulators. Both operands are staged through LDS in a K-contiguous
// layout, 64 K-values (8 chunks of 16 bytes) per row, with the chunk index
// XOR-swizzled by the row so that the 16-byte fragment reads and the staging
// writes are free of bank conflicts. Operands that are not K-contiguous in
// memory are loaded as 8 x 8 blocks of 16-byte rows and transposed in
// registers before the LDS write. Two LDS stages (128 KB of the 160 KB per
// CU) let the global loads of the next K-step overlap the MFMAs of this one,
// with one barrier per K-step.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order is
// remapped so that each XCD receives a contiguous run of tiles, and the run
// walks the tile grid along the dimension whose operand panel it can share in
// that XCD's L2.
#include <hip/hip_runtime.h>

#include "fll_internal.h"

namespace fll {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kChunks = BK / 8;           // 16-byte chunks per LDS row
constexpr int kTileChunks = 256 * kChunks;  // per operand per stage

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_idx(int r, int c) { return r * kChunks + (c ^ swz(r)); }

// Zero the bf16 lanes of a 16-byte chunk at element positions >= keep.
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int keep) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int e0 = 2 * d, e1 = 2 * d + 1;
    unsigned int w = v[d];
    if (e0 >= keep) w &= 0xffff0000u;
    if (e1 >= keep) w &= 0x0000ffffu;
    v[d] = w;
  }
  return v;
}

// Operand rows of the tile come from memory with K contiguous: element
// (row, k) at p[row * ld + k]. Thread t moves chunk t % 8 of rows t / 8 + 32 i.
struct StageK {
  __device__ __forceinline__ static void load(u32x4 (&reg)[8], const unsigned short *p,
                                              int64_t ld, int64_t row0, int64_t nrows,
                                              int64_t k0, int64_t kend, int t) {
    const int c = t & 7;
    const int64_t k = k0 + c * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t row = row0 + (t >> 3) + 32 * i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < nrows && k < kend) {
        v = *reinterpret_cast<const u32x4 *>(p + row * ld + k);
        if (k + 8 > kend) v = keep_first(v, int(kend - k));
      }
      reg[i] = v;
    }
  }
  __device__ __forceinline__ static void store(u32x4 *lds, const u32x4 (&reg)[8], int t) {
    const int c = t & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) lds[lds_idx((t >> 3) + 32 * i, c)] = reg[i];
  }
};

// Operand rows of the tile are contiguous in memory, K is the slow index:
// element (row, k) at p[k * ld + row]. Thread t loads an 8 x 8 block (8
// K-values of 8 consecutive rows) and transposes it in registers.
// A partial 8-row chunk at the end of the rows is read whole: callers
// guarantee the row pitch covers it, and rows >= nrows only feed output
// rows or columns that are never stored.
struct StageMN {
  __device__ __forceinline__ static void load(u32x4 (&reg)[8], const unsigned short *p,
                                              int64_t ld, int64_t row0, int64_t nrows,
                                              int64_t k0, int64_t kend, int t) {
    const int64_t row = row0 + (t & 31) * 8;
    const int64_t kb = k0 + (t >> 5) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = kb + j;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < nrows && k < kend) v = *reinterpret_cast<const u32x4 *>(p + k * ld + row);
      reg[j] = v;
    }
  }
  __device__ __forceinline__ static void store(u32x4 *lds, const u32x4 (&in)[8], int t) {
    const int rb = (t & 31) * 8;
    const int c = t >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = i >> 1;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned int x = in[2 * e][d], y = in[2 * e + 1][d];
        o[e] = (i & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      lds[lds_idx(rb + i, c)] = o;
    }
  }
};

struct GemmDesc {
  const unsigned short *A;
  int64_t lda;
  const unsigned short *B;
  int64_t ldb;
  int64_t M, N, K;
  int64_t split_len;  // K per split
  int tiles_m, tiles_n, splits;
  int m_fastest;      // tile order: 1 = walk M first (share B), 0 = walk N first
};

// Logits epilogue: S = (acc + b[n]) * inv_tau, fp32.
struct EpiLogits {
  float *S;
  int64_t lds;
  const unsigned short *bias;
  float inv_tau;
  __device__ __forceinline__ float col_bias(int64_t n) const {
    return bias ? __uint_as_float(unsigned(bias[n]) << 16) : 0.0f;
  }
  __device__ __forceinline__ void put(int64_t m, int64_t n, float v, float bn, int) const {
    S[m * lds + n] = (v + bn) * inv_tau;
  }
};

__device__ __forceinline__ unsigned short f2bf(float f) {
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// dX epilogue: bf16 store when unsplit, fp32 partial per split otherwise.
struct EpiDx {
  unsigned short *out;
  int64_t ldo;
  float *partial;
  int64_t M, N;
  __device__ __forceinline__ float col_bias(int64_t) const { return 0.0f; }
  __device__ __forceinline__ void put(int64_t m, int64_t n, float v, float, int split) const {
    if (partial)
      partial[(int64_t(split) * M + m) * N + n] = v;
    else
      out[m * ldo + n] = f2bf(v);
  }
};

// dW epilogue: fp32 store or read-modify-write (tiles own disjoint rows).
struct EpiDw {
  float *dW;
  int64_t ld;
  int accumulate;
  __device__ __forceinline__ float col_bias(int64_t) const { return 0.0f; }
  __device__ __forceinline__ void put(int64_t m, int64_t n, float v, float, int) const {
    float *p = dW + m * ld + n;
    *p = accumulate ? *p + v : v;
  }
};

template <class SA, class SB, class Epi>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmDesc d, Epi epi) {
  __shared__ u32x4 lds[2][2][kTileChunks];  // [stage][A, B]: 128 KB

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a
  // contiguous run of the logical tile sequence.
  const int T = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b & 7, j = b >> 3;
  const int per = T >> 3, rem = T & 7;
  const int tl = xcd * per + (xcd < rem ? xcd : rem) + j;
  const int tiles_mn = d.tiles_m * d.tiles_n;
  const int split = tl / tiles_mn;
  const int tmn = tl - split * tiles_mn;
  int tm, tn;
  if (d.m_fastest) {
    tm = tmn % d.tiles_m;
    tn = tmn / d.tiles_m;
  } else {
    tn = tmn % d.tiles_n;
    tm = tmn / d.tiles_n;
  }
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t kbeg = int64_t(split) * d.split_len;
  const int64_t kend = min(d.K, kbeg + d.split_len);

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][k][e] = 0.0f;

  const int nkt = kend > kbeg ? int((kend - kbeg + BK - 1) / BK) : 0;
  u32x4 ra[8], rb[8];
  if (nkt > 0) {
    SA::load(ra, d.A, d.lda, m0, d.M, kbeg, kend, t);
    SB::load(rb, d.B, d.ldb, n0, d.N, kbeg, kend, t);
    SA::store(lds[0][0], ra, t);
    SB::store(lds[0][1], rb, t);
  }
  __syncthreads();

  const int frow = lane & 31;   // fragment row within a 32-block
  const int fhalf = lane >> 5;  // which 8 of the 16 K-values
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
      const int64_t k0 = kbeg + int64_t(kt + 1) * BK;
      SA::load(ra, d.A, d.lda, m0, d.M, k0, kend, t);
      SB::load(rb, d.B, d.ldb, n0, d.N, k0, kend, t);
    }
    const u32x4 *la = lds[cur][0];
    const u32x4 *lb = lds[cur][1];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks * 2 + fhalf;
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 x = la[lds_idx(wm * 128 + i * 32 + frow, c)];
        af[i] = __builtin_bit_cast(bf16x8, x);
        u32x4 y = lb[lds_idx(wn * 128 + i * 32 + frow, c)];
        bf[i] = __builtin_bit_cast(bf16x8, y);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[i][k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[k], acc[i][k], 0, 0, 0);
    }
    if (more) {
      SA::store(lds[cur ^ 1][0], ra, t);
      SB::store(lds[cur ^ 1][1], rb, t);
    }
    __syncthreads();
  }

  // Accumulator layout of the 32 x 32 block: lane l holds column l % 32;
  // register r holds row 8 (r / 4) + 4 (l / 32) + r % 4.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t n = n0 + wn * 128 + k * 32 + (lane & 31);
    if (n >= d.N) continue;
    const float bn = epi.col_bias(n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + fhalf * 4 + (r & 3);
        if (m < d.M) epi.put(m, n, acc[i][k][r], bn, split);
      }
    }
  }
}

inline int cdiv(int64_t a, int64_t b) { return int((a + b - 1) / b); }

template <class SA, class SB, class Epi>
void launch(const GemmDesc &d0, const Epi &epi, hipStream_t st) {
  GemmDesc d = d0;
  d.tiles_m = cdiv(d.M, BM);
  d.tiles_n = cdiv(d.N, BN);
  const int64_t blocks = int64_t(d.tiles_m) * d.tiles_n * d.splits;
  if (blocks <= 0) return;
  hipLaunchKernelGGL((gemm_kernel<SA, SB, Epi>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                     st, d, epi);
}

}  // namespace

void launch_logits_bf16(const void *X, int64_t ldx, const void *W, int64_t ldw,
                        const void *b, float inv_tau, float *S, int64_t lds, int64_t M,
                        int64_t N, int64_t K, hipStream_t st) {
  GemmDesc d{};
  d.A = static_cast<const unsigned short *>(X);
  d.lda = ldx;
  d.B = static_cast<const unsigned short *>(W);
  d.ldb = ldw;
  d.M = M;
  d.N = N;
  d.K = K;
  d.split_len = K;
  d.splits = 1;
  d.m_fastest = 1;  // tiles sharing a W panel run together
  EpiLogits e{S, lds, static_cast<const unsigned short *>(b), inv_tau};
  launch<StageK, StageK>(d, e, st);
}

void launch_dx_bf16(const void *dZ, int64_t ldz, const void *W, int64_t ldw, void *dX,
                    int64_t ldo, float *partial, int64_t M, int64_t N, int64_t K,
                    int64_t splits, int64_t split_len, hipStream_t st) {
  GemmDesc d{};
  d.A = static_cast<const unsigned short *>(dZ);
  d.lda = ldz;
  d.B = static_cast<const unsigned short *>(W);
  d.ldb = ldw;
  d.M = M;
  d.N = N;
  d.K = K;
  d.split_len = splits > 1 ? split_len : K;
  d.splits = int(splits);
  d.m_fastest = 1;  // tiles sharing a W panel run together
  EpiDx e{static_cast<unsigned short *>(dX), ldo, splits > 1 ? partial : nullptr, M, N};
  launch<StageK, StageMN>(d, e, st);
}

void launch_dw_bf16(const void *dZ, int64_t ldz, const void *X, int64_t ldx, float *dW,
                    int64_t M, int64_t N, int64_t K, int accumulate, hipStream_t st) {
  GemmDesc d{};
  d.A = static_cast<const unsigned short *>(dZ);
  d.lda = ldz;
  d.B = static_cast<const unsigned short *>(X);
  d.ldb = ldx;
  d.M = M;
  d.N = N;
  d.K = K;
  d.split_len = K;
  d.splits = 1;
  d.m_fastest = 0;  // tiles sharing a dZ^T panel run together
  EpiDw e{dW, N, accumulate};
  launch<StageMN, StageMN>(d, e, st);
}

}  // namespace fll
