// bf16 MFMA GEMMs of the fused lm_head loss for gfx950 (CDNA4, wave64).
//
// The three products of one token chunk [frozen lm_head GRPO page, Summary:
// the forward logits and the grad_logits^T @ hidden weight gradient;
// FusedLinearKLDivLoss page, Details: fp32 weight-gradient accumulation]:
//
//   logits  S  = (X W^T + b) / tau     A = X    [C x H]   K-contiguous
//                                      B = W    [V x H]   K-contiguous
//   dX      dX = dZ W                  A = dZ   [C x V]   K-contiguous
//                                      B = W    (K = V)   N-contiguous
//   dW      dW (+)= dZ^T X             A = dZ^T (K = C)   M-contiguous
//                                      B = X    (K = C)   N-contiguous
//
// One kernel template serves all three. A workgroup of 256 threads (four
// wavefronts in a 2 x 2 grid) computes a 256 x 256 tile; each wavefront owns
// 128 x 128 of it as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 with fp32
// accumulators (256 AGPRs).
//
// Staging. Each K-step of 32 moves a 256 x 32 slice of each operand from
// global memory straight into LDS with buffer_load_dwordx4 ... lds (no
// registers, no LDS write instructions). Four LDS stages of 32 KB are in
// flight, so a slice is requested about two and a half K-steps before its
// MFMAs run. The buffer descriptors give zero fill for rows past the end of
// an operand; K-chunks past the end are pointed outside the descriptor's
// range and read as zero as well.
//   K-contiguous operands keep their memory layout in LDS: 256 rows of 64
//   bytes, 16-byte chunks XOR-swizzled by row, read with ds_read_b128.
//   MN-contiguous operands also keep their layout: 32 K-rows of 512 bytes,
//   chunks XOR-swizzled by K-row, read with ds_read_b64_tr_b16, whose
//   16-lane transpose hands each lane four consecutive K-values of its own
//   column; two such reads form one MFMA operand of eight K-values.
// MFMA fragments are double-buffered in registers: the reads for the next
// 16-deep half-step are issued between the MFMAs of the current one.
//
// Tile order. Workgroups are dispatched round-robin over the 8 XCDs. The
// logical tile sequence walks groups of G tile-rows (or tile-columns), the
// short side fastest inside a group; optionally each XCD first receives a
// contiguous run of that sequence. Which combination keeps the most operand
// slices in L2 (and shares MALL fills across XCDs) was measured per product
// on the head shapes (C = 4096, H = 4096, V = 128256):
//   logits: groups of 16 tile-rows in dispatch order (each XCD keeps two X
//           panels resident while all XCDs stream the same W panels);
//   dX:     groups of 4 tile-columns in dispatch order;
//   dW:     groups of 8 tile-rows, one contiguous run per XCD.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "fll_internal.h"

namespace fll {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

#ifndef FLL_GEMM_STAGES
#define FLL_GEMM_STAGES 4
#endif
constexpr int BM = 256, BN = 256, BK = 32, NSTAGE = FLL_GEMM_STAGES;
constexpr int kThreads = 256;
constexpr int kOperandBytes = 256 * BK * 2;     // 16 KB per operand per stage
constexpr int kStageBytes = 2 * kOperandBytes;  // 32 KB
constexpr int kLoadsPerStage = 8;               // per thread: 4 for A, 4 for B
// Loads still in flight when stage s is needed: the later full stages, plus
// the A half of the newest one (prologue: the later full stages only).
constexpr int kVmcntLoop = kLoadsPerStage * (NSTAGE - 3) + kLoadsPerStage / 2;
constexpr int kVmcntPrologue = kLoadsPerStage * (NSTAGE - 2);
constexpr unsigned kOOB = 0x80000000u;          // offset outside every descriptor
constexpr unsigned kMaxRecords = 0x7fffffffu;
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format

// Swizzles of the 16-byte chunk index. K-contiguous tiles (4 chunks per row):
// the 32 rows that one ds_read_b128 touches spread over all banks.
// MN-contiguous tiles (32 chunks per K-row): the four K-rows that a 16-lane
// group of ds_read_b64_tr_b16 touches land on distinct banks.
__device__ __forceinline__ int swz_k(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int swz_mn(int k) {
  return (0x6ca0 >> ((k & 3) * 4)) & 15;  // {0, 10, 12, 6}[k & 3]
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes <= 0 ? 0 : (bytes > int64_t(kMaxRecords) ? int64_t(kMaxRecords) : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                           kRsrcWord3);
}

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, LDS_AS void *dst,
                                           unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// ---- K-contiguous operand: element (row, k) at p[row * ld + k] -------------
struct OpK {
  const unsigned short *p;
  int64_t ld, row0, nrows;
  unsigned voff[4];  // byte offsets of this thread's 4 chunks from (row0, k0)
  int kc[4];         // their K offsets within the slice
  unsigned fa[2];    // fragment read byte offsets (half-step 0 and 1)

  __device__ __forceinline__ void init(const unsigned short *p_, int64_t ld_, int64_t row0_,
                                       int64_t nrows_, int wave, int lane, int wr) {
    p = p_;
    ld = ld_;
    row0 = row0_;
    nrows = nrows_;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (wave * 4 + i) * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz_k(r);
      voff[i] = unsigned((int64_t(r) * ld + 8 * c) * 2);
      kc[i] = 8 * c;
    }
    const int r = wr + (lane & 31);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * h + (lane >> 5);
      fa[h] = unsigned(r * 64 + 16 * (c ^ swz_k(r)));
    }
  }
  __device__ __forceinline__ void issue_one(LDS_AS char *stage, int wave, int i, int64_t k0,
                                            int64_t kend) const {
    const __amdgpu_buffer_rsrc_t r = rsrc(p + row0 * ld + k0, ((nrows - row0) * ld - k0) * 2);
    const unsigned v = (k0 + kc[i] < kend) ? voff[i] : kOOB;
    load_lds16(r, stage + (wave * 4 + i) * 1024, v);
  }
  __device__ __forceinline__ void issue(LDS_AS char *stage, int wave, int64_t k0,
                                        int64_t kend) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_one(stage, wave, i, k0, kend);
  }
  static constexpr int kReads = 4;  // LDS reads per half-step
  // Read number x (0..3) of a half-step: block x (rows wr + 32 x ...).
  __device__ __forceinline__ void read(bf16x8 (&f)[4], const LDS_AS char *stage, int x,
                                       int h) const {
    const LDS_AS char *b = stage + fa[h] + x * 2048;
    asm volatile("ds_read_b128 %0, %1" : "=v"(f[x]) : "v"(b));
  }
};

// ---- MN-contiguous operand: element (row, k) at p[k * ld + row] ------------
struct OpMN {
  const unsigned short *p;
  int64_t ld, col0;
  unsigned voff[4];  // byte offsets of this thread's 4 chunks from (k0, col0)
  unsigned fb[4];    // transpose-read byte offsets, block i (half-step 0, h 0)

  __device__ __forceinline__ void init(const unsigned short *p_, int64_t ld_, int64_t col0_,
                                       int wave, int lane, int wr) {
    p = p_;
    ld = ld_;
    col0 = col0_;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = (wave * 4 + i) * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swz_mn(kr);
      voff[i] = unsigned((int64_t(kr) * ld + 8 * c) * 2);
    }
    // 16-lane group G, lane q: K-row 8 (G >> 1) + (q >> 2), columns
    // wr + 32 i + 16 (G & 1) + 4 (q & 3) .. + 3.
    const int G = lane >> 4, q = lane & 15;
    const int k = 8 * (G >> 1) + (q >> 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = wr + 32 * i + 16 * (G & 1) + 4 * (q & 3);
      const int c = col >> 3, half = (col >> 2) & 1;
      fb[i] = unsigned(k * 512 + 16 * (c ^ swz_mn(k)) + 8 * half);
    }
  }
  __device__ __forceinline__ void issue_one(LDS_AS char *stage, int wave, int i, int64_t k0,
                                            int64_t kend) const {
    const __amdgpu_buffer_rsrc_t r = rsrc(p + k0 * ld + col0, ((kend - k0) * ld - col0) * 2);
    load_lds16(r, stage + (wave * 4 + i) * 1024, voff[i]);
  }
  __device__ __forceinline__ void issue(LDS_AS char *stage, int wave, int64_t k0,
                                        int64_t kend) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_one(stage, wave, i, k0, kend);
  }
  static constexpr int kReads = 8;  // LDS reads per half-step
  // Read number x (0..7) of a half-step: block x / 2, K-values 4 (x % 2) .. + 3
  // of each lane's eight (the two halves of the MFMA operand).
  __device__ __forceinline__ void read(bf16x8 (&f)[4], const LDS_AS char *stage, int x,
                                       int h) const {
    const int i = x >> 1;
    const LDS_AS char *b = stage + fb[i] + h * 16 * 512 + (x & 1) * 4 * 512;
    i16x4 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(b));
    auto w = __builtin_bit_cast(i16x8, f[i]);
    if (x & 1) {
      w = __builtin_shufflevector(w, __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1),
                                  0, 1, 2, 3, 8, 9, 10, 11);
    } else {
      w = __builtin_shufflevector(w, __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1),
                                  8, 9, 10, 11, 4, 5, 6, 7);
    }
    f[i] = __builtin_bit_cast(bf16x8, w);
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
  int group;          // tile-rows (or tile-columns) per group of the tile order
  int n_first;        // 1: groups of tile-columns, N fastest inside a group
  int xcd_remap;      // 1: give each XCD a contiguous run of the tile order
};

// Logits epilogue: S = (acc + b[n]) * inv_tau, fp32, plus the row statistics
// of each 128-column half-tile: max and sum of exp(S - max) over its columns
// below N, written as stats[m * n_stat + n / 128] (when stats is given).
struct EpiLogits {
  static constexpr bool kRowStats = true;
  static constexpr bool kReadModifyWrite = false;
  float *S;
  int64_t lds;
  const unsigned short *bias;
  float inv_tau;
  float2 *stats;
  int64_t n_stat;
  __device__ __forceinline__ float col_bias(int64_t n) const {
    return bias ? __uint_as_float(unsigned(bias[n]) << 16) : 0.0f;
  }
};

__device__ __forceinline__ unsigned short f2bf(float f) {
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// dX epilogue: bf16 store when unsplit, fp32 partial per split otherwise.
// Stores four consecutive columns n .. n + 3 of row m (n is a multiple of 4).
struct EpiDx {
  static constexpr bool kRowStats = false;
  static constexpr bool kReadModifyWrite = false;
  unsigned short *out;
  int64_t ldo;
  float *partial;
  int64_t M, N;
  __device__ __forceinline__ void store4(int64_t m, int64_t n, int64_t nmax, float4 v,
                                         int split) const {
    const float ve[4] = {v.x, v.y, v.z, v.w};
    if (partial) {
      float *p = partial + (int64_t(split) * M + m) * N + n;
      if (n + 4 <= nmax) {
        *reinterpret_cast<float4 *>(p) = v;
      } else {
        for (int e = 0; e < 4; ++e)
          if (n + e < nmax) p[e] = ve[e];
      }
    } else {
      unsigned short *p = out + m * ldo + n;
      if (n + 4 <= nmax) {
        uint2 pk;
        pk.x = unsigned(f2bf(v.x)) | (unsigned(f2bf(v.y)) << 16);
        pk.y = unsigned(f2bf(v.z)) | (unsigned(f2bf(v.w)) << 16);
        *reinterpret_cast<uint2 *>(p) = pk;
      } else {
        for (int e = 0; e < 4; ++e)
          if (n + e < nmax) p[e] = f2bf(ve[e]);
      }
    }
  }
};

// dW epilogue: fp32 store, or read-modify-write across token chunks (each
// tile owns its rows, so there are no atomics).
struct EpiDw {
  static constexpr bool kRowStats = false;
  static constexpr bool kReadModifyWrite = true;
  float *dW;
  int64_t ld;
  int accumulate;
  __device__ __forceinline__ float4 load4(int64_t m, int64_t n, int64_t nmax) const {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!accumulate) return v;
    const float *p = dW + m * ld + n;
    if (n + 4 <= nmax) return *reinterpret_cast<const float4 *>(p);
    if (n + 0 < nmax) v.x = p[0];
    if (n + 1 < nmax) v.y = p[1];
    if (n + 2 < nmax) v.z = p[2];
    return v;
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, int64_t nmax, float4 v,
                                         int) const {
    float *p = dW + m * ld + n;
    if (n + 4 <= nmax) {
      *reinterpret_cast<float4 *>(p) = v;
    } else {
      const float ve[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 4; ++e)
        if (n + e < nmax) p[e] = ve[e];
    }
  }
};

// The inner loop's MFMAs and LDS fragment reads are volatile inline assembly,
// so they issue in exactly the order written: each half-step interleaves the
// reads of the next half-step's fragments and a quarter of the next stage's
// loads with its 16 MFMAs. The compiler neither sees the reads' latency nor
// treats the asm as MFMAs, so the LDS waits are explicit and the accumulators
// rest a few cycles before the epilogue reads them.
__device__ __forceinline__ void mfma(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <bool A_K, bool B_K, class Epi>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmDesc d, Epi epi) {
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * kStageBytes];
  LDS_AS char *lds = (LDS_AS char *)smem;

  // ---- tile: optional XCD remap, then grouped order ----
  const int T = gridDim.x;
  const int b = blockIdx.x;
  int tl = b;
  if (d.xcd_remap) {
    const int xcd = b & 7, j = b >> 3;
    const int per = T >> 3, rem = T & 7;
    tl = xcd * per + (xcd < rem ? xcd : rem) + j;
  }
  const int tiles_mn = d.tiles_m * d.tiles_n;
  const int split = tl / tiles_mn;
  const int tmn = tl - split * tiles_mn;
  int tm, tn;
  if (d.n_first) {
    const int gsz = d.group * d.tiles_m;
    const int grp = tmn / gsz;
    const int first = grp * d.group;
    const int gn = min(d.group, d.tiles_n - first);
    const int local = tmn - grp * gsz;
    tn = first + local % gn;
    tm = local / gn;
  } else {
    const int gsz = d.group * d.tiles_n;
    const int grp = tmn / gsz;
    const int first = grp * d.group;
    const int gm = min(d.group, d.tiles_m - first);
    const int local = tmn - grp * gsz;
    tm = first + local % gm;
    tn = local / gm;
  }
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t kbeg = int64_t(split) * d.split_len;
  const int64_t kend = min(d.K, kbeg + d.split_len);

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  using OA = typename std::conditional<A_K, OpK, OpMN>::type;
  using OB = typename std::conditional<B_K, OpK, OpMN>::type;
  OA opa;
  OB opb;
  if constexpr (A_K) opa.init(d.A, d.lda, m0, d.M, wave, lane, wm * 128);
  else opa.init(d.A, d.lda, m0, wave, lane, wm * 128);
  if constexpr (B_K) opb.init(d.B, d.ldb, n0, d.N, wave, lane, wn * 128);
  else opb.init(d.B, d.ldb, n0, wave, lane, wn * 128);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][k][e] = 0.0f;

  const int nkt = kend > kbeg ? int((kend - kbeg + BK - 1) / BK) : 0;
  auto stageA = [&](int s) { return lds + (s % NSTAGE) * kStageBytes; };
  auto stageB = [&](int s) { return lds + (s % NSTAGE) * kStageBytes + kOperandBytes; };
  auto issue = [&](int s) {
    const int64_t k0 = kbeg + int64_t(s) * BK;
    opa.issue(stageA(s), wave, k0, kend);
    opb.issue(stageB(s), wave, k0, kend);
  };

  if (nkt > 0) {
    // prologue: three stages in flight, wait for the first
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s) issue(s);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kVmcntPrologue) : "memory");
    __builtin_amdgcn_s_barrier();
  }

  bf16x8 fa[2][4], fb[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[0][i] = fa[1][i] = bf16x8{};
    fb[0][i] = fb[1][i] = bf16x8{};
  }
  if (nkt > 0) {
#pragma unroll
    for (int x = 0; x < OA::kReads; ++x) opa.read(fa[0], stageA(0), x, 0);
#pragma unroll
    for (int x = 0; x < OB::kReads; ++x) opb.read(fb[0], stageB(0), x, 0);
  }

  // One half-step: 16 MFMAs on (ca, cb); between them the reads of (na, nb)
  // from the given stages and, after MFMAs 0, 4, 8, 12, one stage load each.
  auto half = [&](bf16x8 (&ca)[4], bf16x8 (&cb)[4], bf16x8 (&na)[4], bf16x8 (&nb)[4],
                  const LDS_AS char *sa, const LDS_AS char *sb, int h, auto &&load) {
    constexpr int ea = 16 / OA::kReads, eb = 16 / OB::kReads;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      mfma(acc[x >> 2][x & 3], cb[x & 3], ca[x >> 2]);
      if (x % ea == 0) opa.read(na, sa, x / ea, h);
      if (x % eb == eb / 2) opb.read(nb, sb, x / eb, h);
      if ((x & 3) == 0) load(x >> 2);
    }
  };

  for (int kt = 0; kt < nkt; ++kt) {
    const int64_t k_next = kbeg + int64_t(kt + NSTAGE - 1) * BK;
    // [B] half-step 0 of stage kt; read half-step 1 of stage kt; request the
    // A slice of stage kt + NSTAGE - 1 (past the end: zero-filled, unread).
    wait_lds();
    half(fa[0], fb[0], fa[1], fb[1], stageA(kt), stageB(kt), 1,
         [&](int q) { opa.issue_one(stageA(kt + NSTAGE - 1), wave, q, k_next, kend); });
    // [C] stage kt + 1 complete in LDS for every wave: of the loads issued so
    // far only the later stages (8 per thread each) and the A half of stage
    // kt + NSTAGE - 1 (4) may still be in flight.
    wait_lds();
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kVmcntLoop) : "memory");
    __builtin_amdgcn_s_barrier();
    // [D] half-step 1 of stage kt; read half-step 0 of stage kt + 1; request
    // the B slice of stage kt + NSTAGE - 1.
    half(fa[1], fb[1], fa[0], fb[0], stageA(kt + 1), stageB(kt + 1), 0,
         [&](int q) { opb.issue_one(stageB(kt + NSTAGE - 1), wave, q, k_next, kend); });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // The MFMAs take the B fragment as their first operand, so each 32 x 32
  // accumulator block holds the transposed product: lane l owns output row
  // m = l % 32 of the block, and register r holds column
  // 8 (r / 4) + 4 (l / 32) + r % 4. A lane therefore owns, for each of its
  // four rows, 64 of the wave's 128 columns in runs of four (16-byte
  // stores), and lane l ^ 32 owns the other 64.
  const int lrow = lane & 31;
  const int lcol = 4 * (lane >> 5);
  if constexpr (Epi::kRowStats) {
    const int64_t nh = n0 + wn * 128;  // first column of this 128-column half-tile
    float bias[4][4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t n = nh + k * 32 + 8 * q + lcol + e;
          bias[k][q][e] = n < d.N ? epi.col_bias(n) : 0.0f;
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + i * 32 + lrow;
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = nh + k * 32 + 8 * q + lcol;
          float4 v;
          v.x = (acc[i][k][4 * q + 0] + bias[k][q][0]) * epi.inv_tau;
          v.y = (acc[i][k][4 * q + 1] + bias[k][q][1]) * epi.inv_tau;
          v.z = (acc[i][k][4 * q + 2] + bias[k][q][2]) * epi.inv_tau;
          v.w = (acc[i][k][4 * q + 3] + bias[k][q][3]) * epi.inv_tau;
          acc[i][k][4 * q + 0] = v.x;
          acc[i][k][4 * q + 1] = v.y;
          acc[i][k][4 * q + 2] = v.z;
          acc[i][k][4 * q + 3] = v.w;
          float *dst = epi.S + m * epi.lds + n;
          if (n + 4 <= d.N) {
            if (m < d.M) *reinterpret_cast<float4 *>(dst) = v;
            mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
          } else {
            const float ve[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < d.N) {
                if (m < d.M) dst[e] = ve[e];
                mx = fmaxf(mx, ve[e]);
              }
          }
        }
      }
      if (epi.stats) {
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        float se = 0.0f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (nh + k * 32 + 8 * q + lcol + e < d.N) se += __expf(acc[i][k][4 * q + e] - mx);
        }
        se += __shfl_xor(se, 32, 64);
        if (lane < 32 && m < d.M && nh < d.N)
          epi.stats[m * epi.n_stat + (nh >> 7)] = make_float2(mx, se);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + i * 32 + lrow;
      if (m >= d.M) continue;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (Epi::kReadModifyWrite) {
          // old values of the block's 16 columns first, all loads in flight
          float4 old[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + wn * 128 + k * 32 + 8 * q + lcol;
            old[q] = epi.load4(m, n, d.N);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + wn * 128 + k * 32 + 8 * q + lcol;
            const float4 v = make_float4(old[q].x + acc[i][k][4 * q + 0],
                                         old[q].y + acc[i][k][4 * q + 1],
                                         old[q].z + acc[i][k][4 * q + 2],
                                         old[q].w + acc[i][k][4 * q + 3]);
            epi.store4(m, n, d.N, v, split);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + wn * 128 + k * 32 + 8 * q + lcol;
            const float4 v = make_float4(acc[i][k][4 * q + 0], acc[i][k][4 * q + 1],
                                         acc[i][k][4 * q + 2], acc[i][k][4 * q + 3]);
            epi.store4(m, n, d.N, v, split);
          }
        }
      }
    }
  }
}

inline int cdiv(int64_t a, int64_t b) { return int((a + b - 1) / b); }

template <bool A_K, bool B_K, class Epi>
void launch(const GemmDesc &d0, const Epi &epi, hipStream_t st) {
  GemmDesc d = d0;
  d.tiles_m = cdiv(d.M, BM);
  d.tiles_n = cdiv(d.N, BN);
  const int64_t blocks = int64_t(d.tiles_m) * d.tiles_n * d.splits;
  if (blocks <= 0) return;
  hipLaunchKernelGGL((gemm_kernel<A_K, B_K, Epi>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                     st, d, epi);
}

}  // namespace

void launch_logits_bf16(const void *X, int64_t ldx, const void *W, int64_t ldw,
                        const void *b, float inv_tau, float *S, int64_t lds, float2 *stats,
                        int64_t n_stat, int64_t M, int64_t N, int64_t K, hipStream_t st) {
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
  d.group = 16;       // measured best for the head shapes: see the tile-order note
  d.n_first = 0;
  d.xcd_remap = 0;
  EpiLogits e{S, lds, static_cast<const unsigned short *>(b), inv_tau, stats, n_stat};
  launch<true, true>(d, e, st);
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
  d.group = 4;
  d.n_first = 1;
  d.xcd_remap = 0;
  EpiDx e{static_cast<unsigned short *>(dX), ldo, splits > 1 ? partial : nullptr, M, N};
  launch<true, false>(d, e, st);
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
  d.group = 8;
  d.n_first = 0;
  d.xcd_remap = 1;
  EpiDw e{dW, N, accumulate};
  launch<false, false>(d, e, st);
}

}  // namespace fll
