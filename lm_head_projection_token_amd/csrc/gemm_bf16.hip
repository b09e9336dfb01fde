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
//                                      B = X^T  (K = C)   K-contiguous (the chunk's
//                                                         X transposed once)
//
// One kernel template serves all three. A workgroup of 256 threads (four
// wavefronts in a 2 x 2 grid) computes a 256 x 256 tile; each wavefront owns
// 128 x 128 of it as 8 x 8 blocks of v_mfma_f32_16x16x32_bf16 with fp32
// accumulators (256 AGPRs). This shape, rather than 32 x 32 x 16 blocks,
// because with random operands the chip's power limit sets the clock: an
// MFMA-only loop held 2.07 GHz with 16 x 16 x 32 against 1.72-1.77 GHz with
// 32 x 32 x 16 at the same issue rate (2.38 GHz for both on constant data).
//
// Staging. Each K-step of 32 consumes a 256 x 32 slice of each operand,
// moved from global memory straight into LDS with buffer_load_dwordx4 ...
// lds (no registers, no LDS write instructions). Four 16 KB slots per
// operand (128 KB of LDS) hold four K-slices. The buffer descriptors give
// zero fill for rows past the end of an operand; K-chunks past the end are
// pointed outside the descriptor's range and read as zero as well.
//   K-contiguous operands are loaded a pair of slices at a time: one load
//   instruction covers 8 rows x 128 contiguous bytes (two slices of the same
//   8 rows, whole cache lines), so the texture path handles half the rows
//   per instruction that single slices (16 rows x 64 bytes, half lines)
//   would need: measured 10 % off the logits GEMM and 4-5 % off dX. In LDS
//   the slices of a pair sit 512 bytes apart inside 2 KB blocks of 8 rows,
//   16-byte chunks XOR-swizzled by row, read with ds_read_b128. A pair is
//   loaded during the odd K-step that frees its two slots, about one and a
//   half K-steps before its first slice is read.
//   MN-contiguous operands (B of dX, A of dW) load one slice per K-step,
//   four steps ahead (about two and a half K-steps before it is read): a
//   shorter lead cost dX and dW 1-2 %, and their loads already cover whole
//   lines.
//   MN-contiguous operands keep their memory layout: 32 K-rows of 512 bytes
//   per slot (each load already covers whole lines), chunks XOR-swizzled by
//   K-row, read with ds_read_b64_tr_b16, whose 16-lane transpose hands each
//   lane four consecutive K-values of its own column; two such reads form one
//   MFMA operand of eight K-values.
// MFMA fragments are double-buffered in registers: the reads of the next
// K-step's fragments are issued between the 64 MFMAs of the current one.
//
// Tile order. Workgroups are dispatched round-robin over the 8 XCDs. The
// logical tile sequence walks groups of G tile-rows (or tile-columns), the
// short side fastest inside a group; optionally each XCD first receives a
// contiguous run of that sequence. Which combination keeps the most operand
// slices in L2 (and shares MALL fills across XCDs) was measured per product
// on the head shapes (C = 4096, H = 4096, V = 128256):
//   logits: groups of 4 tile-rows, one contiguous run per XCD (each XCD
//           streams its own share of the W panels, 4 X panels at a time);
//   dX:     groups of 4 tile-columns in dispatch order;
//   dW:     groups of 4 tile-columns, one contiguous run per XCD.
// Launched in the loss's own sequence (logits and dX alternating over the
// same W), the orders differ by about 1%; alone, the logits order is ~10%
// faster than a plain dispatch-order one.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

#ifndef FLL_GEMM_STAGES
#define FLL_GEMM_STAGES 4
#endif
constexpr int BM = 256, BN = 256, BK = 32, NSTAGE = FLL_GEMM_STAGES;
constexpr int kThreads = 256;
static_assert(NSTAGE % 2 == 0, "the K-steps alternate between two fragment register sets");
static_assert(NSTAGE == 4, "two pairs of K-slices in flight");
constexpr int kSliceBytes = 256 * BK * 2;       // 16 KB per operand per K-slice
constexpr int kOperandBytes = NSTAGE * kSliceBytes;  // 64 KB per operand
constexpr int kStageBytes = 2 * kSliceBytes;    // 32 KB of LDS per K-slice
// Paired pipeline (both operands K-contiguous): K-slices are loaded in pairs
// (2j, 2j + 1), each thread issuing 8 loads per operand per pair. A pair is
// loaded during the odd K-step that frees its slots; at the top of an even
// K-step the next pair may still be in flight.
constexpr int kLoadsPerPair = 16;
// Single pipeline (an MN-contiguous operand, whose loads already cover whole
// cache lines): each K-step loads the slice NSTAGE steps ahead, 4 loads per
// operand per thread; when a slice is needed the loads of the two later ones
// may be in flight (in the prologue, of the other NSTAGE - 1).
constexpr int kLoadsPerSlice = 8;
constexpr int kVmcntLoop = kLoadsPerSlice * (NSTAGE - 2);
constexpr int kVmcntPrologue = kLoadsPerSlice * (NSTAGE - 1);
// Epilogue slab: 16 rows of the wave's 128 fp32 columns, rows 528 bytes apart.
constexpr int kSlabPitch = 132;                     // floats
constexpr int kSlabBytes = 16 * kSlabPitch * 4;     // 8448 per wave
static_assert(4 * kSlabBytes + BN * 4 + BM * 4 <= NSTAGE * kStageBytes,
              "epilogue slabs and bias table reuse the stages");
constexpr unsigned kOOB = 0x80000000u;          // offset outside every descriptor
constexpr unsigned kMaxRecords = 0x7fffffffu;
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format
constexpr int kNonTemporal = 2;                 // cache policy of a buffer load: nt

// Swizzles of the 16-byte chunk index. K-contiguous tiles (4 chunks per row):
// the 16 rows that 16 lanes of one ds_read_b128 touch spread over all banks.
// MN-contiguous tiles (32 chunks per K-row): a 16-lane group of
// ds_read_b64_tr_b16 touches four K-rows k .. k + 3 and the group beside it
// the four eight below, all at the same two chunks; {0, 10, 12, 6} by k & 3,
// XOR 2 when k & 8, puts those eight K-rows on distinct banks.
__device__ __forceinline__ int swz_k(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int swz_mn(int k) {
  return ((0x6ca0 >> ((k & 3) * 4)) & 15) ^ ((k >> 2) & 2);  // {0, 10, 12, 6}[k & 3] ^ 2 [k & 8]
}

// Buffer descriptor of `bytes` bytes from `base` (clamped to [0, 2^31 - 1]).
// The clamp works on the two 32-bit halves: with 64-bit signed compares the
// compiler emits vector compares writing scalar registers, and the scalar
// selects waiting on them stall the wavefront inside the MFMA stream.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  const uint64_t u = uint64_t(bytes);
  const unsigned hi = unsigned(u >> 32), lo = unsigned(u);
  unsigned n;
  asm("s_cmp_eq_u32 %[hi], 0\n\t"              // fits in 32 bits?
      "s_cselect_b32 %[n], %[lo], %[mx]\n\t"
      "s_cmp_gt_u32 %[n], %[mx]\n\t"            // above 2^31 - 1?
      "s_cselect_b32 %[n], %[mx], %[n]\n\t"
      "s_cmp_lt_i32 %[hi], 0\n\t"               // negative?
      "s_cselect_b32 %[n], 0, %[n]"
      : [n] "=&s"(n)
      : [lo] "s"(lo), [hi] "s"(hi), [mx] "s"(kMaxRecords)
      : "scc");
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                           kRsrcWord3);
}

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, LDS_AS void *dst,
                                           unsigned voff, unsigned soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// ---- K-contiguous operand: element (row, k) at p[row * ld + k] -------------
// LDS layout: 32 blocks of 8 rows, 2 KB each; inside a block the four K-slice
// slots lie 512 bytes apart, each 8 rows x 64 bytes with the 16-byte chunks
// XOR-swizzled by row. One load instruction covers one block of both slices
// of a pair: lanes 0-31 the first slice, lanes 32-63 the second, i.e. 8 rows
// x 128 contiguous bytes of global memory, whole cache lines.
struct OpK {
  const unsigned short *p;
  int64_t ld, row0, nrows, kbeg;
  unsigned voff[8];  // byte offsets of this thread's 8 pair chunks from (row0, k0)
  int kc[2];         // their K offsets within the pair (by block parity)
  unsigned fa;       // LDS address of this lane's fragment reads (block 0, slot 0)
  __amdgpu_buffer_rsrc_t whole;  // the tile's rows from (row0, kbeg) to the end

  __device__ __forceinline__ void init(const unsigned short *p_, int64_t ld_, int64_t row0_,
                                       int64_t nrows_, int64_t kbeg_, int wave, int lane,
                                       int wr, unsigned lds_base) {
    p = p_;
    ld = ld_;
    row0 = row0_;
    nrows = nrows_;
    kbeg = kbeg_;
    whole = rsrc(p + row0 * ld + kbeg, ((nrows - row0) * ld - kbeg) * 2);
    // lane l of load i: row 8 (8 wave + i) + ((l >> 2) & 7), slice l >> 5 of
    // the pair, chunk (l & 3) of the slot
    const int h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (wave * 8 + i) * 8 + ((lane >> 2) & 7);
      const int c = (lane & 3) ^ swz_k(r);
      voff[i] = unsigned((int64_t(r) * ld + 32 * h + 8 * c) * 2);
      if (i < 2) kc[i] = 32 * h + 8 * c;  // the swizzle repeats with the block parity
    }
    // lane l: row l % 16 of each 16-row block, K-values 8 (l / 16) .. + 7
    const int r = wr + (lane & 15);
    const int c = lane >> 4;
    fa = lds_base + unsigned((r >> 3) * 2048 + (r & 7) * 64 + 16 * (c ^ swz_k(r)));
  }
  // Load block i of this thread's share of the pair of slices starting at
  // K = k0 into the slots slot0, slot0 + 1 (`ops`: the operand's LDS base).
  // CHECK: the pair may end before k0 + 2 BK, so chunks past kend are pointed
  // outside the descriptor. Full pairs (CHECK false) use one descriptor for
  // the whole tile and step through K with the scalar offset: a row below
  // nrows stays inside the descriptor at every k0 < K <= ld, and a row past
  // it lies outside at every k0, whether or not the range check counts the
  // scalar offset.
  template <bool CHECK>
  __device__ __forceinline__ void issue_pair(LDS_AS char *ops, int slot0, int wave, int i,
                                             int64_t k0, int64_t kend) const {
    LDS_AS char *dst = ops + (wave * 8 + i) * 2048 + slot0 * 512;
    if constexpr (CHECK) {
      const __amdgpu_buffer_rsrc_t r = rsrc(p + row0 * ld + k0, ((nrows - row0) * ld - k0) * 2);
      const unsigned v = k0 + kc[i & 1] < kend ? voff[i] : kOOB;
      load_lds16(r, dst, v);
    } else {
      load_lds16(whole, dst, voff[i], unsigned(k0 - kbeg) * 2u);
    }
  }
  // (named by the code for MN-contiguous operands, never called here)
  template <bool CHECK>
  __device__ void issue_one(LDS_AS char *, int, int, int, int64_t, int64_t) const {
    static_assert(CHECK && !CHECK, "K-contiguous operands load pairs of slices");
  }
  static constexpr int kReads = 8;  // LDS reads per K-step
  // Read X (0..7) of the K-step whose slice is in slot SLOT: block X (rows
  // wr + 16 X ..; adding 16 rows leaves the swizzle unchanged). The slot and
  // block offsets are instruction immediates.
  template <int SLOT, int X>
  __device__ __forceinline__ void read(bf16x8 (&f)[8]) const {
    asm volatile("ds_read_b128 %0, %1 offset:%2"
                 : "=v"(f[X])
                 : "v"(fa), "i"(SLOT * 512 + X * 4096));
  }
};

// ---- MN-contiguous operand: element (row, k) at p[k * ld + row] ------------
struct OpMN {
  const unsigned short *p;
  int64_t ld, col0;
  unsigned voff[4];  // byte offsets of this thread's 4 chunks from (k0, col0)
  unsigned fb[8];    // LDS addresses of the transpose reads, block i

  __device__ __forceinline__ void init(const unsigned short *p_, int64_t ld_, int64_t col0_,
                                       int wave, int lane, int wr, unsigned lds_base) {
    p = p_;
    ld = ld_;
    col0 = col0_;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = (wave * 4 + i) * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swz_mn(kr);
      voff[i] = unsigned((int64_t(kr) * ld + 8 * c) * 2);
    }
    // 16-lane group G, lane q: K-row 8 G + (q >> 2), columns
    // wr + 16 i + 4 (q & 3) .. + 3; after the transpose lane q holds column
    // wr + 16 i + q, K-values 8 G .. + 3 (and + 4 .. + 7 from the K-rows four
    // below, whose swizzle is the same).
    const int G = lane >> 4, q = lane & 15;
    const int k = 8 * G + (q >> 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int col = wr + 16 * i + 4 * (q & 3);
      const int c = col >> 3, half = (col >> 2) & 1;
      fb[i] = lds_base + unsigned(k * 512 + 16 * (c ^ swz_mn(k)) + 8 * half);
    }
  }
  // Load chunk i (0..3) of the slice starting at K = k0 into slot `slot`.
  template <bool CHECK>
  __device__ __forceinline__ void issue_one(LDS_AS char *ops, int slot, int wave, int i,
                                            int64_t k0, int64_t kend) const {
    const __amdgpu_buffer_rsrc_t r = rsrc(p + k0 * ld + col0, ((kend - k0) * ld - col0) * 2);
    load_lds16(r, ops + slot * kSliceBytes + (wave * 4 + i) * 1024, voff[i]);
  }
  // Load block i (0..7) of the pair of slices starting at K = k0 into the
  // slots slot0, slot0 + 1 (`ops`: the operand's LDS base); each slot holds
  // 32 K-rows of 512 bytes. K-rows past kend lie outside the descriptor and
  // read as zero, so no per-lane check is needed.
  template <bool CHECK>
  __device__ __forceinline__ void issue_pair(LDS_AS char *ops, int slot0, int wave, int i,
                                             int64_t k0, int64_t kend) const {
    const int t = i >> 2;  // slice of the pair
    const int64_t k = k0 + int64_t(t) * BK;
    const __amdgpu_buffer_rsrc_t r = rsrc(p + k * ld + col0, ((kend - k) * ld - col0) * 2);
    load_lds16(r, ops + (slot0 + t) * kSliceBytes + (wave * 4 + (i & 3)) * 1024, voff[i & 3]);
  }
  static constexpr int kReads = 16;  // LDS reads per K-step
  // Read X (0..15) of the K-step whose slice is in slot SLOT: block X / 2,
  // K-values 4 (X % 2) .. + 3 of each lane's eight (the two halves of the
  // MFMA operand).
  template <int SLOT, int X>
  __device__ __forceinline__ void read(bf16x8 (&f)[8]) const {
    constexpr int i = X >> 1;
    i16x4 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(v)
                 : "v"(fb[i]), "i"(SLOT * kSliceBytes + (X & 1) * 4 * 512));
    auto w = __builtin_bit_cast(i16x8, f[i]);
    if constexpr (X & 1) {
      w = __builtin_shufflevector(w, __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1),
                                  0, 1, 2, 3, 8, 9, 10, 11);
    } else {
      w = __builtin_shufflevector(w, __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1),
                                  8, 9, 10, 11, 4, 5, 6, 7);
    }
    f[i] = __builtin_bit_cast(bf16x8, w);
  }
};

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order.
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

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
// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction per pair; a NaN stays a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ unsigned short f2bf(float f) {
  return (unsigned short)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Logits epilogue: S row-major, pitch lds elements, fp32 or (B16) bf16
// rounded to nearest even. Stores four consecutive columns n .. n + 3 of row
// m (n is a multiple of 4).
template <bool B16>
struct EpiLogits {
  static constexpr bool kRowStats = true;
  static constexpr bool kSeedAcc = false;
  static constexpr bool kColSums = false;
  void *S;
  int64_t lds;
  const unsigned short *bias;
  float inv_tau;
  float2 *stats;
  int64_t n_stat;
  const int64_t *labels;  // label_logit: see launch_logits_bf16
  int64_t label_row0;
  float *label_logit;
  __device__ __forceinline__ float col_bias(int64_t n) const {
    return bias ? __uint_as_float(unsigned(bias[n]) << 16) : 0.0f;
  }
  // store4_in: the four columns are inside the matrix. Non-temporal: the
  // chunk's logits (GBs) are read once, by the row kernel, after the whole
  // GEMM; streaming them past the caches measured 2.5 % off the GEMM and 3 %
  // off the row kernel.
  __device__ __forceinline__ void store4_in(int64_t m, int64_t n, f32x4 v, int) const {
    if constexpr (B16) {
      u32x2 pk;
      pk.x = pack_bf16x2(v.x, v.y);
      pk.y = pack_bf16x2(v.z, v.w);
      __builtin_nontemporal_store(
          pk, reinterpret_cast<u32x2 *>(static_cast<unsigned short *>(S) + m * lds + n));
    } else {
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(static_cast<float *>(S) + m * lds + n));
    }
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, int64_t nmax, float4 v,
                                         int) const {
    const float ve[4] = {v.x, v.y, v.z, v.w};
    if constexpr (B16) {
      unsigned short *p = static_cast<unsigned short *>(S) + m * lds + n;
      if (n + 4 <= nmax) {
        uint2 pk;
        pk.x = pack_bf16x2(v.x, v.y);
        pk.y = pack_bf16x2(v.z, v.w);
        *reinterpret_cast<uint2 *>(p) = pk;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < nmax) p[e] = f2bf(ve[e]);
      }
    } else {
      float *p = static_cast<float *>(S) + m * lds + n;
      if (n + 4 <= nmax) {
        *reinterpret_cast<float4 *>(p) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < nmax) p[e] = ve[e];
      }
    }
  }
};

// dX epilogue: bf16 store when unsplit, fp32 partial per split otherwise.
// Stores four consecutive columns n .. n + 3 of row m (n is a multiple of 4).
struct EpiDx {
  static constexpr bool kRowStats = false;
  static constexpr bool kSeedAcc = false;
  static constexpr bool kColSums = false;
  unsigned short *out;
  int64_t ldo;
  float *partial;
  int64_t M, N;
  __device__ __forceinline__ void store4_in(int64_t m, int64_t n, f32x4 v, int split) const {
    if (partial) {
      *reinterpret_cast<f32x4 *>(partial + (int64_t(split) * M + m) * N + n) = v;
    } else {
      uint2 pk;
      pk.x = pack_bf16x2(v.x, v.y);
      pk.y = pack_bf16x2(v.z, v.w);
      *reinterpret_cast<uint2 *>(out + m * ldo + n) = pk;
    }
  }
  __device__ __forceinline__ void store4(int64_t m, int64_t n, int64_t nmax, float4 v,
                                         int split) const {
    const float ve[4] = {v.x, v.y, v.z, v.w};
    if (partial) {
      float *p = partial + (int64_t(split) * M + m) * N + n;
      if (n + 4 <= nmax) {
        *reinterpret_cast<float4 *>(p) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < nmax) p[e] = ve[e];
      }
    } else {
      unsigned short *p = out + m * ldo + n;
      if (n + 4 <= nmax) {
        uint2 pk;
        pk.x = pack_bf16x2(v.x, v.y);
        pk.y = pack_bf16x2(v.z, v.w);
        *reinterpret_cast<uint2 *>(p) = pk;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < nmax) p[e] = f2bf(ve[e]);
      }
    }
  }
};

// dW: fp32, accumulated across token chunks (each tile owns its rows, so
// there are no atomics). On every chunk after the first the accumulators
// start from the tile's old values, loaded together with the first operand
// slices, so the epilogue only stores: the fp32 read overlaps the start of
// the K loop instead of following it. The interior tiles' loads and stores
// are non-temporal: dW (GBs) is touched once per chunk.
// db (when given) is formed in the same tiles: the tiles of N-block 0 also
// sum their dZ^T rows over the chunk's tokens, with MFMAs against a
// fragment of ones [frozen lm_head GRPO page, Summary: the bias gradient
// with the weight's, only when asked for].
struct EpiDw {
  static constexpr bool kRowStats = false;
  static constexpr bool kSeedAcc = true;
  static constexpr bool kColSums = true;
  float *dW;
  int64_t ld;
  int accumulate;
  float *db;  // [M] fp32, or null
  __device__ __forceinline__ f32x4 load4_in(int64_t m, int64_t n) const {
    if (!accumulate) return f32x4{0.f, 0.f, 0.f, 0.f};
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(dW + m * ld + n));
  }
  __device__ __forceinline__ void store4_in(int64_t m, int64_t n, f32x4 v, int) const {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(dW + m * ld + n));
  }
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
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < nmax) p[e] = ve[e];
    }
  }
};

// The inner loop's MFMAs and LDS fragment reads are volatile inline assembly,
// so they issue in exactly the order written: each K-step interleaves the
// reads of the next K-step's fragments and its share of the slice loads
// with its 64 MFMAs. The compiler neither sees the reads' latency nor
// treats the asm as MFMAs, so the LDS waits are explicit and the accumulators
// rest a few cycles before the epilogue reads them.
__device__ __forceinline__ void mfma(f32x4 &acc, const bf16x8 &a, const bf16x8 &b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// max of three floats (v_max3_f32). fmaxf on values read from accumulator
// registers would first quiet each input with an extra v_max_f32 copy.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one output row of
// a 16 x 16 block) with the gfx950 lane swaps: v_permlane16_swap exchanges
// rows of 16 lanes pairwise and v_permlane32_swap the two halves, so after a
// swap of a value with itself the two results hold x[l] and x[l ^ 16] (or
// x[l ^ 32]) in every lane, in either order. VALU only: no LDS round trip
// as a ds_bpermute would take.
__device__ __forceinline__ float quad_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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
  const int lane = t & 63;
  // The wavefront index is uniform: in a scalar register, every LDS
  // destination of the staging loads is scalar arithmetic.
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const unsigned lds_base = unsigned(reinterpret_cast<uintptr_t>(lds));

  // K-contiguous operands load pairs of slices, MN-contiguous ones single
  // slices: both paired (logits), one paired and the other single (dX: A
  // paired; dW over the transposed X: B paired), both single otherwise.
  constexpr bool PAIRED = A_K && B_K;
  constexpr bool HYBRID = A_K != B_K;
  using OA = typename std::conditional<A_K, OpK, OpMN>::type;
  using OB = typename std::conditional<B_K, OpK, OpMN>::type;
  OA opa;
  OB opb;
  if constexpr (A_K) opa.init(d.A, d.lda, m0, d.M, kbeg, wave, lane, wm * 128, lds_base);
  else opa.init(d.A, d.lda, m0, wave, lane, wm * 128, lds_base);
  if constexpr (B_K)
    opb.init(d.B, d.ldb, n0, d.N, kbeg, wave, lane, wn * 128, lds_base + kOperandBytes);
  else opb.init(d.B, d.ldb, n0, wave, lane, wn * 128, lds_base + kOperandBytes);
  LDS_AS char *lds_a = lds, *lds_b = lds + kOperandBytes;
  // hybrid: the paired (K-contiguous) operand and the single one, with their
  // LDS bases
  auto &opP = [&]() -> auto & {
    if constexpr (B_K && !A_K) return opb;
    else return opa;
  }();
  auto &opS = [&]() -> auto & {
    if constexpr (B_K && !A_K) return opa;
    else return opb;
  }();
  LDS_AS char *lds_P = (B_K && !A_K) ? lds_b : lds_a;
  LDS_AS char *lds_S = (B_K && !A_K) ? lds_a : lds_b;

  // acc[i][j]: the 16 x 16 block of rows wm * 128 + 16 i, columns wn * 128 + 16 j
  f32x4 acc[8][8];
  const int64_t mw = m0 + wm * 128, nw = n0 + wn * 128;
  // every column of this wave is below N / every row and column is inside
  const bool full = nw + 128 <= d.N;
  const bool interior = full && mw + 128 <= d.M;
  if constexpr (Epi::kSeedAcc) {
    // The tile's old values, in the accumulator layout (lane l: row
    // 16 i + l % 16, columns 16 j + 4 (l / 16) .. + 3), loaded straight into
    // the accumulators before the operand slices, so the prologue's wait
    // covers them. One descriptor per tile: rows past M lie outside its
    // range and read as zero, and so does everything on the first chunk
    // (range 0: no branch, the loads return zeros without a memory access);
    // a column group past N (N is a multiple of 4) is pointed outside it.
    const int64_t rows_left = d.M - m0;
    const int64_t range =
        epi.accumulate ? (rows_left < BM ? rows_left : BM) * epi.ld * 4 : int64_t(0);
    const __amdgpu_buffer_rsrc_t r = rsrc(epi.dW + m0 * epi.ld, range);
    // element (m, n) lies (m - m0) * ld + n floats past the descriptor's base
    const unsigned lane_off =
        unsigned(((wm * 128 + (lane & 15)) * epi.ld + nw + 4 * (lane >> 4)) * 4);
    const int64_t nc = nw + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned vi = lane_off + unsigned(i * 16 * epi.ld * 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const unsigned v = full || nc + 16 * j < d.N ? vi + 64u * j : kOOB;
        acc[i][j] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, v, 0, kNonTemporal));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // db: the wave holding the first 128 columns of N-block 0 sums its 128
  // rows of A over K: each lane adds the eight K-values of its fragments
  // with v_dot2 against ones, the four K-groups are merged at the end
  bool col_sums = false;
  if constexpr (Epi::kColSums) col_sums = epi.db != nullptr && tn == 0 && wn == 0;
  float csum[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) csum[i] = 0.0f;

  // K-step kt (the last one may be partial) multiplies the fragments of
  // slice kt, held in registers; meanwhile it reads the fragments of slice
  // kt + 1 from its slot into the other register set and issues loads into
  // slots already consumed (see the staging note at the top). The loop is
  // unrolled by NSTAGE (even), so every slot offset and register set below
  // is a compile-time constant.
  const int nkt = kend > kbeg ? int((kend - kbeg + BK - 1) / BK) : 0;
  const int nkt_full = kend > kbeg ? int((kend - kbeg) / BK) : 0;

  bf16x8 fa[2][8], fb[2][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fa[0][i] = fa[1][i] = bf16x8{};
    fb[0][i] = fb[1][i] = bf16x8{};
  }
  if (nkt > 0) {
    // prologue: all NSTAGE slices in flight; wait for the first, read it
    if constexpr (PAIRED) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int64_t k0 = kbeg + int64_t(2 * pr) * BK;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          opa.template issue_pair<true>(lds_a, 2 * pr, wave, q, k0, kend);
          opb.template issue_pair<true>(lds_b, 2 * pr, wave, q, k0, kend);
        }
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerPair) : "memory");
    } else if constexpr (HYBRID) {
      // in the order the steady state issues them: single 0, single 1,
      // pair (0, 1), single 2, single 3, pair (2, 3); slice 0 of both needs
      // all but the last 16
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int sl = 2 * pr + t;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            opS.template issue_one<true>(lds_S, sl, wave, q, kbeg + int64_t(sl) * BK, kend);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          opP.template issue_pair<true>(lds_P, 2 * pr, wave, q, kbeg + int64_t(2 * pr) * BK, kend);
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerPair) : "memory");
    } else {
#pragma unroll
      for (int sl = 0; sl < NSTAGE; ++sl) {
        const int64_t k0 = kbeg + int64_t(sl) * BK;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          opa.template issue_one<true>(lds_a, sl, wave, q, k0, kend);
          opb.template issue_one<true>(lds_b, sl, wave, q, k0, kend);
        }
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kVmcntPrologue) : "memory");
    }
    __builtin_amdgcn_s_barrier();
    static_for<OA::kReads>([&](auto X) __attribute__((always_inline)) {
      opa.template read<0, decltype(X)::value>(fa[0]);
    });
    static_for<OB::kReads>([&](auto X) __attribute__((always_inline)) {
      opb.template read<0, decltype(X)::value>(fb[0]);
    });
  }

  auto kstep = [&](auto U_, auto CHECK_, int kt) __attribute__((always_inline)) {
    constexpr int u = decltype(U_)::value;
    constexpr bool CHECK = decltype(CHECK_)::value;
    constexpr int cur = u & 1, nxt = cur ^ 1;
    constexpr int slot_nxt = (u + 1) % NSTAGE;  // slice kt + 1
    // Paired: odd steps load the pair kt + 3, kt + 4 into the slots of
    // kt - 1 and kt, both free once every wave is past this step's barrier.
    // Single: every step loads slice kt + NSTAGE into the slot of slice kt.
    // Hybrid: every step loads B's slice kt + NSTAGE into the slot of slice
    // kt, odd steps then A's pair kt + 3, kt + 4.
    constexpr bool load_pair = PAIRED && (u & 1);
    constexpr int slot_load = PAIRED ? (u + 3) % NSTAGE : u;
    const int64_t k_load = kbeg + int64_t(kt + (PAIRED ? 3 : NSTAGE)) * BK;
    constexpr int slot_pair = (u + 3) % NSTAGE;
    const int64_t k_pair = kbeg + int64_t(kt + 3) * BK;
    // Slice kt + 1 is in LDS for every wave, and every wave has its slice-kt
    // fragments. Of this thread's loads, those still allowed in flight are:
    // paired, those of the pair after the one holding slice kt + 1 (none at
    // odd steps, whose slice kt + 1 starts the most recently loaded pair);
    // single, those of slices kt + 2 and kt + 3.
    // hybrid: at even steps the single operand's slices kt + 2, kt + 3 and
    // the paired operand's pair after the one holding slice kt + 1 (16); at
    // odd steps only the single slice loaded by the step before (4), since
    // the pair holding slice kt + 1 was the last thing issued before it.
    constexpr int vm = PAIRED   ? (load_pair ? 0 : kLoadsPerPair)
                       : HYBRID ? ((u & 1) ? 4 : kLoadsPerPair)
                                : kVmcntLoop;
    wait_lds();
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(vm) : "memory");
    __builtin_amdgcn_s_barrier();
    // 64 MFMAs; between them the reads of slice kt + 1 and the loads: paired,
    // at odd steps, the 16 of the next pair (8 of A, then 8 of B); single, 8
    // per step (4 of A, then 4 of B).
    // A's read r follows MFMA ea * r, B's read r MFMA eb / 2 + eb * r. The
    // spacing was measured per product: the logits GEMM spreads its reads
    // over the whole step (closer spacings ran it 1-2 % slower); dX issues
    // its 16 transpose reads of W every second MFMA, done by mid-step so
    // their latency is covered before the next step's wait (dX 3.3 %
    // faster than one every fourth); dW its 8 reads of the transposed X
    // every sixth (about 1 %).
    constexpr int ea = 64 / OA::kReads;
    constexpr int eb = (A_K && !B_K) ? 2 : (!A_K && B_K) ? 6 : 64 / OB::kReads;
    static_assert(ea * (OA::kReads - 1) < 64 && eb / 2 + eb * (OB::kReads - 1) < 64,
                  "every read of slice kt + 1 is issued inside the step");
    static_for<64>([&](auto X_) __attribute__((always_inline)) {
      constexpr int x = decltype(X_)::value;
      mfma(acc[x >> 3][x & 7], fb[cur][x & 7], fa[cur][x >> 3]);
      if constexpr (x % ea == 0) opa.template read<slot_nxt, x / ea>(fa[nxt]);
      if constexpr (x >= eb / 2 && (x - eb / 2) % eb == 0 && (x - eb / 2) / eb < OB::kReads)
        opb.template read<slot_nxt, (x - eb / 2) / eb>(fb[nxt]);
      if constexpr (load_pair && (x & 3) == 2) {
        constexpr int q = x >> 2;
        if constexpr (q < 8)
          opa.template issue_pair<CHECK>(lds_a, slot_load, wave, q, k_load, kend);
        else
          opb.template issue_pair<CHECK>(lds_b, slot_load, wave, q - 8, k_load, kend);
      }
      if constexpr (HYBRID && (u & 1) && (x & 3) == 2) {
        constexpr int q = x >> 2;  // the single slice's 4 loads, then the pair's 8
        if constexpr (q < 4)
          opS.template issue_one<CHECK>(lds_S, slot_load, wave, q, k_load, kend);
        else if constexpr (q < 12)
          opP.template issue_pair<CHECK>(lds_P, slot_pair, wave, q - 4, k_pair, kend);
      }
      if constexpr (HYBRID && !(u & 1) && (x & 15) == 4)
        opS.template issue_one<CHECK>(lds_S, slot_load, wave, x >> 4, k_load, kend);
      if constexpr (!PAIRED && !HYBRID && (x & 7) == 4) {
        constexpr int q = x >> 3;
        if constexpr (q < 4)
          opa.template issue_one<CHECK>(lds_a, slot_load, wave, q, k_load, kend);
        else
          opb.template issue_one<CHECK>(lds_b, slot_load, wave, q - 4, k_load, kend);
      }
    });
    if constexpr (Epi::kColSums) {
      if (col_sums) {
        // the four bf16 pairs of each fragment, taken with shuffles: an
        // element of a bit-cast vector passed to the builtin compiled to the
        // first pair four times
        const bf16x2_t one2 = {1.0, 1.0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x8 f = fa[cur][i];
          float c = csum[i];
          c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 0, 1), one2, c, false);
          c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 2, 3), one2, c, false);
          c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 4, 5), one2, c, false);
          c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 6, 7), one2, c, false);
          csum[i] = c;
        }
      }
    }
  };

  // Full-speed steps: the slice each one loads lies wholly before kend.
  const int fast_end = nkt_full - NSTAGE;
  int kt = 0;
  for (; kt + NSTAGE <= fast_end; kt += NSTAGE)
    static_for<NSTAGE>([&](auto U) __attribute__((always_inline)) {
      kstep(U, std::false_type{}, kt + decltype(U)::value);
    });
  // The last steps load partial or empty slices.
  for (; kt < nkt; kt += NSTAGE)
    static_for<NSTAGE>([&](auto U) __attribute__((always_inline)) {
      if (kt + decltype(U)::value < nkt) kstep(U, std::true_type{}, kt + decltype(U)::value);
    });
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // The MFMAs take the B fragment as their first operand, so each 16 x 16
  // accumulator block holds the transposed product: lane l owns output row
  // m = l % 16 of the block and its four consecutive columns
  // 4 (l / 16) .. + 3, so acc[i][j] of lane l is row 16 i + l % 16,
  // columns 16 j + 4 (l / 16) .. + 3 of the wave's 128 x 128. Lanes l, l ^ 16,
  // l ^ 32 and l ^ 48 share a row.
  //
  // Stored as they lie, a 64-lane store would write 16 rows x 64 bytes, half
  // a cache line per row; the write path then runs far below its rate. So
  // each 16-row slab of the wave's tile passes through LDS (the staging
  // buffers are idle now): written in the accumulator layout, read back so
  // that one instruction covers two rows x 128 columns, i.e. 512 contiguous
  // bytes per row. Rows of the slab sit 528 bytes apart in LDS, which spreads
  // both the writes and the reads over all banks.
  __syncthreads();  // every wave is done reading the staging buffers
  // The bias of the tile's 256 columns (0 past N) goes to LDS after the four
  // waves' slabs: read per slab, it is not held in registers across the
  // epilogue.
  LDS_AS float *btab = (LDS_AS float *)(lds + 4 * kSlabBytes);
  // and the labels of the tile's 256 rows when the label logits are asked
  // for (-1: no label in [0, N))
  LDS_AS int *ltab = (LDS_AS int *)(lds + 4 * kSlabBytes + BN * 4);
  if constexpr (Epi::kRowStats) {
    if (epi.bias) btab[t] = n0 + t < d.N ? epi.col_bias(n0 + t) : 0.0f;
    if (epi.label_logit) {
      const int64_t y = m0 + t < d.M ? epi.labels[epi.label_row0 + m0 + t] : -1;
      ltab[t] = y >= 0 && y < d.N ? int(y) : -1;
    }
    if (epi.bias || epi.label_logit) __syncthreads();
  }
  LDS_AS float *slab = (LDS_AS float *)(lds + wave * kSlabBytes);
  const int lrow = lane & 15;
  const int lcol = 4 * (lane >> 4);
  const int crow = lane >> 5;        // coalesced layout: row 2 j + crow of the slab,
  const int ccol = 4 * (lane & 31);  // columns ccol .. ccol + 3 of the wave's 128
  constexpr float kLog2e = 1.4426950408889634f;

  // db: the chunk's column sums, added to what earlier chunks left (each row
  // of db belongs to one tile: no atomics)
  if constexpr (Epi::kColSums) {
    if (col_sums) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = quad_sum(csum[i]);  // lanes q, q + 16, q + 32, q + 48
        const int64_t m = mw + 16 * i + lane;
        if (lane < 16 && m < d.M) epi.db[m] = epi.accumulate ? epi.db[m] + t : t;
      }
    }
  }

  // One 16-row slab; I is a compile-time constant so that acc[I] stays in
  // registers (a runtime index would move the accumulators to scratch).
  auto do_slab = [&](auto I_) __attribute__((always_inline)) {
    constexpr int i = decltype(I_)::value;
    // keep each slab's register working set to itself
    __builtin_amdgcn_sched_barrier(0);
    // this lane's 32 values of the slab: v[j] = columns 16 j + lcol + 0..3
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = acc[i][j];
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(v[j]));  // copied here, not earlier
    if constexpr (Epi::kRowStats) {
      // S = (acc + b) / tau, then this row's max and sum of exp over the
      // wave's 128 columns below N, merged over the four lanes of the row.
      const int64_t m = mw + i * 16 + lrow;
      if (epi.bias) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4 b = *(const LDS_AS f32x4 *)(btab + wn * 128 + 16 * j + lcol);
          v[j] = (v[j] + b) * epi.inv_tau;
        }
      } else if (epi.inv_tau != 1.0f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] *= epi.inv_tau;
      }
      if (epi.stats) {
        // column of element e of v[j]: nw + 16 j + lcol + e
        float mx = -INFINITY;
        if (full) {
          // two independent chains of max3
          float ma = max3(v[0].x, v[0].y, v[0].z), mb = max3(v[1].x, v[1].y, v[1].z);
          ma = max3(ma, v[0].w, v[2].x);
          mb = max3(mb, v[1].w, v[3].x);
#pragma unroll
          for (int j = 2; j < 8; j += 2) {
            ma = max3(ma, v[j].y, v[j].z);
            mb = max3(mb, v[j + 1].y, v[j + 1].z);
            ma = j + 2 < 8 ? max3(ma, v[j].w, v[j + 2].x) : vmax(ma, v[j].w);
            mb = j + 3 < 8 ? max3(mb, v[j + 1].w, v[j + 3].x) : vmax(mb, v[j + 1].w);
          }
          mx = vmax(ma, mb);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nw + 16 * j + lcol + e < d.N) mx = fmaxf(mx, v[j][e]);
        }
        mx = quad_max(mx);
        // exp(v - mx) = 2^((v - mx) log2(e)), the difference taken first so
        // the maximum itself adds exactly 1 (with v log2(e) - mx log2(e) as
        // one fma, the rounding of mx log2(e) left a one-entry vocabulary a
        // log-sum-exp an ulp off its logit, and exact zeros became 1e-7)
        const float mxs = mx == -INFINITY ? 0.0f : mx;
        float se = 0.0f;
        if (full) {
          // four independent sums (one per element of the 4-column group)
          float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s4[e] += __builtin_amdgcn_exp2f((v[j][e] - mxs) * kLog2e);
          se = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        } else if (mx != -INFINITY) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nw + 16 * j + lcol + e < d.N)
                se += __builtin_amdgcn_exp2f((v[j][e] - mxs) * kLog2e);
        }
        se = quad_sum(se);
        if (lane < 16 && m < d.M && nw < d.N)
          epi.stats[m * epi.n_stat + (nw >> 7)] = make_float2(mx, se);
      }
    }

#pragma unroll
    for (int j = 0; j < 8; ++j)
      *(LDS_AS f32x4 *)(slab + lrow * kSlabPitch + 16 * j + lcol) = v[j];
    if constexpr (Epi::kRowStats) {
      // the label's fp32 logit, if it lies in this wave's 128 columns: one
      // lane per row of the slab reads it back from the slab
      if (epi.label_logit && lane < 16) {
        const int off = ltab[wm * 128 + i * 16 + lane] - int(nw);
        if (off >= 0 && off < 128)
          epi.label_logit[epi.label_row0 + mw + i * 16 + lane] = slab[lane * kSlabPitch + off];
      }
    }
    // A wave's LDS operations complete in order, so the reads see the writes;
    // all eight are issued before the first store waits for them.
    f32x4 rd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rd[j] = *(const LDS_AS f32x4 *)(slab + (2 * j + crow) * kSlabPitch + ccol);
    int64_t mrow = mw + i * 16 + crow;
    asm volatile("" : "+v"(mrow));  // row addresses are formed here, per slab
    if (interior) {
#pragma unroll
      for (int j = 0; j < 8; ++j) epi.store4_in(mrow + 2 * j, nw + ccol, rd[j], split);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (mrow + 2 * j < d.M)
          epi.store4(mrow + 2 * j, nw + ccol, d.N,
                     make_float4(rd[j].x, rd[j].y, rd[j].z, rd[j].w), split);
    }
  };
  static_for<8>([&](auto I) __attribute__((always_inline)) { do_slab(I); });
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
                        const void *b, float inv_tau, void *S, int64_t lds, int s_bf16,
                        float2 *stats, int64_t n_stat, int64_t M, int64_t N, int64_t K,
                        const int64_t *labels, int64_t label_row0, float *label_logit,
                        hipStream_t st) {
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
  d.group = 4;        // measured best for the head shapes: see the tile-order note
  d.n_first = 0;
  d.xcd_remap = 1;
  const auto *bias = static_cast<const unsigned short *>(b);
  if (!labels) label_logit = nullptr;
  if (s_bf16)
    launch<true, true>(d, EpiLogits<true>{S, lds, bias, inv_tau, stats, n_stat, labels,
                                          label_row0, label_logit},
                       st);
  else
    launch<true, true>(d, EpiLogits<false>{S, lds, bias, inv_tau, stats, n_stat, labels,
                                           label_row0, label_logit},
                       st);
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

void launch_dw_bf16(const void *dZ, int64_t ldz, const void *XT, int64_t ldxt, float *dW,
                    float *db, int64_t M, int64_t N, int64_t K, int accumulate,
                    hipStream_t st) {
  GemmDesc d{};
  d.A = static_cast<const unsigned short *>(dZ);
  d.lda = ldz;
  d.B = static_cast<const unsigned short *>(XT);
  d.ldb = ldxt;
  d.M = M;
  d.N = N;
  d.K = K;
  d.split_len = K;
  d.splits = 1;
  d.group = 4;
  d.n_first = 1;
  d.xcd_remap = 1;
  EpiDw e{dW, N, accumulate, db};
  launch<false, true>(d, e, st);
}

}  // namespace fll
