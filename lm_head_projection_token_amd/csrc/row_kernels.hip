// Row-wise and reduction kernels of the fused lm_head loss (gfx950, wave64).
//
// The fused row kernel is the softmax / loss / dlogits step between the
// logits GEMM and the gradient GEMMs: for one token row it forms the
// log-sum-exp over the vocabulary, the row's loss term and the row's dlogits,
// and writes the dlogits in place over the row's logits [FusedLinearKLDivLoss
// page, Details: the log-softmax backward is computed in place on the saved
// log-probs]. It streams the row from HBM with 16-byte coalesced loads; the
// reductions run in registers, then across the wavefront with lane shuffles,
// then across the wavefronts of the workgroup through LDS.
#include <hip/hip_runtime.h>
#include <math.h>

#include "fll_internal.h"

namespace fll {
namespace {

// One workgroup of 12 wavefronts per row, each thread with 4 groups of four
// elements in flight per strip: measured fastest of 256..1024 threads x 4 or 8
// groups for every head at V = 128256 (8-20 % ahead of 4 waves x 8 groups).
constexpr int kRowThreads = 768;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kUnroll = 4;  // float4 groups per thread per strip
constexpr int kStrip = kRowThreads * kUnroll;  // float4 groups per strip

constexpr int HEAD_KL = 0;
constexpr int HEAD_SEL = 1;
constexpr int HEAD_CE = 2;  // the selective head with the opposite sign
constexpr int HEAD_JSD = 3;
constexpr int HEAD_PPO = 4;    // clipped surrogate on the selective log-prob
constexpr int HEAD_CISPO = 5;  // clipped ratio as a gradient-free weight

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Combine two (max, sum of exp(x - max)) pairs.
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

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

// bf16 dZ rows are read by the GEMMs in 8-element chunks; the slots from V to
// the next multiple of 8 are zeroed so a partial last chunk adds nothing.
__device__ __forceinline__ void zero_pad(unsigned short *Zb, int64_t V, int tid) {
  const int64_t pad = (8 - (V & 7)) & 7;
  if (tid < pad) Zb[V + tid] = 0;
}

struct Load4 {
  float v[4];
};

// Loads elements [4g, 4g + 4) of a row (clipped at V), 16-byte loads when the
// group is whole and the row is 16-byte aligned.
__device__ __forceinline__ Load4 load_group(const float *row, int64_t g, int64_t V,
                                            bool vec_ok) {
  Load4 r;
  const int64_t e = 4 * g;
  if (vec_ok && e + 4 <= V) {
    float4 x = *reinterpret_cast<const float4 *>(row + e);
    r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = (e + i < V) ? row[e + i] : 0.0f;
  }
  return r;
}

// The same for the last read of a row: a non-temporal load, so the streamed
// row does not displace reused lines in the caches.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Load4 load_group_last(const float *row, int64_t g, int64_t V,
                                                 bool vec_ok) {
  Load4 r;
  const int64_t e = 4 * g;
  if (vec_ok && e + 4 <= V) {
    const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(row + e));
    r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = (e + i < V) ? row[e + i] : 0.0f;
  }
  return r;
}

// A row of the chunk's logits: fp32, or (SB) bf16 widened to fp32 on load.
__device__ __forceinline__ float bf2f(unsigned short h) { return __uint_as_float(unsigned(h) << 16); }
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
template <bool SB>
struct SRow;
template <>
struct SRow<false> {
  const float *p;
  __device__ __forceinline__ Load4 load(int64_t g, int64_t V) const {
    return load_group(p, g, V, true);
  }
  __device__ __forceinline__ Load4 load_last(int64_t g, int64_t V) const {
    return load_group_last(p, g, V, true);
  }
  __device__ __forceinline__ float at(int64_t v) const { return p[v]; }
};
template <>
struct SRow<true> {
  const unsigned short *p;  // rows are 128-byte aligned, so groups are 8-byte aligned
  template <bool LAST>
  __device__ __forceinline__ Load4 get(int64_t g, int64_t V) const {
    Load4 r;
    const int64_t e = 4 * g;
    if (e + 4 <= V) {
      const u32x2_t *q = reinterpret_cast<const u32x2_t *>(p + e);
      const u32x2_t x = LAST ? __builtin_nontemporal_load(q) : *q;
      r.v[0] = __uint_as_float(x.x << 16);
      r.v[1] = __uint_as_float(x.x & 0xffff0000u);
      r.v[2] = __uint_as_float(x.y << 16);
      r.v[3] = __uint_as_float(x.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) r.v[i] = (e + i < V) ? bf2f(p[e + i]) : 0.0f;
    }
    return r;
  }
  __device__ __forceinline__ Load4 load(int64_t g, int64_t V) const { return get<false>(g, V); }
  __device__ __forceinline__ Load4 load_last(int64_t g, int64_t V) const {
    return get<true>(g, V);
  }
  __device__ __forceinline__ float at(int64_t v) const { return bf2f(p[v]); }
};

// Block-wide reduction helpers: wave shuffles, then the wavefronts' partials
// combined in a fixed order by thread 0 through LDS.
__device__ __forceinline__ float block_sum(float v, float (*red)[8], int slot, int lane,
                                           int wave) {
  v = wave_sum(v);
  if (lane == 0) red[wave][slot] = v;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < kRowWaves; ++w) t += red[w][slot];
  return t;
}

template <int HEAD, bool SB>
__global__ __launch_bounds__(kRowThreads) void row_kernel(RowArgs a) {
  __shared__ float red[kRowWaves][8];
  __shared__ float bcast[8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t lr = blockIdx.x;
  const int64_t gr = a.row0 + lr;
  const int64_t V = a.V;
  char *rowp = reinterpret_cast<char *>(a.S) + lr * a.s_pitch * (SB ? 2 : 4);
  static_assert(HEAD != HEAD_JSD, "the JSD head has its own row kernel");
  float *Srow = reinterpret_cast<float *>(rowp);                 // fp32 logits / dZ
  unsigned short *Zb = reinterpret_cast<unsigned short *>(rowp);  // bf16 dZ
  SRow<SB> sr{reinterpret_cast<decltype(SRow<SB>::p)>(rowp)};
  const int64_t ngroups = (V + 3) / 4;

  int64_t y = 0;
  bool valid = true;
  if (a.labels) {
    y = a.labels[gr];
    valid = (y != a.ignore_index);
  }
  const bool bad_label = HEAD != HEAD_KL && valid && (y < 0 || y >= V);
  if (!valid || bad_label) {
    // The row takes no part: its dlogits are zero.
    for (int64_t g = tid; g < ngroups; g += kRowThreads) {
      const int64_t e = 4 * g;
      for (int i = 0; i < 4; ++i) {
        if (e + i < V) {
          if (SB || a.dz_bf16) Zb[e + i] = 0;
          else Srow[e + i] = 0.0f;
        }
      }
    }
    if (tid == 0) a.rowval[gr] = bad_label ? NAN : 0.0f;
    if (SB || a.dz_bf16) zero_pad(Zb, V, tid);
    return;
  }

  const float *q = HEAD == HEAD_KL ? a.target + gr * V : nullptr;
  const bool q_vec = HEAD == HEAD_KL && (V % 4 == 0) &&
                     ((reinterpret_cast<uintptr_t>(a.target) & 15) == 0);

  // ---- statistics: max and sum exp (from the GEMM's block statistics, or a
  // pass over the logits), and for KL sum q, sum q log max(q, eps) ----
  float m = -INFINITY, s = 0.0f;
  float sq = 0.0f, sqlogq = 0.0f, sqx = 0.0f;
  if (a.stats) {
    const float2 *st = a.stats + lr * a.n_stat;
    for (int64_t t = tid; t < a.n_stat; t += kRowThreads) {
      const float2 p = st[t];
      lse_merge(m, s, p.x, p.y);
    }
    if (HEAD == HEAD_KL) {
      for (int64_t g = tid; g < ngroups; g += kRowThreads) {
        Load4 t = load_group(q, g, V, q_vec);
        const int64_t e = 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (e + i < V) {
            sq += t.v[i];
            // q = 0 adds exactly 0 whatever eps is [FusedLinearKLDivLoss
            // page, Details: 0 log 0 contributes 0]
            sqlogq += t.v[i] > 0.0f ? t.v[i] * __logf(fmaxf(t.v[i], a.eps)) : 0.0f;
          }
        }
      }
    }
  } else {
    for (int64_t g = tid; g < ngroups; g += kRowThreads) {
      Load4 x = sr.load(g, V);
      const int64_t e = 4 * g;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e + i < V) mx = fmaxf(mx, x.v[i]);
      if (mx > m) {
        s *= __expf(m - mx);
        m = mx;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e + i < V) s += __expf(x.v[i] - m);
      if (HEAD == HEAD_KL) {
        Load4 t = load_group(q, g, V, q_vec);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (e + i < V) {
            const float qi = t.v[i];
            sq += qi;
            sqlogq += qi > 0.0f ? qi * __logf(fmaxf(qi, a.eps)) : 0.0f;
            sqx += qi * x.v[i];
          }
        }
      }
    }
  }
  float s_label = 0.0f;
  // read before any write; with bf16 chunk logits the logits GEMM left the
  // fp32 logit of the label in label_logit (the per-row buffer this kernel
  // overwrites at the end)
  if (HEAD != HEAD_KL && tid == 0) s_label = a.label_logit ? a.label_logit[gr] : sr.at(y);

  // wave reduction, then across waves in a fixed order
  {
    float wm = wave_max(m);
    float ws = (m == -INFINITY) ? 0.0f : s * __expf(m - wm);
    ws = wave_sum(ws);
    if (lane == 0) {
      red[wave][0] = wm;
      red[wave][1] = ws;
    }
    if (HEAD == HEAD_KL) {
      float a0 = wave_sum(sq), a1 = wave_sum(sqlogq), a2 = wave_sum(sqx);
      if (lane == 0) {
        red[wave][2] = a0;
        red[wave][3] = a1;
        red[wave][4] = a2;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    float M = red[0][0], Ssum = red[0][1];
    float Q = 0.f, A = 0.f, B = 0.f;
    for (int w = 1; w < kRowWaves; ++w) lse_merge(M, Ssum, red[w][0], red[w][1]);
    if (HEAD == HEAD_KL)
      for (int w = 0; w < kRowWaves; ++w) {
        Q += red[w][2];
        A += red[w][3];
        B += red[w][4];
      }
    const float l = M + __logf(Ssum);
    if (HEAD == HEAD_SEL) a.rowval[gr] = s_label - l;            // log p(y)
    if (HEAD == HEAD_CE) a.rowval[gr] = l - s_label;             // -log p(y)
    if (HEAD == HEAD_KL && !a.stats) a.rowval[gr] = A - B + Q * l;  // sum_v q log q - q (S - l)
    if (HEAD == HEAD_PPO || HEAD == HEAD_CISPO) {
      // rho = p(y) / p_old(y), c = clip(rho, 1 - low, 1 + high); the row's
      // term L and k = dL / d log p(y) [frozen lm_head GRPO page, Summary:
      // the GRPO family on the selective log-prob]
      const float adv = a.weights ? a.weights[gr] : 1.0f;
      const float lp = s_label - l;
      const float rho = expf(lp - a.old_logprobs[gr]);
      const float c = fminf(fmaxf(rho, 1.0f - a.clip_low), 1.0f + a.clip_high);
      float L, k;
      if (HEAD == HEAD_PPO) {
        // -min(rho A, c A); the unclipped product takes ties and carries the
        // gradient -rho A, the clipped one is constant in log p(y)
        const float u = rho * adv, cl = c * adv;
        L = -fminf(u, cl);
        k = u <= cl ? -u : 0.0f;
      } else {
        L = -c * adv * lp;  // CISPO: c is a weight with no gradient
        k = -c * adv;
      }
      a.rowval[gr] = L;
      bcast[3] = k;
    }
    bcast[0] = l;
    bcast[1] = Q;
    bcast[2] = A;
  }
  __syncthreads();
  const float l = bcast[0];
  const float g = a.sc->g;
  float coef;  // dS = coef * (...) below
  float Qr = 0.f;
  if (HEAD == HEAD_KL) {
    coef = g * a.inv_tau;
    Qr = bcast[1];
  } else if (HEAD == HEAD_PPO || HEAD == HEAD_CISPO) {
    coef = g * bcast[3] * a.inv_tau;  // dS = g k (onehot - p)
  } else {
    // selective: dS = g w (onehot - p); cross-entropy: dS = g w (p - onehot)
    const float w = a.weights ? a.weights[gr] : 1.0f;
    coef = (HEAD == HEAD_CE ? -g : g) * w * a.inv_tau;
  }

  // ---- dZ = dS / tau, written in place (bf16 with non-temporal stores: the
  // next reader is the dX GEMM, after the whole chunk) ----
  // The bf16 dZ of element v goes to bytes [2v, 2v + 2) of the row. Over
  // fp32 logits those are float slots that an earlier strip (or this strip,
  // before the barrier) has already read; each strip's loads complete before
  // its barrier. Over bf16 logits each thread overwrites only the elements
  // it has just read, so no barrier is needed.
  float bq = 0.0f;  // KL with block statistics: sum q S, accumulated here
  for (int64_t base = 0; base < ngroups; base += kStrip) {
    Load4 xs[kUnroll];
    Load4 qs[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t g = base + u * kRowThreads + tid;
      if (g < ngroups) {
        xs[u] = sr.load_last(g, V);
        if (HEAD == HEAD_KL) qs[u] = load_group_last(q, g, V, q_vec);
      }
    }
    if constexpr (!SB) __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t g = base + u * kRowThreads + tid;
      if (g >= ngroups) continue;
      const int64_t e = 4 * g;
      float d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __expf(xs[u].v[i] - l);
        if (HEAD == HEAD_KL) {
          d[i] = coef * (Qr * p - qs[u].v[i]);
          if (e + i < V) bq += qs[u].v[i] * xs[u].v[i];
        } else {
          d[i] = coef * (((e + i) == y ? 1.0f : 0.0f) - p);
        }
      }
      if (SB || a.dz_bf16) {
        if (e + 4 <= V) {
          uint2 pk;
          pk.x = pack_bf16x2(d[0], d[1]);
          pk.y = pack_bf16x2(d[2], d[3]);
          __builtin_nontemporal_store(u32x2_t{pk.x, pk.y}, reinterpret_cast<u32x2_t *>(Zb + e));
        } else {
          for (int i = 0; i < 4; ++i)
            if (e + i < V) Zb[e + i] = f2bf(d[i]);
        }
      } else {
        if (e + 4 <= V) {
          *reinterpret_cast<float4 *>(Srow + e) = make_float4(d[0], d[1], d[2], d[3]);
        } else {
          for (int i = 0; i < 4; ++i)
            if (e + i < V) Srow[e + i] = d[i];
        }
      }
    }
  }
  if (HEAD == HEAD_KL && a.stats) {
    const float B = block_sum(bq, red, 5, lane, wave);
    if (tid == 0) a.rowval[gr] = bcast[2] - B + Qr * l;
  }
  // Every read of this row finished before the last strip's barrier.
  if (SB || a.dz_bf16) zero_pad(Zb, V, tid);
}

// Jensen-Shannon head [FusedLinearKLDivLoss page, Summary: the fused JSD
// loss, teacher side with its own projection]. One workgroup per token row.
// With lp = T - lse(T) (teacher), lq = S - lse(S) (model), p = e^lp,
// q = e^lq and lm = log((p + q) / 2):
//   JS_r = 1/2 sum_v p (lp - lm) + 1/2 sum_v q (lq - lm)
//   dS_v = g q_v (1/2 (lq_v - lm_v) - 1/2 sum_u q_u (lq_u - lm_u))
// (the derivative of JS in q_v is 1/2 (lq_v - lm_v); the softmax Jacobian
// subtracts its q-weighted mean). A first pass forms both sums — the second
// enters every dS_v — and a second pass writes dZ = dS / tau in place over S.
// lm is formed in the log domain, lm = max(lp, lq) + log((1 + e^-|lp - lq|) / 2),
// so no probability that underflows can make a term undefined.
struct JsdTerms {
  float q;        // model probability
  float gq;       // lq - lm
  float tp, tq;   // p (lp - lm), q (lq - lm)
};
__device__ __forceinline__ JsdTerms jsd_terms(float s, float t, float lse_s, float lse_t) {
  const float lq = s - lse_s, lp = t - lse_t;
  const float d = lp - lq;
  const float r = __expf(-fabsf(d));           // e^-|lp - lq|, in (0, 1]
  const float big = __expf(fmaxf(lp, lq));     // the larger of p and q
  const float l1 = __logf(0.5f + 0.5f * r);    // lm - max(lp, lq), in [-log 2, 0]
  const float p = d >= 0.f ? big : big * r;
  const float q = d >= 0.f ? big * r : big;
  const float gp = (d >= 0.f ? 0.f : d) - l1;  // lp - lm
  const float gq = (d >= 0.f ? -d : 0.f) - l1; // lq - lm
  return JsdTerms{q, gq, p * gp, q * gq};
}

template <bool SB>
__global__ __launch_bounds__(kRowThreads) void jsd_row_kernel(RowArgs a) {
  __shared__ float red[kRowWaves][8];
  __shared__ float bcast[8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t lr = blockIdx.x;
  const int64_t gr = a.row0 + lr;
  const int64_t V = a.V;
  const int64_t row_bytes = a.s_pitch * (SB ? 2 : 4);
  char *rowp = reinterpret_cast<char *>(a.S) + lr * row_bytes;
  const char *trowp = reinterpret_cast<const char *>(a.T) + lr * row_bytes;
  float *Srow = reinterpret_cast<float *>(rowp);                 // fp32 logits / dZ
  unsigned short *Zb = reinterpret_cast<unsigned short *>(rowp);  // bf16 dZ
  using P = decltype(SRow<SB>::p);
  SRow<SB> sr{reinterpret_cast<P>(rowp)}, tr{reinterpret_cast<P>(trowp)};
  const int64_t ngroups = (V + 3) / 4;

  const bool valid = !a.labels || a.labels[gr] != a.ignore_index;
  if (!valid) {
    for (int64_t g = tid; g < ngroups; g += kRowThreads) {
      const int64_t e = 4 * g;
      for (int i = 0; i < 4; ++i)
        if (e + i < V) {
          if (SB || a.dz_bf16) Zb[e + i] = 0;
          else Srow[e + i] = 0.0f;
        }
    }
    if (tid == 0) a.rowval[gr] = 0.0f;
    if (SB || a.dz_bf16) zero_pad(Zb, V, tid);
    return;
  }

  // ---- log-sum-exp of both rows: from the GEMMs' block statistics, or a pass
  float ms = -INFINITY, ss = 0.0f, mt = -INFINITY, st = 0.0f;
  if (a.stats) {
    const float2 *sa = a.stats + lr * a.n_stat;
    const float2 *sb = a.stats_t + lr * a.n_stat;
    for (int64_t t = tid; t < a.n_stat; t += kRowThreads) {
      const float2 x = sa[t], y = sb[t];
      lse_merge(ms, ss, x.x, x.y);
      lse_merge(mt, st, y.x, y.y);
    }
  } else {
    for (int64_t g = tid; g < ngroups; g += kRowThreads) {
      const Load4 x = sr.load(g, V), y = tr.load(g, V);
      const int64_t e = 4 * g;
      float mx = -INFINITY, my = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e + i < V) {
          mx = fmaxf(mx, x.v[i]);
          my = fmaxf(my, y.v[i]);
        }
      float sx = 0.0f, sy = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e + i < V) {
          sx += __expf(x.v[i] - mx);
          sy += __expf(y.v[i] - my);
        }
      lse_merge(ms, ss, mx, sx);
      lse_merge(mt, st, my, sy);
    }
  }
  {
    const float wms = wave_max(ms), wmt = wave_max(mt);
    const float wss = wave_sum(ms == -INFINITY ? 0.0f : ss * __expf(ms - wms));
    const float wst = wave_sum(mt == -INFINITY ? 0.0f : st * __expf(mt - wmt));
    if (lane == 0) {
      red[wave][0] = wms;
      red[wave][1] = wss;
      red[wave][2] = wmt;
      red[wave][3] = wst;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float m1 = red[0][0], s1 = red[0][1], m2 = red[0][2], s2 = red[0][3];
    for (int w = 1; w < kRowWaves; ++w) {
      lse_merge(m1, s1, red[w][0], red[w][1]);
      lse_merge(m2, s2, red[w][2], red[w][3]);
    }
    bcast[0] = m1 + __logf(s1);
    bcast[1] = m2 + __logf(s2);
  }
  __syncthreads();
  const float lse_s = bcast[0], lse_t = bcast[1];

  // ---- pass 1: both halves of the divergence
  float A = 0.0f, B = 0.0f;
  for (int64_t g = tid; g < ngroups; g += kRowThreads) {
    const Load4 x = sr.load(g, V), y = tr.load(g, V);
    const int64_t e = 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e + i < V) {
        const JsdTerms j = jsd_terms(x.v[i], y.v[i], lse_s, lse_t);
        A += j.tp;
        B += j.tq;
      }
  }
  A = wave_sum(A);
  B = wave_sum(B);
  if (lane == 0) {
    red[wave][4] = A;
    red[wave][5] = B;
  }
  __syncthreads();
  float Ar = 0.0f, Br = 0.0f;
  for (int w = 0; w < kRowWaves; ++w) {
    Ar += red[w][4];
    Br += red[w][5];
  }
  if (tid == 0) a.rowval[gr] = 0.5f * (Ar + Br);
  const float coef = a.sc->g * a.inv_tau;  // dZ = g (dJS/dS) / tau
  const float half_b = 0.5f * Br;

  // ---- pass 2: dZ in place, strip by strip (over fp32 logits every load of
  // a strip lands before its barrier, and the bf16 dZ of element v only
  // covers float slots of elements < v; over bf16 logits each thread
  // overwrites only what it has just read)
  for (int64_t base = 0; base < ngroups; base += kStrip) {
    Load4 xs[kUnroll], ys[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t g = base + u * kRowThreads + tid;
      if (g < ngroups) {
        xs[u] = sr.load_last(g, V);
        ys[u] = tr.load_last(g, V);
      }
    }
    if constexpr (!SB) __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t g = base + u * kRowThreads + tid;
      if (g >= ngroups) continue;
      const int64_t e = 4 * g;
      float d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const JsdTerms j = jsd_terms(xs[u].v[i], ys[u].v[i], lse_s, lse_t);
        d[i] = coef * j.q * (0.5f * j.gq - half_b);
      }
      if (SB || a.dz_bf16) {
        if (e + 4 <= V) {
          uint2 pk;
          pk.x = pack_bf16x2(d[0], d[1]);
          pk.y = pack_bf16x2(d[2], d[3]);
          __builtin_nontemporal_store(u32x2_t{pk.x, pk.y}, reinterpret_cast<u32x2_t *>(Zb + e));
        } else {
          for (int i = 0; i < 4; ++i)
            if (e + i < V) Zb[e + i] = f2bf(d[i]);
        }
      } else {
        if (e + 4 <= V) {
          *reinterpret_cast<float4 *>(Srow + e) = make_float4(d[0], d[1], d[2], d[3]);
        } else {
          for (int i = 0; i < 4; ++i)
            if (e + i < V) Srow[e + i] = d[i];
        }
      }
    }
  }
  if (SB || a.dz_bf16) zero_pad(Zb, V, tid);
}

__global__ __launch_bounds__(1024) void prep_kernel(const int64_t *labels, int64_t BT,
                                                    int64_t ignore_index, int head,
                                                    int reduction, int64_t V,
                                                    DevScalars *sc) {
  __shared__ long long part[1024];
  long long n = 0;
  if (labels) {
    for (int64_t r = threadIdx.x; r < BT; r += blockDim.x) n += (labels[r] != ignore_index);
  } else if (threadIdx.x == 0) {
    n = BT;
  }
  part[threadIdx.x] = n;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const long long nv = part[0];
    double g;
    if (nv == 0) g = 0.0;
    else if (reduction == 2) g = 1.0;                       // sum
    else if (reduction == 1 && (head == 0 || head == 3))
      g = 1.0 / (double(nv) * double(V));                   // KL and JSD mean
    else g = 1.0 / double(nv);                              // batchmean; selective mean
    sc->n_valid = nv;
    sc->g = float(g);
    sc->pad = 0.0f;
  }
}

__global__ __launch_bounds__(1024) void finalize_kernel(const float *rowval,
                                                        const float *weights, int64_t BT,
                                                        const DevScalars *sc, float *loss) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t r = threadIdx.x; r < BT; r += blockDim.x) {
    const double w = weights ? double(weights[r]) : 1.0;
    acc += w * double(rowval[r]);
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = float(double(sc->g) * part[0]);
}


// db column sums. Stage 1: block (x, y) sums rows [y R / kDbSplits,
// (y + 1) R / kDbSplits) of columns 256 x .. 256 x + 255 — each thread four
// adjacent columns read with one 8-byte (bf16) or 16-byte (fp32) load per
// row, the four row groups of the block added in a fixed order — into
// P[y][v]. Stage 2 adds the kDbSplits partials of each column in order, so
// the result does not depend on scheduling.
constexpr int kColX = 64, kColY = 4, kColW = 4;
template <bool BF16>
__global__ __launch_bounds__(kColX *kColY) void colsum_kernel(const void *dZ, int64_t ldz,
                                                              int64_t rows, int64_t V,
                                                              float *P) {
  __shared__ float part[kColY][kColX][kColW];
  const int tx = threadIdx.x, ty = threadIdx.y;
  const int64_t v = (int64_t(blockIdx.x) * kColX + tx) * kColW;
  const int64_t r0 = rows * blockIdx.y / kDbSplits, r1 = rows * (blockIdx.y + 1) / kDbSplits;
  float s[kColW] = {0.f, 0.f, 0.f, 0.f};
  if (v < V) {
    const bool whole = v + kColW <= V;
#pragma unroll 4
    for (int64_t r = r0 + ty; r < r1; r += kColY) {
      if (BF16) {
        const unsigned short *row = static_cast<const unsigned short *>(dZ) + r * ldz + v;
        if (whole) {
          const uint2 u = *reinterpret_cast<const uint2 *>(row);
          s[0] += __uint_as_float(u.x << 16);
          s[1] += __uint_as_float(u.x & 0xffff0000u);
          s[2] += __uint_as_float(u.y << 16);
          s[3] += __uint_as_float(u.y & 0xffff0000u);
        } else {
#pragma unroll
          for (int e = 0; e < kColW; ++e)
            if (v + e < V) s[e] += __uint_as_float(unsigned(row[e]) << 16);
        }
      } else {
        const float *row = static_cast<const float *>(dZ) + r * ldz + v;
        if (whole) {
          const float4 u = *reinterpret_cast<const float4 *>(row);
          s[0] += u.x;
          s[1] += u.y;
          s[2] += u.z;
          s[3] += u.w;
        } else {
#pragma unroll
          for (int e = 0; e < kColW; ++e)
            if (v + e < V) s[e] += row[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kColW; ++e) part[ty][tx][e] = s[e];
  __syncthreads();
  if (ty == 0 && v < V) {
    float* out = P + int64_t(blockIdx.y) * V;
#pragma unroll
    for (int e = 0; e < kColW; ++e) {
      float t = 0.f;
      for (int y = 0; y < kColY; ++y) t += part[y][tx][e];
      if (v + e < V) out[v + e] = t;
    }
  }
}

__global__ void colsum_reduce_kernel(const float *P, int64_t V, float *db, int accumulate) {
  const int64_t v = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (v >= V) return;
  float t = 0.f;
  for (int y = 0; y < kDbSplits; ++y) t += P[int64_t(y) * V + v];
  db[v] = accumulate ? db[v] + t : t;
}

__global__ void dx_reduce_kernel(const float *P, int64_t splits, int64_t M, int64_t N,
                                 void *dX, int64_t ldo, int out_bf16) {
  const int64_t n4 = N / 4;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= M * n4) return;
  const int64_t m = i / n4, c = (i % n4) * 4;
  float4 acc = *reinterpret_cast<const float4 *>(P + m * N + c);
  for (int64_t s = 1; s < splits; ++s) {
    float4 x = *reinterpret_cast<const float4 *>(P + (s * M + m) * N + c);
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  if (out_bf16) {
    uint2 pk;
    pk.x = pack_bf16x2(acc.x, acc.y);
    pk.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2 *>(static_cast<unsigned short *>(dX) + m * ldo + c) = pk;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(dX) + m * ldo + c) = acc;
  }
}

// bf16 transpose through LDS: a 64 x 64 tile per 256-thread workgroup,
// read and written along rows (each thread four elements of a row per
// pass); the LDS row pitch of 65 halfwords keeps the column reads spread
// over the banks. XT's columns from `rows` to the next multiple of 8 are
// written as zeros: the GEMM reads K in groups of 8, and a group that
// straddles the end must add nothing (the bytes there may hold anything,
// e.g. the dX partial sums that share the buffer).
constexpr int kTr = 64;
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const unsigned short *X,
                                                             int64_t ldx, int64_t rows,
                                                             int64_t cols, unsigned short *XT,
                                                             int64_t ldt) {
  __shared__ unsigned short tile[kTr][kTr + 1];
  const int64_t rows8 = (rows + 7) & ~int64_t(7);
  const int64_t r0 = int64_t(blockIdx.y) * kTr, c0 = int64_t(blockIdx.x) * kTr;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
  for (int i = ty; i < kTr; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? X[r * ldx + c] : (unsigned short)0;
  }
  __syncthreads();
  for (int i = ty; i < kTr; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows8) XT[c * ldt + r] = tile[tx][i];
  }
}

__global__ void fill_kernel(float *p, int64_t n, float v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

}  // namespace

void launch_prep(const int64_t *labels, int64_t BT, int64_t ignore_index, int head,
                 int reduction, int64_t V, DevScalars *sc, hipStream_t st) {
  hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(1024), 0, st, labels, BT, ignore_index,
                     head, reduction, V, sc);
}

template <bool SB>
void launch_row_t(const RowArgs &a, hipStream_t st) {
  if (a.head == HEAD_KL)
    hipLaunchKernelGGL((row_kernel<HEAD_KL, SB>), dim3(a.rows), dim3(kRowThreads), 0, st, a);
  else if (a.head == HEAD_SEL)
    hipLaunchKernelGGL((row_kernel<HEAD_SEL, SB>), dim3(a.rows), dim3(kRowThreads), 0, st, a);
  else if (a.head == HEAD_CE)
    hipLaunchKernelGGL((row_kernel<HEAD_CE, SB>), dim3(a.rows), dim3(kRowThreads), 0, st, a);
  else if (a.head == HEAD_JSD)
    hipLaunchKernelGGL(jsd_row_kernel<SB>, dim3(a.rows), dim3(kRowThreads), 0, st, a);
  else if (a.head == HEAD_PPO)
    hipLaunchKernelGGL((row_kernel<HEAD_PPO, SB>), dim3(a.rows), dim3(kRowThreads), 0, st, a);
  else if (a.head == HEAD_CISPO)
    hipLaunchKernelGGL((row_kernel<HEAD_CISPO, SB>), dim3(a.rows), dim3(kRowThreads), 0, st,
                       a);
}

void launch_row(const RowArgs &a, hipStream_t st) {
  if (a.rows <= 0) return;
  if (a.s_bf16) launch_row_t<true>(a, st);
  else launch_row_t<false>(a, st);
}

void launch_colsum(const void *dZ, int dz_bf16, int64_t ldz, int64_t rows, int64_t V,
                   float *P, float *db, int accumulate, hipStream_t st) {
  const int64_t blocks = (V + kColX * kColW - 1) / (kColX * kColW);
  if (dz_bf16)
    hipLaunchKernelGGL(colsum_kernel<true>, dim3(blocks, kDbSplits), dim3(kColX, kColY), 0,
                       st, dZ, ldz, rows, V, P);
  else
    hipLaunchKernelGGL(colsum_kernel<false>, dim3(blocks, kDbSplits), dim3(kColX, kColY), 0,
                       st, dZ, ldz, rows, V, P);
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((V + 255) / 256), dim3(256), 0, st, P, V, db,
                     accumulate);
}

void launch_dx_reduce(const float *P, int64_t splits, int64_t M, int64_t N, void *dX,
                      int64_t ldo, int out_bf16, hipStream_t st) {
  const int64_t n = M * (N / 4);
  if (n <= 0) return;
  const int threads = 256;
  hipLaunchKernelGGL(dx_reduce_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0,
                     st, P, splits, M, N, dX, ldo, out_bf16);
}

void launch_finalize(const float *rowval, const float *weights, int64_t BT,
                     const DevScalars *sc, float *loss, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, st, rowval, weights, BT, sc,
                     loss);
}

void launch_transpose_bf16(const void *X, int64_t ldx, int64_t rows, int64_t cols, void *XT,
                           int64_t ldt, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return;
  const int64_t rows8 = (rows + 7) & ~int64_t(7);  // ldt >= rows8
  const dim3 grid(unsigned((cols + kTr - 1) / kTr), unsigned((rows8 + kTr - 1) / kTr));
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, st,
                     static_cast<const unsigned short *>(X), ldx, rows, cols,
                     static_cast<unsigned short *>(XT), ldt);
}

void launch_fill(float *p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, st, p, n, v);
}

}  // namespace fll
