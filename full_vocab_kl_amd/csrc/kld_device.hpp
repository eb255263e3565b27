// Device-side building blocks shared by the libkld kernels (gfx950, wave64).
//
// Online per-row state for KL(p || q) over a vocabulary ("Qwen3.8-27B
// fidelity suite v5", opening paragraphs: the metric KL(BF16 || candidate);
// "Qwen3.8-27B Quantization Challenge", "How the references were made":
// f32 distributions over the full vocabulary).
//
// For a reference row a and candidate row b the state keeps, over the ids
// seen so far, the maxima ma, mb and, with offsets ra = ref(ma), rb = ref(mb)
// (ref(m) = m, or 0 while the side has seen only -inf):
//   sa = sum_j 2^((a_j - ra) L2E),  sb = sum_j 2^((b_j - rb) L2E),
//   t  = sum_j 2^((a_j - ra) L2E) ((a_j - ra) - (b_j - rb)).
// Then lse_a = ra + ln sa, lse_b = rb + ln sb and, exactly,
//   KL = t/sa + ln(sb/sa)
// (sum_j p_j (a_j - b_j) = t/sa + ra - rb, and the offsets cancel).  Taking
// every difference against the running maxima keeps t exact to f32 rounding
// of O(1) numbers even when the two rows carry large opposite offsets.  When
// a maximum moves by D the sums are rescaled by 2^(-D L2E) and t is rebased
// by sa * D (reference side: t -= sa D before the rescale; candidate side:
// t += sa D).  The argmax of each side is the running maximum plus its lowest
// id.  Partial states over disjoint id ranges merge associatively; merging in
// a fixed order keeps results bitwise reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kld {

constexpr float kL2E = 1.4426950408889634f;   // log2(e) rounded to f32
constexpr double kLn2 = 0.69314718055994530942;
constexpr int kNoId = 0x7fffffff;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kFltMax = 3.402823466e38f;

struct RowState {
  float ma, sa, t, mb, sb;
  int ia, ib;
};

__host__ __device__ inline RowState empty_state() {
  RowState s;
  s.ma = kNegInf; s.sa = 0.f; s.t = 0.f; s.mb = kNegInf; s.sb = 0.f;
  s.ia = kNoId; s.ib = kNoId;
  return s;
}

// Offset a side's differences are taken against: its maximum, or 0 while it
// has seen only -inf (so that -inf elements give 2^-inf = 0, never NaN).
__device__ __forceinline__ float ref_of(float m) { return m == kNegInf ? 0.f : m; }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Factor that moves a sum taken against offset ref(m_old) to ref(m_new).
__device__ __forceinline__ float rescale(float m_old, float m_new) {
  return m_old == kNegInf ? 0.f : exp2_fast((m_old - ref_of(m_new)) * kL2E);
}

__device__ __forceinline__ bool beats(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Bring state x to the offsets of maxima (ma, mb) >= x's own.
__device__ __forceinline__ void rebase(const RowState &x, float ma, float mb, float &sa, float &t,
                                       float &sb) {
  const float fa = rescale(x.ma, ma), fb = rescale(x.mb, mb);
  const float da = ref_of(ma) - ref_of(x.ma), db = ref_of(mb) - ref_of(x.mb);
  // x.sa == 0 means x saw no finite reference id: nothing to rebase
  const float tt = x.sa == 0.f ? x.t : fmaf(x.sa, db - da, x.t);
  sa = x.sa * fa;
  t = tt * fa;
  sb = x.sb * fb;
}

// Associative merge of two partial states over disjoint id ranges.
__device__ inline RowState merge(const RowState &x, const RowState &y) {
  RowState r;
  r.ma = fmaxf(x.ma, y.ma);
  r.mb = fmaxf(x.mb, y.mb);
  float xs, xt, xb, ys, yt, yb;
  rebase(x, r.ma, r.mb, xs, xt, xb);
  rebase(y, r.ma, r.mb, ys, yt, yb);
  r.sa = xs + ys;
  r.t = xt + yt;
  r.sb = xb + yb;
  r.ia = beats(x.ma, x.ia, y.ma, y.ia) ? x.ia : y.ia;
  r.ib = beats(x.mb, x.ib, y.mb, y.ib) ? x.ib : y.ib;
  return r;
}

__device__ __forceinline__ RowState shfl_xor_state(const RowState &s, int mask) {
  RowState o;
  o.ma = __shfl_xor(s.ma, mask); o.sa = __shfl_xor(s.sa, mask); o.t = __shfl_xor(s.t, mask);
  o.mb = __shfl_xor(s.mb, mask); o.sb = __shfl_xor(s.sb, mask);
  o.ia = __shfl_xor(s.ia, mask); o.ib = __shfl_xor(s.ib, mask);
  return o;
}

// Butterfly over the 64 lanes of a wave: every lane ends with the merge of
// all 64 states.  The pairing order is fixed, so the result is reproducible.
__device__ __forceinline__ RowState wave_merge(RowState s) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    RowState o = shfl_xor_state(s, m);
    // merge in lane order so both partners compute the identical value
    const bool lower = (threadIdx.x & m) == 0;
    s = lower ? merge(s, o) : merge(o, s);
  }
  return s;
}

// Per-position results from a complete state (f64 arithmetic on the f32 sums).
struct RowResult {
  float kl, lse_a, lse_b;
  int ia, ib;
};

__device__ inline RowResult finish(const RowState &s) {
  RowResult r;
  const double sa = (double)s.sa, sb = (double)s.sb, t = (double)s.t;
  double kl;
  if (isnan(sa) || isnan(sb) || !(sa > 0.0) || !(sb > 0.0)) {
    kl = __builtin_nan("");
  } else if (isnan(t)) {
    // t turns NaN only through 0 * inf: a finite reference logit whose
    // weight underflowed met a -inf candidate logit, so q = 0 where p > 0.
    kl = __builtin_inf();
  } else {
    kl = t / sa + log(sb / sa);
    if (kl < 0.0) kl = 0.0;   // rounding below the true value (KL >= 0)
  }
  r.kl = kl == 0.0 ? 0.0f : (float)kl;   // canonical +0
  r.lse_a = (float)((double)ref_of(s.ma) + log(sa));
  r.lse_b = (float)((double)ref_of(s.mb) + log(sb));
  r.ia = s.ia == kNoId ? 0 : s.ia;   // all ids -inf: every id ties, the lowest is 0
  r.ib = s.ib == kNoId ? 0 : s.ib;
  return r;
}

// ---- f64 accumulation of partial states -------------------------------------
// The final merges over splits or vocabulary tiles run in f64: partial sums
// arrive in f32, the running sums, rebase factors and t are kept in f64, so
// the merge order adds no rounding visible at the f32 result.
struct RowStateD {
  float ma, mb;
  double sa, t, sb;
  int ia, ib;
};

__device__ inline RowStateD empty_state_d() {
  RowStateD s;
  s.ma = kNegInf; s.mb = kNegInf; s.sa = 0.0; s.t = 0.0; s.sb = 0.0;
  s.ia = kNoId; s.ib = kNoId;
  return s;
}

__device__ inline RowStateD to_d(const RowState &x) {
  RowStateD s;
  s.ma = x.ma; s.mb = x.mb; s.sa = x.sa; s.t = x.t; s.sb = x.sb; s.ia = x.ia; s.ib = x.ib;
  return s;
}

// exp(m_old - ref(m_new)) in f64: the factor that moves a sum to the new offset.
__device__ __forceinline__ double rescale_d(float m_old, float m_new) {
  return m_old == kNegInf ? 0.0 : exp((double)m_old - (double)ref_of(m_new));
}

__device__ inline void rebase_d(const RowStateD &x, float ma, float mb, double &sa, double &t,
                                double &sb) {
  const double fa = rescale_d(x.ma, ma), fb = rescale_d(x.mb, mb);
  const double da = (double)ref_of(ma) - (double)ref_of(x.ma);
  const double db = (double)ref_of(mb) - (double)ref_of(x.mb);
  const double tt = x.sa == 0.0 ? x.t : fma(x.sa, db - da, x.t);
  sa = x.sa * fa;
  t = tt * fa;
  sb = x.sb * fb;
}

__device__ inline RowStateD merge_d(const RowStateD &x, const RowStateD &y) {
  RowStateD r;
  r.ma = fmaxf(x.ma, y.ma);
  r.mb = fmaxf(x.mb, y.mb);
  double xs, xt, xb, ys, yt, yb;
  rebase_d(x, r.ma, r.mb, xs, xt, xb);
  rebase_d(y, r.ma, r.mb, ys, yt, yb);
  r.sa = xs + ys;
  r.t = xt + yt;
  r.sb = xb + yb;
  r.ia = beats(x.ma, x.ia, y.ma, y.ia) ? x.ia : y.ia;
  r.ib = beats(x.mb, x.ib, y.mb, y.ib) ? x.ib : y.ib;
  return r;
}

__device__ inline RowResult finish_d(const RowStateD &s, double *lse_a = nullptr,
                                     double *lse_b = nullptr) {
  RowResult r;
  double kl;
  if (isnan(s.sa) || isnan(s.sb) || !(s.sa > 0.0) || !(s.sb > 0.0)) {
    kl = __builtin_nan("");
  } else if (isnan(s.t)) {
    kl = __builtin_inf();   // 0 * inf: p > 0 where q = 0 (see finish)
  } else {
    kl = s.t / s.sa + log(s.sb / s.sa);
    if (kl < 0.0) kl = 0.0;
  }
  const double la = (double)ref_of(s.ma) + log(s.sa), lb = (double)ref_of(s.mb) + log(s.sb);
  if (lse_a) *lse_a = la;
  if (lse_b) *lse_b = lb;
  r.kl = kl == 0.0 ? 0.0f : (float)kl;
  r.lse_a = (float)la;
  r.lse_b = (float)lb;
  r.ia = s.ia == kNoId ? 0 : s.ia;
  r.ib = s.ib == kNoId ? 0 : s.ib;
  return r;
}

// ---- top-k keys ------------------------------------------------------------
// A 64-bit key per (value, id): order-preserving bits of the value in the high
// word (-0 folded onto +0), the complemented id in the low word, so a larger
// key means a larger value, and among equal values the lower id.
__device__ __forceinline__ uint32_t ord32(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t topk_key(float x, int id) {
  return ((uint64_t)ord32(x) << 32) | (uint64_t)(~(uint32_t)id);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_id(uint64_t k) { return (int)(~(uint32_t)k); }

// Block-wide bitonic sort, descending, of buf[0, n) (LDS), n a power of two;
// NT = threads in the block.  Every thread of the block must call it.
template <int NT>
__device__ void bitonic_desc(uint64_t *buf, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += NT) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t a = buf[i], b = buf[p];
          const bool first_half = (i & k) == 0;
          if (first_half ? (a < b) : (a > b)) { buf[i] = b; buf[p] = a; }
        }
      }
      __syncthreads();
    }
  }
}


// Descending bitonic sort of one value per lane across the 64 lanes of a wave
// (lane 0 ends with the largest).
__device__ __forceinline__ float wave_sort_desc(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float o = __shfl_xor(x, j);
      const bool desc = (lane & k) == 0, lower = (lane & j) == 0;
      x = (desc == lower) ? fmaxf(x, o) : fminf(x, o);
    }
  return x;
}
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = __shfl_xor(x, j);
      const bool desc = (lane & k) == 0, lower = (lane & j) == 0;
      x = (desc == lower) ? (o > x ? o : x) : (o < x ? o : x);
    }
  return x;
}

// Block-wide (256 threads) selection of the R largest nonzero keys among the
// K keys each thread holds (0 = no key; nonzero keys are distinct).  Radix
// select, 8 bits per pass from the top: a 256-bin LDS histogram of the keys
// that match the digits fixed so far, and wave 0 finds the bin that holds the
// wanted rank; the passes stop early once that bin holds exactly the keys
// still wanted (then every key at or above it is selected and the smallest of
// them is the R-th).  Returns the R-th largest key, or 0 when fewer than R keys
// are nonzero; stores the selected keys (every nonzero key when fewer than R)
// in top[0..R-1], zero-filled, in no particular order.  LDS scratch: hist[256],
// sh[6] 8-byte aligned; every thread of the block must call it.
template <int K, int R = 64>
__device__ __forceinline__ uint64_t block_select_top(const uint64_t (&k)[K], uint64_t *top,
                                                     uint32_t *hist, uint32_t *sh) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  uint32_t need = R;
  int shift = 64;        // keys are selected by their bits at and above `shift`
  bool found = true;
  for (int pass = 0; pass < 8; ++pass) {
    const int sh8 = 56 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < K; ++q) {
      const uint64_t x = k[q];
      if (x != 0ull && (pass == 0 || (x >> (sh8 + 8)) == (prefix >> (sh8 + 8))))
        atomicAdd(&hist[(x >> sh8) & 255], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4 l .. 4 l + 3; count the keys in higher bins
      uint32_t c[4], s4 = 0;
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) { c[bq] = hist[4 * tid + bq]; s4 += c[bq]; }
      uint32_t suf = s4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(suf, o);
        if (tid + o < 64) suf += t;
      }
      uint32_t above = suf - s4;
      int bin = -1;
      uint32_t left = 0, cnt = 0;
#pragma unroll
      for (int bq = 3; bq >= 0; --bq) {
        if (bin < 0 && above < need && above + c[bq] >= need) {
          bin = 4 * tid + bq; left = need - above; cnt = c[bq];
        }
        above += c[bq];
      }
      const uint64_t m = __ballot(bin >= 0);
      if (m == 0ull) {
        if (tid == 0) sh[0] = 0xffffffffu;
      } else {
        const int src = __ffsll((long long)m) - 1;
        const int bb = __shfl(bin, src);
        const uint32_t ll = __shfl(left, src), cc = __shfl(cnt, src);
        if (tid == 0) { sh[0] = (uint32_t)bb; sh[1] = ll; sh[3] = cc; }
      }
    }
    __syncthreads();
    const uint32_t dd = sh[0];
    need = sh[1];
    const uint32_t bucket = sh[3];
    __syncthreads();
    if (dd == 0xffffffffu) { found = false; break; }
    prefix |= (uint64_t)dd << sh8;
    shift = sh8;
    if (bucket == need) break;   // every key of the bucket is selected: the set is fixed
  }
  // Selected: the keys whose bits at and above `shift` reach the prefix (all
  // nonzero keys when fewer than R exist).  T = the smallest selected key.
  if (tid == 0) { sh[2] = 0; sh[4] = 0xffffffffu; sh[5] = 0xffffffffu; }
  __syncthreads();
  unsigned long long *tmin = reinterpret_cast<unsigned long long *>(sh + 4);
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const uint64_t x = k[q];
    if (x != 0ull && (!found || (shift == 64 ? true : (x >> shift) >= (prefix >> shift)))) {
      top[atomicAdd(&sh[2], 1u)] = x;
      atomicMin(tmin, (unsigned long long)x);
    }
  }
  __syncthreads();
  const uint32_t cnt = sh[2];
  const uint64_t T = found ? (uint64_t)*tmin : 0ull;
  for (uint32_t i = cnt + tid; i < R; i += 256) top[i] = 0ull;
  __syncthreads();
  return T;
}

template <int K>
__device__ __forceinline__ uint64_t block_select64(const uint64_t (&k)[K], uint64_t *top,
                                                   uint32_t *hist, uint32_t *sh) {
  return block_select_top<K, 64>(k, top, hist, sh);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

// Round f32 to fp16 bits, nearest-even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace kld
