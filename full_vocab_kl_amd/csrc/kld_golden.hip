// Golden records and the 513-cell score ("Qwen3.8-27B Quantization
// Challenge": "Golden distributions", "The score").
//
// golden_export_kernel: one block per reference row.  One streaming pass keeps
// the online log-sum-exp state and the entropy sum (f32 per round, f64 across
// rounds) and filters the 512 largest (value, id) keys through an LDS
// candidate buffer behind a threshold key (first from a sample of the row,
// then the 512th best so far whenever the buffer nears full and is cut).  The
// 512 are sorted by a block bitonic network and written with their f32
// log-probs.  The probability of every id outside the 512 is summed directly
// in the same pass -- ids below the threshold as they stream by, candidates
// as cuts drop them -- so a tiny tail mass keeps its relative accuracy
// instead of coming out of 1 - sum of the listed probabilities.
//
// coarse_partial_kernel + coarse_finalize_kernel: a candidate row is split
// into ranges of at most 131,072 ids, one block each.  A block sets the
// record's listed ids of its range in an LDS bitmap and streams the range
// once, keeping the online log-sum-exp state and, separately, the mass of the
// unlisted ids (the candidate's tail cell, summed directly so that a tiny
// tail keeps its relative accuracy).  The finalize kernel merges a row's
// ranges in order (f64), gathers the 512 listed logits and sums the cells in
// f64 in a fixed order, one wave per row.
#include <type_traits>

#include "kld.h"
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int GT = 256;                  // threads per block
constexpr int GE = 8;                    // consecutive elements per thread and round
constexpr int GROUND = GT * GE;          // elements per round
constexpr int GK = KLD_GOLDEN_TOPK;      // listed ids per record
constexpr int GCAP = 4096;               // candidate keys per block
static_assert(GCAP % GT == 0 && GCAP - GROUND >= GK, "buffer holds the kept keys plus a round");

__device__ __forceinline__ float ld_f32(const float *r, int64_t j) { return r[j]; }
__device__ __forceinline__ float ld_f32(const uint16_t *r, int64_t j) { return bf16_to_f32(r[j]); }

// The GE elements at pos (a multiple of GE) of a row; elements at or past hi
// read as -inf.  Aligned rows take 16-byte loads when the run is in range.
template <typename T, bool ALIGNED>
__device__ __forceinline__ void load_run(const T *__restrict__ row, int64_t pos, int64_t hi,
                                         float (&x)[GE]) {
  if (ALIGNED && pos + GE <= hi) {
    if constexpr (sizeof(T) == 4) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(row + pos);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(row + pos + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
    } else {
      const u32x4 q = *reinterpret_cast<const u32x4 *>(row + pos);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(q[e] << 16);
        x[2 * e + 1] = __uint_as_float(q[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < GE; ++e) x[e] = pos + e < hi ? ld_f32(row, pos + e) : kNegInf;
  }
}

// Online state of one thread: maximum m, S = sum e^(z - m), U = sum e^(z - m) (z - m)
// (the entropy sum), W = sum e^(z - m) over a subset (the unlisted ids).
struct LseState {
  float m;
  double s, u, w;
};

__device__ __forceinline__ LseState lse_merge(const LseState &a, const LseState &b) {
  if (b.m == kNegInf) return a;
  if (a.m == kNegInf) return b;
  const float m = fmaxf(a.m, b.m);
  const double fa = exp((double)a.m - (double)m), fb = exp((double)b.m - (double)m);
  LseState r;
  r.m = m;
  r.s = a.s * fa + b.s * fb;
  // (z - m) = (z - a.m) + (a.m - m)
  r.u = fa * (a.u + ((double)a.m - (double)m) * a.s) + fb * (b.u + ((double)b.m - (double)m) * b.s);
  r.w = a.w * fa + b.w * fb;
  return r;
}

// Block-wide merge (fixed butterfly, then the four waves in order); every
// thread gets the result.
__device__ LseState lse_block(LseState st, LseState *xw) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    LseState q;
    q.m = __shfl_xor(st.m, o);
    q.s = __shfl_xor(st.s, o);
    q.u = __shfl_xor(st.u, o);
    q.w = __shfl_xor(st.w, o);
    st = (threadIdx.x & o) ? lse_merge(q, st) : lse_merge(st, q);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) xw[wave] = st;
  __syncthreads();
  LseState r = xw[0];
#pragma unroll
  for (int w = 1; w < GT / 64; ++w) r = lse_merge(r, xw[w]);
  __syncthreads();
  return r;
}

// Fold one round's f32 partial sums (relative to m) into the thread's state,
// after raising m to the round maximum bm when it grew.
__device__ __forceinline__ void raise_max(LseState &st, float bm) {
  if (bm > st.m) {
    if (st.m != kNegInf) {
      const double f = exp((double)st.m - (double)bm);
      st.u = f * (st.u + ((double)st.m - (double)bm) * st.s);
      st.s *= f;
      st.w *= f;
    }
    st.m = bm;
  }
}

struct GoldenShared {
  uint64_t buf[GCAP];
  uint64_t top[GK];
  uint32_t hist[256];
  LseState xw[GT / 64];
  uint64_t thr;
  int cnt;
  int cut;                      // the buffer has been cut to its GK best
  int kept;                     // keys kept by a cut
  int wcnt[GT / 64];            // per wave: keys at or above a trial prefix
  uint32_t wthr[GT / 64];       // per wave: sampled threshold value
  __align__(8) uint32_t sel[6];
};

// Cut the candidate buffer to its GK best keys (distinct; 0 = none) and make
// the GK-th the threshold; the mass of every dropped key is added to the
// thread's unlisted sum (st.w), so the tail is summed directly in one pass.  The GK-th key is found bit by bit from the top:
// a bit is kept if at least GK keys reach the prefix (each thread counts its
// keys, a butterfly sums a wave's counts, LDS the four waves').  No
// histogram: keys that share their high bits would pile onto one bin.
__device__ void golden_compact(GoldenShared &sh, LseState &st) {
  uint64_t k[GCAP / GT];
  const int cnt = sh.cnt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < GCAP / GT; ++q) {
    const int e = q * GT + (int)threadIdx.x;
    k[q] = e < cnt ? sh.buf[e] : 0ull;
  }
  uint64_t t = 0;   // stays 0 when fewer than GK keys exist: all are kept
  if (cnt > GK) {
    for (int b = 63; b >= 0; --b) {
      const uint64_t c = t | (1ull << b);
      int n = 0;
#pragma unroll
      for (int q = 0; q < GCAP / GT; ++q) n += k[q] >= c ? 1 : 0;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o);
      if (lane == 0) sh.wcnt[wave] = n;
      __syncthreads();
      int tot = 0;
#pragma unroll
      for (int w = 0; w < GT / 64; ++w) tot += sh.wcnt[w];
      __syncthreads();
      if (tot >= GK) t = c;
    }
  }
  // the dropped keys' mass (each key is in one thread's slice)
#pragma unroll
  for (int q = 0; q < GCAP / GT; ++q) {
    if (k[q] != 0ull && k[q] < t) {
      const float x = key_value(k[q]);
      if (x != kNegInf) {   // (a -inf logit has no mass)
        raise_max(st, x);
        st.w += exp((double)x - (double)st.m);
      }
    }
  }
  // the kept keys (exactly GK when t > 0) in any order, then zeros
  if (threadIdx.x == 0) sh.kept = 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < GCAP / GT; ++q)
    if (k[q] != 0ull && k[q] >= t) sh.top[atomicAdd(&sh.kept, 1)] = k[q];
  __syncthreads();
  const int kept = sh.kept;
  for (int i = kept + (int)threadIdx.x; i < GK; i += GT) sh.top[i] = 0ull;
  for (int i = (int)threadIdx.x; i < kept; i += GT) sh.buf[i] = sh.top[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    sh.cnt = kept;
    // GK keys at or above t exist, so no other key below t can be among
    // the GK best (keys are distinct)
    if (t != 0ull) sh.thr = t;
  }
  __syncthreads();
}

template <typename T, bool ALIGNED>
__global__ __launch_bounds__(GT) void golden_export_kernel(
    const T *__restrict__ logits, int64_t ld, int64_t v, const int32_t *__restrict__ target,
    int32_t *__restrict__ ids, float *__restrict__ lp, float *__restrict__ rec) {
  __shared__ GoldenShared sh;
  const int64_t row = blockIdx.x;
  const T *r = logits + row * ld;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Starting threshold from a sample of the row: 16 evenly spread ids per
  // thread; each wave takes the value of the 5th best key of its 1,024 (a
  // bit search on the top 32 key bits, counts summed over the lanes) and the
  // block the smallest of the four.  Keys below it are never appended, so
  // the buffer rarely needs cutting before the end.  If fewer than GK keys
  // reach it, the candidates are collected again from no threshold (below).
  {
    uint64_t sk[GCAP / GT];
#pragma unroll
    for (int q = 0; q < GCAP / GT; ++q) {
      const int64_t p = ((int64_t)(q * GT + (int)threadIdx.x) * v) / GCAP;
      const float x = ld_f32(r, p);
      sk[q] = x == x ? topk_key(x, (int)p) : 0ull;
    }
    uint32_t pre = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t c = pre | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < GCAP / GT; ++q) cnt += (uint32_t)(sk[q] >> 32) >= c ? 1 : 0;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
      if (cnt >= 5) pre = c;
    }
    if (lane == 0) sh.wthr[wave] = pre;
  }
  if (threadIdx.x == 0) sh.cnt = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = sh.wthr[0];
    for (int w = 1; w < GT / 64; ++w) m = sh.wthr[w] < m ? sh.wthr[w] : m;
    sh.thr = (uint64_t)m << 32;   // a key with that value and any id reaches it
    sh.cut = 0;
  }
  __syncthreads();
  const uint64_t thr0 = sh.thr;

  LseState st{kNegInf, 0.0, 0.0, 0.0};
  const int64_t rounds = (v + GROUND - 1) / GROUND;
  // each round's elements are loaded one round ahead, so the loads are in
  // flight while the previous round is processed (and waits at its barrier)
  float xn[GE];
  load_run<T, ALIGNED>(r, (int64_t)threadIdx.x * GE, v, xn);
  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t pos = rd * GROUND + (int64_t)threadIdx.x * GE;
    float x[GE];
#pragma unroll
    for (int e = 0; e < GE; ++e) x[e] = xn[e];
    if (rd + 1 < rounds) load_run<T, ALIGNED>(r, pos + GROUND, v, xn);
    float bm = kNegInf;
#pragma unroll
    for (int e = 0; e < GE; ++e) bm = fmaxf(bm, x[e]);
    raise_max(st, bm);
    float ps = 0.f, pu = 0.f, pw = 0.f;
    float w[GE];
#pragma unroll
    for (int e = 0; e < GE; ++e) w[e] = 0.f;
    if (st.m != kNegInf) {
#pragma unroll
      for (int e = 0; e < GE; ++e) {
        const float d = x[e] - st.m;
        w[e] = exp2_fast(d * kL2E);
        ps += w[e];
        pu = fmaf(w[e], fmaxf(d, -kFltMax), pu);   // a -inf logit (w = 0) adds exactly 0
      }
    }
    // candidates: keys above the threshold (NaN logits are never listed);
    // the rest are outside the GK best, their mass goes to the tail
    const uint64_t th = sh.thr;
#pragma unroll
    for (int e = 0; e < GE; ++e) {
      if (pos + e < v && x[e] == x[e]) {
        const uint64_t key = topk_key(x[e], (int)(pos + e));
        if (key > th) sh.buf[atomicAdd(&sh.cnt, 1)] = key;
        else pw += w[e];
      }
    }
    st.s += (double)ps;
    st.u += (double)pu;
    st.w += (double)pw;
    __syncthreads();
    if (sh.cnt > GCAP - GROUND) {
      golden_compact(sh, st);
      if (threadIdx.x == 0) sh.cut = 1;
      __syncthreads();
    }
  }
  // Fewer than GK keys reached the sampled threshold and no cut raised it:
  // the GK best may include keys below it, so collect the candidates (and
  // the tail) again from no threshold; the other sums are complete.
  if (thr0 != 0ull && sh.cut == 0 && sh.cnt < GK) {
    __syncthreads();
    if (threadIdx.x == 0) { sh.cnt = 0; sh.thr = 0ull; }
    st.w = 0.0;
    __syncthreads();
    for (int64_t rd = 0; rd < rounds; ++rd) {
      const int64_t pos = rd * GROUND + (int64_t)threadIdx.x * GE;
      float x[GE];
      load_run<T, ALIGNED>(r, pos, v, x);
      const uint64_t th = sh.thr;
      float pw = 0.f;
#pragma unroll
      for (int e = 0; e < GE; ++e) {
        if (pos + e < v && x[e] == x[e]) {
          const uint64_t key = topk_key(x[e], (int)(pos + e));
          if (key > th) sh.buf[atomicAdd(&sh.cnt, 1)] = key;
          else if (st.m != kNegInf) pw += exp2_fast((x[e] - st.m) * kL2E);
        }
      }
      st.w += (double)pw;
      __syncthreads();
      if (sh.cnt > GCAP - GROUND) golden_compact(sh, st);
    }
  }
  golden_compact(sh, st);
  // the GK best keys, sorted descending (zero keys -- fewer than GK valid
  // ids -- sort last)
  __syncthreads();
  bitonic_desc<GT>(sh.top, GK);
  const LseState tot = lse_block(st, sh.xw);
  const double ls = log(tot.s);
  const double lse = (double)tot.m + ls;
  for (int i = (int)threadIdx.x; i < GK; i += GT) {
    const uint64_t key = sh.top[i];
    ids[row * GK + i] = key ? key_id(key) : 0;
    lp[row * GK + i] = key ? (float)((double)key_value(key) - lse) : kNegInf;
  }
  const double tail = tot.w / tot.s;   // every id outside the GK listed ones, summed directly
  if (threadIdx.x == 0) {
    float nll = __builtin_nanf("");
    if (target) {
      const int32_t tg = target[row];
      if (tg >= 0 && (int64_t)tg < v) nll = (float)(lse - (double)ld_f32(r, tg));
    }
    rec[row * 3 + 0] = nll;
    rec[row * 3 + 1] = (float)(ls - tot.u / tot.s);   // H = ln S - U / S
    rec[row * 3 + 2] = (float)tail;
  }
}

constexpr int CMAXW = 4096;              // bitmap words per range: 131,072 ids (16 KB)

// The VEC elements at pos of a row (pos a multiple of VEC); past hi: -inf.
template <typename T, int VEC, bool ALIGNED>
__device__ __forceinline__ void load_vecn(const T *__restrict__ row, int64_t pos, int64_t hi,
                                          float (&x)[VEC]) {
  if (ALIGNED && pos + VEC <= hi) {
    if constexpr (sizeof(T) == 4) {
      const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + pos));
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = q[e];
    } else {
      const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + pos));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(q[e] << 16);
        x[2 * e + 1] = __uint_as_float(q[e] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) x[e] = pos + e < hi ? ld_f32(row, pos + e) : kNegInf;
  }
}

template <typename T, int VEC, int U, bool ALIGNED>
__global__ __launch_bounds__(GT) void coarse_partial_kernel(
    const T *__restrict__ cand, int64_t ld, int64_t v, int64_t chunk, int splits,
    const int32_t *__restrict__ ids, LseState *__restrict__ part) {
  __shared__ uint32_t listed[CMAXW];   // the record's ids in [lo, hi), bit (id - lo)
  __shared__ LseState xw[GT / 64];
  const int64_t row = blockIdx.x / splits;
  const int split = (int)(blockIdx.x % splits);
  const int64_t lo = (int64_t)split * chunk;
  const int64_t hi = lo + chunk < v ? lo + chunk : v;
  const T *r = cand + row * ld;
  const int nw = (int)((hi - lo + 31) >> 5);   // bitmap words of this range
  for (int w = (int)threadIdx.x; w < nw; w += GT) listed[w] = 0u;
  __syncthreads();
  for (int i = (int)threadIdx.x; i < GK; i += GT) {
    const int32_t id = ids[row * GK + i];
    if ((int64_t)id >= lo && (int64_t)id < hi) {
      const int64_t o = id - lo;
      atomicOr(&listed[o >> 5], 1u << (o & 31));
    }
  }
  __syncthreads();

  constexpr int64_t kStride = (int64_t)GT * VEC;
  LseState st{kNegInf, 0.0, 0.0, 0.0};
  const int64_t rounds = (hi - lo + kStride * U - 1) / (kStride * U);
  // Aligned rows: the whole vectors of [lo, hi) are read through a buffer
  // resource (vectors past it read 0 and touch no memory), so a round's loads
  // carry no branch and are all in flight together; elements past hi become
  // -inf and a vector straddling hi is completed element by element.
  const int len = (int)(hi - lo);   // a range spans at most 131,072 ids
  const int nvec = len / VEC * VEC;
  __amdgpu_buffer_rsrc_t rs;
  if constexpr (ALIGNED)
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(r + lo), (short)0,
                                           nvec * (int)sizeof(T), 0x00020000);
  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t base = lo + rd * kStride * U + (int64_t)threadIdx.x * VEC;
    float x[U][VEC];
    if constexpr (ALIGNED) {
      typedef typename std::conditional<sizeof(T) == 4, f32x4, u32x4>::type Raw;
      Raw q[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        q[u] = __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(
                   rs, (int)(base + u * kStride - lo) * (int)sizeof(T), 0, 2 /* streaming */));
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          if constexpr (sizeof(T) == 4) x[u][e] = q[u][e];
          else x[u][e] = __uint_as_float((e & 1) ? (q[u][e >> 1] & 0xffff0000u) : (q[u][e >> 1] << 16));
        }
        const int64_t p = base + u * kStride;
        if (p + VEC > hi) {   // the last vectors of the range only
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            x[u][e] = p + e < hi ? (p - lo >= nvec ? ld_f32(r, p + e) : x[u][e]) : kNegInf;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) load_vecn<T, VEC, false>(r, base + u * kStride, hi, x[u]);
    }
    float bm = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) bm = fmaxf(bm, x[u][e]);
    raise_max(st, bm);
    float ps = 0.f, pw = 0.f;
    if (st.m != kNegInf) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // offsets from lo are multiples of VEC, so the vector's flags sit in one word
        const int64_t o = base + u * kStride - lo;
        const uint32_t flags = o < hi - lo ? listed[o >> 5] >> (o & 31) : 0u;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float w = exp2_fast((x[u][e] - st.m) * kL2E);
          ps += w;
          if (!((flags >> e) & 1u)) pw += w;
        }
      }
    }
    st.s += (double)ps;
    st.w += (double)pw;
  }
  const LseState tot = lse_block(st, xw);
  if (threadIdx.x == 0) part[row * splits + split] = tot;
}

__global__ __launch_bounds__(GT) void coarse_finalize_kernel(
    const LseState *__restrict__ part, int splits, int64_t n, const void *__restrict__ cand,
    int dtype, int64_t ld, int64_t v, const int32_t *__restrict__ ids,
    const float *__restrict__ lp, const float *__restrict__ rec, float *__restrict__ kl) {
  const int64_t row = (int64_t)blockIdx.x * (GT / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  LseState tot = part[row * splits];
  for (int i = 1; i < splits; ++i) tot = lse_merge(tot, part[row * splits + i]);
  const double lse = (double)tot.m + log(tot.s);
  const double q_t = tot.w / tot.s;
  double acc = 0.0;
  int flags = 0;   // 1: an id outside [0, v); 2: p > 0 against q = 0
  for (int i = lane; i < GK; i += 64) {
    const int32_t id = ids[row * GK + i];
    if (id < 0 || (int64_t)id >= v) { flags |= 1; continue; }
    const double l = (double)lp[row * GK + i];
    const double p = exp(l);
    if (p == 0.0) continue;
    const float z = dtype == 0 ? reinterpret_cast<const float *>(cand)[row * ld + id]
                               : bf16_to_f32(reinterpret_cast<const uint16_t *>(cand)[row * ld + id]);
    if (z == kNegInf) { flags |= 2; continue; }
    acc += p * (l - ((double)z - lse));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    acc += __shfl_xor(acc, o);
    flags |= __shfl_xor(flags, o);
  }
  if (lane == 0) {
    const double p_t = (double)rec[row * 3 + 2];
    if (p_t > 0.0) {
      if (q_t == 0.0) flags |= 2;
      else acc += p_t * (log(p_t) - log(q_t));
    }
    const bool nan_in = !(tot.s > 0.0) || tot.s != tot.s || tot.m != tot.m ||
                        tot.m == __builtin_huge_valf();
    kl[row] = (flags & 1) || nan_in ? __builtin_nanf("") : (flags & 2) ? __builtin_huge_valf()
                                                                     : (float)acc;
  }
}

}  // namespace

hipError_t launch_golden_export(const void *logits, int dtype, int64_t n, int64_t v, int64_t ld,
                                bool aligned, const int32_t *target, int32_t *ids, float *lp,
                                float *rec, hipStream_t stream) {
  const dim3 grid((unsigned)n), block(GT);
  if (dtype == 0) {
    if (aligned)
      hipLaunchKernelGGL((golden_export_kernel<float, true>), grid, block, 0, stream,
                         (const float *)logits, ld, v, target, ids, lp, rec);
    else
      hipLaunchKernelGGL((golden_export_kernel<float, false>), grid, block, 0, stream,
                         (const float *)logits, ld, v, target, ids, lp, rec);
  } else {
    if (aligned)
      hipLaunchKernelGGL((golden_export_kernel<uint16_t, true>), grid, block, 0, stream,
                         (const uint16_t *)logits, ld, v, target, ids, lp, rec);
    else
      hipLaunchKernelGGL((golden_export_kernel<uint16_t, false>), grid, block, 0, stream,
                         (const uint16_t *)logits, ld, v, target, ids, lp, rec);
  }
  return hipGetLastError();
}

CoarseGeom coarse_geom(int64_t n, int64_t v) {
  // ranges of at most 131,072 ids, a multiple of 256, and about 2048 blocks
  // (more, smaller ranges measured slower: each adds a partial state to merge)
  int64_t want = n > 0 ? (2048 + n - 1) / n : 1;
  const int64_t min_splits = (v + 131071) / 131072;
  const int64_t max_splits = (v + 4095) / 4096;
  if (want > max_splits) want = max_splits;
  if (want < min_splits) want = min_splits;
  if (want < 1) want = 1;
  int64_t chunk = (v + want - 1) / want;
  chunk = (chunk + 255) / 256 * 256;
  CoarseGeom g;
  g.chunk = chunk;
  g.splits = (int)((v + chunk - 1) / chunk);
  return g;
}

size_t coarse_state_bytes() { return sizeof(LseState); }

hipError_t launch_coarse_kl(const void *cand, int dtype, int64_t n, int64_t v, int64_t ld,
                            bool aligned, const int32_t *ids, const float *lp, const float *rec,
                            float *kl, void *part_ws, hipStream_t stream) {
  const CoarseGeom g = coarse_geom(n, v);
  LseState *part = static_cast<LseState *>(part_ws);
  const dim3 grid((unsigned)(n * g.splits)), block(GT);
  if (dtype == 0) {
    if (aligned)
      hipLaunchKernelGGL((coarse_partial_kernel<float, 4, 4, true>), grid, block, 0, stream,
                         (const float *)cand, ld, v, g.chunk, g.splits, ids, part);
    else
      hipLaunchKernelGGL((coarse_partial_kernel<float, 4, 4, false>), grid, block, 0, stream,
                         (const float *)cand, ld, v, g.chunk, g.splits, ids, part);
  } else {
    if (aligned)
      hipLaunchKernelGGL((coarse_partial_kernel<uint16_t, 8, 2, true>), grid, block, 0, stream,
                         (const uint16_t *)cand, ld, v, g.chunk, g.splits, ids, part);
    else
      hipLaunchKernelGGL((coarse_partial_kernel<uint16_t, 8, 2, false>), grid, block, 0, stream,
                         (const uint16_t *)cand, ld, v, g.chunk, g.splits, ids, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(coarse_finalize_kernel, dim3((unsigned)((n + 3) / 4)), block, 0, stream, part,
                     g.splits, n, cand, dtype, ld, v, ids, lp, rec, kl);
  return hipGetLastError();
}

}  // namespace kld
